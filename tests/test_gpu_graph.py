"""The C-ABI calls captured in a HIP graph give the eager result on every replay.

The library enqueues only kernels on the caller's stream (no memsets, no
allocations), so a captured fwd+bwd step must replay to the same bits as the
eager call; replays are interleaved with eager work and synchronisation.
"""
import numpy as np
import pytest
import torch

from evoformer_biased_attention_amd import inputs as I
from tests.helpers import to_device

pytestmark = pytest.mark.gpu


CASES = [
    (I.CONFIGS["tiny_row"], None),
    (I.CONFIGS["msa_row"], None),
    # rows longer than one key tile, planned in chunks (a 24 MiB partial
    # budget): bwd_q3 and bwd_fin launched once per chunk
    (I.custom("graph_chunked_l640_d64_bf16", 2, 24, 640, 2, 64, "bf16", 0.05, 1.0, 51), 24 << 20),
    # rows longer than one key tile without a pair bias: bwd_q3 walks every
    # key tile of its slices (no partials)
    (I.custom("graph_l600_nopair_bf16", 1, 16, 600, 2, 32, "bf16", 0.05, None, 53), None),
]


@pytest.mark.parametrize("cfg,budget", CASES, ids=[c.name for c, _ in CASES])
def test_graph_replay_matches_eager(cfg, budget):
    from evoformer_biased_attention_amd.attention import attn_bwd, attn_fwd

    print(f"case graph replay {cfg.name} shape={cfg.shape} partial budget={budget}", flush=True)
    bits = I.make_inputs(cfg)
    q, k, v, m, p, do = (to_device(bits[n], cfg.dtype) for n in ("q", "k", "v", "mask_bias", "pair_bias", "dout"))
    out_e, lse_e = attn_fwd(q, k, v, m, p)
    g_e = attn_bwd(q, k, v, m, p, out_e, lse_e, do, partial_budget=budget)
    torch.cuda.synchronize()
    # the outputs the call has (dmask, dpair are None without their bias)
    ref = [t.clone() for t in (out_e, lse_e, g_e["dq"], g_e["dk"], g_e["dv"], g_e["dmask"], g_e["dpair"])
           if t is not None]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        attn_fwd(q, k, v, m, p)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out_g, lse_g = attn_fwd(q, k, v, m, p)
        g_g = attn_bwd(q, k, v, m, p, out_g, lse_g, do, partial_budget=budget)
    got = [t for t in (out_g, lse_g, g_g["dq"], g_g["dk"], g_g["dv"], g_g["dmask"], g_g["dpair"]) if t is not None]
    assert len(got) == len(ref)
    for rep in range(4):
        graph.replay()
        torch.cuda.synchronize()
        for a_, b_ in zip(got, ref):
            assert torch.equal(a_, b_), f"replay {rep} differs"
        # eager work between replays
        attn_fwd(q, k, v, m, p)
        torch.cuda.synchronize()
