"""Evoformer biased attention on MI355X (gfx950): fused HIP kernels behind a C ABI.

    from evoformer_biased_attention_amd import evoformer_attention
    out = evoformer_attention(Q, K, V, [mask_bias, pair_bias])

The compute path is libevoattn.so (built in-tree by ``build.py``); importing
this package does not load it, the first call does, and fails loudly if it is
missing.
"""


def __getattr__(name):
    # lazy: keep `import evoformer_biased_attention_amd.inputs` free of torch/HIP
    if name in ("evoformer_attention", "DS4Sci_EvoformerAttention", "EvoformerFusedAttention", "attn_fwd",
                "attn_bwd", "workspace_f32_views"):
        from . import attention
        return getattr(attention, name)
    raise AttributeError(name)
