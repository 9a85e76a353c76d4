"""Write worked_example.json: a 2-query, 2-key problem solved by hand.

Nothing here calls the oracle or the GPU path; every expected value is the
closed form written below.  B = N = H = D = 1 (so scale = 1), L = 2.

    q = [1, 0], k = [1, 0], v = [4, 8], dO = [2, 1]
    mask = [0, 1 + ln 3], pair = [[0, 0], [1, -ln 3]]

Row 0: S = [1, 1 + ln 3] -> P = [1/4, 3/4], O = 7, lse = 1 + ln 4.
Row 1: S = [1, 1]        -> P = [1/2, 1/2], O = 6, lse = 1 + ln 2.
dP = dO_i v_j = [[8, 16], [4, 8]]; delta = [14, 6];
dS = P (dP - delta) = [[-1.5, 1.5], [-1, 1]];
dV = P^T dO = [1, 2]; dQ = dS k = [-1.5, -1]; dK = dS^T q = [-1.5, 1.5];
dmask = column sums of dS = [-2.5, 2.5]; dpair = dS.
"""
import json
import math
import os

ln2, ln3, ln4 = math.log(2.0), math.log(3.0), math.log(4.0)
ex = {
    "what": "hand-derived closed form, see make_worked_example.py",
    "q": [[[[[1.0]], [[0.0]]]]],
    "k": [[[[[1.0]], [[0.0]]]]],
    "v": [[[[[4.0]], [[8.0]]]]],
    "dout": [[[[[2.0]], [[1.0]]]]],
    "mask_bias": [[[[[0.0, 1.0 + ln3]]]]],
    "pair_bias": [[[[[0.0, 0.0], [1.0, -ln3]]]]],
    "expect_out": [7.0, 6.0],
    "expect_lse": [1.0 + ln4, 1.0 + ln2],
    "expect_dv": [1.0, 2.0],
    "expect_dq": [-1.5, -1.0],
    "expect_dk": [-1.5, 1.5],
    "expect_dmask": [-2.5, 2.5],
    "expect_dpair": [-1.5, 1.5, -1.0, 1.0],
}
with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "worked_example.json"), "w") as f:
    json.dump(ex, f, indent=1)
