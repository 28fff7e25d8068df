"""GPU parity of the backward's thin-grid paths against the float64 oracle.

With few batch*head pairs the library changes the backward's work split (the
grid sizes below are what selects each path; every case here is thin):
  - dQ kernel: one 32-query block per wave, and two wave groups per query
    block that split its key tiles and add their fp32 partial dQ through LDS
    (D = 32, 64, 128);
  - dK/dV kernel: two wave groups per key block that split its query steps
    (query head and tile) and add their fp32 partial dK, dV (D = 32, 64).
The shapes drive the split's edge cases: one key tile (the second dQ group has
none), one query step (the second dK/dV group has none), an odd number of
steps, steps that cross query heads (grouped heads), ragged tails, windows
that empty whole tiles, and S_q != S_k.  Every element of dQ, dK, dV is
compared with the oracle's gradients on the same stored inputs (O and lse from
the oracle as stored).
"""
import math

import pytest
import torch

import oracle
import workloads
from parity_util import DT, check_grad, to_f64

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU visible", allow_module_level=True)

import exact_tiled_attention_06_amd as fa  # noqa: E402

fa.library()  # fails loudly when libfa.so is missing

DEV = "cuda:0"


def fp32(x):
    return float(torch.tensor(x, dtype=torch.float32))


# (B, H, H_kv, S_q, S_k, window)
CASES = [
    (1, 1, 1, 20, 20, (-1, -1)),      # one tile each way: second groups idle
    (1, 2, 1, 33, 40, (-1, -1)),      # two query heads per K/V head, ragged
    (1, 3, 1, 97, 97, (-1, -1)),      # three heads: step split crosses heads, odd count
    (2, 2, 2, 161, 161, (-1, -1)),    # five tiles: odd split
    (1, 4, 2, 300, 700, (-1, -1)),    # S_q < S_k
    (1, 2, 2, 700, 300, (-1, -1)),    # S_q > S_k
    (1, 2, 1, 400, 400, (70, 0)),     # window: whole tiles outside
    (1, 2, 2, 260, 260, (30, 45)),    # two-sided window
]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_thin_grid_bwd_elementwise(dtype, D, causal):
    scale = fp32(1 / math.sqrt(D))
    seed = 9700 + D + (100 if causal else 0)
    for (B, H, Hkv, Sq, Sk, window) in CASES:
        q, _, _ = workloads.make_inputs(B, H, Sq, D, dtype, seed)
        _, k, v = workloads.make_inputs(B, Hkv, Sk, D, dtype, seed + 1)
        dout = workloads.make_grad(B, H, Sq, D, dtype, seed + 2)
        seed += 3
        o, lse = oracle.attention(to_f64(q), to_f64(k), to_f64(v), causal, scale, window)
        o = torch.from_numpy(o).to(DT[dtype])
        lse = torch.from_numpy(lse).to(torch.float32)
        args = [x.to(DEV) for x in (q, k, v, o, lse, dout)]
        dq, dk, dv = fa.backward(*args, causal=causal, scale=scale, window=window)
        torch.cuda.synchronize()
        ref = oracle.attention_bwd(to_f64(q), to_f64(k), to_f64(v), to_f64(dout), causal, scale, window)
        what = f"{dtype} D={D} causal={causal} B,H,Hkv={B},{H},{Hkv} Sq,Sk={Sq},{Sk} window={window}"
        for nm, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
            check_grad(to_f64(g), r, dtype, f"{nm} {what}")
