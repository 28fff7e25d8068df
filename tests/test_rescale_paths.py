"""GPU parity with scores that grow along the keys, on shapes that reach every
forward kernel's rescale code.

The kernels keep a lazy reference maximum: a tile is exponentiated against
the running m, and only when a row's partial sum leaves range is m moved to
the new maximum and O and l multiplied by exp2(m_old - m_new) ("Inside
FlashAttention", section 2.3; "T5 讲解", section ④, the online softmax's
rescale).  Random normal inputs rarely take that path.  Here positive queries
meet keys scaled up along the sequence (0.2 to 3.0), so a row's maximum grows
by 40 to 65 in log2 units over the keys and most rows leave range one to four
times (a CPU replay of the rule on these inputs), in the middle of the steady
loop as well as on the edge tiles; a wave rescales when any of its rows does.  The shapes
are chosen for the kernel they run on; every element of O and lse is compared
with the float64 oracle.
"""
import math

import pytest
import torch

import oracle
import workloads
from parity_util import DT, check_lse, check_o, to_f64

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU visible", allow_module_level=True)

import exact_tiled_attention_06_amd as fa  # noqa: E402

fa.library()  # fails loudly when libfa.so is missing

DEV = "cuda:0"


def fp32(x):
    return float(torch.tensor(x, dtype=torch.float32))


def growing(B, H, S, D, dtype, seed):
    q, k, v = workloads.make_inputs(B, H, S, D, dtype, seed)
    ramp = torch.linspace(0.2, 3.0, S).reshape(1, 1, S, 1)
    k = (k.float().abs() * ramp).to(DT[dtype])
    q = (q.float().abs() + 0.5).to(DT[dtype])
    return q, k, v


# (B, H, S, D, dtype, kernel the shape runs on)
CASES = [
    (4, 16, 2000, 64, "f16", "two-block kernel (fa_fwd_ex), key split (forward)"),
    (4, 16, 2048, 32, "bf16", "two-block kernel (fa_fwd_ex), key split (forward)"),
    (4, 16, 1000, 16, "f16", "one-block kernel, 128-row workgroups; key split (forward)"),
    (4, 16, 2000, 128, "bf16", "one-block kernel, 8-wave workgroups"),
    (8, 1, 4096, 128, "f16", "one-block kernel, 4-wave workgroups; key split (forward)"),
    (8, 1, 3000, 64, "f16", "thin-grid kernel, 64-row blocks, half-step loop"),
    (8, 1, 1500, 64, "f16", "thin-grid kernel, 32-row blocks, plain loop"),
    (2, 1, 1024, 16, "f16", "thin-grid kernel, 32-row blocks, one k-step (D = 16)"),
    (8, 1, 1024, 128, "bf16", "thin-grid kernel, 32-row blocks, accumulators in AGPRs (D = 128)"),
    (1, 2, 300, 64, "f32", "fp32 matrix-core kernel"),
]


@pytest.mark.parametrize("B,H,S,D,dtype,kernel", CASES)
@pytest.mark.parametrize("causal", [False, True])
def test_growing_scores_every_kernel(B, H, S, D, dtype, kernel, causal):
    what = f"{dtype} B={B} H={H} S={S} D={D} causal={causal} ({kernel})"
    print(f"\ngrowing scores: {what}", flush=True)
    q, k, v = growing(B, H, S, D, dtype, 3100 + D + S)
    scale = fp32(1 / math.sqrt(D))
    o_ref, l_ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v), causal, scale)
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    # through the binding (with the workspace of the key split where it applies)
    o, lse = fa.forward(qd, kd, vd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    check_o(to_f64(o), o_ref, dtype, f"O forward {what}")
    check_lse(to_f64(lse), l_ref, f"lse forward {what}")
    # and without a workspace (the unsplit kernel)
    o2, l2 = torch.empty_like(qd), torch.empty_like(lse)
    fa.check(fa.fa_fwd_ex(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o2.data_ptr(), l2.data_ptr(), B, H, H, S, S,
                          D, int(causal), -1, -1, scale, fa.DTYPE_CODES[q.dtype],
                          torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    check_o(to_f64(o2), o_ref, dtype, f"O fa_fwd_ex {what}")
    check_lse(to_f64(l2), l_ref, f"lse fa_fwd_ex {what}")


@pytest.mark.parametrize("D,window", [(64, (300, 0)), (128, (200, 50)), (32, (-1, 100))])
def test_growing_scores_window_kernels(D, window):
    """The window kernels (two-block at D = 32, 64; plain loop at D = 128) on
    a grid of 512+ workgroups."""
    B, H, S, dtype = 4, 16, 2048, "f16"
    print(f"\ngrowing scores, window {window}: B={B} H={H} S={S} D={D}", flush=True)
    q, k, v = growing(B, H, S, D, dtype, 3300 + D)
    scale = fp32(1 / math.sqrt(D))
    o_ref, l_ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v), True, scale, window)
    o, lse = fa.forward(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, scale=scale, window=window)
    torch.cuda.synchronize()
    check_o(to_f64(o), o_ref, dtype, f"O window {window} D={D}")
    check_lse(to_f64(lse), l_ref, f"lse window {window} D={D}")
