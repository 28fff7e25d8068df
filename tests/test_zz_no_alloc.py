"""fa_bwd_noalloc (the backward with the library's static D workspace, for
callers that cannot allocate) against fa_bwd_ex (the same kernels with a
caller-provided workspace), through the C ABI: bit-identical dQ, dK, dV on two
calls in a row, the second on a smaller problem, so that the static array's
contents left by the first call cannot leak into the second.  The workspace
limit is refused before any launch."""
import math

import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU visible", allow_module_level=True)

import exact_tiled_attention_06_amd as fa  # noqa: E402

fa.library()  # fails loudly when libfa.so is missing

DEV = "cuda:0"


def fp32(x):
    return float(torch.tensor(x, dtype=torch.float32))


def run_both(B, H, Hkv, Sq, Sk, D, dtype, causal, window, seed):
    q, _, _ = workloads.make_inputs(B, H, Sq, D, dtype, seed)
    _, k, v = workloads.make_inputs(B, Hkv, Sk, D, dtype, seed + 1)
    dout = workloads.make_grad(B, H, Sq, D, dtype, seed + 2)
    q, k, v, dout = (x.to(DEV) for x in (q, k, v, dout))
    scale = fp32(1 / math.sqrt(D))
    o, lse = fa.forward(q, k, v, causal=causal, scale=scale, window=window)
    code = fa.DTYPE_CODES[q.dtype]
    stream = torch.cuda.current_stream().cuda_stream
    wl, wr = window
    outs = []
    for noalloc in (False, True):
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ptrs = [t.data_ptr() for t in (q, k, v, o, dout, lse, dq, dk, dv)]
        if noalloc:
            st = fa.fa_bwd_noalloc(*ptrs, B, H, Hkv, Sq, Sk, D, int(causal), wl, wr, scale, code, stream)
        else:
            delta = torch.empty((B, H, Sq), dtype=torch.float32, device=DEV)
            st = fa.fa_bwd_ex(*ptrs, delta.data_ptr(), B, H, Hkv, Sq, Sk, D, int(causal), wl, wr, scale, code,
                              stream)
        fa.check(st)
        outs.append((dq, dk, dv))
    torch.cuda.synchronize()
    return outs


def assert_identical(outs, what):
    for name, a, b in zip(("dQ", "dK", "dV"), outs[0], outs[1]):
        assert torch.equal(a, b), f"{name} of fa_bwd_noalloc differs from fa_bwd_ex ({what})"


def test_noalloc_matches_workspace_entry_twice():
    # first a large problem (the multi-head causal shape: 262,144 rows of D),
    # then a smaller one with grouped heads, S_q != S_k and a window
    outs = run_both(4, 16, 16, 4096, 4096, 64, "f16", True, (-1, -1), 8300)
    assert_identical(outs, "B=4 H=16 S=4096 D=64 causal")
    outs = run_both(2, 4, 2, 700, 300, 128, "bf16", False, (50, 20), 8310)
    assert_identical(outs, "B=2 H=4 H_kv=2 S_q=700 S_k=300 D=128 window (50, 20)")


def test_noalloc_rejects_oversized_problem():
    # 4,194,305 rows of D: refused with FA_ERR_WORKSPACE before any HIP call
    # (the pointers are never dereferenced)
    P = 1 << 20
    st = fa.fa_bwd_noalloc(P, 2 * P, 3 * P, 4 * P, 5 * P, 6 * P, 7 * P, 8 * P, 9 * P, 1, 1, 1, 4194305, 64, 64,
                           0, -1, -1, 0.125, fa.FA_DTYPE_F16, 0)
    assert st == fa.FA_ERR_WORKSPACE
    with pytest.raises(ValueError):
        fa.check(st)
