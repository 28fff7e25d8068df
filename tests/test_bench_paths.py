"""GPU checks of bench.py's own backward call on small problems.

The backward timing calls the C ABI directly; with grouped K/V heads it must
hand the library the K/V head count of k (an entry that takes H_kv = H would
address K/V heads past the allocation), size dK and dV like k, and pass the
workload's window.  Its gradients must equal, bit for bit, those of the
validated binding on the same inputs (the same kernels on the same data).
"""
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU visible", allow_module_level=True)

import bench  # noqa: E402
import exact_tiled_attention_06_amd as fa  # noqa: E402

fa.library()  # fails loudly when libfa.so is missing


@pytest.mark.parametrize("hkv,window", [(2, (-1, -1)), (1, (64, 0)), (8, (-1, -1))])
def test_backward_call_matches_binding(hkv, window):
    w = workloads.Workload("bench_path_check", 2, 8, 384, 64, "f16", (True,), 4242, hkv=hkv, window=window)
    print(f"\nbench backward call: B=2 H=8 H_kv={w.kv_heads} S=384 D=64 window={window}", flush=True)
    call, (dq_b, dk_b, dv_b) = bench.backward_call(fa, torch, w, True)
    fa.check(call())
    torch.cuda.synchronize()
    q, k, v = (x.to("cuda:0") for x in workloads.workload_inputs(w))
    assert k.shape[1] == w.kv_heads and dk_b.shape == k.shape and dv_b.shape == v.shape
    dout = workloads.make_grad(w.B, w.H, w.S, w.D, w.dtype, w.seed + 1000).to("cuda:0")
    win = None if window == (-1, -1) else window
    o, lse = fa.forward(q, k, v, causal=True, scale=w.scale, window=win)
    dq, dk, dv = fa.backward(q, k, v, o, lse, dout, causal=True, scale=w.scale, window=win)
    torch.cuda.synchronize()
    assert torch.equal(dq_b, dq) and torch.equal(dk_b, dk) and torch.equal(dv_b, dv)
    # and the timing loop runs on the same call
    wall, avg_ms, (settle_ms, settle_n) = bench.time_backward(fa, torch, w, True, 3, 1, settle_ms=5.0)
    assert wall > 0 and avg_ms > 0 and settle_ms >= 5.0 and settle_n >= 10
