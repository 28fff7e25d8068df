"""GPU parity of grouped K/V heads (GQA / MQA) and sliding windows
(fa_fwd_ex, fa_bwd_ex through the C ABI) against the float64 oracle.

window = (left, right): query i attends to keys i - left .. i + right (and
none past i when causal); -1 leaves a side unlimited ("Inside
FlashAttention", section 6.1).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_util import DT, check_grad, check_lse, check_o, to_f64

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU visible", allow_module_level=True)

import exact_tiled_attention_06_amd as fa  # noqa: E402

fa.library()  # fails loudly when libfa.so is missing

DEV = "cuda:0"


def fp32(x):
    return float(torch.tensor(x, dtype=torch.float32))


def inputs(B, H, Hkv, S, D, dtype, seed):
    q, _, _ = workloads.make_inputs(B, H, S, D, dtype, seed)
    _, k, v = workloads.make_inputs(B, Hkv, S, D, dtype, seed + 1)
    dout = workloads.make_grad(B, H, S, D, dtype, seed + 2)
    return q, k, v, dout


def gpu_fwd(q, k, v, causal, scale, window):
    o, lse = fa.forward(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=scale, window=window)
    torch.cuda.synchronize()
    return o, lse


WINDOWS = [(0, 0), (5, -1), (40, 0), (17, 33), (-1, 9), (100, 100), (1, 1)]
HEADS = [(4, 4), (4, 2), (4, 1), (6, 3)]


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_window_and_groups_elementwise(dtype, D, causal):
    seed = 6000 + D
    scale = fp32(1 / math.sqrt(D))
    for S, window, (H, Hkv) in [(31, (5, -1), (4, 2)), (200, (40, 0), (4, 1)), (333, (17, 33), (6, 3)),
                                (130, (0, 0), (4, 4)), (257, (-1, 9), (4, 2)), (96, (100, 100), (2, 1)),
                                (333, (-1, -1), (6, 2))]:
        q, k, v, _ = inputs(1, H, Hkv, S, D, dtype, seed)
        seed += 3
        o, lse = gpu_fwd(q, k, v, causal, scale, window)
        o_ref, l_ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v), causal, scale, window)
        what = f"{dtype} D={D} causal={causal} S={S} window={window} H,Hkv={H},{Hkv}"
        check_o(to_f64(o), o_ref, dtype, f"O {what}")
        check_lse(to_f64(lse), l_ref, f"lse {what}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_window_and_groups_elementwise(dtype, D, causal):
    """O and lse from the oracle (as stored), gradients against the oracle's."""
    seed = 7000 + D
    scale = fp32(1 / math.sqrt(D))
    for S, window, (H, Hkv) in [(31, (5, -1), (4, 2)), (200, (40, 0), (4, 1)), (333, (17, 33), (6, 3)),
                                (130, (0, 0), (4, 4)), (257, (-1, 9), (4, 2)), (300, (-1, -1), (4, 1))]:
        q, k, v, dout = inputs(1, H, Hkv, S, D, dtype, seed)
        seed += 3
        o, lse = oracle.attention(to_f64(q), to_f64(k), to_f64(v), causal, scale, window)
        o = torch.from_numpy(o).to(DT[dtype])
        lse = torch.from_numpy(lse).to(torch.float32)
        args = [x.to(DEV) for x in (q, k, v, o, lse, dout)]
        dq, dk, dv = fa.backward(*args, causal=causal, scale=scale, window=window)
        torch.cuda.synchronize()
        ref = oracle.attention_bwd(to_f64(q), to_f64(k), to_f64(v), to_f64(dout), causal, scale, window)
        what = f"{dtype} D={D} causal={causal} S={S} window={window} H,Hkv={H},{Hkv}"
        for nm, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
            check_grad(to_f64(g), r, dtype, f"{nm} {what}")


def test_ex_defaults_match_plain_entries_bitwise():
    """fa_fwd_ex / fa_bwd_ex with H_kv = H and no window (or a window wider than S)
    launch exactly what fa_fwd / fa_bwd launch."""
    q, k, v, dout = inputs(2, 4, 4, 1000, 64, "f16", 8000)
    qd, kd, vd, dd = (x.to(DEV) for x in (q, k, v, dout))
    o1, l1 = fa.forward(qd, kd, vd, causal=True)
    o2, l2 = fa.forward(qd, kd, vd, causal=True, window=(5000, 1000))
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    g1 = fa.backward(qd, kd, vd, o1, l1, dd, causal=True)
    g2 = fa.backward(qd, kd, vd, o1, l1, dd, causal=True, window=(-1, 1000))
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_gqa_equals_replicated_heads():
    """Grouped heads on the GPU equal the GPU's own multi-head result on K/V
    replicated per query head (forward bitwise; dK, dV the group sums)."""
    B, H, Hkv, S, D = 2, 8, 2, 512, 64
    q, k, v, dout = inputs(B, H, Hkv, S, D, "bf16", 8100)
    qd, kd, vd, dd = (x.to(DEV) for x in (q, k, v, dout))
    kr, vr = (x.repeat_interleave(H // Hkv, dim=1).contiguous() for x in (kd, vd))
    for causal in (False, True):
        o1, l1 = fa.forward(qd, kd, vd, causal=causal)
        o2, l2 = fa.forward(qd, kr, vr, causal=causal)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        dq1, dk1, dv1 = fa.backward(qd, kd, vd, o1, l1, dd, causal=causal)
        dq2, dk2, dv2 = fa.backward(qd, kr, vr, o2, l2, dd, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(dq1, dq2)
        for g, gr in ((dk1, dk2), (dv1, dv2)):
            summed = gr.float().reshape(B, Hkv, H // Hkv, S, D).sum(2)
            check_grad(to_f64(g), to_f64(summed), "bf16", "GQA dK/dV vs replicated group sums")


def test_window_full_size_sampled():
    """B=4 H=16 H_kv=4 S=4096 D=64 fp16, causal with a 512-key left window:
    sampled rows of O and lse, sampled dQ / dK / dV positions."""
    B, H, Hkv, S, D = 4, 16, 4, 4096, 64
    window = (512, 0)
    q, k, v, dout = inputs(B, H, Hkv, S, D, "f16", 8200)
    scale = fp32(1 / math.sqrt(D))
    qd, kd, vd, dd = (x.to(DEV) for x in (q, k, v, dout))
    o, lse = fa.forward(qd, kd, vd, causal=True, scale=scale, window=window)
    dq, dk, dv = fa.backward(qd, kd, vd, o, lse, dd, causal=True, scale=scale, window=window)
    torch.cuda.synchronize()
    rng = np.random.default_rng(8200)
    heads = [0, 21, B * H - 1]
    rows = np.array(sorted({bh * S + t for bh in heads for t in
                            [0, 1, 511, 512, 513, 1023, 1024, 4095] + list(rng.integers(0, S, 48))}), dtype=np.int64)
    o_ref, l_ref = oracle.attention_rows(to_f64(q), to_f64(k), to_f64(v), True, scale, rows, window)
    check_o(to_f64(o).reshape(-1, D)[rows], o_ref, "f16", "O windowed GQA")
    check_lse(to_f64(lse).reshape(-1)[rows], l_ref, "lse windowed GQA")
    kvheads = [0, 7, B * Hkv - 1]
    krows = np.array(sorted({kh * S + t for kh in kvheads for t in
                             [0, 31, 32, 3583, 3584, 4095] + list(rng.integers(0, S, 32))}), dtype=np.int64)
    rq, rk, rv = oracle.attention_bwd_rows(to_f64(q), to_f64(k), to_f64(v), to_f64(dout), True, scale, rows,
                                           krows, window)
    check_grad(to_f64(dq).reshape(-1, D)[rows], rq, "f16", "dQ windowed GQA")
    check_grad(to_f64(dk).reshape(-1, D)[krows], rk, "f16", "dK windowed GQA")
    check_grad(to_f64(dv).reshape(-1, D)[krows], rv, "f16", "dV windowed GQA")
