"""GPU parity of the backward (fa_bwd, through the C ABI) against the float64 oracle.

Small ragged shapes compare every element of dQ, dK, dV, with O and lse taken
from the oracle (rounded to their storage types) so that only the backward is
under test; end-to-end cases run the GPU forward first, as a training step
does.  The full-size workloads compare sampled positions (dQ of a query, dK and
dV of a key), which the oracle computes one by one, and check on every head
properties that hold at any size.
"""
import math

import numpy as np
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


def oracle_fwd_stored(q, k, v, causal, scale, dtype):
    """Oracle O rounded to the input type and lse rounded to float32 (what a forward stores)."""
    o, lse = oracle.attention(to_f64(q), to_f64(k), to_f64(v), causal, scale)
    return (torch.from_numpy(o).to(DT[dtype]).contiguous(),
            torch.from_numpy(lse).to(torch.float32).contiguous())


def gpu_bwd(q, k, v, o, lse, dout, causal, scale):
    args = [x.to(DEV) for x in (q, k, v, o, lse, dout)]
    dq, dk, dv = fa.backward(*args, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return dq, dk, dv


def check_all(got, ref, dtype, what):
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        check_grad(to_f64(g), r, dtype, f"{name} {what}")


SMALL_SHAPES = [
    (1, 1, 1),      # one row, one key: dQ = dK = 0, dV = dO
    (1, 2, 31),     # less than one tile
    (2, 1, 64),     # two whole tiles
    (1, 2, 128),    # one block of 128 rows
    (2, 2, 333),    # several blocks, ragged tail
    (1, 3, 520),    # ragged tail of 8 rows
]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_small_shapes_elementwise(dtype, D, causal):
    seed = 3000 + D
    scale = fp32(1 / math.sqrt(D))
    for (B, H, S) in SMALL_SHAPES:
        q, k, v = workloads.make_inputs(B, H, S, D, dtype, seed)
        dout = workloads.make_grad(B, H, S, D, dtype, seed + 7)
        seed += 1
        o, lse = oracle_fwd_stored(q, k, v, causal, scale, dtype)
        got = gpu_bwd(q, k, v, o, lse, dout, causal, scale)
        ref = oracle.attention_bwd(to_f64(q), to_f64(k), to_f64(v), to_f64(dout), causal, scale)
        check_all(got, ref, dtype, f"{dtype} D={D} causal={causal} B,H,S={B},{H},{S}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_end_to_end(dtype, causal):
    """GPU forward, then GPU backward from its O and lse, against the oracle's gradients."""
    for D, (B, H, S) in [(64, (2, 2, 333)), (128, (1, 2, 260)), (32, (1, 1, 700))]:
        q, k, v = workloads.make_inputs(B, H, S, D, dtype, 4000 + S)
        dout = workloads.make_grad(B, H, S, D, dtype, 4100 + S)
        scale = fp32(1 / math.sqrt(D))
        qd, kd, vd, dd = (x.to(DEV) for x in (q, k, v, dout))
        o, lse = fa.forward(qd, kd, vd, causal=causal, scale=scale)
        dq, dk, dv = fa.backward(qd, kd, vd, o, lse, dd, causal=causal, scale=scale)
        torch.cuda.synchronize()
        ref = oracle.attention_bwd(to_f64(q), to_f64(k), to_f64(v), to_f64(dout), causal, scale)
        check_all((dq, dk, dv), ref, dtype, f"end-to-end {dtype} D={D} causal={causal}")


@pytest.mark.parametrize("scale", [1.0, 0.3, 0.01])
def test_bwd_scale_values(scale):
    """Peaked (scale 1) and nearly flat (0.01) softmax rows."""
    B, H, S, D = 1, 2, 300, 64
    q, k, v = workloads.make_inputs(B, H, S, D, "f16", 4200)
    dout = workloads.make_grad(B, H, S, D, "f16", 4201)
    scale = fp32(scale)
    for causal in (False, True):
        o, lse = oracle_fwd_stored(q, k, v, causal, scale, "f16")
        got = gpu_bwd(q, k, v, o, lse, dout, causal, scale)
        ref = oracle.attention_bwd(to_f64(q), to_f64(k), to_f64(v), to_f64(dout), causal, scale)
        check_all(got, ref, "f16", f"scale={scale} causal={causal}")


def test_bwd_single_key_closed_form():
    """S = 1: P = 1, so dV = dO exactly and dQ, dK vanish (dP - D = 0)."""
    q, k, v = workloads.make_inputs(2, 3, 1, 64, "f16", 4300)
    dout = workloads.make_grad(2, 3, 1, 64, "f16", 4301)
    _, lse = oracle.attention(to_f64(q), to_f64(k), to_f64(v), True, 0.125)  # = 0.125 * <q, k>
    lse = torch.from_numpy(lse).to(torch.float32).contiguous()
    dq, dk, dv = gpu_bwd(q, k, v, v.clone(), lse, dout, True, 0.125)
    assert torch.equal(dv.cpu(), dout)
    assert float(dq.abs().max()) <= 1e-3 and float(dk.abs().max()) <= 1e-3


def test_bwd_deterministic():
    q, k, v = workloads.make_inputs(2, 4, 1000, 64, "f16", 4400)
    dout = workloads.make_grad(2, 4, 1000, 64, "f16", 4401)
    qd, kd, vd, dd = (x.to(DEV) for x in (q, k, v, dout))
    o, lse = fa.forward(qd, kd, vd, causal=True)
    a = fa.backward(qd, kd, vd, o, lse, dd, causal=True)
    b = fa.backward(qd, kd, vd, o, lse, dd, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_argument_errors_raise():
    q = torch.zeros((1, 1, 64, 64), dtype=torch.float32, device=DEV)
    lse = torch.zeros((1, 1, 64), dtype=torch.float32, device=DEV)
    with pytest.raises(ValueError):
        fa.backward(q, q, q, q, lse, q)  # fp32 has no backward
    q = torch.zeros((1, 1, 64, 48), dtype=torch.float16, device=DEV)
    with pytest.raises(ValueError):
        fa.backward(q, q, q, q, lse, q)  # head dim 48


def test_bwd_empty_inputs():
    for shape in [(0, 2, 64, 64), (1, 0, 64, 64), (1, 2, 0, 64)]:
        q = torch.zeros(shape, dtype=torch.float16, device=DEV)
        lse = torch.zeros(shape[:3], dtype=torch.float32, device=DEV)
        dq, dk, dv = fa.backward(q, q.clone(), q.clone(), q.clone(), lse, q.clone(), causal=True)
        assert dq.shape == shape and dk.shape == shape and dv.shape == shape


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_d16_two_block_grid_elementwise(dtype, causal):
    """D = 16 on a grid of 256+ dQ workgroups (B=1 H=64 S=1024): the dQ kernel's
    two-query-block instance; every element of dQ, dK, dV against the oracle."""
    B, H, S, D = 1, 64, 1024, 16
    scale = fp32(1 / math.sqrt(D))
    q, k, v = workloads.make_inputs(B, H, S, D, dtype, 8100)
    dout = workloads.make_grad(B, H, S, D, dtype, 8101)
    o, lse = oracle_fwd_stored(q, k, v, causal, scale, dtype)
    got = gpu_bwd(q, k, v, o, lse, dout, causal, scale)
    ref = oracle.attention_bwd(to_f64(q), to_f64(k), to_f64(v), to_f64(dout), causal, scale)
    check_all(got, ref, dtype, f"D=16 B,H,S={B},{H},{S} causal={causal}")


@pytest.mark.parametrize("D", [16, 64])
def test_bwd_window_blocks_without_keys(D):
    """S_q = 2048 queries over S_k = 512 keys with a window (64, 0), causal, B=4
    H=16: whole query blocks of the full-grid dQ kernel have no key tile (they
    must stage nothing and write dQ = 0); every element against the oracle."""
    B, H, Sq, Sk, window = 4, 16, 2048, 512, (64, 0)
    dtype = "f16"
    scale = fp32(1 / math.sqrt(D))
    q, _, _ = workloads.make_inputs(B, H, Sq, D, dtype, 8200 + D)
    _, k, v = workloads.make_inputs(B, H, Sk, D, dtype, 8201 + D)
    dout = workloads.make_grad(B, H, Sq, D, dtype, 8202 + D)
    o, lse = oracle.attention(to_f64(q), to_f64(k), to_f64(v), True, scale, window)
    o = torch.from_numpy(o).to(DT[dtype])
    lse = torch.from_numpy(lse).to(torch.float32)
    args = [x.to(DEV) for x in (q, k, v, o, lse, dout)]
    dq, dk, dv = fa.backward(*args, causal=True, scale=scale, window=window)
    torch.cuda.synchronize()
    ref = oracle.attention_bwd(to_f64(q), to_f64(k), to_f64(v), to_f64(dout), True, scale, window)
    check_all((dq, dk, dv), ref, dtype, f"D={D} Sq={Sq} Sk={Sk} window={window}")
    assert torch.count_nonzero(dq[:, :, Sk + window[0]:]) == 0, "rows without keys must get dQ = 0"


# ----------------------------------------------------------- full-size workloads


def sampled_positions(B, H, S, heads, n_random, seed):
    """Flat positions (b*H + h)*S + t in the given heads: both sides of every
    32/128-row boundary (tile and workgroup edges), the ends, and random ones."""
    rng = np.random.default_rng(seed)
    pos = set()
    for bh in heads:
        base = bh * S
        for t in (0, 1, S - 2, S - 1):
            pos.add(base + t)
        for blk in (32, 128):
            for edge in range(blk, S, blk * max(1, S // (blk * 6))):
                pos.update({base + edge - 1, base + edge})
        pos.update(int(base + x) for x in rng.integers(0, S, size=n_random))
    return np.array(sorted(pos), dtype=np.int64)


def check_properties(q, dout, dq, dk, dv, dtype, what):
    """On every head: finite values, sum_j dV_j = sum_i dO_i, sum_j dK_j = 0
    (normwise against the sums of magnitudes, with the input-type roundings)."""
    for t in (dq, dk, dv):
        assert torch.isfinite(t.float()).all(), f"{what}: non-finite gradient"
    u = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}[dtype]
    dv64, dk64 = dv.double(), dk.double()
    mass = (dv64.sum(2) - dout.to(dv.device).double().sum(2)).abs()
    scale_v = dv64.abs().sum(2) + 1.0
    assert float((mass / scale_v).max()) <= 8 * u, f"{what}: sum_j dV_j != sum_i dO_i"
    shift = dk64.sum(2).abs() / (dk64.abs().sum(2) + 1e-30)
    assert float(shift.max()) <= 16 * u, f"{what}: sum_j dK_j != 0"


@pytest.mark.parametrize("name", ["multihead_causal", "batch_f16"])
def test_bwd_workload_sampled(name):
    w = workloads.BY_NAME[name]
    q, k, v = workloads.workload_inputs(w)
    dout = workloads.make_grad(w.B, w.H, w.S, w.D, w.dtype, w.seed + 1000)
    qd, kd, vd, dd = (x.to(DEV) for x in (q, k, v, dout))
    BH = w.B * w.H
    heads = sorted({0, BH // 2, BH - 1})
    pos = sampled_positions(w.B, w.H, w.S, heads, n_random=96, seed=w.seed)
    for causal in w.causal:
        o, lse = fa.forward(qd, kd, vd, causal=causal, scale=w.scale)
        dq, dk, dv = fa.backward(qd, kd, vd, o, lse, dd, causal=causal, scale=w.scale)
        torch.cuda.synchronize()
        ref = oracle.attention_bwd_rows(to_f64(q), to_f64(k), to_f64(v), to_f64(dout), causal, w.scale, pos)
        for nm, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
            check_grad(to_f64(g).reshape(-1, w.D)[pos], r, w.dtype, f"{nm} {name} causal={causal}")
        check_properties(q, dout, dq, dk, dv, w.dtype, f"{name} causal={causal}")


def test_bwd_long_seq_sampled():
    """B=8 H=1 S=16384 D=128 bf16 causal: dQ of sampled query rows and dK, dV of
    sampled key rows in three heads (both sides of tile and workgroup edges, the
    ends, random positions) against the oracle, plus the invariants on every head."""
    w = workloads.BY_NAME["long_seq_bf16"]
    q, k, v = workloads.workload_inputs(w)
    dout = workloads.make_grad(w.B, w.H, w.S, w.D, w.dtype, w.seed + 1000)
    qd, kd, vd, dd = (x.to(DEV) for x in (q, k, v, dout))
    o, lse = fa.forward(qd, kd, vd, causal=True, scale=w.scale)
    dq, dk, dv = fa.backward(qd, kd, vd, o, lse, dd, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    heads = [0, 3, w.B * w.H - 1]
    pos = sampled_positions(w.B, w.H, w.S, heads, n_random=24, seed=w.seed)
    ref = oracle.attention_bwd_rows(to_f64(q), to_f64(k), to_f64(v), to_f64(dout), True, w.scale, pos)
    for nm, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        err = check_grad(to_f64(g).reshape(-1, w.D)[pos], r, w.dtype, f"{nm} long_seq_bf16")
        print(f"\nparity long_seq_bf16 backward {nm} at {len(pos)} positions: normwise {err:.3e}", flush=True)
    check_properties(q, dout, dq, dk, dv, w.dtype, "long_seq_bf16")
