"""GPU parity of queries and keys of different length (S_q != S_k; fa_fwd_ex,
fa_bwd_ex through the C ABI) against the float64 oracle.

Query i and key j sit at positions i and j: keys at or past S_k do not exist
and causal masking compares the positions, so query i sees keys
0..min(i, S_k - 1) (the CS336 write-up's forward kernel, its causal-mask and
N_QUERIES / N_KEYS tail sections).  A row that a window leaves with no key
has O = 0 and lse = -inf.
"""
import itertools
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


def rect_inputs(B, H, Hkv, Sq, Sk, D, dtype, seed):
    q, _, _ = workloads.make_inputs(B, H, Sq, D, dtype, seed)
    _, k, v = workloads.make_inputs(B, Hkv, Sk, D, dtype, seed + 1)
    dout = workloads.make_grad(B, H, Sq, D, dtype, seed + 2)
    return q, k, v, dout


def gpu_fwd(q, k, v, causal, scale, window=None):
    o, lse = fa.forward(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=scale, window=window)
    torch.cuda.synchronize()
    return o, lse


def check_rows(o, lse, o_ref, l_ref, dtype, what):
    """Rows the oracle leaves without a key must be O = 0, lse = -inf exactly;
    the others within the usual tolerances."""
    o, lse = to_f64(o), to_f64(lse)
    empty = np.isneginf(l_ref)
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: rows without keys differ"
    assert np.all(o[empty] == 0.0), f"{what}: O of a row without keys must be 0"
    check_o(o[~empty], o_ref[~empty], dtype, f"O {what}")
    check_lse(lse[~empty], l_ref[~empty], f"lse {what}")


# (S_q, S_k): longer and shorter key runs, ragged tails, a single query or key
SHAPES = [(300, 1000), (1000, 300), (77, 129), (129, 77), (512, 64), (64, 512), (1, 200), (200, 1), (33, 2049)]
HEADS = [(4, 4), (4, 2), (4, 1), (6, 3)]


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_rect_elementwise(dtype, D, causal):
    seed = 9000 + D
    scale = fp32(1 / math.sqrt(D))
    for (Sq, Sk), (H, Hkv) in zip(SHAPES, itertools.cycle(HEADS)):
        q, k, v, _ = rect_inputs(1, H, Hkv, Sq, Sk, D, dtype, seed)
        seed += 3
        o, lse = gpu_fwd(q, k, v, causal, scale)
        o_ref, l_ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v), causal, scale)
        what = f"{dtype} D={D} causal={causal} Sq={Sq} Sk={Sk} H,Hkv={H},{Hkv}"
        check_o(to_f64(o), o_ref, dtype, f"O {what}")
        check_lse(to_f64(lse), l_ref, f"lse {what}")


RECT_WINDOWS = [(700, 300, (50, 0)), (300, 700, (20, 40)), (450, 130, (0, 0)), (130, 450, (-1, 5)),
                (600, 96, (60, 10))]


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_rect_window_empty_rows(dtype, D, causal):
    """Windows with S_q > S_k leave rows without keys (O = 0, lse = -inf)."""
    seed = 9100 + D
    scale = fp32(1 / math.sqrt(D))
    for Sq, Sk, window in RECT_WINDOWS:
        q, k, v, _ = rect_inputs(1, 4, 2, Sq, Sk, D, dtype, seed)
        seed += 3
        o, lse = gpu_fwd(q, k, v, causal, scale, window)
        o_ref, l_ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v), causal, scale, window)
        check_rows(o, lse, o_ref, l_ref, dtype, f"{dtype} D={D} causal={causal} Sq={Sq} Sk={Sk} window={window}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_rect_elementwise(dtype, D, causal):
    """O and lse from the oracle (as stored; -inf for rows without keys),
    gradients against the oracle's: keys no query sees get dK = dV = 0."""
    seed = 9200 + D
    scale = fp32(1 / math.sqrt(D))
    cases = [(300, 1000, (-1, -1)), (1000, 300, (-1, -1)), (77, 129, (-1, -1)), (64, 512, (-1, -1)),
             (700, 300, (50, 0)), (300, 700, (20, 40)), (600, 96, (60, 10))]
    for (Sq, Sk, window), (H, Hkv) in zip(cases, itertools.cycle(HEADS)):
        q, k, v, dout = rect_inputs(1, H, Hkv, Sq, Sk, D, dtype, seed)
        seed += 3
        o, lse = oracle.attention(to_f64(q), to_f64(k), to_f64(v), causal, scale, window)
        o = torch.from_numpy(o).to(DT[dtype])
        lse = torch.from_numpy(lse).to(torch.float32)
        args = [x.to(DEV) for x in (q, k, v, o, lse, dout)]
        dq, dk, dv = fa.backward(*args, causal=causal, scale=scale, window=window)
        torch.cuda.synchronize()
        ref = oracle.attention_bwd(to_f64(q), to_f64(k), to_f64(v), to_f64(dout), causal, scale, window)
        what = f"{dtype} D={D} causal={causal} Sq={Sq} Sk={Sk} window={window} H,Hkv={H},{Hkv}"
        for nm, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
            check_grad(to_f64(g), r, dtype, f"{nm} {what}")


@pytest.mark.parametrize("D,dtype", [(64, "f16"), (32, "f16"), (128, "bf16"), (16, "f16")])
def test_rect_large_grid_sampled(D, dtype):
    """Grids of 512+ workgroups (the two-block and large-tile kernels): B=4 H=16
    H_kv=4, S_q = 3000, S_k = 5000 and the reverse, causal and not; sampled rows
    of O, lse, dQ and key rows of dK, dV."""
    B, H, Hkv = 4, 16, 4
    scale = fp32(1 / math.sqrt(D))
    rng = np.random.default_rng(9300 + D)
    for (Sq, Sk), causal in itertools.product([(3000, 5000), (5000, 3000)], [True, False]):
        q, k, v, dout = rect_inputs(B, H, Hkv, Sq, Sk, D, dtype, 9300 + D + Sq)
        qd, kd, vd, dd = (x.to(DEV) for x in (q, k, v, dout))
        o, lse = fa.forward(qd, kd, vd, causal=causal, scale=scale)
        what = f"{dtype} D={D} causal={causal} Sq={Sq} Sk={Sk}"
        heads = [0, 13, B * H - 1]
        rows = np.array(sorted({bh * Sq + t for bh in heads for t in
                                [0, 1, Sq - 1, min(Sq, Sk) - 1, min(Sq, Sk) % Sq] +
                                list(rng.integers(0, Sq, 24))}), dtype=np.int64)
        o_ref, l_ref = oracle.attention_rows(to_f64(q), to_f64(k), to_f64(v), causal, scale, rows)
        check_o(to_f64(o).reshape(-1, D)[rows], o_ref, dtype, f"O {what}")
        check_lse(to_f64(lse).reshape(-1)[rows], l_ref, f"lse {what}")
        if dtype == "f32":
            continue
        dq, dk, dv = fa.backward(qd, kd, vd, o, lse, dd, causal=causal, scale=scale)
        torch.cuda.synchronize()
        kvheads = [0, B * Hkv - 1]
        krows = np.array(sorted({kh * Sk + t for kh in kvheads for t in
                                 [0, 31, Sk - 1, min(Sq, Sk) - 1, min(Sq, Sk) % Sk] +
                                 list(rng.integers(0, Sk, 12))}), dtype=np.int64)
        rq, rk, rv = oracle.attention_bwd_rows(to_f64(q), to_f64(k), to_f64(v), to_f64(dout), causal, scale,
                                               rows, krows)
        check_grad(to_f64(dq).reshape(-1, D)[rows], rq, dtype, f"dQ {what}")
        check_grad(to_f64(dk).reshape(-1, D)[krows], rk, dtype, f"dK {what}")
        check_grad(to_f64(dv).reshape(-1, D)[krows], rv, dtype, f"dV {what}")


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_no_keys_or_no_queries(dtype):
    """S_k = 0: every row is empty (O = 0, lse = -inf; dQ = 0).  S_q = 0: the
    backward's dK, dV are 0.  Outputs start as NaN so that every write shows."""
    B, H, D = 2, 4, 64
    q, k, v, dout = rect_inputs(B, H, H, 100, 0, D, dtype, 9400)
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((B, H, 100), float("nan"), dtype=torch.float32, device=DEV)
    fa.forward(qd, kd, vd, causal=False, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))
    if dtype == "f32":
        return
    dq, dk, dv = fa.backward(qd, kd, vd, o, lse, dout.to(DEV), causal=True)
    torch.cuda.synchronize()
    assert torch.all(dq == 0) and dk.numel() == 0 and dv.numel() == 0
    q, k, v, dout = rect_inputs(B, H, 2, 0, 300, D, dtype, 9401)
    qd, kd, vd, dd = (x.to(DEV) for x in (q, k, v, dout))
    o = torch.empty_like(qd)
    lse = torch.empty((B, H, 0), dtype=torch.float32, device=DEV)
    dq, dk, dv = fa.backward(qd, kd, vd, o, lse, dd, causal=False)
    torch.cuda.synchronize()
    assert dq.numel() == 0 and torch.all(dk == 0) and torch.all(dv == 0)


def test_square_ex_equals_plain_bitwise():
    """S_q = S_k through the extended entry points launches what the plain ones do."""
    q, k, v, dout = rect_inputs(2, 4, 4, 777, 777, 64, "bf16", 9500)
    qd, kd, vd, dd = (x.to(DEV) for x in (q, k, v, dout))
    o1, l1 = fa.forward(qd, kd, vd, causal=True)
    o2 = torch.empty_like(qd)
    l2 = torch.empty((2, 4, 777), dtype=torch.float32, device=DEV)
    st = torch.cuda.current_stream().cuda_stream
    fa.check(fa.fa_fwd(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o2.data_ptr(), l2.data_ptr(), 2, 4, 777, 64, 1,
                       fp32(1 / 8), fa.DTYPE_CODES[torch.bfloat16], st))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
