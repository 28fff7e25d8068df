"""Seeded random shapes across the forward's and backward's kernel choices,
each compared element by element with the float64 oracle.

Which kernel runs depends on the grid (batch x heads x query blocks of 256,
128, 64 or 32 rows), the head dimension, the mask, the window, S_q against S_k
and whether a workspace is given.  The fixed-shape tests pin each rule at a
few points; here a seeded generator draws shapes inside each regime (large
grids, the grids the key split serves, grids between the split and the large
tile at D = 128, thin grids, queries and keys of different length, windows,
grouped K/V heads), with ragged lengths throughout, so that the boundaries
between the rules are crossed at sizes nobody picked by hand.  The case list
is the same on every run; each case prints its parameters before it runs.

What is compared is what the pages define: O and the natural-log lse of exact
attention ("T5 讲解：FlashAttention forward", section ①; "Inside
FlashAttention", section 2.4), and for fp16 / bf16 the gradients of the
recompute backward ("从零训练语言模型（第二部分）", section "反向传播").
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
FULL_GRID = 512  # workgroups that fill the GPU twice over (the dispatch's threshold)


def fp32(x):
    return float(torch.tensor(x, dtype=torch.float32))


def cdiv(a, b):
    return -(-a // b)


def heads(rng, need_bh, max_b=8):
    """(B, H, H_kv) with H = G * H_kv, G in {1, 2, 4}, and B * H >= need_bh."""
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 4]))
    h = hkv * g
    b = max(1, cdiv(need_bh, h))
    while b > max_b:  # too many batches: widen the heads instead
        hkv *= 2
        h = hkv * g
        b = max(1, cdiv(need_bh, h))
    return b, h, hkv


def window_of(rng):
    return tuple(int(x) for x in rng.choice([-1, 0, 3, 17, 64, 200, 700], size=2))


def make_cases():
    rng = np.random.default_rng(20261202)
    cases = []
    # large grids: the two-block kernel (D = 32, 64: 256 rows), the one-block
    # kernel on 128 rows (D = 16) and on 8-wave 256-row workgroups (D = 128)
    for i in range(8):
        D = [32, 64, 16, 128][i % 4]
        S = int(rng.integers(500, 2200))
        rows = 128 if D == 16 else 256
        B, H, Hkv = heads(rng, cdiv(FULL_GRID, cdiv(S, rows)))
        win = window_of(rng) if i >= 6 else None
        cases.append(dict(kind="large", B=B, H=H, Hkv=Hkv, Sq=S, Sk=S, D=D, dtype=["f16", "bf16"][i % 2],
                          causal=bool(rng.integers(0, 2)) or i < 2, window=win))
    # the key split's grids: causal, no window, S_q = S_k, the whole grid
    # resident: n query blocks x B*H = 512 at D = 16, 32, 64; at D = 128,
    # n 128-row blocks x B*H = 256 with 64-row blocks reaching 512 (S in the
    # upper half of its last 128-row block)
    for i, (D, n) in enumerate([(64, 2), (64, 8), (32, 4), (32, 16), (16, 4), (16, 16), (128, 8), (128, 16)]):
        rows = 128 if D in (16, 128) else 256
        lo = (n - 1) * rows + (65 if D == 128 else 1)
        S = int(rng.integers(lo, n * rows + 1))
        bh = (FULL_GRID if D != 128 else 256) // n
        hkv = int(rng.choice([1, 2]))
        H = 2 * hkv if bh % (2 * hkv) == 0 else hkv
        cases.append(dict(kind="split", B=bh // H, H=H, Hkv=hkv, Sq=S, Sk=S, D=D, dtype=["f16", "bf16"][i % 2],
                          causal=True, window=None))
    # D = 128 grids between the key split and the large tile (128 rows)
    for i in range(2):
        S = int(rng.integers(2100, 4000))
        bh = int(rng.integers(cdiv(FULL_GRID, cdiv(S, 64)), cdiv(FULL_GRID, cdiv(S, 256))))
        cases.append(dict(kind="mid128", B=bh, H=1, Hkv=1, Sq=S, Sk=S, D=128, dtype=["bf16", "f16"][i],
                          causal=bool(i), window=None))
    # thin grids (keys split across the waves of a workgroup), fp32 included
    for i in range(10):
        D = int(rng.choice([16, 32, 64, 128]))
        B, H, Hkv = heads(rng, int(rng.integers(1, 9)), max_b=2)
        S = int(rng.integers(1, 3000))
        cases.append(dict(kind="thin", B=B, H=H, Hkv=Hkv, Sq=S, Sk=S, D=D, dtype=["f16", "bf16", "f32"][i % 3],
                          causal=bool(i % 2), window=window_of(rng) if i % 4 == 3 else None))
    # queries and keys of different length, with and without windows
    for i in range(8):
        D = int(rng.choice([16, 32, 64, 128]))
        B, H, Hkv = heads(rng, int(rng.integers(1, 33)), max_b=4)
        Sq, Sk = (int(x) for x in rng.integers(1, 1800, size=2))
        cases.append(dict(kind="rect", B=B, H=H, Hkv=Hkv, Sq=Sq, Sk=Sk, D=D, dtype=["f16", "bf16", "f32"][i % 3],
                          causal=bool(i % 2), window=window_of(rng) if i >= 4 else None))
    return cases


def make_bwd_cases():
    rng = np.random.default_rng(20261203)
    cases = []
    for i in range(10):
        D = [16, 32, 64, 128][i % 4]
        if i < 4:  # grids of at least 512 dK/dV workgroups (128 keys each)
            S = int(rng.integers(300, 1300))
            B, H, Hkv = heads(rng, cdiv(FULL_GRID, cdiv(S, 128)))
            # K/V heads set the dK/dV grid: widen B until it is full
            while B * Hkv * cdiv(S, 128) < FULL_GRID:
                B += 1
            Sq = Sk = S
        else:
            B, H, Hkv = heads(rng, int(rng.integers(1, 17)), max_b=4)
            Sq = int(rng.integers(1, 1500))
            Sk = Sq if i < 7 else int(rng.integers(1, 1500))
        cases.append(dict(kind="bwd", B=B, H=H, Hkv=Hkv, Sq=Sq, Sk=Sk, D=D, dtype=["f16", "bf16"][i % 2],
                          causal=bool(rng.integers(0, 2)), window=window_of(rng) if i in (5, 8) else None))
    return cases


CASES = make_cases()
BWD_CASES = make_bwd_cases()


def case_id(c):
    w = "" if c["window"] is None else f"-w{c['window'][0]}_{c['window'][1]}"
    return (f"{c['kind']}-{c['dtype']}-B{c['B']}H{c['H']}kv{c['Hkv']}-S{c['Sq']}x{c['Sk']}-D{c['D']}"
            f"-{'c' if c['causal'] else 'n'}{w}")


def inputs(c, seed):
    q, _, _ = workloads.make_inputs(c["B"], c["H"], c["Sq"], c["D"], c["dtype"], seed)
    _, k, v = workloads.make_inputs(c["B"], c["Hkv"], c["Sk"], c["D"], c["dtype"], seed + 1)
    return q, k, v


def check_rows(o, lse, o_ref, l_ref, dtype, what):
    """Rows the oracle leaves without a key are O = 0, lse = -inf exactly; the
    others within the parity tolerances."""
    o, lse = to_f64(o), to_f64(lse)
    empty = np.isneginf(l_ref)
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: rows without keys differ"
    assert np.all(o[empty] == 0.0), f"{what}: O of a row without keys must be 0"
    check_o(o[~empty], o_ref[~empty], dtype, f"O {what}")
    check_lse(lse[~empty], l_ref[~empty], f"lse {what}")


def test_cases_reach_every_regime():
    """The generator's shapes land where they are meant to (host arithmetic
    only): the split cases need the workspace the library sizes for them, the
    others none, and every family is present."""
    kinds = {c["kind"] for c in CASES}
    assert kinds == {"large", "split", "mid128", "thin", "rect"}
    for c in CASES:
        code = fa.DTYPE_CODES[DT[c["dtype"]]]
        wl, wr = (-1, -1) if c["window"] is None else c["window"]
        nb = fa.fa_fwd_workspace_bytes(c["B"], c["H"], c["Hkv"], c["Sq"], c["Sk"], c["D"], int(c["causal"]), wl, wr,
                                       code)
        assert (nb > 0) == (c["kind"] == "split"), case_id(c)
        assert c["H"] % c["Hkv"] == 0


@pytest.mark.parametrize("c", CASES, ids=case_id)
def test_fuzz_forward(c):
    what = case_id(c)
    print(f"\nfuzz forward {what}", flush=True)
    seed = 9000 + CASES.index(c) * 3
    q, k, v = inputs(c, seed)
    scale = fp32(1 / math.sqrt(c["D"]))
    o_ref, l_ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v), c["causal"], scale, c["window"])
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    o, lse = fa.forward(qd, kd, vd, causal=c["causal"], scale=scale, window=c["window"])
    torch.cuda.synchronize()
    check_rows(o, lse, o_ref, l_ref, c["dtype"], what)
    if c["kind"] == "split":
        # the same problem without a workspace: the unsplit kernel
        o2 = torch.empty_like(qd)
        l2 = torch.empty_like(lse)
        st = fa.fa_fwd_ex(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o2.data_ptr(), l2.data_ptr(), c["B"],
                          c["H"], c["Hkv"], c["Sq"], c["Sk"], c["D"], 1, -1, -1, scale,
                          fa.DTYPE_CODES[q.dtype], torch.cuda.current_stream().cuda_stream)
        fa.check(st)
        torch.cuda.synchronize()
        check_rows(o2, l2, o_ref, l_ref, c["dtype"], what + " (no workspace)")


@pytest.mark.parametrize("c", BWD_CASES, ids=case_id)
def test_fuzz_backward(c):
    """dQ, dK, dV from the oracle's own O and lse (as stored in the input
    type), against the oracle's gradients."""
    what = case_id(c)
    print(f"\nfuzz backward {what}", flush=True)
    seed = 9500 + BWD_CASES.index(c) * 4
    q, k, v = inputs(c, seed)
    dout = workloads.make_grad(c["B"], c["H"], c["Sq"], c["D"], c["dtype"], seed + 2)
    scale = fp32(1 / math.sqrt(c["D"]))
    q64, k64, v64, d64 = (to_f64(x) for x in (q, k, v, dout))
    o_ref, l_ref = oracle.attention(q64, k64, v64, c["causal"], scale, c["window"])
    dq_ref, dk_ref, dv_ref = oracle.attention_bwd(q64, k64, v64, d64, c["causal"], scale, c["window"])
    o = torch.from_numpy(o_ref).to(DT[c["dtype"]])
    lse = torch.from_numpy(l_ref).to(torch.float32)
    dq, dk, dv = fa.backward(q.to(DEV), k.to(DEV), v.to(DEV), o.to(DEV), lse.to(DEV), dout.to(DEV),
                             causal=c["causal"], scale=scale, window=c["window"])
    torch.cuda.synchronize()
    check_grad(to_f64(dq), dq_ref, c["dtype"], f"dQ {what}")
    check_grad(to_f64(dk), dk_ref, c["dtype"], f"dK {what}")
    check_grad(to_f64(dv), dv_ref, c["dtype"], f"dV {what}")
