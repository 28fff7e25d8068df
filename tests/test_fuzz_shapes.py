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
from fuzz_cases import BWD_CASES, CASES, case_id
from parity_util import DT, check_grad, check_lse, check_o, to_f64

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU visible", allow_module_level=True)

import exact_tiled_attention_06_amd as fa  # noqa: E402

fa.library()  # fails loudly when libfa.so is missing

DEV = "cuda:0"


def fp32(x):
    return float(torch.tensor(x, dtype=torch.float32))


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
