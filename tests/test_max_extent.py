"""GPU checks at the largest key extent the matrix-core kernels address.

One head's K (or V) of S_k rows of D fp16 values must stay below 2^31 bytes
(the kernels read it through a buffer resource with a 32-bit extent; larger
calls return FA_ERR_TOO_LARGE).  These tests run 96 queries against
S_k = 2^24 - 32 keys at D = 64, i.e. 2^31 - 4096 bytes per head, with K and V
zero except for one key j* at the very end.  The softmax then has a closed form
evaluated here in float64 from the stored values (no value comes from the
GPU path):

    s_i = scale <q_i, k*>,  w_i = e^{s_i} / (e^{s_i} + S_k - 1)
    O_i = w_i v*,   lse_i = ln(e^{s_i} + S_k - 1)

and the gradients follow from the definition (P_ij = w_i at j*, else
p_i = 1 / (e^{s_i} + S_k - 1); dP_ij = <dO_i, v*> at j*, else 0):

    dQ_i  = scale w_i (1 - w_i) <dO_i, v*> k*
    dV_j* = sum_i w_i dO_i,    dV_j = sum_i p_i dO_i            (j != j*)
    dK_j* = scale sum_i w_i (1 - w_i) <dO_i, v*> q_i,
    dK_j  = -scale sum_i p_i w_i <dO_i, v*> q_i                 (j != j*)

Causal, query i sees keys 0..i only, never j*: O = 0 and lse = ln(i + 1).
"""
import math

import numpy as np
import pytest
import torch

from parity_util import check_grad, check_lse, check_o, to_f64

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU visible", allow_module_level=True)

import exact_tiled_attention_06_amd as fa  # noqa: E402

fa.library()  # fails loudly when libfa.so is missing

DEV = "cuda:0"
D = 64
SQ = 96
SK = (1 << 24) - 32  # S_k * D * 2 = 2^31 - 4096 bytes per head


def fp32(x):
    return float(torch.tensor(x, dtype=torch.float32))


def setup(seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    q = torch.randn((1, 1, SQ, D), generator=g).to(torch.float16)
    kstar = (torch.randn((D,), generator=g) * 0.6).to(torch.float16)
    vstar = torch.randn((D,), generator=g).to(torch.float16)
    dout = torch.randn((1, 1, SQ, D), generator=g).to(torch.float16)
    k = torch.zeros((1, 1, SK, D), dtype=torch.float16, device=DEV)
    v = torch.zeros((1, 1, SK, D), dtype=torch.float16, device=DEV)
    k[0, 0, SK - 1] = kstar.to(DEV)
    v[0, 0, SK - 1] = vstar.to(DEV)
    return q, kstar, vstar, dout, k, v


def closed_form(q, kstar, vstar, dout, scale):
    q64, k64, v64, do64 = (to_f64(x).reshape(-1, D) if x.dim() > 1 else to_f64(x) for x in (q, kstar, vstar, dout))
    s = scale * (q64 @ k64)                       # [SQ]
    z = np.exp(s) + (SK - 1)                      # softmax denominators
    w = np.exp(s) / z
    p = 1.0 / z
    o = w[:, None] * v64[None, :]
    lse = np.log(z)
    g = do64 @ v64                                # <dO_i, v*>
    dq = scale * (w * (1 - w) * g)[:, None] * k64[None, :]
    dv_star = (w[:, None] * do64).sum(0)
    dv_rest = (p[:, None] * do64).sum(0)
    dk_star = scale * ((w * (1 - w) * g)[:, None] * q64).sum(0)
    dk_rest = -scale * ((p * w * g)[:, None] * q64).sum(0)
    return o, lse, dq, dk_star, dk_rest, dv_star, dv_rest


def test_forward_at_the_largest_key_extent():
    q, kstar, vstar, _, k, v = setup(9600)
    scale = fp32(1 / math.sqrt(D))
    o, lse = fa.forward(q.to(DEV), k, v, causal=False, scale=scale)
    torch.cuda.synchronize()
    o_ref, l_ref, *_ = closed_form(q, kstar, vstar, torch.zeros_like(q), scale)
    check_o(to_f64(o).reshape(SQ, D), o_ref, "f16", "O at the largest key extent")
    check_lse(to_f64(lse).reshape(SQ), l_ref, "lse at the largest key extent")
    # causal: query i sees keys 0..i (all zero): O = 0, lse = ln(i + 1)
    o, lse = fa.forward(q.to(DEV), k, v, causal=True, scale=scale)
    torch.cuda.synchronize()
    assert torch.all(o == 0)
    check_lse(to_f64(lse).reshape(SQ), np.log(np.arange(1, SQ + 1, dtype=np.float64)),
              "causal lse at the largest key extent")


def test_backward_at_the_largest_key_extent():
    q, kstar, vstar, dout, k, v = setup(9601)
    scale = fp32(1 / math.sqrt(D))
    qd, dd = q.to(DEV), dout.to(DEV)
    o, lse = fa.forward(qd, k, v, causal=False, scale=scale)
    dq, dk, dv = fa.backward(qd, k, v, o, lse, dd, causal=False, scale=scale)
    torch.cuda.synchronize()
    _, _, dq_ref, dk_star, dk_rest, dv_star, dv_rest = closed_form(q, kstar, vstar, dout, scale)
    check_grad(to_f64(dq).reshape(SQ, D), dq_ref, "f16", "dQ at the largest key extent")
    # every key but j* has the same gradient, computed by the same arithmetic
    for g in (dk, dv):
        assert torch.equal(g[0, 0, 1:SK - 1], g[0, 0, :1].expand(SK - 2, D)), "keys other than j* differ"
    for nm, g, star, rest in (("dK", dk, dk_star, dk_rest), ("dV", dv, dv_star, dv_rest)):
        got = to_f64(g[0, 0, [0, SK // 2, SK - 2, SK - 1]])
        ref = np.stack([rest, rest, rest, star])
        check_grad(got, ref, "f16", f"{nm} at the largest key extent")
