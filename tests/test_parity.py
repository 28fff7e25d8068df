"""GPU parity: the HIP kernels (through the C ABI) against the float64 CPU oracle.

Every case compares every element of O and lse: small ragged shapes, and every
workload of the five configurations at full size, in the launch configuration
the benchmark times (the oracle runs multi-threaded over the whole workload).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_util import check_lse, check_o, lse_errors, to_f64

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU visible", allow_module_level=True)

import exact_tiled_attention_06_amd as fa  # noqa: E402

fa.library()  # fails loudly when libfa.so is missing

DEV = "cuda:0"


def run_gpu(q, k, v, causal, scale=None):
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    o, lse = fa.forward(qd, kd, vd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse


def fp32_scale(x):
    return float(torch.tensor(x, dtype=torch.float32))


def full_check(q, k, v, causal, dtype, scale=None, what=""):
    D = q.shape[-1]
    scale = fp32_scale(1.0 / math.sqrt(D) if scale is None else scale)
    o, lse = run_gpu(q, k, v, causal, scale)
    o_ref, l_ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v), causal, scale)
    e_o = check_o(to_f64(o), o_ref, dtype, f"O {what}")
    check_lse(to_f64(lse), l_ref, f"lse {what}")
    return o, lse, e_o, lse_errors(to_f64(lse), l_ref)


# ----------------------------------------------------------------- small shapes

SMALL_SHAPES = [
    (1, 1, 1),      # one row, one key
    (1, 2, 31),     # less than one tile
    (2, 1, 64),     # exactly one key tile
    (1, 2, 128),    # one query block of 128
    (2, 2, 333),    # several query blocks and key tiles, ragged tail
    (1, 3, 520),    # ragged tail of 8 rows
]


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_small_shapes_elementwise(dtype, D, causal):
    seed = 1000 + D
    for (B, H, S) in SMALL_SHAPES:
        q, k, v = workloads.make_inputs(B, H, S, D, dtype, seed)
        seed += 1
        full_check(q, k, v, causal, dtype, what=f"{dtype} D={D} causal={causal} B,H,S={B},{H},{S}")


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
def test_growing_scores_force_rescales(dtype, causal):
    """Keys scaled up along the sequence make the running maximum grow on every tile,
    so every tile rescales the accumulator (the pitfall of forgetting acc *= alpha)."""
    B, H, S, D = 1, 2, 700, 64
    q, k, v = workloads.make_inputs(B, H, S, D, dtype, 77)
    ramp = torch.linspace(0.2, 3.0, S).reshape(1, 1, S, 1)
    k = (k.float() * ramp).to(q.dtype)
    q = (q.float().abs() + 0.5).to(q.dtype)  # positive queries against a growing key ramp
    k = k.abs()
    full_check(q, k, v, causal, dtype, what="growing scores")


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_scale_values(dtype):
    B, H, S, D = 1, 2, 300, 64
    q, k, v = workloads.make_inputs(B, H, S, D, dtype, 88)
    for scale in (1.0, 0.01, 0.3):
        for causal in (False, True):
            full_check(q, k, v, causal, dtype, scale=scale, what=f"scale={scale} causal={causal}")


def test_q_equals_k_aliasing():
    B, H, S, D = 1, 2, 256, 64
    q, _, v = workloads.make_inputs(B, H, S, D, "f16", 99)
    qd, vd = q.to(DEV), v.to(DEV)
    o, lse = fa.forward(qd, qd, vd, causal=True)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(to_f64(q), to_f64(q), to_f64(v), True, fp32_scale(1 / 8))
    check_o(to_f64(o), o_ref, "f16")
    check_lse(to_f64(lse), l_ref)


# ------------------------------------------------------------ pins on the GPU


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("D", [16, 64, 128])
def test_causal_row0_is_v0(dtype, D):
    """Causal row 0 sees key 0 only: p = 1, l = 1, so O[0] = V[0] (bit-exact for fp16/bf16)."""
    B, H, S = 2, 3, 200
    q, k, v = workloads.make_inputs(B, H, S, D, dtype, 123)
    o, lse = run_gpu(q, k, v, True)
    got = o[:, :, 0].cpu()
    if dtype == "f32":
        assert torch.allclose(got, v[:, :, 0], rtol=1e-6, atol=1e-6)
    else:
        assert torch.equal(got, v[:, :, 0]), "causal row 0 differs from V[0]"
    scale = fp32_scale(1 / math.sqrt(D))
    ref = scale * (to_f64(q)[:, :, 0] * to_f64(k)[:, :, 0]).sum(-1)
    assert np.max(np.abs(to_f64(lse)[:, :, 0] - ref)) <= 1e-4 * max(1.0, np.max(np.abs(ref)))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_last_row_causal_equals_noncausal(dtype):
    """Row S-1 attends to every key with or without the mask; both kernels visit the
    same tiles in the same order, so the results agree exactly."""
    B, H, S, D = 2, 2, 1024, 64
    q, k, v = workloads.make_inputs(B, H, S, D, dtype, 321)
    o1, l1 = run_gpu(q, k, v, False)
    o2, l2 = run_gpu(q, k, v, True)
    assert torch.equal(o1[:, :, -1], o2[:, :, -1])
    assert torch.equal(l1[:, :, -1], l2[:, :, -1])


def test_deterministic():
    q, k, v = workloads.make_inputs(2, 4, 1000, 64, "f16", 5)
    o1, l1 = run_gpu(q, k, v, True)
    o2, l2 = run_gpu(q, k, v, True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_runs_on_the_callers_stream():
    q, k, v = (x.to(DEV) for x in workloads.make_inputs(1, 2, 512, 64, "f16", 6))
    ref_o, ref_l = fa.forward(q, k, v, causal=True)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o, l = fa.forward(q, k, v, causal=True)
    s.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(l, ref_l)


def test_empty_inputs():
    for shape in [(0, 2, 64, 64), (1, 0, 64, 64), (1, 2, 0, 64)]:
        q = torch.zeros(shape, dtype=torch.float16, device=DEV)
        o, lse = fa.forward(q, q.clone(), q.clone(), causal=True)
        assert o.shape == shape and lse.shape == shape[:3]


def test_argument_errors_raise():
    q = torch.zeros((1, 1, 64, 48), dtype=torch.float16, device=DEV)
    with pytest.raises(ValueError):
        fa.forward(q, q, q)
    q = torch.zeros((1, 1, 64, 64), dtype=torch.float16, device=DEV)
    with pytest.raises(ValueError):
        fa.forward(q, q, q, scale=-1.0)
    with pytest.raises(ValueError):
        fa.forward(q, q, q, out=q)  # output aliases the inputs


# ----------------------------------------------------------- full-size workloads

# every named workload of the five configurations: single-head fp32, the
# headless batch (causal and not), the multi-head causal one, the long bf16
# sequence and the 20 points of the causal fp16 sweep -- each compared with the
# oracle on every element of O and lse, in the launch configuration the
# benchmark times
CONFIG_WORKLOADS = (["single_head_f32", "batch_f16", "multihead_causal", "long_seq_bf16"]
                    + [w.name for w in workloads.sweep()])


@pytest.mark.parametrize("name", CONFIG_WORKLOADS)
def test_workload_elementwise(name):
    w = workloads.BY_NAME[name]
    q, k, v = workloads.workload_inputs(w)
    for causal in w.causal:
        # check_lse asserts both the normwise and the elementwise lse forms
        o, lse, e_o, e_l = full_check(q, k, v, causal, w.dtype, w.scale, what=f"{name} causal={causal}")
        print(f"\nparity {name} causal={causal}: max|dO| = {e_o:.3e} "
              f"({'normwise rel' if w.dtype == 'f32' else 'abs'}), lse normwise {e_l[0]:.3e}, "
              f"elementwise {e_l[1]:.3e}", flush=True)
        # properties that hold for every row: finite values and causal row 0 == V[0]
        assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
        if causal and w.dtype != "f32":
            assert torch.equal(o[:, :, 0].cpu(), v[:, :, 0])


def test_outputs_off_device_rejected():
    """out / lse tensors that are not on q's device are refused before any launch."""
    q, k, v = (x.to(DEV) for x in workloads.make_inputs(1, 2, 128, 64, "f16", 11))
    with pytest.raises(ValueError):
        fa.forward(q, k, v, causal=True, out=torch.empty((1, 2, 128, 64), dtype=torch.float16))
    with pytest.raises(ValueError):
        fa.forward(q, k, v, causal=True, lse=torch.empty((1, 2, 128), dtype=torch.float32))
    # the same call with device buffers runs
    o, lse = fa.forward(q, k, v, causal=True, out=torch.empty_like(q),
                        lse=torch.empty((1, 2, 128), dtype=torch.float32, device=DEV))
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
