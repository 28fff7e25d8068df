"""Comparison helpers for the GPU-vs-oracle parity tests.

Tolerances (from the attention forward's accuracy targets; derivation in the
design notes):
  O, fp16 inputs:  max |O_gpu - O_ref| <= 5e-3
  O, bf16 inputs:  max |O_gpu - O_ref| <= 2e-2
  O, fp32 inputs:  max |O_gpu - O_ref| / max |O_ref| <= 1e-4
  lse, all dtypes: max |lse_gpu - lse_ref| / max |lse_ref| <= 1e-4 and, per element,
                   |lse_gpu - lse_ref| <= 1e-4 * max(|lse_ref|, 1)
O_ref and lse_ref are the unrounded float64 oracle values on the same stored inputs.

Gradients (dQ, dK, dV of the backward), normwise:
  max |g_gpu - g_ref| / max(max |g_ref|, 1e-2) <= 4u,  u = 2^-11 (fp16), 2^-8 (bf16):
  the output rounding contributes at most u/2, the rounding of P and dS to the
  input type before their products about u (1.5u worst in a CPU emulation of the
  kernels' arithmetic on the parity shapes), the fp32 parts ~1e-6.  The floor
  holds a gradient that vanishes in exact arithmetic (dQ and dK at S = 1) to an
  absolute bound instead of a ratio to zero.
"""
from __future__ import annotations

import numpy as np
import torch

O_ABS_TOL = {"f16": 5e-3, "bf16": 2e-2}
O_REL_TOL_F32 = 1e-4
LSE_REL_TOL = 1e-4

GRAD_REL_TOL = {"f16": 4 * 2.0 ** -11, "bf16": 4 * 2.0 ** -8}
GRAD_FLOOR = 1e-2

DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def dtype_name(t: torch.dtype) -> str:
    return {v: k for k, v in DT.items()}[t]


def to_f64(x: torch.Tensor) -> np.ndarray:
    """Exact widening of stored fp16/bf16/fp32 values to float64."""
    return x.detach().to("cpu").to(torch.float64).numpy()


def check_o(o_gpu: np.ndarray, o_ref: np.ndarray, dtype: str, what: str = "O") -> float:
    assert o_gpu.shape == o_ref.shape, f"{what}: shape {o_gpu.shape} vs {o_ref.shape}"
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite GPU output"
    if o_gpu.size == 0:
        return 0.0
    err = float(np.max(np.abs(o_gpu - o_ref)))
    if dtype == "f32":
        rel = err / max(float(np.max(np.abs(o_ref))), 1e-30)
        assert rel <= O_REL_TOL_F32, f"{what}: normwise relative error {rel:.3e} > {O_REL_TOL_F32}"
        return rel
    tol = O_ABS_TOL[dtype]
    if err > tol:
        idx = np.unravel_index(np.argmax(np.abs(o_gpu - o_ref)), o_gpu.shape)
        raise AssertionError(f"{what}: max abs error {err:.3e} > {tol} at {idx}: "
                             f"gpu {o_gpu[idx]!r} ref {o_ref[idx]!r}")
    return err


def check_grad(g_gpu: np.ndarray, g_ref: np.ndarray, dtype: str, what: str = "grad") -> float:
    assert g_gpu.shape == g_ref.shape, f"{what}: shape {g_gpu.shape} vs {g_ref.shape}"
    assert np.all(np.isfinite(g_gpu)), f"{what}: non-finite GPU values"
    if g_gpu.size == 0:
        return 0.0
    ref_max = float(np.max(np.abs(g_ref)))
    err = float(np.max(np.abs(g_gpu - g_ref)))
    rel = err / max(ref_max, GRAD_FLOOR)
    tol = GRAD_REL_TOL[dtype]
    if rel > tol:
        idx = np.unravel_index(np.argmax(np.abs(g_gpu - g_ref)), g_gpu.shape)
        raise AssertionError(f"{what}: normwise error {rel:.3e} > {tol:.3e} (max |ref| {ref_max:.3e}) "
                             f"at {idx}: gpu {g_gpu[idx]!r} ref {g_ref[idx]!r}")
    return rel


def check_lse(l_gpu: np.ndarray, l_ref: np.ndarray, what: str = "lse") -> float:
    assert l_gpu.shape == l_ref.shape, f"{what}: shape {l_gpu.shape} vs {l_ref.shape}"
    assert np.all(np.isfinite(l_gpu)), f"{what}: non-finite GPU lse"
    if l_gpu.size == 0:
        return 0.0
    d = np.abs(l_gpu - l_ref)
    rel = float(np.max(d)) / max(float(np.max(np.abs(l_ref))), 1e-30)
    assert rel <= LSE_REL_TOL, f"{what}: normwise relative error {rel:.3e} > {LSE_REL_TOL}"
    elem = d / np.maximum(np.abs(l_ref), 1.0)
    worst = float(np.max(elem))
    if worst > LSE_REL_TOL:
        idx = np.unravel_index(np.argmax(elem), l_gpu.shape)
        raise AssertionError(f"{what}: elementwise error {worst:.3e} > {LSE_REL_TOL} at {idx}")
    return rel


def lse_errors(l_gpu: np.ndarray, l_ref: np.ndarray):
    """(normwise, elementwise) lse errors: max|d| / max|ref| and max |d| / max(|ref|, 1)."""
    if l_gpu.size == 0:
        return 0.0, 0.0
    d = np.abs(l_gpu - l_ref)
    return (float(np.max(d)) / max(float(np.max(np.abs(l_ref))), 1e-30),
            float(np.max(d / np.maximum(np.abs(l_ref), 1.0))))


def sample_rows(B: int, H: int, S: int, n_random: int, seed: int) -> np.ndarray:
    """Flat row indices (b*H + h)*S + i: the first and last rows of every head, rows
    on both sides of every 32/64/128/256-row boundary of a few heads, and random rows."""
    rng = np.random.default_rng(seed)
    rows = set()
    bh_all = B * H
    for bh in range(bh_all):
        rows.update({bh * S, bh * S + S - 1})
    for bh in sorted({0, bh_all - 1, bh_all // 2}):
        for blk in (32, 64, 128, 256):
            for edge in range(blk, S, blk * max(1, S // (blk * 8))):
                for i in (edge - 1, edge):
                    rows.add(bh * S + i)
    rows.update(int(x) for x in rng.integers(0, bh_all * S, size=n_random))
    return np.array(sorted(rows), dtype=np.int64)
