"""Double-precision CPU attention oracle (test infrastructure only).

This package is the parity oracle: plain exact attention and its gradients
evaluated row by row in IEEE double precision (``attn_oracle.c``), with no
tiling and no online softmax.
Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
it.  It shares no code with the HIP path and imports nothing from the product
package.

What it computes follows the definition of exact attention on the pages
("T5 讲解：FlashAttention forward", section ①; "Inside FlashAttention",
section 1.1), the stable softmax with the row maximum subtracted
("从零训练语言模型（第二部分）", section "安全 / 在线 softmax") and the per-row
log-sum-exp ``lse = m + ln l`` ("Inside FlashAttention", section 2.4).  Causal
means query ``i`` sees keys ``0..i`` ("Triton 实现", the naive listing's
upper-triangular mask).

The gradients (``attention_bwd``) follow the backward equations of
"从零训练语言模型（第二部分）", section "反向传播", with the softmax Jacobian's row
term taken as sum_t P_it dP_it from the oracle's own probabilities.

Inputs are the *stored* element values the GPU receives (fp16, bf16 or fp32),
widened exactly to float64 by the caller; ``scale`` is the float32 value that is
handed to the kernel, widened.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "attn_oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

_c_double_p = ctypes.POINTER(ctypes.c_double)
_c_int64_p = ctypes.POINTER(ctypes.c_int64)


def build(source: str = SOURCE, output: str = LIBRARY, extra_flags: Sequence[str] = ()) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math) into a shared library."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
           *extra_flags, "-o", output + ".tmp", source, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(output + ".tmp", output)
    return output


def _as_f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


class Oracle:
    """ctypes handle on one build of ``attn_oracle.c``."""

    def __init__(self, library: str):
        lib = ctypes.CDLL(library)
        lib.oracle_attn_fwd.restype = ctypes.c_int
        lib.oracle_attn_fwd.argtypes = [_c_double_p] * 5 + [ctypes.c_int64] * 4 + [
            ctypes.c_int, ctypes.c_double]
        lib.oracle_attn_fwd_rows.restype = ctypes.c_int
        lib.oracle_attn_fwd_rows.argtypes = [_c_double_p] * 3 + [ctypes.c_int64] * 4 + [
            ctypes.c_int, ctypes.c_double, _c_int64_p, ctypes.c_int64, _c_double_p, _c_double_p]
        lib.oracle_attn_bwd.restype = ctypes.c_int
        lib.oracle_attn_bwd.argtypes = [_c_double_p] * 7 + [ctypes.c_int64] * 4 + [
            ctypes.c_int, ctypes.c_double]
        lib.oracle_attn_bwd_rows.restype = ctypes.c_int
        lib.oracle_attn_bwd_rows.argtypes = [_c_double_p] * 4 + [ctypes.c_int64] * 4 + [
            ctypes.c_int, ctypes.c_double, _c_int64_p, ctypes.c_int64] + [_c_double_p] * 3
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        self._lib = lib
        self.path = library

    @staticmethod
    def _ptr(a: np.ndarray):
        return a.ctypes.data_as(_c_double_p)

    def num_threads(self) -> int:
        return int(self._lib.oracle_num_threads())

    def attention(self, q, k, v, causal: bool, scale: float):
        """Exact attention over all rows.  q, k, v: [B,H,S,D]; returns (o [B,H,S,D], lse [B,H,S])."""
        q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
        if q.ndim != 4 or k.shape != q.shape or v.shape != q.shape:
            raise ValueError(f"q, k, v must share one [B,H,S,D] shape, got {q.shape}, {k.shape}, {v.shape}")
        B, H, S, D = q.shape
        o = np.empty_like(q)
        lse = np.empty((B, H, S), dtype=np.float64)
        rc = self._lib.oracle_attn_fwd(self._ptr(q), self._ptr(k), self._ptr(v), self._ptr(o),
                                       self._ptr(lse), B, H, S, D, int(bool(causal)), float(scale))
        if rc != 0:
            raise ValueError(f"oracle_attn_fwd failed with status {rc}")
        return o, lse

    def attention_rows(self, q, k, v, causal: bool, scale: float, rows):
        """Exact attention for selected flat rows ``(b*H + h)*S + i``.

        Returns (o [n, D], lse [n]) in the order of ``rows``.
        """
        q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
        if q.ndim != 4 or k.shape != q.shape or v.shape != q.shape:
            raise ValueError("q, k, v must share one [B,H,S,D] shape")
        B, H, S, D = q.shape
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n = rows.shape[0]
        o = np.empty((n, D), dtype=np.float64)
        lse = np.empty((n,), dtype=np.float64)
        rc = self._lib.oracle_attn_fwd_rows(
            self._ptr(q), self._ptr(k), self._ptr(v), B, H, S, D, int(bool(causal)), float(scale),
            rows.ctypes.data_as(_c_int64_p), n, self._ptr(o), self._ptr(lse))
        if rc != 0:
            raise ValueError(f"oracle_attn_fwd_rows failed with status {rc}")
        return o, lse

    def attention_bwd(self, q, k, v, dout, causal: bool, scale: float):
        """Gradients of exact attention for upstream gradient ``dout``.

        q, k, v, dout: [B,H,S,D]; returns (dq, dk, dv), each [B,H,S,D].
        """
        q, k, v, dout = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(dout)
        if q.ndim != 4 or any(x.shape != q.shape for x in (k, v, dout)):
            raise ValueError("q, k, v, dout must share one [B,H,S,D] shape")
        B, H, S, D = q.shape
        dq, dk, dv = np.empty_like(q), np.empty_like(q), np.empty_like(q)
        rc = self._lib.oracle_attn_bwd(self._ptr(q), self._ptr(k), self._ptr(v), self._ptr(dout),
                                       self._ptr(dq), self._ptr(dk), self._ptr(dv),
                                       B, H, S, D, int(bool(causal)), float(scale))
        if rc != 0:
            raise ValueError(f"oracle_attn_bwd failed with status {rc}")
        return dq, dk, dv

    def attention_bwd_rows(self, q, k, v, dout, causal: bool, scale: float, rows):
        """Gradients at selected flat positions ``(b*H + h)*S + t``: dQ of query t
        and dK, dV of key t.  Returns (dq [n,D], dk [n,D], dv [n,D])."""
        q, k, v, dout = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(dout)
        if q.ndim != 4 or any(x.shape != q.shape for x in (k, v, dout)):
            raise ValueError("q, k, v, dout must share one [B,H,S,D] shape")
        B, H, S, D = q.shape
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n = rows.shape[0]
        dq, dk, dv = (np.empty((n, D), dtype=np.float64) for _ in range(3))
        rc = self._lib.oracle_attn_bwd_rows(
            self._ptr(q), self._ptr(k), self._ptr(v), self._ptr(dout), B, H, S, D,
            int(bool(causal)), float(scale), rows.ctypes.data_as(_c_int64_p), n,
            self._ptr(dq), self._ptr(dk), self._ptr(dv))
        if rc != 0:
            raise ValueError(f"oracle_attn_bwd_rows failed with status {rc}")
        return dq, dk, dv


_DEFAULT: Optional[Oracle] = None


def default() -> Oracle:
    """The oracle built from this directory's source (built on first use if absent or stale)."""
    global _DEFAULT
    if _DEFAULT is None:
        stale = (not os.path.exists(LIBRARY)
                 or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE))
        if stale:
            build()
        _DEFAULT = Oracle(LIBRARY)
    return _DEFAULT


def attention(q, k, v, causal: bool, scale: float):
    return default().attention(q, k, v, causal, scale)


def attention_rows(q, k, v, causal: bool, scale: float, rows):
    return default().attention_rows(q, k, v, causal, scale, rows)


def attention_bwd(q, k, v, dout, causal: bool, scale: float):
    return default().attention_bwd(q, k, v, dout, causal, scale)


def attention_bwd_rows(q, k, v, dout, causal: bool, scale: float, rows):
    return default().attention_bwd_rows(q, k, v, dout, causal, scale, rows)
