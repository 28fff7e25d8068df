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
upper-triangular mask), in absolute positions when queries and keys differ in
number (the CS336 write-up's forward kernel: ``Sq`` queries, ``Sk`` keys, keys
at or past ``Sk`` absent); a row left with no key has o = 0 and lse = -inf.

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


def _shapes(q, k, v, extra=()):
    """[B,H,Sq,D] queries, [B,Hkv,Sk,D] keys and values (H a multiple of Hkv):
    returns B, H, Hkv, Sq, Sk, D."""
    if q.ndim != 4 or k.ndim != 4 or v.shape != k.shape:
        raise ValueError(f"q must be [B,H,Sq,D] and k, v one [B,Hkv,Sk,D] shape, got {q.shape}, {k.shape}, {v.shape}")
    B, H, Sq, D = q.shape
    if k.shape[0] != B or k.shape[3] != D or k.shape[1] < 1 or H % k.shape[1] != 0:
        raise ValueError(f"k, v shape {k.shape} does not fit q {q.shape} (H must be a multiple of Hkv)")
    for x in extra:
        if x.shape != q.shape:
            raise ValueError(f"expected shape {q.shape}, got {x.shape}")
    return B, H, k.shape[1], Sq, k.shape[2], D


def _window(window):
    wl, wr = (int(window[0]), int(window[1])) if window is not None else (-1, -1)
    if wl < -1 or wr < -1:
        raise ValueError(f"window bounds must be >= -1 (-1: unlimited), got {window}")
    return wl, wr


class Oracle:
    """ctypes handle on one build of ``attn_oracle.c``.

    Keys and values may have fewer heads than the queries (grouped heads:
    query head h reads key/value head h // (H // Hkv)) and another length
    (q [B,H,Sq,D], k and v [B,Hkv,Sk,D]); ``window = (left, right)`` limits
    query i to keys i - left .. i + right (-1: no limit on that side).
    """

    def __init__(self, library: str):
        lib = ctypes.CDLL(library)
        I64, I, D_ = ctypes.c_int64, ctypes.c_int, ctypes.c_double
        lib.oracle_attn_fwd_ex.restype = I
        lib.oracle_attn_fwd_ex.argtypes = [_c_double_p] * 5 + [I64] * 6 + [I, I64, I64, D_]
        lib.oracle_attn_fwd_rows_ex.restype = I
        lib.oracle_attn_fwd_rows_ex.argtypes = [_c_double_p] * 3 + [I64] * 6 + [I, I64, I64, D_] + [
            _c_int64_p, I64, _c_double_p, _c_double_p]
        lib.oracle_attn_bwd_ex.restype = I
        lib.oracle_attn_bwd_ex.argtypes = [_c_double_p] * 7 + [I64] * 6 + [I, I64, I64, D_]
        lib.oracle_attn_bwd_rows_ex.restype = I
        lib.oracle_attn_bwd_rows_ex.argtypes = [_c_double_p] * 4 + [I64] * 6 + [I, I64, I64, D_] + [
            _c_int64_p, I64, _c_double_p, _c_int64_p, I64, _c_double_p, _c_double_p]
        lib.oracle_num_threads.restype = I
        lib.oracle_num_threads.argtypes = []
        self._lib = lib
        self.path = library

    @staticmethod
    def _ptr(a: np.ndarray):
        return a.ctypes.data_as(_c_double_p)

    def num_threads(self) -> int:
        return int(self._lib.oracle_num_threads())

    def attention(self, q, k, v, causal: bool, scale: float, window=None):
        """Exact attention over all rows: returns (o [B,H,Sq,D], lse [B,H,Sq])."""
        q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
        B, H, Hkv, Sq, Sk, D = _shapes(q, k, v)
        wl, wr = _window(window)
        o = np.empty_like(q)
        lse = np.empty((B, H, Sq), dtype=np.float64)
        rc = self._lib.oracle_attn_fwd_ex(self._ptr(q), self._ptr(k), self._ptr(v), self._ptr(o),
                                          self._ptr(lse), B, H, Hkv, Sq, Sk, D, int(bool(causal)), wl, wr,
                                          float(scale))
        if rc != 0:
            raise ValueError(f"oracle_attn_fwd_ex failed with status {rc}")
        return o, lse

    def attention_rows(self, q, k, v, causal: bool, scale: float, rows, window=None):
        """Exact attention for selected flat query rows ``(b*H + h)*Sq + i``:
        returns (o [n, D], lse [n]) in the order of ``rows``."""
        q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
        B, H, Hkv, Sq, Sk, D = _shapes(q, k, v)
        wl, wr = _window(window)
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n = rows.shape[0]
        o = np.empty((n, D), dtype=np.float64)
        lse = np.empty((n,), dtype=np.float64)
        rc = self._lib.oracle_attn_fwd_rows_ex(
            self._ptr(q), self._ptr(k), self._ptr(v), B, H, Hkv, Sq, Sk, D, int(bool(causal)), wl, wr,
            float(scale), rows.ctypes.data_as(_c_int64_p), n, self._ptr(o), self._ptr(lse))
        if rc != 0:
            raise ValueError(f"oracle_attn_fwd_rows_ex failed with status {rc}")
        return o, lse

    def attention_bwd(self, q, k, v, dout, causal: bool, scale: float, window=None):
        """Gradients for upstream gradient ``dout`` [B,H,Sq,D]: returns
        (dq [B,H,Sq,D], dk [B,Hkv,Sk,D], dv [B,Hkv,Sk,D])."""
        q, k, v, dout = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(dout)
        B, H, Hkv, Sq, Sk, D = _shapes(q, k, v, (dout,))
        wl, wr = _window(window)
        dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(k)
        rc = self._lib.oracle_attn_bwd_ex(self._ptr(q), self._ptr(k), self._ptr(v), self._ptr(dout),
                                          self._ptr(dq), self._ptr(dk), self._ptr(dv),
                                          B, H, Hkv, Sq, Sk, D, int(bool(causal)), wl, wr, float(scale))
        if rc != 0:
            raise ValueError(f"oracle_attn_bwd_ex failed with status {rc}")
        return dq, dk, dv

    def attention_bwd_rows(self, q, k, v, dout, causal: bool, scale: float, rows, krows=None, window=None):
        """Gradients at selected positions: dQ of flat query rows ``rows``
        ((b*H + h)*Sq + t) and dK, dV of flat key rows ``krows`` ((b*Hkv + hk)*Sk + t;
        default: the same indices as ``rows``).  Returns (dq [n,D], dk [m,D], dv [m,D])."""
        q, k, v, dout = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(dout)
        B, H, Hkv, Sq, Sk, D = _shapes(q, k, v, (dout,))
        wl, wr = _window(window)
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        krows = rows if krows is None else np.ascontiguousarray(np.asarray(krows, dtype=np.int64))
        n, m = rows.shape[0], krows.shape[0]
        dq = np.empty((n, D), dtype=np.float64)
        dk, dv = np.empty((m, D), dtype=np.float64), np.empty((m, D), dtype=np.float64)
        rc = self._lib.oracle_attn_bwd_rows_ex(
            self._ptr(q), self._ptr(k), self._ptr(v), self._ptr(dout), B, H, Hkv, Sq, Sk, D,
            int(bool(causal)), wl, wr, float(scale), rows.ctypes.data_as(_c_int64_p), n, self._ptr(dq),
            krows.ctypes.data_as(_c_int64_p), m, self._ptr(dk), self._ptr(dv))
        if rc != 0:
            raise ValueError(f"oracle_attn_bwd_rows_ex failed with status {rc}")
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


def attention(q, k, v, causal: bool, scale: float, window=None):
    return default().attention(q, k, v, causal, scale, window)


def attention_rows(q, k, v, causal: bool, scale: float, rows, window=None):
    return default().attention_rows(q, k, v, causal, scale, rows, window)


def attention_bwd(q, k, v, dout, causal: bool, scale: float, window=None):
    return default().attention_bwd(q, k, v, dout, causal, scale, window)


def attention_bwd_rows(q, k, v, dout, causal: bool, scale: float, rows, krows=None, window=None):
    return default().attention_bwd_rows(q, k, v, dout, causal, scale, rows, krows, window)
