"""FlashAttention-2 forward and backward for AMD Instinct MI355X (gfx950): Python binding of libfa.so.

Argument marshalling only: every step of the attention runs in the HIP kernels
behind the C ABI declared in ``include/fa.h``.  PyTorch supplies device memory
and the current stream; this module never computes attention itself and has no
CPU fallback -- the first call (or ``library()``) fails loudly when the library
is not built.  The library is loaded on first use so that the build step can
import this package before the library exists.

    fa_fwd(q, k, v, o, lse, B, H, S, D, causal, scale, dtype, stream)
        the C entry point with raw device pointers (ints) and sizes;
    fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, S, D, causal, scale, dtype, stream)
        the C backward entry point;
    fa_status_string(status)
        the C status description;
    forward(q, k, v, causal=False, scale=None, window=None) -> (o, lse)
        convenience on torch tensors q [B,H,S_q,D], k and v [B,H_kv,S_k,D]:
        allocates o (input dtype), lse (float32 [B,H,S_q]) and the workspace
        fa_fwd_workspace_bytes asks for (none for most problems) and calls
        fa_fwd_ws on the current stream.  The default scale is 1/sqrt(D)
        ("T5 讲解：FlashAttention forward", section ⑥).
    fa_fwd_ex / fa_bwd_ex(...)
        the C entry points with grouped K/V heads (H_kv), separate query and
        key lengths (S_q, S_k) and a sliding window;
    fa_fwd_workspace_bytes(...), fa_fwd_ws(...)
        the workspace the forward uses to split the longest causal query
        blocks over two workgroups, and fa_fwd_ex with that workspace;
    fa_fwd_single_buffered(...)
        race check: fa_fwd's two-block kernel with single-buffered K/V staging;
    fa_bwd_noalloc(...)
        fa_bwd_ex without the delta workspace argument (the library's static
        device array), for callers that cannot allocate;
    backward(q, k, v, o, lse, dout, causal=False, scale=None, window=None) -> (dq, dk, dv)
        gradients for the upstream gradient dout, from the forward's o and lse;
        allocates the outputs and the D workspace and calls fa_bwd.
"""
from __future__ import annotations

import ctypes
import math
import os
import struct

import torch  # loads the HIP runtime that libfa.so binds to (same soname)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_HERE, "libfa.so")

FA_OK = 0
FA_ERR_NULL_POINTER = 1
FA_ERR_SHAPE = 2
FA_ERR_HEAD_DIM = 3
FA_ERR_DTYPE = 4
FA_ERR_CAUSAL = 5
FA_ERR_SCALE = 6
FA_ERR_ALIAS = 7
FA_ERR_TOO_LARGE = 8
FA_ERR_LAUNCH = 9
FA_ERR_ALIGNMENT = 10
FA_ERR_WINDOW = 11
FA_ERR_WORKSPACE = 12
FA_ERR_UNSUPPORTED = 13

FA_DTYPE_F32 = 0
FA_DTYPE_F16 = 1
FA_DTYPE_BF16 = 2

DTYPE_CODES = {torch.float32: FA_DTYPE_F32, torch.float16: FA_DTYPE_F16, torch.bfloat16: FA_DTYPE_BF16}

# argument problems map to ValueError, runtime problems to RuntimeError
_VALUE_ERRORS = {FA_ERR_NULL_POINTER, FA_ERR_SHAPE, FA_ERR_HEAD_DIM, FA_ERR_DTYPE, FA_ERR_CAUSAL,
                 FA_ERR_SCALE, FA_ERR_ALIAS, FA_ERR_TOO_LARGE, FA_ERR_ALIGNMENT, FA_ERR_WINDOW,
                 FA_ERR_WORKSPACE, FA_ERR_UNSUPPORTED}


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIBRARY):
        raise ImportError(
            f"{LIBRARY} is not built; build it with `python -m exact_tiled_attention_06_amd.build` "
            "(there is no CPU fallback)")
    lib = ctypes.CDLL(LIBRARY)
    lib.fa_fwd.restype = ctypes.c_int
    lib.fa_fwd.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_void_p] + [ctypes.c_int64] * 4 + [
        ctypes.c_int, ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
    lib.fa_bwd.restype = ctypes.c_int
    lib.fa_bwd.argtypes = [ctypes.c_void_p] * 10 + [ctypes.c_int64] * 4 + [
        ctypes.c_int, ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
    I64, I, F, P = ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_void_p
    lib.fa_fwd_ex.restype = I
    lib.fa_fwd_ex.argtypes = [P] * 5 + [I64] * 6 + [I, I64, I64, F, I, P]
    lib.fa_bwd_ex.restype = I
    lib.fa_bwd_ex.argtypes = [P] * 10 + [I64] * 6 + [I, I64, I64, F, I, P]
    lib.fa_fwd_workspace_bytes.restype = I64
    lib.fa_fwd_workspace_bytes.argtypes = [I64] * 6 + [I, I64, I64, I]
    lib.fa_fwd_ws.restype = I
    lib.fa_fwd_ws.argtypes = [P] * 5 + [I64] * 6 + [I, I64, I64, F, I, P, I64, P]
    lib.fa_fwd_single_buffered.restype = I
    lib.fa_fwd_single_buffered.argtypes = [P] * 5 + [I64] * 4 + [I, F, I, P]
    lib.fa_bwd_noalloc.restype = I
    lib.fa_bwd_noalloc.argtypes = [P] * 9 + [I64] * 6 + [I, I64, I64, F, I, P]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_status_string.argtypes = [ctypes.c_int]
    return lib


_lib: ctypes.CDLL | None = None


def library() -> ctypes.CDLL:
    """libfa.so, loaded on first use (so that the build step can import this
    package before the library exists); raises ImportError when it is not built."""
    global _lib
    if _lib is None:
        _lib = _load()
    return _lib


class FaError(RuntimeError):
    def __init__(self, status: int):
        super().__init__(f"attention call failed: {fa_status_string(status)} (status {status})")
        self.status = status


class FaValueError(ValueError):
    def __init__(self, status: int):
        super().__init__(f"attention call rejected its arguments: {fa_status_string(status)} (status {status})")
        self.status = status


def fa_status_string(status: int) -> str:
    return library().fa_status_string(int(status)).decode()


def fa_fwd(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, S: int, D: int,
           causal: int, scale: float, dtype: int, stream: int) -> int:
    """The C entry point: raw device addresses and sizes; returns the status code."""
    return int(library().fa_fwd(q, k, v, o, lse, B, H, S, D, int(causal), float(scale), int(dtype), stream))


def fa_bwd(q: int, k: int, v: int, o: int, dout: int, lse: int, dq: int, dk: int, dv: int, delta: int,
           B: int, H: int, S: int, D: int, causal: int, scale: float, dtype: int, stream: int) -> int:
    """The C backward entry point: raw device addresses and sizes; returns the status code."""
    return int(library().fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, S, D, int(causal),
                                float(scale), int(dtype), stream))


def fa_fwd_ex(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, H_kv: int, S_q: int, S_k: int,
              D: int, causal: int, window_left: int, window_right: int, scale: float, dtype: int,
              stream: int) -> int:
    """The C forward with grouped K/V heads, query and key lengths S_q, S_k and a
    sliding window; returns the status code."""
    return int(library().fa_fwd_ex(q, k, v, o, lse, B, H, H_kv, S_q, S_k, D, int(causal), int(window_left),
                                   int(window_right), float(scale), int(dtype), stream))


def fa_fwd_workspace_bytes(B: int, H: int, H_kv: int, S_q: int, S_k: int, D: int, causal: int,
                           window_left: int, window_right: int, dtype: int) -> int:
    """Bytes of the workspace with which fa_fwd_ws splits the longest causal
    query blocks over two workgroups; 0 when the problem runs without one."""
    return int(library().fa_fwd_workspace_bytes(B, H, H_kv, S_q, S_k, D, int(causal), int(window_left),
                                                int(window_right), int(dtype)))


def fa_fwd_ws(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, H_kv: int, S_q: int, S_k: int,
              D: int, causal: int, window_left: int, window_right: int, scale: float, dtype: int,
              workspace: int, workspace_bytes: int, stream: int) -> int:
    """fa_fwd_ex with a caller-given device workspace (see fa_fwd_workspace_bytes);
    returns the status code."""
    return int(library().fa_fwd_ws(q, k, v, o, lse, B, H, H_kv, S_q, S_k, D, int(causal), int(window_left),
                                   int(window_right), float(scale), int(dtype), workspace, int(workspace_bytes),
                                   stream))


def fa_bwd_ex(q: int, k: int, v: int, o: int, dout: int, lse: int, dq: int, dk: int, dv: int, delta: int,
              B: int, H: int, H_kv: int, S_q: int, S_k: int, D: int, causal: int, window_left: int,
              window_right: int, scale: float, dtype: int, stream: int) -> int:
    """The C backward with grouped K/V heads, query and key lengths S_q, S_k and a
    sliding window; returns the status code."""
    return int(library().fa_bwd_ex(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, H_kv, S_q, S_k, D,
                                   int(causal), int(window_left), int(window_right), float(scale), int(dtype),
                                   stream))


def fa_fwd_single_buffered(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, S: int, D: int,
                           causal: int, scale: float, dtype: int, stream: int) -> int:
    """Race check: fa_fwd on the two-block kernel with single-buffered K/V
    staging (bit-identical results expected); returns the status code."""
    return int(library().fa_fwd_single_buffered(q, k, v, o, lse, B, H, S, D, int(causal), float(scale),
                                                int(dtype), stream))


def fa_bwd_noalloc(q: int, k: int, v: int, o: int, dout: int, lse: int, dq: int, dk: int, dv: int,
                   B: int, H: int, H_kv: int, S_q: int, S_k: int, D: int, causal: int, window_left: int,
                   window_right: int, scale: float, dtype: int, stream: int) -> int:
    """fa_bwd_ex without the delta workspace (the library's static array, for
    callers that cannot allocate); returns the status code."""
    return int(library().fa_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, B, H, H_kv, S_q, S_k, D, int(causal),
                                        int(window_left), int(window_right), float(scale), int(dtype), stream))


def _fp32(x: float) -> float:
    """x rounded to the nearest float32 (the C ABI's scale argument), without
    a tensor round trip on every call."""
    x = float(x)
    try:
        return struct.unpack("f", struct.pack("f", x))[0]
    except OverflowError:  # beyond float32: the library rejects the non-finite scale
        return math.copysign(math.inf, x)


def _window(window):
    if window is None:
        return -1, -1
    wl, wr = int(window[0]), int(window[1])
    return wl, wr


def _kv_shape_ok(q: torch.Tensor, k: torch.Tensor) -> bool:
    """k is [B,H_kv,S_k,D] for q [B,H,S_q,D]: same B and D, H a multiple of H_kv."""
    if k.dim() != 4 or k.shape[0] != q.shape[0] or k.shape[3] != q.shape[3]:
        return False
    hq, hk = q.shape[1], k.shape[1]
    return (hq == 0 and hk == 0) or (hk >= 1 and hq % hk == 0)


def check(status: int) -> None:
    if status == FA_OK:
        return
    if status in _VALUE_ERRORS:
        raise FaValueError(status)
    raise FaError(status)


def forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
            scale: float | None = None, out: torch.Tensor | None = None,
            lse: torch.Tensor | None = None, window=None):
    """Attention forward on device tensors q [B,H,S_q,D], k and v [B,H_kv,S_k,D]
    (H a multiple of H_kv); returns (o [B,H,S_q,D], lse [B,H,S_q]).  Causal means
    query i sees keys 0..i; ``window = (left, right)`` limits query i to keys
    i - left .. i + right (-1: unlimited side).  A row left with no key gets
    o = 0 and lse = -inf."""
    if q.dim() != 4:
        raise ValueError(f"q must be [B,H,S_q,D], got shape {tuple(q.shape)}")
    if not _kv_shape_ok(q, k) or v.shape != k.shape:
        raise ValueError(f"k, v must share a [B,H_kv,S_k,D] shape with q's B and D and H a multiple of H_kv: "
                         f"{tuple(q.shape)}, {tuple(k.shape)}, {tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in DTYPE_CODES:
        raise ValueError(f"q, k, v must share one of {list(DTYPE_CODES)}; got {q.dtype}, {k.dtype}, {v.dtype}")
    if not (q.is_cuda and k.is_cuda and v.is_cuda) or not (k.device == q.device and v.device == q.device):
        raise RuntimeError("q, k, v must be device tensors on one device")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    B, H, S, D = q.shape
    S_k = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    scale = _fp32(scale)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor of q's shape and dtype")
    if lse.shape != (B, H, S) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor of shape [B,H,S]")
    # the kernels write through these pointers: a host (or other-device) buffer
    # would hand the GPU an address it must not touch
    if out.device != q.device or lse.device != q.device:
        raise ValueError(f"out and lse must be on q's device {q.device}; got {out.device}, {lse.device}")
    stream = torch.cuda.current_stream(q.device).cuda_stream
    wl, wr = _window(window)
    code = DTYPE_CODES[q.dtype]
    # the workspace of the key split of the longest causal blocks (0 bytes for
    # most problems: then this is fa_fwd_ex)
    nbytes = fa_fwd_workspace_bytes(B, H, k.shape[1], S, S_k, D, int(bool(causal)), wl, wr, code)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device) if nbytes > 0 else None
    status = fa_fwd_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                       B, H, k.shape[1], S, S_k, D, int(bool(causal)), wl, wr, scale, code,
                       ws.data_ptr() if ws is not None else 0, nbytes, stream)
    check(status)
    return out, lse


def backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
             dout: torch.Tensor, causal: bool = False, scale: float | None = None, window=None):
    """Attention backward (fp16 / bf16): returns (dq, dk, dv), dk and dv shaped like k.

    q, o, dout are [B,H,S_q,D], k and v [B,H_kv,S_k,D]; o and lse are the
    forward's outputs for the same q, k, v, causal, scale and window; the
    D = rowsum(dout * o) workspace is allocated here."""
    ts = (q, k, v, o, dout)
    if q.dim() != 4 or o.shape != q.shape or dout.shape != q.shape or not _kv_shape_ok(q, k) or v.shape != k.shape:
        raise ValueError("q, o, dout must share one [B,H,S_q,D] shape and k, v one [B,H_kv,S_k,D] shape")
    if any(t.dtype != q.dtype for t in ts) or q.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("q, k, v, o, dout must share dtype float16 or bfloat16")
    if not all(t.is_cuda and t.device == q.device for t in ts + (lse,)):
        raise RuntimeError("all tensors must be device tensors on one device")
    if not all(t.is_contiguous() for t in ts + (lse,)):
        raise ValueError("all tensors must be contiguous")
    B, H, S, D = q.shape
    if lse.shape != (B, H, S) or lse.dtype != torch.float32:
        raise ValueError("lse must be a float32 tensor of shape [B,H,S]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    scale = _fp32(scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(k)
    delta = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    wl, wr = _window(window)
    status = fa_bwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                       dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(), B, H, k.shape[1], S,
                       k.shape[2], D, int(bool(causal)), wl, wr, scale, DTYPE_CODES[q.dtype], stream)
    check(status)
    return dq, dk, dv
