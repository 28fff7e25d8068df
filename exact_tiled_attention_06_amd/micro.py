"""Issue-rate microbenchmarks of the gfx950 instructions the attention kernels
use (binding of libfa_micro.so, declared in ``include/fa_micro.h``).

``table()`` runs every probe once on cuda:0 and returns rows of cycles per
instruction or per body, from which the vector-side bound of the attention
loop is stated: per attended (query, key) pair the forward issues one
exponential and a few vector ALU operations besides its 4*D matrix-core FLOPs
("Inside FlashAttention", section 4.1).
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_HERE, "libfa_micro.so")

OP_EXP, OP_FMA, OP_ADD, OP_CVT, OP_EXP16, OP_PKADD16, OP_MAX3 = range(7)
OP_NAMES = {OP_EXP: "v_exp_f32", OP_FMA: "v_fma_f32", OP_ADD: "v_add_f32", OP_CVT: "v_cvt_pk_f16_f32",
            OP_EXP16: "v_exp_f16", OP_PKADD16: "v_pk_add_f16", OP_MAX3: "v_max3_f32"}
MIXED, PRODUCTS, VECTOR, SPLIT = range(4)

_lib = None


def library() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            raise ImportError(f"{LIBRARY} is not built; build it with `python -m exact_tiled_attention_06_amd.build`")
        lib = ctypes.CDLL(LIBRARY)
        lib.fa_micro.restype = ctypes.c_int
        lib.fa_micro.argtypes = [ctypes.c_int] * 6 + [ctypes.c_void_p, ctypes.c_void_p]
        _lib = lib
    return _lib


def run(op: int, k: int, agpr: bool, mode: int, waves: int, iters: int = 2000) -> list:
    """Cycles each wave's loop took (one workgroup of `waves` waves on cuda:0)."""
    out = torch.zeros(waves, dtype=torch.int64, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    rc = library().fa_micro(op, k, int(agpr), mode, waves, iters, out.data_ptr(), stream)
    if rc != 0:
        raise RuntimeError(f"fa_micro({op}, {k}, {agpr}, {mode}, {waves}) failed with status {rc}")
    torch.cuda.synchronize()
    return [int(x) for x in out.cpu()]


def table(iters: int = 2000) -> list:
    """Every probe once; each row: what ran, and cycles per unit of work per wave."""
    rows = []

    def add(kind, unit_desc, per_unit, **kw):
        rows.append(dict(kind=kind, unit=unit_desc, cycles=round(per_unit, 2), **kw))

    run(OP_EXP, 4, False, VECTOR, 4, 10)  # warm up the clocks and the code objects
    # vector instructions alone: 32 per body, one and two waves per SIMD
    for op in OP_NAMES:
        for waves in (4, 8):
            c = run(op, 4, False, VECTOR, waves, iters)
            add("vector", f"{OP_NAMES[op]}, {waves // 4} wave(s)/SIMD", max(c) / (iters * 32),
                op=OP_NAMES[op], waves_per_simd=waves // 4)
    # matrix products alone: 8 per body on 4 independent accumulators
    for agpr in (False, True):
        for waves in (4, 8):
            c = run(OP_EXP, 0, agpr, PRODUCTS, waves, iters)
            add("mfma", f"32x32x16 f16, acc in {'AGPR' if agpr else 'VGPR'}, {waves // 4} wave(s)/SIMD",
                max(c) / (iters * 8), agpr=agpr, waves_per_simd=waves // 4)
    # one MFMA then k vector instructions, in every wave
    for agpr in (False, True):
        for op in (OP_EXP, OP_FMA):
            for k in (1, 2, 4, 8, 16):
                for waves in (4, 8):
                    c = run(op, k, agpr, MIXED, waves, iters)
                    add("mixed", f"MFMA + {k} x {OP_NAMES[op]}, acc in {'AGPR' if agpr else 'VGPR'}, "
                                 f"{waves // 4} wave(s)/SIMD", max(c) / (iters * 8),
                        op=OP_NAMES[op], k=k, agpr=agpr, waves_per_simd=waves // 4)
    # two waves per SIMD, one running MFMAs only and one vector work only
    for agpr in (False, True):
        for op in (OP_EXP, OP_FMA):
            for k in (2, 4, 8, 16):
                c = run(op, k, agpr, SPLIT, 8, iters)
                add("split", f"SIMD shared by an MFMA-only wave and a {8 * k} x {OP_NAMES[op]} wave, acc in "
                             f"{'AGPR' if agpr else 'VGPR'}: cycles per body, MFMA wave / vector wave",
                    max(c[:4]) / iters, vector_wave_cycles=round(max(c[4:]) / iters, 2),
                    op=OP_NAMES[op], k=k, agpr=agpr)
    return rows
