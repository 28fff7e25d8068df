"""Seeded synthetic attention workloads.

This module only draws inputs: it holds none of the attention arithmetic, so the
oracle and the HIP path can both be fed from it without sharing any of the
method's code.

Every input is ``torch.randn`` of shape [B, H, S, D], drawn in float32 on the
CPU from ``torch.Generator().manual_seed(seed)`` in the order q, k, v, then
rounded to the workload dtype (round to nearest even).  This mirrors the pages'
own workloads, which are all standard-normal random tensors ("T5 讲解：
FlashAttention forward", section ①, test scale B=4, H=16, S=4096, D=64 fp16; the
CS336 write-up's benchmark harnesses).

The named workloads:

  single_head_f32     B=1 H=1  S=256   D=64  fp32  non-causal         seed 1
  batch_f16           B=8 H=1  S=4096  D=64  fp16  causal and not      seed 2
  multihead_causal    B=4 H=16 S=4096  D=64  fp16  causal             seed 3
  long_seq_bf16       B=8 H=1  S=16384 D=128 bf16  causal             seed 4
  gqa_causal          B=4 H=16 H_kv=4 S=4096 D=64 fp16 causal   seed 5
  window_causal       B=2 H=16 S=8192 D=64 fp16 causal, window (1024, 0)  seed 6
  sweep_D{d}_S{s}     B=8 H=1  D in {16,32,64,128} x S in {256,1024,4096,8192,16384}
                      fp16 causal, seeds 500..519 in D-major order
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Tuple

import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
# integer codes of the C ABI's dtype argument
DTYPE_CODES = {"f32": 0, "f16": 1, "bf16": 2}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    S: int
    D: int
    dtype: str
    causal: Tuple[bool, ...]
    seed: int
    hkv: int = 0                         # key/value heads (0: as many as query heads)
    window: Tuple[int, int] = (-1, -1)   # (left, right); -1: unlimited side

    @property
    def kv_heads(self) -> int:
        return self.hkv or self.H

    @property
    def scale(self) -> float:
        """1/sqrt(D), rounded to float32 (the value the kernel receives)."""
        return float(torch.tensor(1.0 / math.sqrt(self.D), dtype=torch.float32))

    def flops(self, causal: bool) -> float:
        """4*B*H*S^2*D, halved for causal; with a window, 4*B*H*D times the number
        of (query, key) pairs the window admits."""
        if self.window == (-1, -1):
            f = 4.0 * self.B * self.H * self.S * self.S * self.D
            return f / 2 if causal else f
        wl, wr = self.window
        i = torch.arange(self.S, dtype=torch.float64)
        lo = torch.clamp(i - wl, min=0) if wl >= 0 else torch.zeros_like(i)
        hi = i if causal else torch.full_like(i, self.S - 1)
        if wr >= 0:
            hi = torch.minimum(hi, torch.clamp(i + wr, max=self.S - 1))
        pairs = float((hi - lo + 1).sum())
        return 4.0 * self.B * self.H * pairs * self.D

    def hbm_bytes(self) -> int:
        """Q, K, V read once, O written once (element size e), lse written in fp32."""
        e = torch.tensor([], dtype=DTYPES[self.dtype]).element_size()
        n = self.B * self.H * self.S
        nkv = self.B * self.kv_heads * self.S
        return 2 * n * self.D * e + 2 * nkv * self.D * e + 4 * n


def make_inputs(B: int, H: int, S: int, D: int, dtype: str, seed: int):
    """q, k, v as CPU tensors of ``dtype``: randn in float32 from ``seed`` (q, k, v order), then rounded."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    shape = (B, H, S, D)
    out = []
    for _ in range(3):
        x = torch.randn(shape, dtype=torch.float32, generator=g)
        out.append(x.to(DTYPES[dtype]).contiguous())
    return tuple(out)


def make_grad(B: int, H: int, S: int, D: int, dtype: str, seed: int):
    """An upstream gradient dO for the backward: randn [B,H,S,D] in float32 from
    ``seed``, rounded to ``dtype`` (drawn apart from q, k, v)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    x = torch.randn((B, H, S, D), dtype=torch.float32, generator=g)
    return x.to(DTYPES[dtype]).contiguous()


def workload_inputs(w: Workload):
    """q [B,H,S,D]; k, v [B,H_kv,S,D] (drawn after q from the same generator)."""
    if w.kv_heads == w.H:
        return make_inputs(w.B, w.H, w.S, w.D, w.dtype, w.seed)
    g = torch.Generator(device="cpu")
    g.manual_seed(int(w.seed))
    q = torch.randn((w.B, w.H, w.S, w.D), dtype=torch.float32, generator=g).to(DTYPES[w.dtype]).contiguous()
    kv = [torch.randn((w.B, w.kv_heads, w.S, w.D), dtype=torch.float32, generator=g).to(DTYPES[w.dtype]).contiguous()
          for _ in range(2)]
    return q, kv[0], kv[1]


SINGLE_HEAD_F32 = Workload("single_head_f32", 1, 1, 256, 64, "f32", (False,), 1)
BATCH_F16 = Workload("batch_f16", 8, 1, 4096, 64, "f16", (False, True), 2)
MULTIHEAD_CAUSAL = Workload("multihead_causal", 4, 16, 4096, 64, "f16", (True,), 3)
LONG_SEQ_BF16 = Workload("long_seq_bf16", 8, 1, 16384, 128, "bf16", (True,), 4)


def sweep() -> List[Workload]:
    out = []
    seed = 500
    for d in (16, 32, 64, 128):
        for s in (256, 1024, 4096, 8192, 16384):
            out.append(Workload(f"sweep_D{d}_S{s}", 8, 1, s, d, "f16", (True,), seed))
            seed += 1
    return out


# grouped heads and a sliding window ("Inside FlashAttention", section 6.1)
GQA_CAUSAL = Workload("gqa_causal", 4, 16, 4096, 64, "f16", (True,), 5, hkv=4)
WINDOW_CAUSAL = Workload("window_causal", 2, 16, 8192, 64, "f16", (True,), 6, window=(1024, 0))

ALL = [SINGLE_HEAD_F32, BATCH_F16, MULTIHEAD_CAUSAL, LONG_SEQ_BF16, GQA_CAUSAL, WINDOW_CAUSAL] + sweep()
BY_NAME = {w.name: w for w in ALL}
