"""Seeded synthetic inputs for the attention-forward workloads.

This module generates inputs only: it holds none of the attention arithmetic.
Both the HIP path (through the tests and the benchmark) and the CPU oracle
consume exactly the tensors made here.

The workloads follow the kernel benchmarks described in the IPLEX blog
"FlashAttention-2: making long-context attention run efficiently on GPUs",
section "Read the reported speed-ups with their conditions": sequence lengths
from 512 to about 16k, head dimensions 64 and 128, causal masking on and off,
and a total of 16k tokens per batch.  The pages use synthetic shapes and name
no dataset, so no dataset is stood in for.

Recipe (the pages give none; this is the plainest reading):
  * Q, K, V are i.i.d. N(0, 1) float32 drawn on the CPU from a seeded
    ``torch.Generator`` in the order Q, K, V;
  * the long-sequence causal workload additionally multiplies, per (b, h),
    exactly round(0.01 * S) key rows by 8 (rows picked by a seeded randperm,
    drawn after V in b-major, h-minor order) -- a peaky-softmax stress;
  * the float32 values are then rounded to the workload dtype with
    round-to-nearest-even (torch's cast).  Scaling by 8 is a power of two and
    commutes with that rounding.
  * scale = float32(1 / sqrt(d)).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "SWEEP", "DECODE", "DecodeWorkload", "make_inputs", "make_inputs_kv",
           "default_scale", "torch_dtype"]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    S: int
    d: int
    dtype: str          # "fp16" or "bf16"
    causal: bool
    seed: int
    peaky_frac: float = 0.0   # fraction of K rows per head multiplied by peaky_mult
    peaky_mult: float = 8.0

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads, in order: tiny, short-sequence batch, mid-sequence causal,
# long-sequence causal with peaky keys, single-sequence stress.
WORKLOADS = (
    Workload("tiny", 1, 2, 128, 64, "fp16", False, 1001),
    Workload("short_seq_batch", 32, 32, 512, 64, "bf16", False, 1002),
    Workload("mid_seq_causal", 8, 16, 2048, 128, "bf16", True, 1003),
    Workload("long_seq_causal", 2, 16, 8192, 128, "bf16", True, 1004, peaky_frac=0.01),
    Workload("single_seq_stress", 1, 32, 16384, 64, "fp16", False, 1005),
)
WORKLOADS_BY_NAME = {w.name: w for w in WORKLOADS}

# The pages' kernel-benchmark grid (same blog section): S from 512 to 16k,
# d in {64, 128}, causal off and on, 16k tokens per batch (B = 16384 / S).
# The pages give no head count; H = 2048 / d (a 2048-wide model) is taken.
# bf16 throughout; seeds 2001.. in grid order.
SWEEP = tuple(
    Workload(f"sweep_S{S}_d{d}_{'causal' if causal else 'full'}", 16384 // S, 2048 // d, S, d, "bf16", causal,
             2001 + i)
    for i, (S, d, causal) in enumerate(
        (S, d, causal) for d in (64, 128) for causal in (False, True)
        for S in (512, 1024, 2048, 4096, 8192, 16384)))
SWEEP_BY_NAME = {w.name: w for w in SWEEP}


def torch_dtype(name: str) -> torch.dtype:
    return {"fp16": torch.float16, "bf16": torch.bfloat16}[name]


def default_scale(d: int) -> float:
    """float32(1/sqrt(d)), returned as a Python float holding that fp32 value."""
    return float(np.float32(1.0 / math.sqrt(d)))


def peaky_rows(w: Workload, g: torch.Generator) -> torch.Tensor:
    """[B, H, n] indices of the K rows to scale (drawn after Q, K, V)."""
    n = int(round(w.peaky_frac * w.S))
    out = torch.empty((w.B, w.H, n), dtype=torch.int64)
    for b in range(w.B):
        for h in range(w.H):
            out[b, h] = torch.randperm(w.S, generator=g)[:n]
    return out


def make_inputs(w: Workload, seed: int | None = None):
    """Return (q, k, v) as contiguous CPU tensors [B, H, S, d] of w.dtype."""
    g = torch.Generator().manual_seed(w.seed if seed is None else seed)
    shape = (w.B, w.H, w.S, w.d)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    if w.peaky_frac > 0:
        rows = peaky_rows(w, g)
        for b in range(w.B):
            for h in range(w.H):
                k[b, h, rows[b, h]] *= w.peaky_mult
    dt = torch_dtype(w.dtype)
    return q.to(dt).contiguous(), k.to(dt).contiguous(), v.to(dt).contiguous()


def make_inputs_kv(B: int, H: int, Sq: int, Sk: int, d: int, dtype: str, seed: int):
    """(q [B, H, Sq, d], k, v [B, H, Sk, d]) by the same recipe as make_inputs:
    i.i.d. N(0, 1) float32 drawn in the order Q, K, V, rounded to dtype."""
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((B, H, Sq, d), generator=g, dtype=torch.float32)
    k = torch.randn((B, H, Sk, d), generator=g, dtype=torch.float32)
    v = torch.randn((B, H, Sk, d), generator=g, dtype=torch.float32)
    dt = torch_dtype(dtype)
    return q.to(dt).contiguous(), k.to(dt).contiguous(), v.to(dt).contiguous()


@dataclass(frozen=True)
class DecodeWorkload:
    """Sq new queries per head over Sk cached keys (token-by-token decoding)."""
    name: str
    B: int
    H: int
    Sq: int
    Sk: int
    d: int
    dtype: str
    causal: bool
    seed: int

    def inputs(self):
        return make_inputs_kv(self.B, self.H, self.Sq, self.Sk, self.d, self.dtype, self.seed)


# Decoding workloads.  The pages contrast decoding with prompt processing but
# give no decoding shapes; these take the benchmark grid's model widths (2048
# = H * d) with one new token per sequence, at three batch / context mixes of
# equal K/V size (1 GiB of bf16 K and V per call): many short contexts, a
# typical batch, one long context.  The new token is the last position of
# its sequence, so the end-aligned causal mask keeps every key; causal is on.
DECODE = (
    DecodeWorkload("decode_B64_S2048_d64", 64, 32, 1, 2048, 64, "bf16", True, 3001),
    DecodeWorkload("decode_B16_S8192_d128", 16, 16, 1, 8192, 128, "bf16", True, 3002),
    DecodeWorkload("decode_B1_S131072_d128", 1, 16, 1, 131072, 128, "bf16", True, 3003),
)
DECODE_BY_NAME = {w.name: w for w in DECODE}

# Wide heads (d = 192, 256; beyond the pages' grid): the grid's 16k tokens at
# S = 4096 with 8 heads, bf16.
WIDE = (
    Workload("wide_S4096_d256_full", 4, 8, 4096, 256, "bf16", False, 3101),
    Workload("wide_S4096_d256_causal", 4, 8, 4096, 256, "bf16", True, 3102),
    Workload("wide_S4096_d192_full", 4, 8, 4096, 192, "bf16", False, 3103),
)
