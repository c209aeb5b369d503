"""Seeded synthetic inputs for masked attention forward.

This module only draws numbers and describes workloads (shapes, sparse modes, lengths,
seeds). It holds none of the attention arithmetic, so the fp64 oracle and the HIP path can
both be fed from it. Everything is drawn with torch's CPU generator: float32 N(0, 1)
values, then rounded (round-to-nearest-even) to the working dtype.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def randn(shape, dtype: torch.dtype, seed: int) -> torch.Tensor:
    """float32 N(0,1) from a seeded CPU generator, cast to ``dtype``."""
    g = torch.Generator().manual_seed(int(seed))
    return torch.randn(tuple(shape), generator=g, dtype=torch.float32).to(dtype)


def lengths_uniform(count: int, lo: int, hi: int, seed: int) -> List[int]:
    """``count`` integers uniform in [lo, hi] (inclusive) from a seeded CPU generator."""
    g = torch.Generator().manual_seed(int(seed))
    return [int(x) for x in torch.randint(lo, hi + 1, (count,), generator=g)]


def cumulative_ends(lengths) -> List[int]:
    """Cumulative end offsets, one per sequence, without a leading zero (e.g. [3, 2] -> [3, 5])."""
    out, acc = [], 0
    for n in lengths:
        acc += int(n)
        out.append(acc)
    return out


def alibi_slopes(n_heads: int) -> List[float]:
    """Per-head alibi slopes 2^(-8 (h + 1) / N), h = 0 .. N-1."""
    return [2.0 ** (-8.0 * (h + 1) / n_heads) for h in range(n_heads)]


@dataclass
class Workload:
    """One synthetic attention-forward problem."""

    name: str
    layout: str                 # "BNSD" | "BSND" | "TND"
    dtype: str                  # "f32" | "f16" | "bf16"
    B: int
    N: int
    D: int
    Sq: int = 0                 # BNSD / BSND
    Skv: int = 0
    qlens: Optional[List[int]] = None   # TND per-sequence lengths
    kvlens: Optional[List[int]] = None
    sparse_mode: int = 0
    pre_tokens: int = 0
    next_tokens: int = 0
    prefix: Optional[List[int]] = None
    alibi: bool = False
    seed: int = 0
    scale: Optional[float] = None
    extra: dict = field(default_factory=dict)

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.D)

    @property
    def actual_seq_qlen(self):
        return cumulative_ends(self.qlens) if self.qlens is not None else None

    @property
    def actual_seq_kvlen(self):
        return cumulative_ends(self.kvlens) if self.kvlens is not None else None

    def shapes(self):
        """(q shape, k/v shape) in the workload's layout."""
        if self.layout == "BNSD":
            return (self.B, self.N, self.Sq, self.D), (self.B, self.N, self.Skv, self.D)
        if self.layout == "BSND":
            return (self.B, self.Sq, self.N, self.D), (self.B, self.Skv, self.N, self.D)
        return (sum(self.qlens), self.N, self.D), (sum(self.kvlens), self.N, self.D)

    def tensors(self):
        """Seeded CPU tensors q, k, v in the workload's dtype and layout."""
        qs, ks = self.shapes()
        dt = DTYPES[self.dtype]
        if "page_example" in self.extra:
            # (B, seq, d_head) from the exercise page, as BNSD with one head.
            q, k, v = page_example_tensors(self.extra["page_example"])
            return tuple(x.unsqueeze(1).to(dt).contiguous() for x in (q, k, v))
        return (randn(qs, dt, self.seed * 3 + 0), randn(ks, dt, self.seed * 3 + 1),
                randn(ks, dt, self.seed * 3 + 2))

    def slopes(self):
        return alibi_slopes(self.N) if self.alibi else None

    def mask(self):
        """(atten_mask, mask_bcast) of a sparse_mode=1 workload, else (None, None).

        "upper_triangle": one uint8 [1, 1, Sq, Skv] tensor shared by every batch and head, 1
        (masked) where j - i > Skv - Sq: the rightDownCausal pattern handed over as an explicit
        mask."""
        if self.extra.get("mask") == "upper_triangle":
            m = torch.ones(self.Sq, self.Skv, dtype=torch.uint8).triu(1 + self.Skv - self.Sq)
            return m[None, None].contiguous(), [1, 1]
        return None, None


NO_MASK = 2 ** 62   # a pre/next value that reaches past any sequence: "no mask" in mode 0


def page_example_tensors(example: int):
    """The two input specs of the tiling exercise page, in float64, shape (B, seq, d_head).

    Example 1 seeds torch's global generator with 42 and draws q, k, v = randn(2, 12, 16) in
    that order. Example 2 prints no seed: it is drawn here right after example 1 in the same
    session, i.e. from the generator state example 1 left behind.
    """
    torch.manual_seed(42)
    q1 = torch.randn(2, 12, 16, dtype=torch.float64)
    k1 = torch.randn(2, 12, 16, dtype=torch.float64)
    v1 = torch.randn(2, 12, 16, dtype=torch.float64)
    if example == 1:
        return q1, k1, v1
    q2 = torch.randn(1, 7, 8, dtype=torch.float64)
    k2 = torch.randn(1, 7, 8, dtype=torch.float64)
    v2 = torch.randn(1, 7, 8, dtype=torch.float64)
    return q2, k2, v2


def workloads() -> dict:
    """The named workloads: parity cases and the benchmark shape."""
    w = {}
    w["tiny_f32"] = Workload("tiny_f32", "BNSD", "f32", 2, 1, 16, 12, 12, sparse_mode=0,
                             pre_tokens=NO_MASK, next_tokens=NO_MASK, seed=42, scale=0.25,
                             extra={"page_example": 1})
    w["tiny_f32_causal"] = Workload("tiny_f32_causal", "BNSD", "f32", 2, 1, 16, 12, 12,
                                    sparse_mode=0, pre_tokens=12, next_tokens=0, seed=42,
                                    scale=0.25, extra={"page_example": 1})
    w["causal_2048"] = Workload("causal_2048", "BNSD", "bf16", 4, 32, 128, 2048, 2048,
                                sparse_mode=3, seed=2)
    w["band_8192"] = Workload("band_8192", "BNSD", "bf16", 2, 32, 128, 8192, 8192,
                              sparse_mode=4, pre_tokens=1024, next_tokens=0, seed=3)
    w["band_neg_16"] = Workload("band_neg_16", "BNSD", "bf16", 1, 1, 128, 16, 16,
                                sparse_mode=0, pre_tokens=9, next_tokens=-3, seed=31)
    w["band_neg_8192"] = Workload("band_neg_8192", "BNSD", "bf16", 2, 32, 128, 8192, 8192,
                                  sparse_mode=0, pre_tokens=1024, next_tokens=-256, seed=32)
    w["causal_8192"] = Workload("causal_8192", "BNSD", "bf16", 2, 32, 128, 8192, 8192,
                                sparse_mode=3, seed=8)
    # The headline's shape and inputs with sparseMode=1: the same causal pattern, read from an
    # explicit uint8 mask shared by every batch and head.
    w["causal_8192_mask"] = Workload("causal_8192_mask", "BNSD", "bf16", 2, 32, 128, 8192, 8192,
                                     sparse_mode=1, seed=8, extra={"mask": "upper_triangle"})
    lens = lengths_uniform(16, 128, 4096, seed=4)
    w["varlen_tnd"] = Workload("varlen_tnd", "TND", "bf16", 16, 32, 128, qlens=lens,
                               kvlens=list(lens), sparse_mode=3, seed=4)
    w["prefix_alibi"] = Workload("prefix_alibi", "BNSD", "f16", 4, 16, 128, 4096, 8192,
                                 sparse_mode=5, prefix=lengths_uniform(4, 0, 4096, seed=5),
                                 alibi=True, seed=5)
    w["prefix_alibi_square"] = Workload("prefix_alibi_square", "BNSD", "f16", 4, 16, 128,
                                        4096, 4096, sparse_mode=5,
                                        prefix=lengths_uniform(4, 0, 4096, seed=55),
                                        alibi=True, seed=55)
    # Decode shapes (split-KV path): one query row per sequence against a long K/V, a
    # speculative-decode block of 8 rows, and a varlen decode batch of 32 sequences.
    w["decode_32k"] = Workload("decode_32k", "BNSD", "bf16", 4, 32, 128, 1, 32768, sparse_mode=3, seed=60)
    w["decode_spec8_8k"] = Workload("decode_spec8_8k", "BSND", "bf16", 8, 32, 128, 8, 8192, sparse_mode=3,
                                    seed=61)
    kvl = lengths_uniform(32, 256, 8192, seed=62)
    w["decode_varlen"] = Workload("decode_varlen", "TND", "bf16", 32, 32, 128, qlens=[1] * 32, kvlens=kvl,
                                  sparse_mode=3, seed=62)
    return w
