"""Seeded synthetic inputs for the prefill-attention workloads.

This module holds no attention arithmetic: it only draws lengths, cached
context sizes and bf16 tensors, so that the oracle and the HIP path can be fed
the same bytes.  Values are drawn on the CPU with ``torch.Generator`` from a
fixed seed as float32 N(0, 1) and rounded to bf16 (round-to-nearest-even);
lengths and contexts come from splitmix64 (Steele, Lea and Flood, "Fast
splittable pseudorandom number generators", OOPSLA 2014; the finaliser
constants are Stafford's "Mix13" as published with the algorithm), which is
language-independent.

The workloads stand in for the pages' prompts, which are real text of a few
hundred to several thousand tokens with a long-tailed length mix: a single
Llama-2-7B-shaped layer (32 heads x 128), a varlen batch 10/50/2048 [P3 §1
example batch], chunked prefill of an 8192-token prompt in 512-token chunks
beside decode rows [P3 §3; P2 §2.2], and a long-context log-uniform length
mix.  [P2] "大模型推理优化：Prefill、Decode与KV Cache的工程实践";
[P3] "大模型 Prompt Prefill 阶段的高效 Batching 与算子排布".
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

_MASK64 = (1 << 64) - 1


class SplitMix64:
    """splitmix64: a 64-bit Weyl sequence passed through a bijective mixer."""

    def __init__(self, seed: int):
        self.x = seed & _MASK64

    def next(self) -> int:
        self.x = (self.x + 0x9E3779B97F4A7C15) & _MASK64
        z = self.x
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
        return z ^ (z >> 31)

    def uniform(self) -> float:
        """A double in [0, 1) from the top 53 bits."""
        return (self.next() >> 11) * (1.0 / (1 << 53))


def default_scale(head_dim: int) -> float:
    """1/sqrt(head_dim) rounded to float32, the value a float argument carries."""
    return float(np.float32(1.0 / math.sqrt(head_dim)))


def randn_bf16(gen, shape):
    """float32 N(0,1) from ``gen`` rounded to bf16 (CPU tensor)."""
    import torch
    return torch.randn(*shape, generator=gen, dtype=torch.float32).to(torch.bfloat16)


def generator(seed: int):
    import torch
    g = torch.Generator()
    g.manual_seed(seed)
    return g


def cu_from_lengths(lengths: List[int]) -> List[int]:
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + int(n))
    return cu


def decode_contexts(seed: int = 4, rows: int = 64, lo: int = 256, hi: int = 4096) -> List[int]:
    """Cached context lengths of the decode rows: uniform integers in [lo, hi]."""
    sm = SplitMix64(seed)
    span = hi - lo + 1
    return [lo + int(math.floor(sm.uniform() * span)) for _ in range(rows)]


def loguniform_lengths(seed: int = 5, total: int = 65536, lo: int = 64,
                       hi: int = 32768, tail: Optional[int] = 32768) -> List[int]:
    """Lengths log-uniform in [lo, hi] summing to ``total``, then ``tail`` appended.

    Each draw is floor(exp(ln lo + u (ln hi - ln lo))) clamped to [lo, hi]; a
    draw that reaches the remainder takes the remainder and ends the list; a
    final piece shorter than ``lo`` is merged into the shortest earlier one.
    """
    sm = SplitMix64(seed)
    out: List[int] = []
    remaining = total
    a, b = math.log(lo), math.log(hi)
    while remaining > 0:
        n = int(math.floor(math.exp(a + sm.uniform() * (b - a))))
        n = max(lo, min(hi, n))
        if n >= remaining:
            n = remaining
        out.append(n)
        remaining -= n
    if len(out) > 1 and out[-1] < lo:
        last = out.pop()
        j = int(np.argmin(out))
        out[j] += last
    if tail:
        out.append(int(tail))
    return out


@dataclass
class Varlen:
    """A varlen prefill problem: flattened q [N, H, D], k/v [N, HK, D] plus
    cu_seqlens (HK = num_kv_heads, default H)."""
    name: str
    lengths: List[int]
    num_heads: int
    head_dim: int
    seed: int
    scale: float = 0.0
    cu_seqlens: List[int] = field(default_factory=list)
    num_kv_heads: int = 0

    def __post_init__(self):
        if not self.scale:
            self.scale = default_scale(self.head_dim)
        if not self.num_kv_heads:
            self.num_kv_heads = self.num_heads
        self.cu_seqlens = cu_from_lengths(self.lengths)

    @property
    def num_tokens(self) -> int:
        return self.cu_seqlens[-1]

    @property
    def max_seqlen(self) -> int:
        return max(self.lengths) if self.lengths else 0

    def tensors(self):
        """(q, k, v) as CPU bf16, q [N, H, D] and k, v [N, HK, D], drawn in
        that order from the seed."""
        g = generator(self.seed)
        q = randn_bf16(g, (self.num_tokens, self.num_heads, self.head_dim))
        kv = (self.num_tokens, self.num_kv_heads, self.head_dim)
        k = randn_bf16(g, kv)
        v = randn_bf16(g, kv)
        return q, k, v


@dataclass
class ChunkedStep:
    """One step of chunked prefill: a prompt chunk plus length-1 decode rows.

    Sequence 0 is chunk ``chunk`` of a ``prompt_len`` prompt (``chunk_len``
    new tokens, prefix ``chunk * chunk_len``); sequences 1..R are decode rows
    (1 new token each, prefix = that row's cached context).  The cache is
    [1 + R, HK, cap, D].
    """
    chunk: int
    prompt_len: int
    chunk_len: int
    contexts: List[int]
    num_heads: int
    head_dim: int
    cap: int
    scale: float = 0.0
    num_kv_heads: int = 0  # 0: as many as num_heads

    def __post_init__(self):
        if not self.scale:
            self.scale = default_scale(self.head_dim)
        if not self.num_kv_heads:
            self.num_kv_heads = self.num_heads

    @property
    def lengths(self) -> List[int]:
        return [self.chunk_len] + [1] * len(self.contexts)

    @property
    def prefix_lens(self) -> List[int]:
        return [self.chunk * self.chunk_len] + list(self.contexts)

    @property
    def cu_seqlens(self) -> List[int]:
        return cu_from_lengths(self.lengths)

    @property
    def num_seqs(self) -> int:
        return 1 + len(self.contexts)


class ChunkedWorkload:
    """Chunked prefill of one long prompt beside decode rows (all bf16 N(0,1)).

    Value draw order from ``seed``: prompt q [prompt_len, H, D], k, v
    [prompt_len, HK, D]; decode rows' q [R, H, D], k, v [R, HK, D]; then each
    decode row's cached prefix, K then V, [HK, ctx_r, D].  HK = num_kv_heads
    (default H).
    """

    def __init__(self, prompt_len=8192, chunk_len=512, rows=64, num_heads=32,
                 head_dim=128, seed=4, ctx_lo=256, ctx_hi=4096, cap=None, num_kv_heads=None):
        self.prompt_len = prompt_len
        self.chunk_len = chunk_len
        self.num_heads = num_heads
        self.num_kv_heads = num_kv_heads or num_heads
        self.head_dim = head_dim
        self.seed = seed
        self.contexts = decode_contexts(seed, rows, ctx_lo, ctx_hi) if rows else []
        self.cap = cap if cap is not None else max([prompt_len] + [c + 1 for c in self.contexts])
        self.scale = default_scale(head_dim)
        self.num_chunks = (prompt_len + chunk_len - 1) // chunk_len

    def step(self, c: int) -> ChunkedStep:
        n = min(self.chunk_len, self.prompt_len - c * self.chunk_len)
        st = ChunkedStep(c, self.prompt_len, self.chunk_len, self.contexts,
                         self.num_heads, self.head_dim, self.cap, self.scale, self.num_kv_heads)
        if n != self.chunk_len:
            raise ValueError("prompt length must be a multiple of the chunk length")
        return st

    def tensors(self):
        """Returns dict with prompt q/k/v, decode q/k/v and per-row prefix K/V lists."""
        g = generator(self.seed)
        H, HK, D = self.num_heads, self.num_kv_heads, self.head_dim
        pq = randn_bf16(g, (self.prompt_len, H, D))
        pk = randn_bf16(g, (self.prompt_len, HK, D))
        pv = randn_bf16(g, (self.prompt_len, HK, D))
        R = len(self.contexts)
        dq = randn_bf16(g, (R, H, D))
        dk = randn_bf16(g, (R, HK, D))
        dv = randn_bf16(g, (R, HK, D))
        pre_k, pre_v = [], []
        for ctx in self.contexts:
            pre_k.append(randn_bf16(g, (HK, ctx, D)))
            pre_v.append(randn_bf16(g, (HK, ctx, D)))
        return dict(pq=pq, pk=pk, pv=pv, dq=dq, dk=dk, dv=dv, pre_k=pre_k, pre_v=pre_v)


def workload(name: str):
    """The named synthetic workloads (sizes as in the measurement plan)."""
    if name == "single_T64_H4_D32":
        return Varlen(name, [64], 4, 32, seed=1)
    if name == "varlen_10_50_2048_H32_D128":
        return Varlen(name, [10, 50, 2048], 32, 128, seed=2)
    if name == "single_T2048_H32_D128":
        return Varlen(name, [2048], 32, 128, seed=3)
    if name == "chunked_8192x512_plus_64_decode_H32_D128":
        return ChunkedWorkload(seed=4)
    if name == "longmix_65536_plus_32768_H32_D128":
        return Varlen(name, loguniform_lengths(5), 32, 128, seed=5)
    if name == "single_T2048_H32_KV8_D128":
        return Varlen(name, [2048], 32, 128, seed=6, num_kv_heads=8)
    if name == "chunked_8192x512_plus_64_decode_H32_KV8_D128":
        return ChunkedWorkload(seed=7, num_kv_heads=8)
    raise KeyError(name)


WORKLOADS = [
    "single_T64_H4_D32",
    "varlen_10_50_2048_H32_D128",
    "single_T2048_H32_D128",
    "chunked_8192x512_plus_64_decode_H32_D128",
    "longmix_65536_plus_32768_H32_D128",
    "single_T2048_H32_KV8_D128",
    "chunked_8192x512_plus_64_decode_H32_KV8_D128",
]
