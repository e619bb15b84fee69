"""Seeded synthetic inputs at the shapes of the pages' workloads (Qwen3-shaped).

Used by the tests and by ``bench.py``; it feeds both the HIP library and the
fp64 oracle and holds none of the method's arithmetic: it only draws numbers,
rounds them to bfloat16 (torch's round-to-nearest-even cast) and does the host
bookkeeping of a paged KV cache (page allocation, block tables, slot mapping).

Seeding: every request's data is drawn from a generator seeded by
(workload seed, tensor kind, request id), never by its slot in a batch, so a
request's bytes are identical in every batch it is placed in.  Weights use the
request id ``WEIGHTS``.

Models (Qwen3-8B, Qwen3-235B-A22B) and their weights are not available; N(0, 1)
activations and N(0, 0.02) weights at the models' shapes stand in for them.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

WEIGHTS = 999_983          # request id reserved for weight tensors
_KINDS = {"x": 1, "gamma": 2, "w": 3, "q": 4, "k": 5, "v": 6, "len": 7, "perm": 8,
          "route": 9, "logits": 10, "misc": 11, "gate": 12}

PAGE = 16                  # KV page size (tokens per page)


def seed_of(base: int, kind: str, index: int) -> int:
    return (int(base) * 1_000_003 + _KINDS[kind] * 65_537 + int(index) * 7_919) % (2 ** 62)


def gen(base: int, kind: str, index: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed_of(base, kind, index))
    return g


def randn_bf16(shape, base: int, kind: str, index: int, std: float = 1.0, mean: float = 0.0,
               device="cpu") -> torch.Tensor:
    """N(mean, std^2) drawn in fp32 then rounded to bf16.  Values depend on the
    device that draws them (CPU and GPU generators differ); a test draws once
    and hands the same bytes to the library and to the oracle."""
    x = torch.randn(*shape, generator=gen(base, kind, index, device), dtype=torch.float32, device=device)
    if std != 1.0:
        x = x * std
    if mean != 0.0:
        x = x + mean
    return x.to(torch.bfloat16)


def randn_f32(shape, base: int, kind: str, index: int, std: float = 1.0) -> torch.Tensor:
    x = torch.randn(*shape, generator=gen(base, kind, index), dtype=torch.float32)
    return x * std if std != 1.0 else x


def rand_int(lo: int, hi: int, base: int, kind: str, index: int) -> int:
    """Uniform integer in [lo, hi] (inclusive)."""
    return int(torch.randint(lo, hi + 1, (1,), generator=gen(base, kind, index)).item())


def rows_for_requests(requests: Sequence[int], width: int, base: int, kind: str = "x",
                      std: float = 1.0, device="cpu") -> torch.Tensor:
    """Stack one seeded [width] bf16 row per request id."""
    return torch.stack([randn_bf16((width,), base, kind, r, std=std, device=device) for r in requests]) \
        if len(requests) else torch.empty((0, width), dtype=torch.bfloat16, device=device)


def moe_weights(num_experts: int, hidden: int, ffn: int, base: int, std_up: float = 0.02,
                std_down: float = 0.02, device="cpu"):
    """Expert weights w_up [E, ffn, hidden] and w_down [E, hidden, ffn] (bf16),
    one seeded draw per expert and matrix."""
    w_up = torch.empty((num_experts, ffn, hidden), dtype=torch.bfloat16, device=device)
    w_down = torch.empty((num_experts, hidden, ffn), dtype=torch.bfloat16, device=device)
    for e in range(num_experts):
        w_up[e] = randn_bf16((ffn, hidden), base, "w", WEIGHTS + 2 * e + 1, std=std_up, device=device)
        w_down[e] = randn_bf16((hidden, ffn), base, "w", WEIGHTS + 2 * e + 2, std=std_down, device=device)
    return w_up, w_down


# ---------------------------------------------------------------- paged KV cache

@dataclass
class PagedBatch:
    """Host-side description of a batch of requests over a paged KV pool."""
    seq_lens: List[int]                  # tokens in each request's cache
    block_table: torch.Tensor            # [B, max_pages] int32 (unused entries = -1)
    num_pages: int                       # pool size
    slot_mapping: torch.Tensor           # [sum L] int32: physical slot of every token, request-major
    page_size: int = PAGE

    @property
    def max_pages(self) -> int:
        return int(self.block_table.shape[1])


def allocate_pages(seq_lens: Sequence[int], base: int, page_size: int = PAGE,
                   extra_pages: int = 3, perm_index: int = 0,
                   max_pages: Optional[int] = None) -> PagedBatch:
    """Give every request ceil(L / page) physical pages drawn from a seeded
    random permutation of a pool (plus ``extra_pages`` never used)."""
    need = [(L + page_size - 1) // page_size for L in seq_lens]
    total = sum(need) + extra_pages
    perm = torch.randperm(total, generator=gen(base, "perm", perm_index)).to(torch.int32)
    mp = max(need + [1]) if max_pages is None else max_pages
    bt = torch.full((len(seq_lens), mp), -1, dtype=torch.int32)
    slots = []
    at = 0
    for b, (L, n) in enumerate(zip(seq_lens, need)):
        pages = perm[at:at + n]
        at += n
        bt[b, :n] = pages
        t = torch.arange(L, dtype=torch.int32)
        slots.append(pages[(t // page_size).long()] * page_size + t % page_size)
    sm = torch.cat(slots) if slots else torch.empty((0,), dtype=torch.int32)
    return PagedBatch(list(seq_lens), bt, total, sm, page_size)


def request_kv(request: int, length: int, num_kv_heads: int, head_dim: int, base: int, device="cpu"):
    """Request ``request``'s logical K and V [length, Hkv, D] (bf16), seeded by
    (workload, request id)."""
    k = randn_bf16((length, num_kv_heads, head_dim), base, "k", request, device=device)
    v = randn_bf16((length, num_kv_heads, head_dim), base, "v", request, device=device)
    return k, v


def request_kv_prefix_stable(request: int, length: int, num_kv_heads: int, head_dim: int,
                             base: int, block: int = 256, device="cpu"):
    """Like ``request_kv`` but token rows are drawn per 256-token block, so the
    first L tokens are identical for every total length >= L (growing caches)."""
    ks, vs = [], []
    for blk in range((length + block - 1) // block):
        n = min(block, length - blk * block)
        idx = request * 4096 + blk
        ks.append(randn_bf16((block, num_kv_heads, head_dim), base, "k", idx, device=device)[:n])
        vs.append(randn_bf16((block, num_kv_heads, head_dim), base, "v", idx, device=device)[:n])
    if not ks:
        z = torch.empty((0, num_kv_heads, head_dim), dtype=torch.bfloat16, device=device)
        return z, z.clone()
    return torch.cat(ks), torch.cat(vs)


# ---------------------------------------------------------------- workloads

# Model shapes named by the workloads.
QWEN3_8B = dict(hidden=4096, q_heads=32, kv_heads=8, head_dim=128, mlp=12288, qkv=6144)
QWEN3_235B = dict(hidden=4096, q_heads=64, kv_heads=4, head_dim=128, experts=128, top_k=8,
                  expert_ffn=1536, vocab=151936)
TINY = dict(hidden=512, out=1024, head_dim=64, q_heads=1, kv_heads=1)

SEED_TINY, SEED_DECODE, SEED_MIXED, SEED_LONG, SEED_MOE = 0, 2, 3, 4, 5


def decode_lengths(requests: Sequence[int], base: int, lo: int = 1, hi: int = 4096) -> List[int]:
    """Per-request KV length, uniform in [lo, hi], seeded by request id."""
    return [rand_int(lo, hi, base, "len", r) for r in requests]


def moe_routing(tokens: Sequence[int], num_experts: int, top_k: int, base: int):
    """Per token: top_k distinct experts drawn uniformly, and fp32 weights that are
    the softmax of top_k seeded N(0,1) logits.  Seeded by token id."""
    experts = torch.empty((len(tokens), top_k), dtype=torch.int32)
    logits = torch.empty((len(tokens), top_k), dtype=torch.float32)
    for i, t in enumerate(tokens):
        g = gen(base, "route", t)
        experts[i] = torch.randperm(num_experts, generator=g)[:top_k].to(torch.int32)
        logits[i] = torch.randn(top_k, generator=g)
    weights = torch.softmax(logits, dim=-1)
    return experts, weights
