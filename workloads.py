"""Seeded synthetic inputs for paged decode attention.

This module is shared by the oracle's tests, the GPU parity tests and the
benchmark. It draws random numbers and lays out shapes; it performs none of
the attention arithmetic, none of the paging address arithmetic and none of
the FP8 coding, so that neither side of a parity check can lean on the other.

The shapes stand in for the decode workloads the pages discuss:

* Llama-3.1-8B GQA head shape (32 query heads, 8 KV heads, head dim 128,
  32 layers) -- "LLM에서 KV 캐시는 얼마나 생길까" (froggydisk), section on the
  size of one token, and "The KV Cache Is the New Memory Wall" review, §2.1.
* Llama-3-70B (64 query heads, 8 KV heads, head dim 128, 80 layers) at a
  131,072-token context -- same sources, §2.1 / Tab. 1 and the 128k workloads
  of §4.
* 16-token blocks assigned through a per-sequence block table -- froggydisk,
  section on techniques that shrink the KV cache (PagedAttention).

No dataset is used; every tensor is drawn from a seeded generator.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np

BLOCK_SIZE = 16


@dataclass(frozen=True)
class DecodeWorkload:
    """Shape and value recipe of one decode-step workload."""

    name: str
    seed: int
    b: int                      # sequences in the batch
    layers: int                 # layers run back to back in one step
    n_q: int                    # query heads
    n_kv: int                   # KV heads
    head_dim: int
    ctx: Tuple                  # ("fixed", s) or ("uniform", lo, hi) inclusive
    pool_blocks: Optional[int] = None   # None: exactly the blocks the batch needs
    kv_dtype: str = "bf16"      # "bf16" or "fp8"
    channel_scale: bool = False  # per-(kv-head, channel) magnitudes ~ U[0.5, 2]
    scores: bool = False        # fused cumulative score output requested
    shared_prefix: int = 0      # leading tokens whose blocks every sequence shares (multiple of 16)

    @property
    def g(self) -> int:
        return self.n_q // self.n_kv

    def with_(self, **kw) -> "DecodeWorkload":
        return dataclasses.replace(self, **kw)


# The five workloads.  Names describe the shape; seeds are fixed per workload.
WORKLOADS = {
    "tiny": DecodeWorkload("tiny-g4-d64-s256", seed=1, b=1, layers=1, n_q=4, n_kv=1,
                           head_dim=64, ctx=("fixed", 256), pool_blocks=16),
    "8b_layer": DecodeWorkload("llama3.1-8b-1layer-b1-s32768", seed=2, b=1, layers=1,
                               n_q=32, n_kv=8, head_dim=128, ctx=("fixed", 32768),
                               pool_blocks=4096, channel_scale=True),
    "8b_ragged": DecodeWorkload("llama3.1-8b-32layer-b32-s4k..16k", seed=3, b=32,
                                layers=32, n_q=32, n_kv=8, head_dim=128,
                                ctx=("uniform", 4096, 16384)),
    "70b_long": DecodeWorkload("llama3-70b-80layer-b4-s131072", seed=4, b=4, layers=80,
                               n_q=64, n_kv=8, head_dim=128, ctx=("fixed", 131072)),
    # one GPU's share of the 70B request when its context is split over 8 GPUs
    "70b_shard": DecodeWorkload("llama3-70b-80layer-b4-s16384-context-shard-of-8", seed=6, b=4,
                                layers=80, n_q=64, n_kv=8, head_dim=128, ctx=("fixed", 16384)),
    # 32 requests behind one 16,384-token system prompt whose blocks they all share
    "8b_prefix": DecodeWorkload("llama3.1-8b-8layer-b32-shared16k+1k", seed=7, b=32, layers=8,
                                n_q=32, n_kv=8, head_dim=128, ctx=("fixed", 17408),
                                shared_prefix=16384),
    # a serving batch of 256 requests behind one 8,192-token system prompt
    "8b_prefix256": DecodeWorkload("llama3.1-8b-8layer-b256-shared8k+512", seed=9, b=256, layers=8,
                                   n_q=32, n_kv=8, head_dim=128, ctx=("fixed", 8704),
                                   shared_prefix=8192),
    # 1,024 requests behind one 4,096-token system prompt
    "8b_prefix1024": DecodeWorkload("llama3.1-8b-8layer-b1024-shared4k+256", seed=10, b=1024, layers=8,
                                    n_q=32, n_kv=8, head_dim=128, ctx=("fixed", 4352),
                                    shared_prefix=4096),
    # a large serving batch: 256 requests of 1k..4k tokens
    "8b_batch256": DecodeWorkload("llama3.1-8b-32layer-b256-s1k..4k", seed=8, b=256, layers=32,
                                  n_q=32, n_kv=8, head_dim=128, ctx=("uniform", 1024, 4096)),
    "8b_fp8_scores": DecodeWorkload("llama3.1-8b-fp8-scores-32layer-b32-s8k..32k", seed=5,
                                    b=32, layers=32, n_q=32, n_kv=8, head_dim=128,
                                    ctx=("uniform", 8192, 32768), kv_dtype="fp8",
                                    scores=True),
}


def cdiv(a: int, b: int) -> int:
    return -(-a // b)


def context_lengths(w: DecodeWorkload, rng: Optional[np.random.Generator] = None) -> np.ndarray:
    """Context length per sequence (the current token included)."""
    rng = rng or np.random.default_rng(w.seed)
    if w.ctx[0] == "fixed":
        return np.full(w.b, int(w.ctx[1]), dtype=np.int32)
    lo, hi = int(w.ctx[1]), int(w.ctx[2])
    return rng.integers(lo, hi + 1, size=w.b).astype(np.int32)


def block_tables(w: DecodeWorkload, lens: np.ndarray,
                 rng: Optional[np.random.Generator] = None,
                 pad_value: int = -1) -> Tuple[np.ndarray, int]:
    """Scatter every sequence's logical blocks over a shuffled physical pool.

    Returns ``(table, num_blocks)``; ``table`` is int32 ``[b][max_blocks]`` and
    entries past a sequence's last block hold ``pad_value``.
    """
    rng = rng or np.random.default_rng(w.seed + 1000)
    need = [cdiv(int(s), BLOCK_SIZE) for s in lens]
    shared = w.shared_prefix // BLOCK_SIZE
    if w.shared_prefix % BLOCK_SIZE or any(n < shared for n in need):
        raise ValueError("the shared prefix must be whole blocks inside every sequence")
    total = shared + sum(n - shared for n in need)
    num_blocks = w.pool_blocks if w.pool_blocks is not None else total
    if num_blocks < total:
        raise ValueError(f"pool of {num_blocks} blocks cannot hold {total}")
    perm = rng.permutation(num_blocks).astype(np.int32)
    max_blocks = max(max(need, default=0), 1)
    table = np.full((len(need), max_blocks), pad_value, dtype=np.int32)
    cur = shared
    for i, n in enumerate(need):
        table[i, :shared] = perm[:shared]
        table[i, shared:n] = perm[cur:cur + n - shared]
        cur += n - shared
    return table, num_blocks


def _torch():
    import torch
    return torch


def _gen(device, seed: int):
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def query(w: DecodeWorkload, layer: int, device="cpu"):
    """q, bf16 ``[b][n_q][head_dim]``, N(0, 1) drawn in fp32 then cast."""
    torch = _torch()
    g = _gen(device, w.seed * 1_000_003 + 7919 * layer + 1)
    x = torch.randn((w.b, w.n_q, w.head_dim), generator=g, device=device, dtype=torch.float32)
    return x.to(torch.bfloat16)


def channel_magnitudes(w: DecodeWorkload, device="cpu"):
    """Per-(kv-head, channel) magnitudes ~ U[0.5, 2] for K and for V (fp32)."""
    torch = _torch()
    g = _gen(device, w.seed * 1_000_003 + 17)
    ck = torch.rand((w.n_kv, w.head_dim), generator=g, device=device) * 1.5 + 0.5
    cv = torch.rand((w.n_kv, w.head_dim), generator=g, device=device) * 1.5 + 0.5
    return ck, cv


def keys_values(w: DecodeWorkload, layer: int, n_tokens: int, device="cpu"):
    """Logical K and V of one layer, bf16 ``[n_tokens][n_kv][head_dim]`` each.

    The tokens of all sequences are packed one after another (sequence ``i``
    occupies rows ``offsets[i] : offsets[i] + lens[i]``, see :func:`offsets`).
    Values are N(0, 1) in fp32, times the per-channel magnitude when the
    workload asks for one, then cast to bf16.
    """
    torch = _torch()
    g = _gen(device, w.seed * 1_000_003 + 7919 * layer + 2)
    shape = (n_tokens, w.n_kv, w.head_dim)
    k = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    v = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if w.channel_scale:
        ck, cv = channel_magnitudes(w, device)
        k.mul_(ck)
        v.mul_(cv)
    return k.to(torch.bfloat16), v.to(torch.bfloat16)


def stored_rows(w: DecodeWorkload, lens: np.ndarray):
    """Where the rows generated for a batch sit when a shared prefix is stored
    once: sequence 0's rows (the shared prompt, then its own), then every other
    sequence's own rows, in sequence order.

    Returns ``(first, start, n_rows)``: the first stored token of each sequence
    (0 for sequence 0, the prefix length for the others), the row at which each
    sequence's stored tokens begin, and the number of rows.  Without a shared
    prefix this is ``(0, offsets[:-1], offsets[-1])``.  Sequence i's logical
    rows are rows ``[0, P)`` followed by ``[start[i], start[i] + s_i - P)`` for
    i >= 1, and ``[0, s_0)`` for i = 0.
    """
    lens = np.asarray(lens, dtype=np.int64)
    P = w.shared_prefix if len(lens) else 0
    first = np.full(len(lens), P, dtype=np.int32)
    if len(lens):
        first[0] = 0
    stored = lens - first
    start = np.zeros(len(lens), dtype=np.int64)
    start[1:] = np.cumsum(stored)[:-1]
    return first, start, int(stored.sum())


def offsets(lens: np.ndarray) -> np.ndarray:
    """Row offset of each sequence in the packed logical K/V (length b + 1)."""
    out = np.zeros(len(lens) + 1, dtype=np.int64)
    out[1:] = np.cumsum(np.asarray(lens, dtype=np.int64))
    return out


def initial_scores(w: DecodeWorkload, stride: int, device="cpu"):
    """Cumulative-score array before the step: fp32 ``[b][stride]`` ~ U[0, 1)."""
    torch = _torch()
    g = _gen(device, w.seed * 1_000_003 + 29)
    return torch.rand((w.b, stride), generator=g, device=device, dtype=torch.float32)
