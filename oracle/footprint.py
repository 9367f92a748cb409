"""KV footprint, step bytes and FLOP accounting (oracle; test-only).

* Bytes per token: a K and a V vector per layer and per KV head, each of
  ``head_dim`` elements of ``w`` bytes -- froggydisk "LLM에서 KV 캐시는 얼마나
  생길까", section on the size of one token (and its per-request table); the
  same footprint as the first page's §2.1 / Tab. 1.
* One decode step reads the whole cache once; the new token's own K/V write is
  a 1/s correction and is not counted -- review "The KV Cache Is the New
  Memory Wall", §3.1 and Tab. 8.
* FLOPs: per token, per layer, per query head, 2*d_h for q.k and 2*d_h for the
  weighted V sum.  With the KV bytes above this gives the long-context
  arithmetic intensity 2g/w FLOP/B that the review states in §3.2 (8 FLOP/B
  for BF16 at g = 8, 64 FLOP/B for 2-bit storage).
"""
from __future__ import annotations

import math

BLOCK_SIZE = 16


def kv_bytes_per_token(layers: int, n_kv: int, head_dim: int, bytes_per_elem: float) -> float:
    """2 (K and V) x layers x KV heads x head dim x bytes per element."""
    return 2 * layers * n_kv * head_dim * bytes_per_elem


def request_kv_bytes(tokens: int, layers: int, n_kv: int, head_dim: int,
                     bytes_per_elem: float) -> float:
    """KV bytes held by one request of ``tokens`` tokens (prompt + output)."""
    return tokens * kv_bytes_per_token(layers, n_kv, head_dim, bytes_per_elem)


def decode_flops_per_token(n_q: int, head_dim: int) -> int:
    """FLOPs of one layer for one cached token: q.k and p*v for every query head."""
    return 4 * n_q * head_dim


def long_context_intensity(n_q: int, n_kv: int, bytes_per_elem: float) -> float:
    """FLOP per KV byte as the context grows: FLOPs / KV bytes = 2g / w."""
    return decode_flops_per_token(n_q, 1) / (2 * n_kv * bytes_per_elem)


def step_bytes(context_lens, layers: int, n_q: int, n_kv: int, head_dim: int,
               kv_bytes_per_elem: float, fp8_scales: bool = False,
               score_bytes_per_token: int = 0) -> int:
    """Algorithmic HBM bytes of one decode step over all layers.

    Per layer and sequence: every cached K and V element once, q read and the
    bf16 output written once (2 bytes each), one 4-byte block id per 16-token
    block, and with FP8 two fp32 scales (K and V) per (block, KV head).  A
    fused score update adds ``score_bytes_per_token`` per token once per step.
    Work an implementation adds on top (partials, scratch, over-fetch of a
    block's unused tail) is deliberately not counted.
    """
    total = 0
    for s in context_lens:
        s = int(s)
        nblk = math.ceil(s / BLOCK_SIZE)
        per_layer = (2 * n_kv * head_dim * kv_bytes_per_elem * s
                     + 2 * n_q * head_dim * 2
                     + 4 * nblk
                     + (2 * n_kv * 4 * nblk if fp8_scales else 0))
        total += layers * per_layer + score_bytes_per_token * s
    return int(total)


def step_flops(context_lens, layers: int, n_q: int, head_dim: int) -> int:
    return int(sum(layers * decode_flops_per_token(n_q, head_dim) * int(s)
                   for s in context_lens))
