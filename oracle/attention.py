"""Decode attention in float64, written from its definition (test-only).

For one new token of one sequence and one query head h (froggydisk
"LLM에서 KV 캐시는 얼마나 생길까", section "KV 캐시란"):

* every cached token t gets the score q_h . k_t, divided by sqrt(d_h) before
  the softmax (the page divides by sqrt(128) for head dim 128);
* the softmax turns the scores into weights alpha_t that sum to one;
* the output is the weighted sum of the cached V rows, a d_h-vector;
* query heads share KV heads in groups of g = n_q / n_kv (the page's 8B model:
  32 query heads over 8 KV heads, four per KV head).  Reading: query head h
  uses KV head floor(h / g).
* the context s_i counts every cached token including the current one (the
  new token's K/V is appended before it attends); there is no mask.

``lse`` (the natural log of the softmax denominator taken with the scores'
maximum factored out) is the quantity that lets per-chunk results be merged
exactly: splitting the context into chunks and recombining them by their
log-sum-exp is an exact rewrite of the same softmax.  An empty context gives
output 0 and lse = -inf.
"""
from __future__ import annotations

import math

import numpy as np


def head_group(h: int, n_q: int, n_kv: int) -> int:
    """KV head used by query head h: contiguous groups of g = n_q / n_kv."""
    g = n_q // n_kv
    return h // g


def logits(q_h: np.ndarray, K_j: np.ndarray) -> np.ndarray:
    """Scores of one query head over the cached keys of its KV head."""
    d = q_h.shape[-1]
    return (K_j @ q_h) / math.sqrt(d)


def softmax_weights(l: np.ndarray):
    """alpha_t = exp(l_t - m) / sum_t exp(l_t - m); also returns (m, Z)."""
    m = np.max(l)
    p = np.exp(l - m)
    Z = np.sum(p)
    return p / Z, m, Z


def decode_head(q_h: np.ndarray, K_j: np.ndarray, V_j: np.ndarray):
    """Output and lse of one query head; K_j, V_j are ``[s][d]`` float64."""
    s, d = K_j.shape
    if s == 0:
        return np.zeros(d), -np.inf
    l = logits(q_h, K_j)
    alpha, m, Z = softmax_weights(l)
    return alpha @ V_j, m + math.log(Z)


def decode_sequence(q: np.ndarray, K: np.ndarray, V: np.ndarray):
    """All query heads of one sequence.

    q: ``[n_q][d]``; K, V: ``[s][n_kv][d]`` (logical, contiguous), float64.
    Returns o ``[n_q][d]`` and lse ``[n_q]``.
    """
    n_q, d = q.shape
    n_kv = K.shape[1]
    o = np.zeros((n_q, d))
    lse = np.zeros(n_q)
    for h in range(n_q):
        j = head_group(h, n_q, n_kv)
        o[h], lse[h] = decode_head(q[h], K[:, j, :], V[:, j, :])
    return o, lse


def attention_weights_sequence(q: np.ndarray, K: np.ndarray) -> np.ndarray:
    """alpha ``[n_q][s]`` of one sequence (zero-width for an empty context)."""
    n_q, _ = q.shape
    s, n_kv, _ = K.shape
    out = np.zeros((n_q, s))
    if s == 0:
        return out
    for h in range(n_q):
        j = head_group(h, n_q, n_kv)
        out[h], _, _ = softmax_weights(logits(q[h], K[:, j, :]))
    return out


def chunk_partials(q: np.ndarray, K: np.ndarray, V: np.ndarray, chunk: int, n_chunks=None):
    """Per-chunk (o_c, lse_c) of one sequence, chunks of ``chunk`` tokens.

    o_c is the chunk's own normalised output; an empty chunk has o_c = 0 and
    lse_c = -inf.  Shapes: o_c ``[n_q][n_chunks][d]``, lse_c ``[n_q][n_chunks]``.
    """
    n_q, d = q.shape
    s = K.shape[0]
    if n_chunks is None:
        n_chunks = max(1, -(-s // chunk))
    o_c = np.zeros((n_q, n_chunks, d))
    lse_c = np.full((n_q, n_chunks), -np.inf)
    for c in range(n_chunks):
        lo, hi = c * chunk, min(s, (c + 1) * chunk)
        if lo >= hi:
            continue
        o, lse = decode_sequence(q, K[lo:hi], V[lo:hi])
        o_c[:, c, :] = o
        lse_c[:, c] = lse
    return o_c, lse_c


def merge_partials(o_c: np.ndarray, lse_c: np.ndarray):
    """Recombine chunk partials by log-sum-exp.

    lse = M + log(sum_c exp(lse_c - M)) with M = max_c lse_c, and
    o = sum_c exp(lse_c - lse) * o_c.  Chunks with lse_c = -inf weigh 0; if all
    are empty the result is o = 0, lse = -inf.
    """
    lead = o_c.shape[:-2]
    n_chunks, d = o_c.shape[-2:]
    o_flat = o_c.reshape(-1, n_chunks, d)
    l_flat = lse_c.reshape(-1, n_chunks)
    out = np.zeros((o_flat.shape[0], d))
    lse = np.full(o_flat.shape[0], -np.inf)
    for r in range(o_flat.shape[0]):
        M = np.max(l_flat[r])
        if M == -np.inf:
            continue
        w = np.exp(l_flat[r] - M)
        lse[r] = M + math.log(np.sum(w))
        out[r] = (np.exp(l_flat[r] - lse[r])[:, None] * o_flat[r]).sum(axis=0)
    return out.reshape(*lead, d), lse.reshape(lead)
