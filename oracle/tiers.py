"""Tier-restricted decode, written out plainly (test-only).

gist.science summary of "Not all thinking needs HBM", methodology 1-4:
tokens are sorted into tiers by their cumulative attention score (method 2,
computed by ``scores``): T0 stays in HBM and holds the protected tokens (the
prompt, attention sinks, a recent window) and the highest-scored reasoning
tokens; T1, the middle band, lives in host DDR at full precision and is
prefetched to the GPU before every attention step; T2 is a reduced-precision
CPU copy; T3, the lowest-scored tail, is evicted for good.  Tiers are
reassigned every Delta = 64 decode steps (method 4).  Attention runs over
T0 and T1; since T1 arrives at full precision it contributes exactly the terms
it would have contributed from HBM, so the error depends only on what was
evicted, not on how the kept tokens are split between T0 and T1 (method 3,
Proposition 1).

Readings taken where the summary leaves a choice open:

* the unit of tiering is the 16-token block of the paged pool; a block's
  score is the sum of its tokens' cumulative scores;
* the protected blocks are the first ``protect_first`` blocks (prompt and
  sinks) and the last ``protect_last`` blocks (the recent window, which
  includes the partly filled last block);
* the other blocks are ranked by score, highest first, equal scores by
  position (earlier first); the first ``t0_blocks`` of them go to T0, the next
  ``t1_blocks`` to T1 and the rest to T3; T2 is not used (attention covers
  T0 and T1 only);
* new tokens between two re-tierings belong to the recent window (T0).
"""
from __future__ import annotations

import numpy as np

from . import attention

BLOCK = 16
DELTA = 64
T0, T1, T3 = 0, 1, 3


def block_scores(token_scores, s: int) -> np.ndarray:
    """Sum of the cumulative scores of each block's tokens (the last one partial)."""
    x = np.asarray(token_scores, dtype=np.float64)[:s]
    nb = -(-s // BLOCK)
    out = np.zeros(nb)
    for b in range(nb):
        out[b] = x[b * BLOCK:min(s, (b + 1) * BLOCK)].sum()
    return out


def plan_tiers(scores, protect_first: int, protect_last: int, t0_blocks: int, t1_blocks: int) -> np.ndarray:
    """Tier (T0, T1 or T3) of every block, from the block scores."""
    nb = len(scores)
    tier = np.full(nb, T3, dtype=np.int8)
    protected = set(range(min(protect_first, nb))) | set(range(max(0, nb - protect_last), nb))
    for b in protected:
        tier[b] = T0
    rest = sorted((b for b in range(nb) if b not in protected), key=lambda b: (-scores[b], b))
    for rank, b in enumerate(rest):
        if rank < t0_blocks:
            tier[b] = T0
        elif rank < t0_blocks + t1_blocks:
            tier[b] = T1
    return tier


def retier_due(step: int) -> bool:
    """Tiers are reassigned every DELTA decode steps, starting with step 0."""
    return step % DELTA == 0


def kept_tokens(tier, s: int) -> np.ndarray:
    """Mask of the tokens attention covers: those of T0 and T1 blocks."""
    keep = np.zeros(s, dtype=bool)
    for b, t in enumerate(tier):
        if t in (T0, T1):
            keep[b * BLOCK:min(s, (b + 1) * BLOCK)] = True
    return keep


def restricted_decode(q, K, V, keep):
    """Attention of every query head over the kept tokens only: (o, lse).
    With nothing kept the output is 0 and the lse -inf."""
    keep = np.asarray(keep, dtype=bool)
    return attention.decode_sequence(q, np.asarray(K)[keep], np.asarray(V)[keep])


def restricted_weights(q, K, keep):
    """alpha [n_q][s] of the restricted step: softmax over the kept tokens, exactly 0
    on the others (what the cumulative score adds for this step)."""
    keep = np.asarray(keep, dtype=bool)
    K = np.asarray(K)
    out = np.zeros((np.asarray(q).shape[0], K.shape[0]))
    if keep.any():
        out[:, keep] = attention.attention_weights_sequence(q, K[keep])
    return out
