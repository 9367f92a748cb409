"""Mixed-precision, tier-homogeneous pages, written out plainly (test-only).

"The KV Cache Is the New Memory Wall" review, §5.5 (open direction 1): one
paged layout that carries a precision per block (and a keep mask).  gist.science
summary of "Spherical KV", §2.2: retained states are grouped into pages whose
entries all share one precision tier, so the decode kernel reads them in a
single pass guided by each page's header instead of gathering irregularly.

Readings taken here (the library's choices, restated):

* blocks of each precision live in a pool of that precision (bf16 or FP8
  E4M3 with per-(block, head) scales); a block-table entry names its block's
  precision in bit 30 (set: the FP8 pool) -- the page header; a negative entry
  is a block that is not attended (the keep mask);
* the decode kernel takes the table two entries at a time, so every such pair
  is a tier-homogeneous page: a sequence's row lists one precision's blocks,
  then a -1 if that run has an odd length, then the other precision's blocks;
  the run holding the sequence's partly filled block comes second, with that
  block last, so only the final entry of a row can be partial;
* attention does not depend on the order of the blocks (the softmax sums over
  the whole set), so the rearranged row gives the step over the same tokens.
"""
from __future__ import annotations

import numpy as np

from . import attention

PRECISION_BIT = 1 << 30
BLOCK = 16


def arrange_row(ids_bf16, ids_fp8, fp8_last: bool, tail_tokens: int):
    """Table row and context length of a sequence whose blocks are split over
    the two pools.  The second run (FP8 if ``fp8_last``) follows the first,
    after a -1 if the first has an odd length; the row's last block holds
    ``tail_tokens`` (1..16) tokens, every other block 16."""
    first, second = (list(ids_bf16), list(ids_fp8)) if fp8_last else (list(ids_fp8), list(ids_bf16))
    tag_first = 0 if fp8_last else PRECISION_BIT
    tag_second = PRECISION_BIT if fp8_last else 0
    row = [b | tag_first for b in first]
    if second and len(row) % 2:
        row.append(-1)
    row += [b | tag_second for b in second]
    if not row:
        return [], 0
    return row, BLOCK * (len(row) - 1) + tail_tokens


def pairs_homogeneous(row) -> bool:
    """No pair of entries (2k, 2k+1) mixes the two precisions."""
    for k in range(0, len(row) - 1, 2):
        a, b = row[k], row[k + 1]
        if a >= 0 and b >= 0 and (a & PRECISION_BIT) != (b & PRECISION_BIT):
            return False
    return True


def decode_mixed(q, blocks):
    """One sequence's step over blocks given as (K [n][n_kv][d], V) float64
    arrays holding the values as stored (bf16 values, or FP8 codes times
    scales); the blocks may come in any order."""
    if not blocks:
        n_q, d = np.asarray(q).shape
        return np.zeros((n_q, d)), np.full(n_q, -np.inf)
    K = np.concatenate([k for k, _ in blocks])
    V = np.concatenate([v for _, v in blocks])
    return attention.decode_sequence(q, K, V)
