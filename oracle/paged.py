"""Block-table addressing and the pool layout, written out plainly (test-only).

The cache is cut into fixed 16-token blocks; each request owns a block table
that maps its i-th logical block to a physical block number, and attention
reads the blocks in table order, so scattered physical placement cannot change
the result (froggydisk "LLM에서 KV 캐시는 얼마나 생길까", PagedAttention
paragraph and its three-request block-table example).  Because only a
request's last block can be partly filled, the waste is at most 15 tokens per
request (same paragraph).

The physical layout inside the pool is the library's own choice, documented
in its C header; it is restated here from that documentation, independently
of the library's code:

* element offset of the tile pair of (layer l, physical block p, KV head j):
  ``((l * num_blocks + p) * n_kv + j) * 2 * 16 * head_dim``
* K is kept as 16-byte pieces of n = 16 / w elements (w the element size,
  P = head_dim / n pieces per row).  Channel c has step c // 32 and group
  (c // 8) % 4; a piece holds n / 8 consecutive steps' 8-channel slices of
  one group, so c lies in piece q = 4 (step // (n / 8)) + group of its row,
  at position 8 (step % (n / 8)) + c % 8; with s = (t // 4) % 2 and
  r = 4 (t // 8) + t % 4, piece q of row t is piece number (s P + q) 8 + r
  of the tile (for bf16 a piece is simply channels 8q .. 8q + 7);
* V of in-block row t, channel c: ``+ 16 * head_dim + c * 16 + t`` (channel-major)
* FP8 pools use the same rules with w = 1 (offsets in bytes); the fp32 scale
  of (l, p, j) is at index ``((l * n_kv + j) * num_blocks + p) * 2`` (+0 for
  K, +1 for V): head-major within a layer.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

BLOCK_SIZE = 16


def slot(table_row, t: int) -> int:
    """Physical slot of logical token t: block id times 16 plus in-block row."""
    return int(table_row[t // BLOCK_SIZE]) * BLOCK_SIZE + t % BLOCK_SIZE


def slots_of_sequence(table_row, s: int) -> np.ndarray:
    return np.array([slot(table_row, t) for t in range(s)], dtype=np.int64)


def blocks_needed(s: int) -> int:
    return -(-int(s) // BLOCK_SIZE)


def tail_waste(s: int) -> int:
    """Unused token slots in a request's blocks (only the last one can be partial)."""
    return blocks_needed(s) * BLOCK_SIZE - int(s)


@dataclass(frozen=True)
class PoolLayout:
    num_layers: int
    num_blocks: int
    n_kv: int
    head_dim: int
    elem_bytes: int = 2          # 2 for bf16 pools, 1 for FP8

    def k_in_tile(self, row, ch):
        """Element offset of K[row][ch] from the start of its tile (works on arrays)."""
        n = 16 // self.elem_bytes
        steps_per_piece = n // 8
        pieces_per_row = self.head_dim // n
        s = (row // 4) % 2
        r = 4 * (row // 8) + row % 4
        step, group = ch // 32, (ch // 8) % 4
        q = 4 * (step // steps_per_piece) + group
        piece = (s * pieces_per_row + q) * 8 + r
        return piece * n + 8 * (step % steps_per_piece) + ch % 8

    @property
    def tile_pair_elems(self) -> int:
        return 2 * BLOCK_SIZE * self.head_dim

    @property
    def total_elems(self) -> int:
        return self.num_layers * self.num_blocks * self.n_kv * self.tile_pair_elems

    def tile_base(self, layer: int, block: int, head: int) -> int:
        return ((layer * self.num_blocks + block) * self.n_kv + head) * self.tile_pair_elems

    def k_offset(self, layer: int, block: int, head: int, row: int, ch: int) -> int:
        return self.tile_base(layer, block, head) + int(self.k_in_tile(row, ch))

    def v_offset(self, layer: int, block: int, head: int, row: int, ch: int) -> int:
        return (self.tile_base(layer, block, head) + BLOCK_SIZE * self.head_dim
                + ch * BLOCK_SIZE + row)

    def scale_index(self, layer: int, block: int, head: int, which: int) -> int:
        return ((layer * self.n_kv + head) * self.num_blocks + block) * 2 + which


def scatter(pool: np.ndarray, lay: PoolLayout, layer: int, table_row, K, V) -> None:
    """Write one sequence's logical K/V ``[s][n_kv][d]`` into ``pool`` (flat)."""
    s = K.shape[0]
    for t in range(s):
        p, row = divmod(slot(table_row, t), BLOCK_SIZE)
        for j in range(lay.n_kv):
            for c in range(lay.head_dim):
                pool[lay.k_offset(layer, p, j, row, c)] = K[t, j, c]
                pool[lay.v_offset(layer, p, j, row, c)] = V[t, j, c]


def gather(pool: np.ndarray, lay: PoolLayout, layer: int, table_row, s: int):
    """Read one sequence's logical K/V back out of ``pool`` in table order."""
    K = np.empty((s, lay.n_kv, lay.head_dim), dtype=pool.dtype)
    V = np.empty_like(K)
    for t in range(s):
        p, row = divmod(slot(table_row, t), BLOCK_SIZE)
        for j in range(lay.n_kv):
            for c in range(lay.head_dim):
                K[t, j, c] = pool[lay.k_offset(layer, p, j, row, c)]
                V[t, j, c] = pool[lay.v_offset(layer, p, j, row, c)]
    return K, V


def gather_indices(lay: PoolLayout, layer: int, table_row, s: int):
    """Flat pool indices of a sequence's logical K and V, each ``[s][n_kv][d]``.

    The same formulas as :meth:`PoolLayout.k_offset` / :meth:`v_offset`,
    evaluated for all tokens, heads and channels at once.
    """
    t = np.arange(s, dtype=np.int64)
    blk = np.asarray(table_row, dtype=np.int64)[t // BLOCK_SIZE]
    row = t % BLOCK_SIZE
    heads = np.arange(lay.n_kv, dtype=np.int64)
    ch = np.arange(lay.head_dim, dtype=np.int64)
    base = ((layer * lay.num_blocks + blk)[:, None] * lay.n_kv + heads[None, :]) * lay.tile_pair_elems
    k_idx = base[:, :, None] + lay.k_in_tile(row[:, None, None], ch[None, None, :])
    v_idx = base[:, :, None] + BLOCK_SIZE * lay.head_dim + ch[None, None, :] * BLOCK_SIZE + row[:, None, None]
    return k_idx, v_idx
