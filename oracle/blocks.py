"""The paged engine's block bookkeeping, written out plainly (test-only).

froggydisk "LLM에서 KV 캐시는 얼마나 생길까", section "KV 캐시를 줄이는
기법", PagedAttention and prefix-cache paragraphs:

* the cache memory is cut into 16-token blocks up front and every request has
  a block table: its i-th block lives in physical block table[i];
* a new request gets just enough blocks for its prompt; during decoding a new
  free block is taken and appended to the table when the last block holds 16
  tokens; a finished request returns its blocks to the free list -- so the
  waste is the unfilled tail of the last block, at most 15 tokens;
* several tables may point at one physical block; each block counts the
  requests pointing at it and goes back to the free list when the count
  reaches 0;
* prefix cache: every full block is looked up by a hash of its 16 tokens
  together with all tokens before it; a new prompt is cut into 16-token pieces
  and matched from the front until the first piece that is not found; the
  blocks found are put into the new table as they are and only the rest is
  prefilled; a last piece of fewer than 16 tokens is never hashed or reused;
  finished requests' blocks are kept and, when memory runs short, the ones
  unused for longest are evicted -- only blocks that no request points at.

Readings taken where the page leaves a choice open:

* free blocks are handed out lowest number first (this reproduces the page's
  block-table example for requests A, B, C when the three grow in turn);
* the lookup key is the whole token prefix up to and including the block (the
  exact content the page's hash stands for, so no two different prefixes can
  collide);
* a block is registered in the prefix cache at the moment it becomes full (a
  prompt's full blocks when the request arrives), unless the same prefix is
  registered already -- then it stays private for good;
* blocks never registered go straight back to the free list at count 0;
  registered ones become evictable and are evicted least recently released
  first, and only when no free block is left; a finished request releases
  its blocks from the last to the first, so the front of a prefix outlives
  its tail;
* a call that cannot get all the blocks it needs changes nothing and fails.
"""
from __future__ import annotations

BLOCK = 16


class NoBlocks(Exception):
    """The pool cannot supply the blocks a call needs (nothing was changed)."""


class BlockPool:
    def __init__(self, num_blocks: int, prefix_cache: bool = False):
        self.num_blocks = num_blocks
        self.prefix_cache = prefix_cache
        self.free = list(range(num_blocks))     # never registered (or evicted), unreferenced
        self.ref = [0] * num_blocks
        self.cache = {}                         # token prefix tuple -> block
        self.key_of = {}                        # registered block -> its prefix tuple
        self.evictable = []                     # registered, unreferenced; oldest release first
        self.seqs = {}                          # id -> {"blocks": [...], "len": n, "tokens": [...] or None}
        self.next_id = 0

    # ------------------------------------------------------------ helpers
    def available(self) -> int:
        return len(self.free) + len(self.evictable)

    def _take(self) -> int:
        if self.free:
            b = min(self.free)
            self.free.remove(b)
        else:
            b = self.evictable.pop(0)
            del self.cache[self.key_of.pop(b)]
        self.ref[b] = 1
        return b

    def _release(self, b: int):
        self.ref[b] -= 1
        if self.ref[b] == 0:
            if b in self.key_of:
                self.evictable.append(b)
            else:
                self.free.append(b)

    def _register(self, seq, k: int):
        """Block k of ``seq`` has just become full: record it under its prefix."""
        toks = seq["tokens"]
        if not self.prefix_cache or toks is None:
            return
        b = seq["blocks"][k]
        key = tuple(toks[:BLOCK * (k + 1)])
        if key not in self.cache and b not in self.key_of:
            self.cache[key] = b
            self.key_of[b] = key

    # ------------------------------------------------------------ calls
    def add_sequence(self, n: int, tokens=None):
        """New request with an n-token prompt; returns (id, n_cached)."""
        toks = list(tokens) if tokens is not None else None
        found = []
        if self.prefix_cache and toks is not None:
            for k in range(n // BLOCK):
                b = self.cache.get(tuple(toks[:BLOCK * (k + 1)]))
                if b is None:
                    break
                found.append(b)
        need = -(-n // BLOCK) - len(found)
        reusable_now = sum(1 for b in found if b in self.evictable)
        if need > self.available() - reusable_now:
            raise NoBlocks()
        for b in found:
            if self.ref[b] == 0:
                self.evictable.remove(b)
            self.ref[b] += 1
        blocks = found + [self._take() for _ in range(need)]
        sid = self.next_id
        self.next_id += 1
        self.seqs[sid] = {"blocks": blocks, "len": n, "tokens": toks}
        for k in range(n // BLOCK):
            self._register(self.seqs[sid], k)
        return sid, BLOCK * len(found)

    def append(self, sid: int, n: int = 1, tokens=None):
        """Append n tokens to a request; returns their slots (block * 16 + row)."""
        seq = self.seqs[sid]
        old = seq["len"]
        need = -(-(old + n) // BLOCK) - len(seq["blocks"])
        if need > self.available():
            raise NoBlocks()
        for _ in range(need):
            seq["blocks"].append(self._take())
        seq["len"] = old + n
        if seq["tokens"] is not None:
            # without the new tokens' ids the content is unknown: stop registering
            seq["tokens"] = seq["tokens"] + list(tokens) if tokens is not None else None
        for k in range(old // BLOCK, (old + n) // BLOCK):
            self._register(seq, k)
        return self.slots(sid, old, n)

    def slots(self, sid: int, first: int, n: int):
        blocks = self.seqs[sid]["blocks"]
        return [blocks[t // BLOCK] * BLOCK + t % BLOCK for t in range(first, first + n)]

    def table(self, sid: int):
        return list(self.seqs[sid]["blocks"])

    def length(self, sid: int) -> int:
        return self.seqs[sid]["len"]

    def free_sequence(self, sid: int):
        seq = self.seqs.pop(sid)
        for b in reversed(seq["blocks"]):
            self._release(b)

    def counts(self):
        """(free, evictable, referenced) block counts."""
        used = sum(1 for r in self.ref if r > 0)
        return len(self.free), len(self.evictable), used
