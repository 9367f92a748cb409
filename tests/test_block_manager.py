"""The native block bookkeeping (kvblocks.h) against the oracle's model (no GPU).

Random traffic -- new requests with shared prompt prefixes, decode appends,
finished requests -- is driven through both, on pools small enough that the
prefix cache evicts and calls run out of blocks; after every call the return
values, failures, every live block table, the block counts and every block's
reference count must agree exactly.
"""
import numpy as np
import pytest

import decode_attention_paged_04_amd as kvd
from oracle import blocks


def _golden_tables():
    import json
    import os
    here = os.path.dirname(os.path.abspath(__file__))
    return json.load(open(os.path.join(here, "golden", "block_table_example.json")))["tables"]


def test_page_block_tables():
    bm = kvd.BlockManager(11)
    a, _ = bm.add_sequence(16)
    b, _ = bm.add_sequence(32)
    c, _ = bm.add_sequence(16)
    for sid, n in [(a, 16), (b, 32), (c, 16), (b, 32), (c, 16)]:
        bm.append(sid, n)
    assert {"A": bm.table(a), "B": bm.table(b), "C": bm.table(c)} == _golden_tables()
    assert bm.counts() == (0, 0, 11)
    table, lens = bm.fill_tables([c, a], 6)
    assert table.tolist() == [[3, 7, 10, -1, -1, -1], [0, 4, -1, -1, -1, -1]]
    assert lens.tolist() == [48, 32]


def _compare(bm, ref, live):
    for sid in live:
        assert bm.table(sid) == ref.table(sid), sid
        assert bm.length(sid) == ref.length(sid)
    assert bm.counts() == ref.counts()
    assert [bm.refcount(b) for b in range(ref.num_blocks)] == ref.ref


def _prompt(rng, bases):
    """Token ids sharing prefixes: a random cut of a base prompt plus a random tail."""
    base = bases[int(rng.integers(len(bases)))]
    cut = int(rng.integers(0, len(base) + 1))
    tail = rng.integers(0, 3, int(rng.integers(0, 40))).tolist()
    return base[:cut] + tail


@pytest.mark.parametrize("prefix", [False, True])
@pytest.mark.parametrize("seed", [1, 2, 3])
def test_matches_oracle_under_random_traffic(prefix, seed):
    rng = np.random.default_rng(seed)
    num_blocks = 24
    bm = kvd.BlockManager(num_blocks, prefix_cache=prefix)
    ref = blocks.BlockPool(num_blocks, prefix_cache=prefix)
    bases = [rng.integers(0, 5, 64).tolist() for _ in range(3)]
    live, fails = [], 0
    for step in range(600):
        op = int(rng.integers(4))
        if op == 0 or not live:
            toks = _prompt(rng, bases) if rng.random() < 0.85 else None
            n = len(toks) if toks is not None else int(rng.integers(0, 70))
            try:
                want = ref.add_sequence(n, toks)
            except blocks.NoBlocks:
                want = None
            if want is None:
                with pytest.raises(kvd.KvdError) as e:
                    bm.add_sequence(n, toks)
                assert e.value.status == kvd.KVD_ERR_CAPACITY
                fails += 1
            else:
                assert bm.add_sequence(n, toks) == want, step
                live.append(want[0])
        elif op in (1, 2):
            sid = live[int(rng.integers(len(live)))]
            n = 1 if op == 1 else int(rng.integers(1, 20))
            toks = rng.integers(0, 3, n).tolist() if rng.random() < 0.9 else None
            try:
                want = ref.append(sid, n, toks)
            except blocks.NoBlocks:
                want = None
            if want is None:
                with pytest.raises(kvd.KvdError) as e:
                    bm.append(sid, n, toks)
                assert e.value.status == kvd.KVD_ERR_CAPACITY
                fails += 1
            else:
                assert bm.append(sid, n, toks) == want, step
        else:
            sid = live.pop(int(rng.integers(len(live))))
            ref.free_sequence(sid)
            bm.free_sequence(sid)
        _compare(bm, ref, live)
        if live and step % 50 == 0:
            sid = live[0]
            L = ref.length(sid)
            assert bm.slots(sid, 0, L) == ref.slots(sid, 0, L)
    assert fails > 0            # the pool did run out


def test_prefix_reuse_and_eviction_counts():
    bm = kvd.BlockManager(6, prefix_cache=True)
    T = list(range(100, 148))
    p, n0 = bm.add_sequence(40, T[:40])
    q, n1 = bm.add_sequence(40, T[:40])
    assert (n0, n1) == (0, 32)
    assert bm.table(q)[:2] == bm.table(p)[:2] and bm.refcount(bm.table(p)[0]) == 2
    bm.free_sequence(p)
    bm.free_sequence(q)
    free, cached, used = bm.counts()
    assert (cached, used) == (2, 0) and free == 4
    r, n2 = bm.add_sequence(33, T[:32] + [5])
    assert n2 == 32 and bm.counts() == (3, 0, 3)


def test_errors():
    E = kvd.KvdError
    with pytest.raises(E):
        kvd.BlockManager(0)
    bm = kvd.BlockManager(4)
    with pytest.raises(E):
        bm.append(12345, 1)
    with pytest.raises(E):
        bm.free_sequence(7)
    sid, _ = bm.add_sequence(20)
    with pytest.raises(E):
        bm.slots(sid, 10, 11)                  # past the end
    with pytest.raises(E):
        bm.fill_tables([sid], 1)               # two blocks do not fit
    with pytest.raises(E):
        bm.refcount(4)
    with pytest.raises(E) as e:
        bm.add_sequence(64)                    # needs 4 blocks, 2 are left
    assert e.value.status == kvd.KVD_ERR_CAPACITY
    assert bm.counts() == (2, 0, 2)            # the failed call changed nothing
    bm.free_sequence(sid)
    with pytest.raises(E):
        bm.free_sequence(sid)                  # ids are never reused
    assert bm.counts() == (4, 0, 0)
