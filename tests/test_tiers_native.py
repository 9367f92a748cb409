"""The native tier planner (kvblocks.h, tiers) against the oracle (no GPU)."""
import numpy as np
import pytest

import decode_attention_paged_04_amd as kvd
from oracle import tiers


@pytest.mark.parametrize("seed", range(6))
def test_plan_matches_oracle(seed):
    rng = np.random.default_rng(seed)
    for _ in range(300):
        nb = int(rng.integers(0, 60))
        # coarse scores make ties common, so the tie rule is exercised
        sc = np.round(rng.random(nb) * 6) / 2 if rng.random() < 0.5 else rng.random(nb)
        args = [int(rng.integers(0, 4)), int(rng.integers(0, 4)), int(rng.integers(0, 30)), int(rng.integers(0, 30))]
        want = tiers.plan_tiers(sc, *args)
        got = kvd.tier_plan(sc, *args)
        assert np.array_equal(got, want), (nb, args)


def test_block_scores_match_oracle():
    rng = np.random.default_rng(7)
    for s in (0, 1, 15, 16, 17, 100, 1000):
        # multiples of 2^-12 below 64: every sum is exact in any order
        ts = (rng.integers(0, 64 * 4096, s) / 4096.0).astype(np.float32)
        assert np.array_equal(kvd.tier_block_scores(ts), tiers.block_scores(ts, s))


def test_restrict_marks_evicted_blocks():
    row = np.array([5, 9, 2, 7, 11], dtype=np.int32)
    t = np.array([tiers.T0, tiers.T3, tiers.T1, tiers.T3, tiers.T0], dtype=np.int8)
    assert kvd.tier_restrict(row, t).tolist() == [5, -1, 2, -1, 11]
    keep = tiers.kept_tokens(t, 5 * 16 - 3)
    assert keep.reshape(-1)[:16].all() and not keep[16:32].any()


def test_errors():
    with pytest.raises(kvd.KvdError):
        kvd.tier_plan(np.array([1.0, np.nan]), 0, 0, 1, 1)
    with pytest.raises(kvd.KvdError):
        kvd.tier_plan(np.array([1.0]), -1, 0, 1, 1)
    with pytest.raises(kvd.KvdError):
        kvd.tier_restrict(np.array([1, 2], np.int32), np.array([0, 2], np.int8))


def test_mixed_row_matches_oracle():
    from oracle import mixed
    rng = np.random.default_rng(9)
    for _ in range(500):
        n16, n8 = int(rng.integers(0, 9)), int(rng.integers(0, 9))
        ids = rng.permutation(1000)[:n16 + n8]
        fp8_last = bool(rng.integers(2))
        tail = int(rng.integers(1, 17))
        row, s = kvd.mixed_row(ids[:n16], ids[n16:], fp8_last, tail)
        want_row, want_s = mixed.arrange_row(list(ids[:n16]), list(ids[n16:]), fp8_last, tail)
        assert row.tolist() == want_row and s == want_s
    with pytest.raises(kvd.KvdError):
        kvd.mixed_row([1], [2], True, 0)                 # tail outside 1..16
    with pytest.raises(kvd.KvdError):
        kvd.mixed_row([1 << 30], [], True, 3)            # id does not fit below the bit
