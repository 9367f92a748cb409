"""The benchmark's byte accounting agrees with the oracle's step-byte formula."""
import numpy as np
import pytest

import bench
from oracle import footprint


@pytest.mark.parametrize("fp8,scores", [(False, False), (True, False), (True, True)])
def test_step_bytes_match_oracle(fp8, scores):
    rng = np.random.default_rng(3)
    lens = rng.integers(0, 5000, 7)
    w = 1 if fp8 else 2
    got = bench.algorithmic_step_bytes(lens, 3, 32, 8, 128, w, fp8, scores)
    ref = footprint.step_bytes(lens, 3, 32, 8, 128, w, fp8_scales=fp8,
                               score_bytes_per_token=8 if scores else 0)
    assert got == ref


def test_headline_bytes():
    # 8B-shaped layer at s = 32768: 134,217,728 bytes of K/V plus q, out and block ids
    got = bench.algorithmic_step_bytes([32768], 1, 32, 8, 128, 2, False, False)
    assert got == 134_217_728 + 16_384 + 8_192
    # 70B step: 327,680 B of K/V per token over 80 layers
    got70 = bench.algorithmic_step_bytes([131072] * 4, 80, 64, 8, 128, 2, False, False)
    assert got70 - 4 * 80 * (2 * 64 * 128 * 2 + 4 * 8192) == 4 * 131072 * 327680
