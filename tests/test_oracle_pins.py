"""The oracle against facts outside itself (CPU only)."""
import numpy as np
import pytest

import pins
from oracle import attention, e4m3, footprint, numerics


def test_footprint_matches_printed_tables():
    assert pins.footprint_mismatches() == []


def test_step_bytes_closed_form():
    # 8B-shaped layer at s = 32768: 4096 B of KV per token, q and o 2*32*128*2 B,
    # one 4-byte id per 16-token block
    got = footprint.step_bytes([32768], 1, 32, 8, 128, 2)
    assert got == 32768 * 4096 + 2 * 32 * 128 * 2 + 4 * 2048
    # FP8 halves the KV term and adds two fp32 scales per (block, kv head)
    got8 = footprint.step_bytes([32768], 1, 32, 8, 128, 1, fp8_scales=True)
    assert got8 == 32768 * 2048 + 2 * 32 * 128 * 2 + 4 * 2048 + 2 * 8 * 4 * 2048
    # 70B step of 80 layers at s = 131072: the KV term is 327,680 B per token
    kv = footprint.step_bytes([131072], 80, 64, 8, 128, 2) - 80 * (2 * 64 * 128 * 2 + 4 * 8192)
    assert kv == 131072 * 327680
    assert footprint.step_flops([10], 2, 32, 128) == 2 * 4 * 32 * 128 * 10


def test_bf16_rounding_matches_torch_cast():
    assert pins.bf16_rounding_mismatches() == 0


def test_bf16_exact_roundtrip():
    bits = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    v = numerics.bf16_bits_to_f64(bits)
    fin = np.isfinite(v)
    back = numerics.f64_to_bf16_bits(v[fin])
    # +0 / -0 keep their sign; every finite pattern maps back to itself
    assert np.array_equal(back, bits[fin])


def test_e4m3_decode_all_codes_matches_torch():
    assert pins.e4m3_decode_mismatches() == 0


def test_e4m3_encode_matches_torch_nearest_even():
    assert pins.e4m3_encode_mismatches() == 0


def test_e4m3_page_facts():
    assert pins.e4m3_page_fact_failures() == []


def test_e4m3_saturation_and_sign():
    x = np.array([448.0, 463.9, 464.0, 500.0, 1e30, np.inf, -1e30, -0.0, 0.0], np.float32)
    c = e4m3.encode(x)
    assert c.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x80, 0x00]


def test_attention_matches_torch_sdpa():
    assert pins.sdpa_max_error() < 1e-13


def test_attention_matches_brute_force():
    assert pins.brute_force_max_error() < 1e-13


def test_lse_matches_scipy_logsumexp():
    assert pins.lse_library_max_error() < 1e-12


def test_split_and_merge_is_exact():
    assert pins.split_merge_max_error() < 1e-12


def test_uneven_spans_merge_exactly():
    assert pins.uneven_split_merge_max_error() < 1e-12


def test_merge_edge_cases():
    rng = np.random.default_rng(11)
    oc = rng.standard_normal((3, 4, 8))
    lc = rng.standard_normal((3, 4))
    o, lse = attention.merge_partials(oc, lc)
    # an extra empty chunk changes nothing
    oc2 = np.concatenate([oc, np.zeros((3, 1, 8))], axis=1)
    lc2 = np.concatenate([lc, np.full((3, 1), -np.inf)], axis=1)
    o2, lse2 = attention.merge_partials(oc2, lc2)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    # chunk order does not matter (up to rounding)
    perm = rng.permutation(4)
    o3, lse3 = attention.merge_partials(oc[:, perm], lc[:, perm])
    assert np.max(np.abs(o3 - o)) < 1e-14 and np.max(np.abs(lse3 - lse)) < 1e-14
    # one chunk: identity
    o4, lse4 = attention.merge_partials(oc[:, :1], lc[:, :1])
    assert np.allclose(o4, oc[:, 0], atol=0, rtol=1e-15) and np.array_equal(lse4, lc[:, 0])
    # all empty
    o5, lse5 = attention.merge_partials(np.zeros((2, 3, 4)), np.full((2, 3), -np.inf))
    assert np.all(o5 == 0) and np.all(lse5 == -np.inf)


def test_attention_special_cases():
    assert pins.special_case_failures() == []


def test_block_table_worked_example():
    assert pins.block_table_example_failures() == []


def test_placement_does_not_change_result():
    assert pins.placement_invariance_max_error() == 0.0


def test_scores():
    assert pins.score_failures() == []


def test_fp8_quantisation():
    assert pins.fp8_quant_failures() == []


def test_fp8_append_requantise():
    assert pins.fp8_append_failures() == []


def test_block_manager():
    assert pins.block_manager_failures() == []


def test_tier_restricted_decode():
    assert pins.tier_failures() == []


def test_mixed_precision_rows():
    assert pins.mixed_failures() == []


@pytest.mark.parametrize("g", [1, 2, 4, 8])
@pytest.mark.parametrize("d", [64, 128])
def test_brute_force_grid(g, d):
    """Small contexts 1..40 for every group size and head dim, against torch SDPA."""
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(100 * g + d)
    n_kv = 2
    n_q = g * n_kv
    for s in (1, 2, 15, 16, 17, 31, 40):
        q = rng.standard_normal((n_q, d))
        K = rng.standard_normal((s, n_kv, d))
        V = rng.standard_normal((s, n_kv, d))
        o, _ = attention.decode_sequence(q, K, V)
        ref = F.scaled_dot_product_attention(
            torch.from_numpy(q)[None, :, None], torch.from_numpy(K).permute(1, 0, 2)[None],
            torch.from_numpy(V).permute(1, 0, 2)[None], enable_gqa=True)[0, :, 0].numpy()
        assert np.max(np.abs(o - ref)) < 1e-13


def test_vectorised_gather_indices_match_scalar_layout():
    from oracle import paged
    lay = paged.PoolLayout(num_layers=3, num_blocks=9, n_kv=2, head_dim=8)
    table = [4, 0, 7]
    k_idx, v_idx = paged.gather_indices(lay, 2, table, 37)
    for t in (0, 5, 15, 16, 31, 36):
        p, row = divmod(paged.slot(table, t), 16)
        for j in range(2):
            for c in (0, 3, 7):
                assert k_idx[t, j, c] == lay.k_offset(2, p, j, row, c)
                assert v_idx[t, j, c] == lay.v_offset(2, p, j, row, c)


def test_bf16_ulp():
    from oracle import numerics
    x = np.array([1.0, 1.5, 1.99, 2.0, 3.0, 0.25, -5.0, 1e-40])
    exp = np.array([2.0 ** -7, 2.0 ** -7, 2.0 ** -7, 2.0 ** -6, 2.0 ** -6, 2.0 ** -9, 2.0 ** -5, 2.0 ** -133])
    assert np.array_equal(numerics.bf16_ulp(x), exp)
    # the spacing is the gap to the next bf16 number up
    bits = np.array([0x3F80, 0x4000, 0x3E80, 0x0001], dtype=np.uint16)
    v = numerics.bf16_bits_to_f64(bits)
    nxt = numerics.bf16_bits_to_f64(bits + 1)
    assert np.array_equal(nxt - v, numerics.bf16_ulp(v))
