"""Plant plausible mistakes in the oracle (on the CPU) and check a pin notices.

Each case patches one oracle function with a wrong variant -- a dropped term,
a wrong sign or index, a transposed operand, a wrong constant -- and asserts
that at least one of the pins in ``pins.py`` fails.  The patch is undone after
every case.
"""
import math

import numpy as np
import pytest

import pins
from oracle import attention, blocks, e4m3, footprint, mixed, paged, scores, tiers


def _all_pins_pass() -> bool:
    return (pins.footprint_mismatches() == []
            and pins.e4m3_decode_mismatches() == 0
            and pins.e4m3_encode_mismatches(n=20_000) == 0
            and pins.e4m3_page_fact_failures() == []
            and pins.sdpa_max_error() < 1e-13
            and pins.brute_force_max_error() < 1e-13
            and pins.lse_library_max_error() < 1e-12
            and pins.split_merge_max_error() < 1e-12
            and pins.special_case_failures() == []
            and pins.block_table_example_failures() == []
            and pins.placement_invariance_max_error() == 0.0
            and pins.score_failures() == []
            and pins.fp8_quant_failures() == []
            and pins.fp8_append_failures() == []
            and pins.block_manager_failures() == []
            and pins.tier_failures() == []
            and pins.mixed_failures() == [])


def _modulo_heads(h, n_q, n_kv):
    return h % n_kv


def _no_scale_logits(q_h, K_j):
    return K_j @ q_h


def _natural_scale_logits(q_h, K_j):
    return (K_j @ q_h) / q_h.shape[-1]


def _lse_without_max(q_h, K_j, V_j):
    s, d = K_j.shape
    if s == 0:
        return np.zeros(d), -np.inf
    l = attention.logits(q_h, K_j)
    alpha, m, Z = attention.softmax_weights(l)
    return alpha @ V_j, math.log(Z)


def _merge_unweighted(o_c, lse_c):
    lead = o_c.shape[:-2]
    o = o_c.mean(axis=-2)
    M = np.max(lse_c, axis=-1)
    return o.reshape(*lead, o_c.shape[-1]), M


def _decode_code_bias8(code):
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -7
    return sign * 2.0 ** (e - 8) * (1.0 + m / 8.0)


def _encode_ties_away(y):
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y.astype(np.float64))
    P = e4m3._POS
    hi = np.clip(np.searchsorted(P, a, side="left"), 1, len(P) - 1)
    lo = hi - 1
    code = np.where(a - P[lo] < P[hi] - a, lo, hi)
    code = np.where(a < 448.0, code, 0x7E)
    return (code | (np.signbit(y).astype(np.int64) << 7)).astype(np.uint8)


def _bytes_no_factor2(layers, n_kv, head_dim, w):
    return layers * n_kv * head_dim * w


def _v_token_major(self, layer, block, head, row, ch):
    return self.tile_base(layer, block, head) + 16 * self.head_dim + row * self.head_dim + ch


def _slot_off_by_one(table_row, t):
    return int(table_row[t // 16]) * 16 + (t + 1) % 16


def _layer_inc_no_head_mean(alpha, weight):
    return weight * alpha.sum(axis=0)


def _step_inc_no_head_mean(alphas):
    acc = np.zeros(alphas[0].shape[1])
    for a in alphas:
        acc += a.sum(axis=0)
    return acc / len(alphas)


def _scale_over_256(absmax):
    return (np.asarray(absmax, dtype=np.float32) / np.float32(256.0)).astype(np.float32)


def _append_absmax_new_rows_only(codes, scale, x_new):
    codes = np.asarray(codes, dtype=np.uint8)
    x_new = np.asarray(x_new, dtype=np.float32)
    old = e4m3.decode_table()[codes].astype(np.float32) * np.float32(scale)
    am = np.float32(np.max(np.abs(x_new))) if x_new.size else np.float32(0)
    ns = np.float32(e4m3.scale_of_absmax(am))
    if codes.shape[0] and ns != np.float32(scale):
        codes = e4m3.quantize_tile(old, ns)
    return np.concatenate([codes, e4m3.quantize_tile(x_new, ns)]), ns


def _append_never_reencodes(codes, scale, x_new):
    codes = np.asarray(codes, dtype=np.uint8)
    x_new = np.asarray(x_new, dtype=np.float32)
    old = e4m3.decode_table()[codes].astype(np.float32) * np.float32(scale)
    both = np.concatenate([old.reshape(-1), x_new.reshape(-1)])
    am = np.float32(np.max(np.abs(both))) if both.size else np.float32(0)
    ns = np.float32(e4m3.scale_of_absmax(am))
    return np.concatenate([codes, e4m3.quantize_tile(x_new, ns)]), ns


def _append_new_rows_old_scale(codes, scale, x_new):
    codes = np.asarray(codes, dtype=np.uint8)
    x_new = np.asarray(x_new, dtype=np.float32)
    old = e4m3.decode_table()[codes].astype(np.float32) * np.float32(scale)
    both = np.concatenate([old.reshape(-1), x_new.reshape(-1)])
    am = np.float32(np.max(np.abs(both))) if both.size else np.float32(0)
    ns = np.float32(e4m3.scale_of_absmax(am))
    enc_scale = np.float32(scale) if codes.shape[0] else ns
    if codes.shape[0] and ns != np.float32(scale):
        codes = e4m3.quantize_tile(old, ns)
    return np.concatenate([codes, e4m3.quantize_tile(x_new, enc_scale)]), ns


def _take_highest_first(self):
    if self.free:
        b = max(self.free)
        self.free.remove(b)
    else:
        b = self.evictable.pop(0)
        del self.cache[self.key_of.pop(b)]
    self.ref[b] = 1
    return b


def _take_most_recent(self):
    if self.free:
        b = min(self.free)
        self.free.remove(b)
    else:
        b = self.evictable.pop()
        del self.cache[self.key_of.pop(b)]
    self.ref[b] = 1
    return b


def _release_to_free_list(self, b):
    self.ref[b] -= 1
    if self.ref[b] == 0:
        self.free.append(b)


def _release_ignoring_holders(self, b):
    self.ref[b] = 0
    if b in self.key_of:
        if b not in self.evictable:
            self.evictable.append(b)
    elif b not in self.free:
        self.free.append(b)


def _plan_lowest_first(scores, protect_first, protect_last, t0_blocks, t1_blocks):
    return _orig_plan(-np.asarray(scores), protect_first, protect_last, t0_blocks, t1_blocks)


_orig_plan = tiers.plan_tiers


def _restricted_ignores_mask(q, K, V, keep):
    return attention.decode_sequence(q, np.asarray(K), np.asarray(V))


def _block_scores_max(token_scores, s):
    x = np.asarray(token_scores, dtype=np.float64)[:s]
    nb = -(-s // 16)
    return np.array([x[b * 16:min(s, (b + 1) * 16)].max() for b in range(nb)])


def _arrange_without_pad(ids_bf16, ids_fp8, fp8_last, tail_tokens):
    first, second = (list(ids_bf16), list(ids_fp8)) if fp8_last else (list(ids_fp8), list(ids_bf16))
    tf, ts = (0, 1 << 30) if fp8_last else (1 << 30, 0)
    row = [b | tf for b in first] + [b | ts for b in second]
    return (row, 16 * (len(row) - 1) + tail_tokens) if row else ([], 0)


def _decode_mixed_drops_last(q, blocks):
    return _orig_decode_mixed(q, blocks[:-1])


_orig_decode_mixed = mixed.decode_mixed


MUTATIONS = [
    ("heads modulo instead of grouped", attention, "head_group", _modulo_heads),
    ("logit scale dropped", attention, "logits", _no_scale_logits),
    ("logit scale 1/d", attention, "logits", _natural_scale_logits),
    ("lse without max", attention, "decode_head", _lse_without_max),
    ("merge ignores lse", attention, "merge_partials", _merge_unweighted),
    ("e4m3 bias 8", e4m3, "decode_code", _decode_code_bias8),
    ("e4m3 ties away", e4m3, "encode", _encode_ties_away),
    ("bytes/token missing K+V factor", footprint, "kv_bytes_per_token", _bytes_no_factor2),
    ("V stored token-major", paged.PoolLayout, "v_offset", _v_token_major),
    ("slot off by one", paged, "slot", _slot_off_by_one),
    ("score missing head mean", scores, "layer_increment", _layer_inc_no_head_mean),
    ("score step missing head mean", scores, "step_increment", _step_inc_no_head_mean),
    ("fp8 scale absmax/256", e4m3, "scale_of_absmax", _scale_over_256),
    ("fp8 append absmax of new rows only", e4m3, "append_tile", _append_absmax_new_rows_only),
    ("fp8 append keeps stale codes", e4m3, "append_tile", _append_never_reencodes),
    ("fp8 append encodes new rows with old scale", e4m3, "append_tile", _append_new_rows_old_scale),
    ("blocks handed out highest first", blocks.BlockPool, "_take", _take_highest_first),
    ("evicts the most recently released", blocks.BlockPool, "_take", _take_most_recent),
    ("finished blocks not kept for reuse", blocks.BlockPool, "_release", _release_to_free_list),
    ("release ignores other holders", blocks.BlockPool, "_release", _release_ignoring_holders),
    ("tiers ranked lowest score first", tiers, "plan_tiers", _plan_lowest_first),
    ("restricted decode ignores the kept set", tiers, "restricted_decode", _restricted_ignores_mask),
    ("block score is the max, not the sum", tiers, "block_scores", _block_scores_max),
    ("mixed row without the pad", mixed, "arrange_row", _arrange_without_pad),
    ("mixed step drops a block", mixed, "decode_mixed", _decode_mixed_drops_last),
]


def test_unpatched_oracle_passes_every_pin():
    assert _all_pins_pass()


@pytest.mark.parametrize("name,mod,attr,bad", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, name, mod, attr, bad):
    monkeypatch.setattr(mod, attr, bad)
    if mod is e4m3 and attr == "decode_code":
        monkeypatch.setattr(e4m3, "_POS", np.array([bad(c) for c in range(0x7F)]))
    assert not _all_pins_pass(), f"no pin caught: {name}"
