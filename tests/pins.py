"""Checks that pin the oracle to facts outside itself.

Each function returns the worst deviation (or a bool) of one oracle part
against an independent source: a value the pages print, a closed form, a
library routine, or brute force.  The oracle tests assert on them; the
mutation tests plant plausible mistakes in the oracle and assert that at
least one of them notices.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

from oracle import attention, e4m3, footprint, numerics, paged, scores

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- footprint
def footprint_mismatches() -> list:
    g = _golden("kv_bytes_per_token.json")
    bad = []
    for row in g["per_token"]:
        got = footprint.kv_bytes_per_token(row["layers"], row["n_kv"], row["head_dim"],
                                           row["bytes_per_elem"])
        if got != row["bytes"] or got / 1024 != row["kib"]:
            bad.append(("per_token", row["model"], got))
    for row in g["per_request_gib"]:
        for key, (L, nkv, d) in (("8b", (32, 8, 128)), ("70b", (80, 8, 128))):
            gib = footprint.request_kv_bytes(row["tokens"], L, nkv, d, 2) / 2 ** 30
            if abs(gib - row[key]) > 0.005 + 1e-12:      # the page prints two decimals
                bad.append(("per_request", key, row["tokens"], gib))
    r = g["review_70b"]
    bpt = footprint.kv_bytes_per_token(80, 8, 128, 2)
    if round(bpt / 1e6, 2) != r["mb_per_token_decimal"]:
        bad.append(("mb", bpt))
    if round(footprint.request_kv_bytes(128_000, 80, 8, 128, 2) / 1e9, 1) != r["gb_at_128000"]:
        bad.append(("gb128k",))
    if round(footprint.request_kv_bytes(512_000, 80, 8, 128, 2) / 1e9, 1) != r["gb_at_512000"]:
        bad.append(("gb512k",))
    it = _golden("intensity.json")
    for c in it["cases"]:
        got = footprint.long_context_intensity(c["n_q"], c["n_kv"], c["bytes_per_elem"])
        if got != c["flop_per_byte"]:
            bad.append(("intensity", c, got))
    if round(it["h100_ridge"] / footprint.long_context_intensity(64, 8, 0.25), 1) != it["ratio_2bit_to_ridge"]:
        bad.append(("ridge",))
    return bad


# ---------------------------------------------------------------- bf16
def bf16_rounding_mismatches(n=200_000, seed=0) -> int:
    """Oracle's nearest-even bf16 rounding against torch's fp32 -> bf16 cast."""
    import torch
    rng = np.random.default_rng(seed)
    x = np.concatenate([
        rng.standard_normal(n).astype(np.float32),
        (rng.standard_normal(n) * 1e-38).astype(np.float32),     # subnormal range
        (rng.standard_normal(n) * 1e37).astype(np.float32),
        # exact ties: bf16 values plus half a quantum
        (numerics.bf16_bits_to_f64(rng.integers(0x0080, 0x7F00, n).astype(np.uint16))
         * (1 + 2.0 ** -8)).astype(np.float32),
    ])
    ours = numerics.f64_to_bf16_bits(x.astype(np.float64))
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return int(np.count_nonzero(ours != theirs))


# ---------------------------------------------------------------- e4m3
def e4m3_decode_mismatches() -> int:
    """Decode of all 256 codes against torch.float8_e4m3fn -> float32."""
    import torch
    theirs = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float32)
    theirs = theirs.double().numpy()
    ours = e4m3.decode_table()
    both_nan = np.isnan(ours) & np.isnan(theirs)
    same = both_nan | ((ours == theirs) & (np.signbit(ours) == np.signbit(theirs)))
    return int(np.count_nonzero(~same))


def e4m3_encode_mismatches(n=200_000, seed=1) -> int:
    """Encode against torch's nearest-even cast, inside +-464 where torch does not overflow."""
    import torch
    rng = np.random.default_rng(seed)
    table = e4m3.decode_table()
    fin = table[np.isfinite(table)]
    mids = []
    s = np.sort(np.unique(fin))
    mids = (s[1:] + s[:-1]) / 2                   # exact ties in fp32
    x = np.concatenate([
        (rng.uniform(-463, 463, n)).astype(np.float32),
        (rng.standard_normal(n) * 2.0 ** rng.integers(-12, 6, n)).astype(np.float32),
        mids.astype(np.float32), fin.astype(np.float32),
    ])
    ours = e4m3.encode(x)
    theirs = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # the fast path the quantiser uses must agree too, saturation included
    wide = np.concatenate([x, np.array([464.0, 465.0, 1e30, -1e30, np.inf, -np.inf], np.float32),
                           (rng.uniform(-1e4, 1e4, n)).astype(np.float32)])
    fast_bad = np.count_nonzero(e4m3.encode_nearest_even(wide) != e4m3.encode(wide))
    return int(np.count_nonzero(ours != theirs)) + int(fast_bad)


def e4m3_page_fact_failures() -> list:
    g = _golden("e4m3_facts.json")
    t = e4m3.decode_table()
    bad = []
    fin = t[np.isfinite(t)]
    if np.max(fin) != g["max_finite"]:
        bad.append("max")
    if e4m3.encode(np.array([1e6], np.float32))[0] != e4m3.encode(np.array([448.0], np.float32))[0]:
        bad.append("saturate")
    for sp in g["spacing"]:
        v = np.sort(fin[(fin >= sp["lo"]) & (fin <= sp["hi"])])
        if not np.all(np.diff(v) == sp["step"]):
            bad.append(("spacing", sp))
    for ex in g["examples"]:
        c = e4m3.encode(np.array([ex["in"]], np.float32))[0]
        if t[c] != ex["stored"]:
            bad.append(("example", ex, t[c]))
    b = g["bits"]
    if 2 ** (b["sign"] + b["exponent"] + b["mantissa"]) != len(t):
        bad.append("bits")
    return bad


# ---------------------------------------------------------------- attention
def sdpa_max_error(seed=0) -> float:
    """Oracle decode output against torch scaled_dot_product_attention (float64, GQA)."""
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(seed)
    worst = 0.0
    for (n_q, n_kv, d, s) in [(4, 1, 64, 37), (8, 2, 16, 5), (32, 8, 128, 70), (8, 8, 32, 1),
                              (64, 8, 128, 33), (6, 3, 8, 19)]:
        q = rng.standard_normal((n_q, d))
        K = rng.standard_normal((s, n_kv, d)) * 1.7
        V = rng.standard_normal((s, n_kv, d))
        o, _ = attention.decode_sequence(q, K, V)
        tq = torch.from_numpy(q)[None, :, None, :]
        tk = torch.from_numpy(K).permute(1, 0, 2)[None]
        tv = torch.from_numpy(V).permute(1, 0, 2)[None]
        ref = F.scaled_dot_product_attention(tq, tk, tv, enable_gqa=True)[0, :, 0, :].numpy()
        worst = max(worst, float(np.max(np.abs(o - ref))))
    return worst


def brute_force_max_error(seed=1) -> float:
    """Oracle (o, lse) against explicit pure-Python loops on tiny inputs."""
    rng = np.random.default_rng(seed)
    worst = 0.0
    for (n_q, n_kv, d, s) in [(2, 1, 3, 4), (4, 2, 5, 7), (3, 3, 2, 1), (8, 2, 4, 6)]:
        q = rng.standard_normal((n_q, d))
        K = rng.standard_normal((s, n_kv, d))
        V = rng.standard_normal((s, n_kv, d))
        o, lse = attention.decode_sequence(q, K, V)
        g = n_q // n_kv
        for h in range(n_q):
            j = h // g
            ls = [sum(q[h][c] * K[t][j][c] for c in range(d)) / math.sqrt(d) for t in range(s)]
            den = math.fsum(math.exp(x) for x in ls)
            for c in range(d):
                num = math.fsum(math.exp(ls[t]) * V[t][j][c] for t in range(s))
                worst = max(worst, abs(num / den - o[h][c]))
            worst = max(worst, abs(math.log(den) - lse[h]))
    return worst


def lse_library_max_error(seed=2) -> float:
    """lse against scipy's logsumexp of logits computed by torch matmul."""
    import torch
    from scipy.special import logsumexp
    rng = np.random.default_rng(seed)
    worst = 0.0
    for (n_q, n_kv, d, s) in [(8, 2, 64, 300), (4, 4, 128, 9)]:
        q = rng.standard_normal((n_q, d)) * 3
        K = rng.standard_normal((s, n_kv, d))
        V = rng.standard_normal((s, n_kv, d))
        _, lse = attention.decode_sequence(q, K, V)
        tq = torch.from_numpy(q)
        tk = torch.from_numpy(K).repeat_interleave(n_q // n_kv, dim=1)   # [s][n_q][d]
        lg = torch.einsum("hd,shd->hs", tq, tk).numpy() / np.sqrt(d)
        worst = max(worst, float(np.max(np.abs(lse - logsumexp(lg, axis=1)))))
    return worst


def split_merge_max_error(seed=3) -> float:
    """Merging any chunking's partials reproduces the unsplit result."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((8, 32))
    K = rng.standard_normal((203, 2, 32)) * 2
    V = rng.standard_normal((203, 2, 32))
    o, lse = attention.decode_sequence(q, K, V)
    worst = 0.0
    for chunk in (1, 16, 48, 100, 203, 512):
        oc, lc = attention.chunk_partials(q, K, V, chunk)
        om, lm = attention.merge_partials(oc, lc)
        worst = max(worst, float(np.max(np.abs(om - o))), float(np.max(np.abs(lm - lse))))
    return worst


def uneven_split_merge_max_error(seed=5) -> float:
    """Merging the partials of any contiguous spans that tile the context --
    random cut points, and chunks paired as C + d, C - d (or C - d, C + d) with a
    last chunk left alone -- reproduces the unsplit result."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((8, 32))
    s = 1000
    K = rng.standard_normal((s, 2, 32)) * 2
    V = rng.standard_normal((s, 2, 32))
    o, lse = attention.decode_sequence(q, K, V)

    def merged(bounds):
        spans = list(zip(bounds[:-1], bounds[1:]))
        oc = np.zeros((q.shape[0], len(spans), q.shape[1]))
        lc = np.full((q.shape[0], len(spans)), -np.inf)
        for c, (lo, hi) in enumerate(spans):
            if lo < hi:
                oc[:, c], lc[:, c] = attention.decode_sequence(q, K[lo:hi], V[lo:hi])
        return attention.merge_partials(oc, lc)

    cases = []
    for _ in range(4):
        cuts = np.sort(rng.choice(np.arange(1, s), size=int(rng.integers(1, 12)), replace=False))
        cases.append([0, *cuts.tolist(), s])
    C, d = 224, 32                                   # 5 chunks at C: pairs (0, 1), (2, 3), chunk 4
    for sign in (1, -1):
        b = [0]
        for c in range(5):
            base = (c & ~1) * C
            b.append(min(s, base + C + sign * d if c % 2 == 0 and c + 1 < 5 else (c + 1) * C))
        cases.append(b)
    worst = 0.0
    for bounds in cases:
        om, lm = merged(bounds)
        worst = max(worst, float(np.max(np.abs(om - o))), float(np.max(np.abs(lm - lse))))
    return worst


def special_case_failures(seed=4) -> list:
    rng = np.random.default_rng(seed)
    bad = []
    d = 16
    q = rng.standard_normal((4, d))
    # s = 1: output is V_0 exactly, lse = l_0
    K = rng.standard_normal((1, 2, d))
    V = rng.standard_normal((1, 2, d))
    o, lse = attention.decode_sequence(q, K, V)
    for h in range(4):
        if not np.array_equal(o[h], V[0, h // 2]):
            bad.append("s1")
    # q = 0: uniform weights, o = mean of V, lse = log s
    K = rng.standard_normal((10, 2, d))
    V = rng.standard_normal((10, 2, d))
    o, lse = attention.decode_sequence(np.zeros((4, d)), K, V)
    if np.max(np.abs(o[0] - V[:, 0].mean(0))) > 1e-14 or abs(lse[0] - math.log(10)) > 1e-14:
        bad.append("q0")
    # constant V: output equals the constant
    Vc = np.full((10, 2, d), 0.375)
    o, _ = attention.decode_sequence(q, K, Vc)
    if np.max(np.abs(o - 0.375)) > 1e-15:
        bad.append("constV")
    # one logit far above the rest: output is that token's V
    K = np.zeros((10, 2, d))
    K[7, :, :] = q[0] / np.linalg.norm(q[0]) * 400.0
    o, _ = attention.decode_sequence(q[:1].repeat(4, 0), K, V)
    if np.max(np.abs(o[0] - V[7, 0])) > 1e-12:
        bad.append("dominant")
    # empty context
    o, lse = attention.decode_sequence(q, np.zeros((0, 2, d)), np.zeros((0, 2, d)))
    if np.any(o != 0) or np.any(lse != -np.inf):
        bad.append("empty")
    # weights sum to one
    a = attention.attention_weights_sequence(q, rng.standard_normal((50, 2, d)) * 3)
    if np.max(np.abs(a.sum(1) - 1)) > 1e-12:
        bad.append("sum1")
    return bad


# ---------------------------------------------------------------- paging
def block_table_example_failures() -> list:
    g = _golden("block_table_example.json")
    bs = g["block_size"]
    bad = []
    used = sorted(b for t in g["tables"].values() for b in t)
    if used != list(range(g["pool_blocks"])):
        bad.append("cover")
    lay = paged.PoolLayout(num_layers=1, num_blocks=g["pool_blocks"], n_kv=2, head_dim=8)
    pool = np.full(lay.total_elems, np.nan)
    rng = np.random.default_rng(5)
    data = {}
    for name, table in g["tables"].items():
        s = len(table) * bs - (3 if name != "A" else 0)     # the last block may be partial
        if paged.tail_waste(s) > g["max_waste_tokens"]:
            bad.append(("waste", name))
        K = rng.standard_normal((s, 2, 8))
        V = rng.standard_normal((s, 2, 8))
        paged.scatter(pool, lay, 0, table, K, V)
        data[name] = (table, K, V)
        # the slot of token t lies in physical block table[t // 16] at row t % 16
        for t in range(s):
            p, row = divmod(paged.slot(table, t), bs)
            if p != table[t // bs] or row != t % bs:
                bad.append(("slot", name, t))
    for name, (table, K, V) in data.items():
        K2, V2 = paged.gather(pool, lay, 0, table, K.shape[0])
        if not (np.array_equal(K, K2) and np.array_equal(V, V2)):
            bad.append(("roundtrip", name))
    # documented layout (head_dim 8, bf16: 8 channels per 16-byte piece, one
    # piece per row): K row t in piece 8 ((t // 4) % 2) + 4 (t // 8) + t % 4;
    # V channel-major after the K tile; worked by hand:
    base = lay.tile_base(0, 3, 1)
    for row, ch, want in [(2, 1, 17), (5, 3, 75), (12, 7, 103), (15, 0, 15 * 8)]:
        if lay.k_offset(0, 3, 1, row, ch) - base != want:
            bad.append(("k_layout", row, ch))
    if lay.v_offset(0, 3, 1, 2, 1) - base != 16 * 8 + 1 * 16 + 2:
        bad.append("v_layout")
    # every K element of a tile has its own place inside the K half of the tile
    for d, w in [(8, 2), (64, 2), (128, 2), (64, 1), (128, 1)]:
        L2 = paged.PoolLayout(1, 1, 1, d, elem_bytes=w)
        offs = sorted(int(L2.k_in_tile(r, c)) for r in range(16) for c in range(d))
        if offs != list(range(16 * d)):
            bad.append(("k_permutation", d, w))
    return bad


def placement_invariance_max_error(seed=6) -> float:
    """Paged result (gather through any block table) equals the contiguous result."""
    rng = np.random.default_rng(seed)
    s, n_kv, d, n_q = 75, 2, 8, 4
    K = rng.standard_normal((s, n_kv, d))
    V = rng.standard_normal((s, n_kv, d))
    q = rng.standard_normal((n_q, d))
    o_ref, lse_ref = attention.decode_sequence(q, K, V)
    worst = 0.0
    nb = paged.blocks_needed(s)
    for trial in range(3):
        lay = paged.PoolLayout(1, 12, n_kv, d)
        table = rng.permutation(12)[:nb]
        pool = np.zeros(lay.total_elems)
        paged.scatter(pool, lay, 0, table, K, V)
        K2, V2 = paged.gather(pool, lay, 0, table, s)
        o, lse = attention.decode_sequence(q, K2, V2)
        worst = max(worst, float(np.max(np.abs(o - o_ref))), float(np.max(np.abs(lse - lse_ref))))
    return worst


# ---------------------------------------------------------------- scores
def score_failures(seed=7) -> list:
    rng = np.random.default_rng(seed)
    bad = []
    d, n_q, n_kv, s, L = 16, 8, 2, 40, 3
    alphas = []
    for _ in range(L):
        q = rng.standard_normal((n_q, d))
        K = rng.standard_normal((s, n_kv, d)) * 2
        alphas.append(attention.attention_weights_sequence(q, K))
    inc = scores.step_increment(alphas)
    if abs(inc.sum() - 1.0) > 1e-12:
        bad.append("sum1")
    # per-layer calls with weight 1/L add up to the step increment
    acc = sum(scores.layer_increment(a, 1.0 / L) for a in alphas)
    if np.max(np.abs(acc - inc)) > 1e-15:
        bad.append("layers")
    # uniform attention: every position gains 1/s
    a0 = attention.attention_weights_sequence(np.zeros((n_q, d)), rng.standard_normal((s, n_kv, d)))
    if np.max(np.abs(scores.step_increment([a0]) - 1.0 / s)) > 1e-15:
        bad.append("uniform")
    # brute force: one layer, explicit double loop
    a = alphas[0]
    for t in range(s):
        bf = math.fsum(a[h][t] for h in range(n_q)) / n_q
        if abs(bf - scores.step_increment([a])[t]) > 1e-15:
            bad.append(("bf", t))
            break
    return bad


# ---------------------------------------------------------------- fp8 path
def fp8_quant_failures(seed=8) -> list:
    rng = np.random.default_rng(seed)
    bad = []
    s, n_kv, d = 37, 2, 8                       # last block has 5 rows
    X = (rng.standard_normal((s, n_kv, d)) * 3).astype(np.float32)
    X[16:32, 1, :] = 0                          # an all-zero block
    codes, sc = e4m3.quantize_sequence(X)
    table = e4m3.decode_table()
    for b in range(3):
        for j in range(n_kv):
            rows = X[b * 16:min(s, b * 16 + 16), j]
            am = np.float32(np.max(np.abs(rows)))
            if sc[b, j] != np.float32(am / np.float32(448)):
                bad.append(("scale", b, j))
            c = codes[b * 16:min(s, b * 16 + 16), j]
            if am == 0:
                if np.any(c != 0):
                    bad.append("zero_block")
                continue
            # the element holding the absmax maps to +-448 exactly
            if np.max(np.abs(table[c])) != 448.0:
                bad.append(("max448", b, j))
    # a tile's scale ignores rows past the sequence end (the short last block)
    X2 = X.copy()
    Xext = np.concatenate([X2, np.full((11, n_kv, d), 1e30, np.float32)])
    c2, sc2 = e4m3.quantize_sequence(Xext[:s])
    if not (np.array_equal(c2, codes) and np.array_equal(sc2, sc)):
        bad.append("tail")
    # dequantised values are within half a step of the input
    deq = e4m3.dequantize_sequence(codes, sc)
    rel = np.abs(deq - X) / np.maximum(np.abs(X), 1e-30)
    big = np.abs(X) >= 2 ** -6 * np.repeat(sc, 16, axis=0)[:s, :, None]
    if np.max(rel[big]) > 2.0 ** -4 + 1e-7:
        bad.append("halfstep")
    # power-of-two scale and values on the grid: exact round trip
    Y = np.zeros((1, 1, 4), np.float32)
    Y[0, 0] = [448.0, -3.25, 0.125, 2 ** -9]
    cY, sY = e4m3.quantize_sequence(Y)
    if sY[0, 0] != 1.0 or not np.array_equal(e4m3.dequantize_sequence(cY, sY)[0, 0], Y[0, 0]):
        bad.append("exact")
    return bad


def fp8_append_failures(seed=9) -> list:
    """Appending to partly filled FP8 tiles: reduces to the block quantiser when
    a tile starts empty; scales only grow; the largest element of a nonzero
    tile reads back as +-448; appended rows, and old rows across a re-encode,
    move by at most half an E4M3 step; zero rows leave a tile untouched; on a
    power-of-two grid every value survives a scale doubling exactly."""
    rng = np.random.default_rng(seed)
    bad = []
    table = e4m3.decode_table()
    s, n_kv, d = 37, 2, 8
    X = (rng.standard_normal((s, n_kv, d)) * 3).astype(np.float32)
    X[20, 0, 3] = 40.0                           # a late large value forces a re-encode
    empty_c = np.zeros((0, n_kv, d), np.uint8)
    empty_s = np.zeros((0, n_kv), np.float32)
    # whole sequence in one append == block quantisation
    c_all, s_all = e4m3.append_sequence(empty_c, empty_s, X)
    c_ref, s_ref = e4m3.quantize_sequence(X)
    if not (np.array_equal(c_all, c_ref) and np.array_equal(s_all, s_ref)):
        bad.append("prefill")
    # token by token after a 5-token prefill
    c, sc = e4m3.append_sequence(empty_c, empty_s, X[:5])
    half = 2.0 ** -4 + 1e-6                      # half a step relative, plus fp32 slack
    for t in range(5, s):
        before = e4m3.dequantize_sequence(c, sc)
        c2, sc2 = e4m3.append_sequence(c, sc, X[t:t + 1])
        after = e4m3.dequantize_sequence(c2, sc2)
        nb_old = sc.shape[0]
        if np.any(sc2[:nb_old] < sc):
            bad.append(("monotone", t))
        blk = t // 16
        for j in range(n_kv):
            tile = c2[blk * 16:t + 1, j]
            if sc2[blk, j] != 0 and np.max(np.abs(table[tile])) != 448.0:
                bad.append(("max448", t, j))
        floor = 2.0 ** -6 * np.float64(sc2[blk])[None, :, None]    # below: subnormal grid
        rows = slice(blk * 16, t)
        o_b, o_a = before[rows], after[rows]
        big = np.abs(o_b) >= floor
        if np.any(np.abs(o_a - o_b)[big] > half * np.abs(o_b)[big]):
            bad.append(("old_moved", t))
        if np.any(np.abs(o_a - o_b)[~big] > 2.0 ** -10 * np.broadcast_to(np.float64(sc2[blk])[None, :, None], o_b.shape)[~big] + 1e-30):
            bad.append(("old_moved_sub", t))
        x = X[t].astype(np.float64)
        bigx = np.abs(x) >= floor[0]
        if np.any(np.abs(after[t] - x)[bigx] > half * np.abs(x)[bigx]):
            bad.append(("new_row", t))
        c, sc = c2, sc2
    # zero rows appended under an unchanged scale leave the old codes as they are
    base_c, base_s = e4m3.append_sequence(empty_c, empty_s, X[:3])
    zc, zs = e4m3.append_sequence(base_c, base_s, np.zeros((2, n_kv, d), np.float32))
    if np.array_equal(zs, base_s) and not np.array_equal(zc[:3], base_c):
        bad.append("zero_append")
    # power-of-two grid: scale 1 then 2, every value read back exactly
    g = np.array([[448.0, -3.25, 0.125, 2.0 ** -5]], np.float32).reshape(1, 1, 4)
    gc, gs = e4m3.append_sequence(np.zeros((0, 1, 4), np.uint8), np.zeros((0, 1), np.float32), g)
    g2 = np.array([[896.0, 1.0, -6.5, 0.25]], np.float32).reshape(1, 1, 4)
    gc2, gs2 = e4m3.append_sequence(gc, gs, g2)
    back = e4m3.dequantize_sequence(gc2, gs2)
    if gs[0, 0] != 1.0 or gs2[0, 0] != 2.0 or not np.array_equal(back, np.concatenate([g, g2]).astype(np.float64)):
        bad.append("grid")
    return bad


# ---------------------------------------------------------------- block manager
def _blocks_invariant_failures(bp) -> list:
    """Every block is free, evictable or referenced, exactly once; a block's count
    is the number of live tables holding it; each table has ceil(len/16) blocks."""
    bad = []
    count = [0] * bp.num_blocks
    for sid, seq in bp.seqs.items():
        if len(seq["blocks"]) != -(-seq["len"] // 16):
            bad.append(("waste", sid))
        for b in seq["blocks"]:
            count[b] += 1
    if count != bp.ref:
        bad.append("refcount")
    free, evict = set(bp.free), set(bp.evictable)
    used = {b for b in range(bp.num_blocks) if bp.ref[b] > 0}
    if free & evict or free & used or evict & used or len(free | evict | used) != bp.num_blocks:
        bad.append("partition")
    if len(free) != len(bp.free) or len(evict) != len(bp.evictable):
        bad.append("duplicates")
    return bad


def block_manager_failures(seed=12) -> list:
    from oracle import blocks
    bad = []
    g = _golden("block_table_example.json")
    # the page's three tables: the requests grow in turn, lowest free block first
    bp = blocks.BlockPool(g["pool_blocks"])
    a, _ = bp.add_sequence(16)
    b, _ = bp.add_sequence(32)
    c, _ = bp.add_sequence(16)
    for sid, n in [(a, 16), (b, 32), (c, 16), (b, 32), (c, 16)]:
        bp.append(sid, n)
    got = {"A": bp.table(a), "B": bp.table(b), "C": bp.table(c)}
    if got != g["tables"]:
        bad.append(("example", got))
    for name, sid in [("A", a), ("B", b), ("C", c)]:
        if bp.slots(sid, 0, bp.length(sid)) != [paged.slot(g["tables"][name], t) for t in range(bp.length(sid))]:
            bad.append(("slots", name))
    bad += _blocks_invariant_failures(bp)
    # random traffic without prefix caching: no block is ever shared, waste <= 15
    rng = np.random.default_rng(seed)
    bp = blocks.BlockPool(40)
    live = []
    for _ in range(400):
        op = rng.integers(3)
        try:
            if op == 0 or not live:
                live.append(bp.add_sequence(int(rng.integers(0, 60)))[0])
            elif op == 1:
                bp.append(live[int(rng.integers(len(live)))], int(rng.integers(1, 20)))
            else:
                bp.free_sequence(live.pop(int(rng.integers(len(live)))))
        except blocks.NoBlocks:
            pass
        inv = _blocks_invariant_failures(bp)
        if inv:
            bad.append(("random", inv))
            break
        if max(bp.ref) > 1:
            bad.append("shared_without_prefix_cache")
            break
    # prefix cache
    T = [int(x) for x in rng.integers(0, 1000, 40)]
    bp = blocks.BlockPool(12, prefix_cache=True)
    p, n0 = bp.add_sequence(40, T)
    q, n1 = bp.add_sequence(40, T)
    if n0 != 0 or n1 != 32 or bp.table(q)[:2] != bp.table(p)[:2] or bp.table(q)[2] == bp.table(p)[2]:
        bad.append(("reuse", n0, n1))          # two full blocks reused; the 8-token tail never
    if [bp.ref[x] for x in bp.table(p)] != [2, 2, 1]:
        bad.append("reuse_counts")
    T1 = list(T)
    T1[0] += 1                                  # a different first token: nothing matches
    r, n2 = bp.add_sequence(40, T1)
    T2 = list(T)
    T2[20] += 1                                 # a difference in block 1: block 0 only
    s_, n3 = bp.add_sequence(40, T2)
    if n2 != 0 or n3 != 16:
        bad.append(("first_miss", n2, n3))
    bad += _blocks_invariant_failures(bp)
    # a block that fills during decoding becomes reusable too
    bp.append(p, 8, [7] * 8)
    t_, n4 = bp.add_sequence(48, T + [7] * 8)
    if n4 != 48:
        bad.append(("decode_filled", n4))
    # eviction: only unreferenced blocks, least recently released first
    bp = blocks.BlockPool(4, prefix_cache=True)
    p, _ = bp.add_sequence(32, T[:32])          # blocks 0, 1
    q, _ = bp.add_sequence(16, T[:16])          # shares block 0
    bp.free_sequence(p)                         # block 1 evictable; block 0 still held by q
    x, _ = bp.add_sequence(32)                  # free blocks 2, 3
    y, _ = bp.add_sequence(16)                  # must evict block 1, never block 0
    if bp.table(y) != [1] or bp.ref[0] != 1:
        bad.append(("evict", bp.table(y)))
    before = (list(bp.free), list(bp.evictable), list(bp.ref), {k: list(v["blocks"]) for k, v in bp.seqs.items()})
    try:
        bp.add_sequence(16)                     # nothing left: fails and changes nothing
        bad.append("no_fail")
    except blocks.NoBlocks:
        pass
    after = (list(bp.free), list(bp.evictable), list(bp.ref), {k: list(v["blocks"]) for k, v in bp.seqs.items()})
    if before != after:
        bad.append("atomic")
    # release order: the tail of a finished request is evicted before its head
    bp = blocks.BlockPool(3, prefix_cache=True)
    p, _ = bp.add_sequence(48, T[:32] + [1] * 16)
    bp.free_sequence(p)
    z, _ = bp.add_sequence(16)
    if bp.table(z) != [2]:
        bad.append(("release_order", bp.table(z)))
    return bad


# ---------------------------------------------------------------- tiers
def tier_failures(seed=13) -> list:
    """Tier-restricted decode: all-kept reduces to the plain step; a brute-force
    softmax over the kept tokens; weights 0 off the kept set and summing to 1
    on it; the plan's protected blocks, budgets and ranking; block scores as
    sums; the 64-step schedule; the result depends only on the evicted set."""
    from oracle import tiers
    rng = np.random.default_rng(seed)
    bad = []
    s, n_q, n_kv, d = 37, 4, 2, 8
    q = rng.standard_normal((n_q, d))
    K = rng.standard_normal((s, n_kv, d))
    V = rng.standard_normal((s, n_kv, d))
    o_all, l_all = tiers.restricted_decode(q, K, V, np.ones(s, bool))
    o_ref, l_ref = attention.decode_sequence(q, K, V)
    if not (np.array_equal(o_all, o_ref) and np.array_equal(l_all, l_ref)):
        bad.append("all_kept")
    keep = rng.random(s) < 0.5
    keep[3] = True
    o, lse = tiers.restricted_decode(q, K, V, keep)
    for h in range(n_q):
        j = h // (n_q // n_kv)
        idx = [t for t in range(s) if keep[t]]
        lg = [sum(q[h, c] * K[t, j, c] for c in range(d)) / math.sqrt(d) for t in idx]
        m = max(lg)
        e = [math.exp(x - m) for x in lg]
        z = math.fsum(e)
        want = [math.fsum(e[k] * V[t, j, c] for k, t in enumerate(idx)) / z for c in range(d)]
        if np.max(np.abs(o[h] - np.array(want))) > 1e-13 or abs(lse[h] - (m + math.log(z))) > 1e-13:
            bad.append(("brute", h))
    a = tiers.restricted_weights(q, K, keep)
    if np.any(a[:, ~keep] != 0) or np.max(np.abs(a[:, keep].sum(axis=1) - 1)) > 1e-12:
        bad.append("weights")
    o0, l0 = tiers.restricted_decode(q, K, V, np.zeros(s, bool))
    if np.any(o0 != 0) or not np.all(np.isneginf(l0)):
        bad.append("nothing_kept")
    # block scores: sums over each block's tokens (the last block holds 5)
    ts = np.arange(37, dtype=np.float64)
    if list(tiers.block_scores(ts, 37)) != [120.0, 376.0, 170.0]:
        bad.append("block_scores")
    # the plan
    sc = rng.random(20)
    sc[7] = sc[9]                                # a tie: block 7 ranks before block 9
    tier = tiers.plan_tiers(sc, 2, 3, 5, 4)
    if not all(tier[b] == tiers.T0 for b in (0, 1, 17, 18, 19)):
        bad.append("protected")
    rest = [b for b in range(2, 17)]
    if sum(tier[b] == tiers.T0 for b in rest) != 5 or sum(tier[b] == tiers.T1 for b in rest) != 4:
        bad.append("budgets")
    lo0 = min(sc[b] for b in rest if tier[b] == tiers.T0)
    hi1, lo1 = max(sc[b] for b in rest if tier[b] == tiers.T1), min(sc[b] for b in rest if tier[b] == tiers.T1)
    hi3 = max(sc[b] for b in rest if tier[b] == tiers.T3)
    if not (lo0 >= hi1 and lo1 >= hi3):
        bad.append("ranking")
    tie = tiers.plan_tiers(np.zeros(6), 0, 0, 2, 2)
    if list(tie) != [tiers.T0, tiers.T0, tiers.T1, tiers.T1, tiers.T3, tiers.T3]:
        bad.append("ties")
    if any(t == tiers.T3 for t in tiers.plan_tiers(sc, 2, 3, 10, 10)):
        bad.append("roomy_budget")
    if not (tiers.retier_due(0) and tiers.retier_due(128) and not tiers.retier_due(63)):
        bad.append("delta")
    km = tiers.kept_tokens([tiers.T0, tiers.T3, tiers.T1], 37)
    if not (km[:16].all() and not km[16:32].any() and km[32:].all()):
        bad.append("kept_tokens")
    # Proposition 1: another T0/T1 split with the same evicted blocks gives the same result
    sc3 = rng.random(3)
    p1 = tiers.plan_tiers(sc3, 0, 1, 1, 0)
    p2 = tiers.plan_tiers(sc3, 0, 1, 0, 1)
    if not np.array_equal(p1 == tiers.T3, p2 == tiers.T3) or np.array_equal(p1, p2):
        bad.append("prop1_setup")
    r1 = tiers.restricted_decode(q, K, V, tiers.kept_tokens(p1, s))
    r2 = tiers.restricted_decode(q, K, V, tiers.kept_tokens(p2, s))
    if not (np.array_equal(r1[0], r2[0]) and np.array_equal(r1[1], r2[1])):
        bad.append("prop1")
    return bad


# ---------------------------------------------------------------- mixed precision
def mixed_failures(seed=14) -> list:
    """Mixed-precision rows: every pair one precision, every block once with its
    precision bit, a pad only between an odd first run and a second run, the
    context length; the step over a row's blocks equals the plain step over the
    same tokens whatever their order, FP8 blocks entering as stored."""
    from oracle import e4m3, mixed
    rng = np.random.default_rng(seed)
    bad = []
    for _ in range(200):
        n16, n8 = int(rng.integers(0, 7)), int(rng.integers(0, 7))
        ids = rng.permutation(100)[:n16 + n8]
        a, b = list(ids[:n16]), list(ids[n16:])
        fp8_last = bool(rng.integers(2))
        tail = int(rng.integers(1, 17))
        row, s = mixed.arrange_row(a, b, fp8_last, tail)
        if not mixed.pairs_homogeneous(row):
            bad.append(("homogeneous", a, b, fp8_last))
            break
        real = [e for e in row if e >= 0]
        if sorted(real) != sorted(a + [x | mixed.PRECISION_BIT for x in b]):
            bad.append(("ids", a, b))
            break
        first = a if fp8_last else b
        second = b if fp8_last else a
        pads = row.count(-1)
        if pads != (1 if second and len(first) % 2 else 0):
            bad.append(("pad", a, b, fp8_last))
            break
        if row and (s != 16 * (len(row) - 1) + tail or row[-1] < 0):
            bad.append(("length", a, b))
            break
    # a worked row: bf16 blocks 3, 8, 5 then FP8 blocks 2, 7 (the last holding 9 tokens)
    row, s = mixed.arrange_row([3, 8, 5], [2, 7], True, 9)
    if row != [3, 8, 5, -1, 2 | (1 << 30), 7 | (1 << 30)] or s != 16 * 5 + 9:
        bad.append(("worked", row, s))
    # the step over the blocks, in any order, equals the plain step
    n_q, n_kv, d, s = 4, 2, 16, 16 * 5 + 7
    q = rng.standard_normal((n_q, d))
    K = rng.standard_normal((s, n_kv, d)).astype(np.float32)
    V = rng.standard_normal((s, n_kv, d)).astype(np.float32)
    stored_K, stored_V = K.astype(np.float64).copy(), V.astype(np.float64).copy()
    blocks = []
    for b in range(6):
        lo, hi = 16 * b, min(s, 16 * b + 16)
        if b % 2:                                      # odd blocks stored as FP8
            ck, sk = e4m3.quantize_sequence(K[lo:hi])
            cv, sv = e4m3.quantize_sequence(V[lo:hi])
            stored_K[lo:hi] = e4m3.dequantize_sequence(ck, sk)
            stored_V[lo:hi] = e4m3.dequantize_sequence(cv, sv)
        blocks.append((stored_K[lo:hi], stored_V[lo:hi]))
    o_ref, l_ref = attention.decode_sequence(q, stored_K, stored_V)
    for perm in (list(range(6)), [5, 0, 3, 1, 4, 2], [1, 3, 5, 0, 2, 4]):
        o, l = mixed.decode_mixed(q, [blocks[k] for k in perm])
        if np.max(np.abs(o - o_ref)) > 1e-13 or np.max(np.abs(l - l_ref)) > 1e-13:
            bad.append(("order", perm))
    o0, l0 = mixed.decode_mixed(q, [])
    if np.any(o0 != 0) or not np.all(np.isneginf(l0)):
        bad.append("empty")
    return bad
