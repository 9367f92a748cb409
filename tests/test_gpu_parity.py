"""GPU parity of the HIP path against the float64 oracle (small and ragged sizes).

Every call goes through the C ABI of libkvdecode.  Sizes span several 32-token
pairs, several chunks and a ragged last block; edge cases cover empty and
one-token contexts, stale NaN rows in partly filled blocks, bad block ids,
several layers, block permutations and repeated runs.
"""
import json
import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

LENS = [0, 1, 15, 16, 17, 31, 32, 33, 100, 257, 1000]


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import decode_attention_paged_04_amd as kvd
    import gpu_harness as H
    import workloads as W
    return kvd, H, W, torch


def _workload(W, g, d, n_kv=2, fp8=False, seed=11, layers=1):
    return W.DecodeWorkload(f"grid-g{g}-d{d}", seed=seed, b=len(LENS), layers=layers, n_q=g * n_kv,
                            n_kv=n_kv, head_dim=d, ctx=("fixed", 0),
                            kv_dtype="fp8" if fp8 else "bf16")


def _case(H, W, w, lens=LENS, **kw):
    lens = np.array(lens, dtype=np.int32)
    table, nb = W.block_tables(w, lens, pad_value=-1)
    return H.PagedCase(w, lens=lens, table=table, num_blocks=nb, **kw)


def test_fp8_widening_of_every_code(env):
    kvd, H, W, torch = env
    from oracle import e4m3
    for n in (256, 13):
        codes = torch.arange(256, dtype=torch.uint8, device="cuda")[:n].contiguous()
        out = torch.empty(n, dtype=torch.float32, device="cuda")
        kvd.kvd_debug_fp8_decode(codes, out)
        torch.cuda.synchronize()
        got = out.cpu().double().numpy()
        ref = e4m3.decode_table()[:n]
        both_nan = np.isnan(got) & np.isnan(ref)
        same = both_nan | ((got == ref) & (np.signbit(got) == np.signbit(ref)))
        assert same.all(), np.nonzero(~same)[0][:10]


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_gather_offsets_follow_the_block_table(env, dtype):
    kvd, H, W, torch = env
    from oracle import paged
    here = os.path.dirname(os.path.abspath(__file__))
    ex = json.load(open(os.path.join(here, "golden", "block_table_example.json")))
    rows = [ex["tables"][k] for k in ("A", "B", "C")] + [[2, 11, -5]]   # last row: bad ids
    mb = max(len(r) for r in rows)
    table = np.full((len(rows), mb), -1, dtype=np.int32)
    for i, r in enumerate(rows):
        table[i, :len(r)] = r
    nb, n_kv, d, L = ex["pool_blocks"], 2, 64, 3
    dt = kvd.KVD_FP8_E4M3 if dtype == "fp8" else kvd.KVD_BF16
    pool = kvd.allocate_pool(L, nb, n_kv, d, dt)
    lay = paged.PoolLayout(L, nb, n_kv, d, elem_bytes=1 if dtype == "fp8" else 2)
    n_tok = 16 * mb
    tt = torch.from_numpy(table).cuda()
    for layer in (0, 2):
        ok = torch.empty((len(rows), n_kv, n_tok), dtype=torch.int64, device="cuda")
        ov = torch.empty_like(ok)
        kvd.kvd_debug_gather_offsets(pool, layer, tt, n_tok, ok, ov)
        torch.cuda.synchronize()
        gk, gv = ok.cpu().numpy(), ov.cpu().numpy()
        for i in range(len(rows)):
            for j in range(n_kv):
                for t in range(n_tok):
                    p = int(table[i, t // 16])
                    if 0 <= p < nb:
                        assert gk[i, j, t] == lay.k_offset(layer, p, j, t % 16, 0)
                        assert gv[i, j, t] == lay.v_offset(layer, p, j, t % 16, 0)
                    else:
                        assert gk[i, j, t] == -1 and gv[i, j, t] == -1


@pytest.mark.parametrize("d", [64, 128])
def test_write_bf16_places_every_element(env, d):
    kvd, H, W, torch = env
    from oracle import paged
    w = _workload(W, 2, d, layers=2)
    lens = [1, 16, 17, 40, 0]
    case = _case(H, W, w, lens=lens)
    got = case.pool.kv.cpu().numpy().view(np.uint16)
    lay = case.layout()
    exp = np.full(lay.total_elems, 0xFFFF, dtype=np.uint16)
    for layer in range(2):
        K, V = case.kv[layer]
        Kb = K.view(torch.int16).numpy().view(np.uint16)
        Vb = V.view(torch.int16).numpy().view(np.uint16)
        for i, s in enumerate(lens):
            lo = int(case.offs[i])
            k_idx, v_idx = paged.gather_indices(lay, layer, case.table[i], s)
            exp[k_idx] = Kb[lo:lo + s]
            exp[v_idx] = Vb[lo:lo + s]
    assert np.array_equal(got, exp)


@pytest.mark.parametrize("d", [64, 128])
def test_write_fp8_codes_and_scales_bit_exact(env, d):
    kvd, H, W, torch = env
    from oracle import e4m3, paged
    lens = np.array([1, 16, 17, 40, 0, 33], dtype=np.int32)
    w = _workload(W, 2, d, fp8=True, layers=2)
    table, nb = W.block_tables(w, lens)
    # custom data: an all-zero tile, exact E4M3 midpoints, and tiny values
    case = H.PagedCase(w, lens=lens, table=table, num_blocks=nb, keep_layers=[0, 1])
    n = int(case.offs[-1])
    K, V = case.kv[0]
    Kf, Vf = K.float(), V.float()
    Kf[int(case.offs[1]):int(case.offs[1]) + 16, 0, :] = 0          # seq 1 block 0, head 0
    Vf[int(case.offs[3]) + 16:int(case.offs[3]) + 32, 1, :] = 0     # seq 3 block 1, head 1
    Kf[int(case.offs[2]), 1, :4] = torch.tensor([448.0, 3.125, 3.375, 1e-4])   # ties after scaling
    Vf[int(case.offs[5]):int(case.offs[5]) + 16, 0, :] *= 1e-30      # very small magnitudes
    K2, V2 = Kf.to(torch.bfloat16), Vf.to(torch.bfloat16)
    case.kv[0] = (K2, V2)
    slots = kvd.kvd_slot_mapping(case.table_t, case.lens_t)
    kvd.kvd_write_kv(case.pool, 0, K2.cuda(), V2.cuda(), slots)
    torch.cuda.synchronize()
    got = case.pool.kv.cpu().numpy()
    got_sc = case.pool.scales.cpu().numpy()
    lay = case.layout()
    exp = np.full(lay.total_elems, 0xFF, dtype=np.uint8)
    exp_sc = np.zeros(lay.num_layers * nb * w.n_kv * 2, dtype=np.float32)
    for layer in range(2):
        Kl, Vl = case.kv[layer]
        for i, s in enumerate(lens):
            if s == 0:
                continue
            lo = int(case.offs[i])
            k_idx, v_idx = paged.gather_indices(lay, layer, case.table[i], s)
            ck, sk = e4m3.quantize_sequence(Kl[lo:lo + s].float().numpy())
            cv, sv = e4m3.quantize_sequence(Vl[lo:lo + s].float().numpy())
            exp[k_idx] = ck
            exp[v_idx] = cv
            for b in range(sk.shape[0]):
                p = int(case.table[i, b])
                for j in range(w.n_kv):
                    exp_sc[lay.scale_index(layer, p, j, 0)] = sk[b, j]
                    exp_sc[lay.scale_index(layer, p, j, 1)] = sv[b, j]
    assert np.array_equal(got_sc.view(np.uint32), exp_sc.view(np.uint32))
    assert np.array_equal(got, exp), np.count_nonzero(got != exp)


@pytest.mark.parametrize("g", [1, 4, 8, 16])
@pytest.mark.parametrize("d", [64, 128])
def test_decode_bf16_ragged_grid(env, g, d):
    kvd, H, W, torch = env
    w = _workload(W, g, d, seed=100 + g + d)
    case = _case(H, W, w)
    ref_o, ref_lse = case.oracle(0)
    for chunk in (0, 16, 48, 256):
        H.say(f"g={g} d={d} chunk={chunk}")
        out, lse = case.run(0, chunk=chunk)
        torch.cuda.synchronize()
        H.assert_bf16_close(out, ref_o, what=f"g{g} d{d} chunk{chunk}")
        H.assert_lse_close(lse, ref_lse)
        # s = 0 gives exact zeros and -inf
        assert torch.all(out[0] == 0) and torch.all(torch.isneginf(lse[0]))


@pytest.mark.parametrize("g", [4, 8])
@pytest.mark.parametrize("d", [64, 128])
def test_decode_fp8_ragged_grid(env, g, d):
    kvd, H, W, torch = env
    w = _workload(W, g, d, fp8=True, seed=200 + g + d)
    case = _case(H, W, w)
    ref_o, ref_lse = case.oracle(0)
    for chunk in (0, 32, 256):
        H.say(f"fp8 g={g} d={d} chunk={chunk}")
        out, lse = case.run(0, chunk=chunk)
        torch.cuda.synchronize()
        mx, rel = H.assert_bf16_close(out, ref_o, rel_tol=H.TOL_FP8_REL_L2, what=f"fp8 g{g} d{d}")
        # computing on the decoded codes is exact up to fp32 rounding: hold it to the bf16 bar too
        assert rel <= H.TOL_REL_L2, rel
        H.assert_lse_close(lse, ref_lse)


@pytest.mark.parametrize("fp8", [False, True])
def test_several_layers_are_independent(env, fp8):
    kvd, H, W, torch = env
    w = _workload(W, 4, 128, fp8=fp8, seed=300, layers=3)
    case = _case(H, W, w, lens=[5, 70, 300])
    for layer in range(3):
        out, lse = case.run(layer, chunk=64)
        torch.cuda.synchronize()
        ref_o, ref_lse = case.oracle(layer)
        H.assert_bf16_close(out, ref_o, what=f"layer {layer}")
        H.assert_lse_close(lse, ref_lse)


def test_block_placement_and_reruns_are_bit_identical(env):
    kvd, H, W, torch = env
    w = _workload(W, 8, 128, seed=400)
    lens = np.array([1, 33, 700, 1000], dtype=np.int32)
    outs = []
    for perm_seed in (1, 2, 3):
        table, nb = W.block_tables(w, lens, rng=np.random.default_rng(perm_seed))
        case = H.PagedCase(w, lens=lens, table=table, num_blocks=nb + 7 * perm_seed)
        for _ in range(2):
            out, lse = case.run(0, chunk=128)
            outs.append((out.clone(), lse.clone()))
    torch.cuda.synchronize()
    for o, l in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0][0].view(torch.int16))
        assert torch.equal(l, outs[0][1])


# (b, n_q, n_chunks): the merge spreads a head over 1 to 8 waves (rows per
# wave R = 2 .. 16) and holds 1 to 8 rows per lane, looping past 8R chunks.
# 15 heads: R up to 16, 1 to 8 rows per lane, 300 chunks loop three times;
# 2,048 heads: one wave per head (two with d_h 64), looping past 16 (32)
# chunks; 256 heads: R = 8 with one and four rows per lane.
MERGE_SHAPES = ([(3, 5, nc) for nc in (1, 2, 6, 16, 17, 40, 100, 300)]
                + [(64, 32, nc) for nc in (2, 5, 16, 40)] + [(8, 32, 8), (8, 32, 24)])


@pytest.mark.parametrize("b,n_q,nc", MERGE_SHAPES)
@pytest.mark.parametrize("d", [64, 128])
def test_merge_partials_export(env, b, n_q, nc, d):
    """Every shape of the merge kernel, an empty chunk whose partial holds NaN,
    and a head with every chunk empty, against the oracle's merge."""
    kvd, H, W, torch = env
    from oracle import attention
    rng = np.random.default_rng(5 + nc + d + 1000 * b)
    part_o = rng.standard_normal((b, n_q, nc, d)).astype(np.float32)
    part_lse = (rng.standard_normal((b, n_q, nc)) * 3).astype(np.float32)
    if nc > 1:
        part_lse[0, 1, nc // 2] = -np.inf             # an empty chunk: its o_c is never read
        part_o[0, 1, nc // 2] = np.nan
    part_lse[1, 2, :] = -np.inf                   # all chunks empty
    part_o[1, 2, :] = np.nan
    clean = np.where(np.isnan(part_o), 0.0, part_o)    # what an empty chunk means to the oracle
    ref_o, ref_lse = attention.merge_partials(clean.astype(np.float64), part_lse.astype(np.float64))
    out = torch.empty((b, n_q, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((b, n_q), dtype=torch.float32, device="cuda")
    kvd.kvd_merge_partials(torch.from_numpy(part_o).cuda(), torch.from_numpy(part_lse).cuda(), out, lse)
    torch.cuda.synchronize()
    H.assert_bf16_close(out, ref_o, what=f"merge nc={nc} d={d}")
    H.assert_lse_close(lse, ref_lse)
    assert torch.all(out[1, 2] == 0)


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("chunk", [0, 16, 48, 128])
def test_decode_partials_match_oracle_chunks(env, fp8, chunk):
    """Per-chunk partials against the oracle's, and their merge against the
    one-call result bit for bit (16, 48 and 128 tokens: 63, 21 and 8 chunks;
    0: the library's chunking, one chunk here)."""
    kvd, H, W, torch = env
    from oracle import attention
    w = _workload(W, 8, 128, fp8=fp8, seed=700)
    case = _case(H, W, w)
    part_o, part_lse, C, nc = kvd.kvd_decode_partials(case.pool, 0, case.q[0], case.table_t, case.lens_t,
                                                      case.max_ctx, chunk_tokens=chunk)
    torch.cuda.synchronize()
    po, pl = part_o.cpu().double().numpy(), part_lse.cpu().double().numpy()
    qf = H.bf16_to_f64(case.q[0])
    for i, s in enumerate(LENS):
        K, V = case.logical(0, i)
        oc, lc = attention.chunk_partials(qf[i], K, V, C, n_chunks=nc)
        live = np.isfinite(lc)
        assert np.array_equal(np.isneginf(pl[i]), ~live), (i, s)
        if live.any():
            err = np.abs(po[i][live] - oc[live]) / np.maximum(1.0, np.abs(oc[live]))
            assert err.max() <= 1e-5, (i, s, err.max())
            lerr = np.abs(pl[i][live] - lc[live]) / np.maximum(1.0, np.abs(lc[live]))
            assert lerr.max() <= 1e-5, (i, s, lerr.max())
    # merging them reproduces the one-call result bit for bit
    out = torch.empty_like(case.q[0])
    lse = torch.empty(case.q[0].shape[:2], dtype=torch.float32, device="cuda")
    kvd.kvd_merge_partials(part_o, part_lse, out, lse)
    ref_out, ref_lse = case.run(0, chunk=chunk)
    torch.cuda.synchronize()
    if nc > 1:
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
        assert torch.equal(lse, ref_lse)
    else:
        H.assert_bf16_close(out, case.oracle(0)[0], what="merged single chunk")


@pytest.mark.parametrize("fp8", [False, True])
def test_large_batch_unit_order(env, fp8):
    """150 sequences (more than one 64-lane group of lengths), a fifth of them
    empty: the decode kernel places the chunks that hold tokens before the
    empty ones, locating its unit with a prefix sum over every group.  Each
    chunk's partial, the live/empty pattern, the merged output and the
    single-chunk path must match the oracle."""
    kvd, H, W, torch = env
    from oracle import attention
    rng = np.random.default_rng(41)
    lens = rng.integers(1, 300, 150).astype(np.int32)
    lens[rng.random(150) < 0.2] = 0
    lens[[0, 63, 64, 127, 128, 149]] = [0, 299, 0, 1, 33, 0]     # group edges
    w = W.DecodeWorkload("batch150", seed=42, b=150, layers=1, n_q=8, n_kv=2, head_dim=64,
                         ctx=("fixed", 0), kv_dtype="fp8" if fp8 else "bf16")
    case = _case(H, W, w, lens=lens)
    qf = H.bf16_to_f64(case.q[0])
    for chunk in (32, 96):
        H.say(f"batch150 fp8={fp8} chunk={chunk}")
        part_o, part_lse, C, nc = kvd.kvd_decode_partials(case.pool, 0, case.q[0], case.table_t, case.lens_t,
                                                          case.max_ctx, chunk_tokens=chunk)
        torch.cuda.synchronize()
        po, pl = part_o.cpu().double().numpy(), part_lse.cpu().double().numpy()
        for i, s in enumerate(lens):
            K, V = case.logical(0, i)
            oc, lc = attention.chunk_partials(qf[i], K, V, C, n_chunks=nc)
            live = np.isfinite(lc)
            assert np.array_equal(np.isneginf(pl[i]), ~live), (i, s)
            if live.any():
                err = np.abs(po[i][live] - oc[live]) / np.maximum(1.0, np.abs(oc[live]))
                assert err.max() <= 1e-5, (i, s, err.max())
    ref_o, ref_l = case.oracle(0)
    for chunk in (0, 64, 512):                   # 512: one chunk, the direct path
        out, lse = case.run(0, chunk=chunk)
        torch.cuda.synchronize()
        H.assert_bf16_close(out, ref_o, what=f"batch150 fp8={fp8} chunk={chunk}")
        H.assert_lse_close(lse, ref_l)
        empty = torch.from_numpy(lens == 0).cuda()
        assert torch.all(out[empty] == 0) and torch.all(torch.isneginf(lse[empty]))


def test_bad_block_ids_read_as_zero(env):
    kvd, H, W, torch = env
    w = _workload(W, 4, 64, seed=500)
    lens = np.array([40], dtype=np.int32)
    table, nb = W.block_tables(w, lens)
    case = H.PagedCase(w, lens=lens, table=table, num_blocks=nb)
    bad = case.table_t.clone()
    bad[0, 1] = 1 << 30                      # the second block points outside the pool
    out = torch.empty_like(case.q[0])
    kvd.decode(case.pool, 0, case.q[0], bad, case.lens_t, 40, out=out, chunk_tokens=16)
    torch.cuda.synchronize()
    # the kernel reads zeros for the bad block: K = 0 gives score 0, V = 0 adds nothing
    K, V = case.logical(0, 0)
    K[16:32] = 0
    V[16:32] = 0
    from oracle import attention
    ref, _ = attention.decode_sequence(H.bf16_to_f64(case.q[0])[0], K, V)
    H.assert_bf16_close(out[0], ref, what="bad ids")


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("chunk", [0, 32, 64, 96])
def test_fused_cumulative_scores(env, fp8, chunk):
    kvd, H, W, torch = env
    w = _workload(W, 4, 128, fp8=fp8, seed=600, layers=3)
    lens = [0, 1, 17, 64, 200, 513]
    case = _case(H, W, w, lens=lens)
    stride = case.max_ctx + 5
    init = np.random.default_rng(9).random((len(lens), stride)).astype(np.float32)
    score = torch.from_numpy(init).cuda()
    for layer in range(3):
        out, lse = case.run(layer, chunk=chunk, score=score, weight=1.0 / 3)
        torch.cuda.synchronize()
        ref_o, ref_lse = case.oracle(layer)
        H.assert_bf16_close(out, ref_o, what=f"scores layer {layer}")
    got = score.cpu().double().numpy()
    ref = case.oracle_scores(init, range(len(lens)), 1.0 / 3)
    assert H.score_rel_error(got, ref) <= H.TOL_SCORE_REL
    # every sequence's scores grew by exactly one in total
    for i, s in enumerate(lens):
        if s:
            assert abs((got[i, :s] - init[i, :s]).sum() - 1.0) < 1e-4
        assert np.array_equal(got[i, s:], init[i, s:].astype(np.float64))


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("chunk", [0, 64, 160])
def test_score_increments_alone(env, fp8, chunk):
    """The score update with the array starting at zero, so that the 1e-5
    relative bound applies to each token's increment itself (a nonzero start
    would dominate it): three layers, every token of every sequence."""
    kvd, H, W, torch = env
    w = _workload(W, 4, 128, fp8=fp8, seed=610, layers=3)
    lens = [1, 17, 64, 200, 513, 1000]
    case = _case(H, W, w, lens=lens)
    stride = case.max_ctx + 3
    score = torch.zeros((len(lens), stride), dtype=torch.float32, device="cuda")
    for layer in range(3):
        case.run(layer, chunk=chunk, score=score, weight=1.0 / 3)
    torch.cuda.synchronize()
    got = score.cpu().double().numpy()
    ref = case.oracle_scores(np.zeros((len(lens), stride)), range(len(lens)), 1.0 / 3)
    for i, s in enumerate(lens):
        assert np.all(ref[i, :s] > 0) and np.all(got[i, s:] == 0)
    err = H.score_rel_error(got, ref)
    H.say(f"score increments fp8={fp8} chunk={chunk}: max rel error {err:.2e}")
    assert err <= H.TOL_SCORE_REL, err


def test_tiny_workload(env):
    kvd, H, W, torch = env
    w = W.WORKLOADS["tiny"]
    case = H.PagedCase(w)
    out, lse = case.run(0)
    torch.cuda.synchronize()
    ref_o, ref_lse = case.oracle(0)
    H.assert_bf16_close(out, ref_o, what="tiny")
    H.assert_lse_close(lse, ref_lse)


@pytest.mark.parametrize("b", [2, 64, 65, 150, 512])
def test_chunk_major_order_edges(env, b):
    """The chunk-major order of full chunks at its edges: one sequence per lane (b <= 64, lane 63 owning the last) and up
    to eight (65, 150, 512), exactly 64 chunks of 16 tokens, sequences with no
    full chunk, with every chunk full, and empty ones.  Every unit must be computed once: outputs and lse against the
    oracle."""
    kvd, H, W, torch = env
    rng = np.random.default_rng(50 + b)
    lens = rng.integers(0, 1025, b).astype(np.int32)
    lens[0] = 1024                                     # all 64 chunks full
    lens[-1] = 1024 if b > 2 else 7                    # the last lane
    if b > 4:
        lens[1], lens[2], lens[3] = 0, 15, 16          # empty, no full chunk, one full chunk
    w = _workload(W, 4, 64, seed=51 + b)
    w = w.with_(b=b)
    case = _case(H, W, w, lens=lens)
    out, lse = case.run(0, chunk=16)
    torch.cuda.synchronize()
    ref_o, ref_l = case.oracle(0)
    H.assert_bf16_close(out, ref_o, what=f"chunk-major b={b}")
    H.assert_lse_close(lse, ref_l)


def test_slot_mapping_bit_exact(env):
    """kvd_slot_mapping against the page's rule written out independently:
    token t of sequence i sits in physical block table[i][t // 16], row t % 16
    -- on the block-table example of the PagedAttention paragraph (requests A,
    B, C over 11 blocks) and on a seeded ragged batch with a run of new
    tokens per sequence, negative entries and empty sequences."""
    kvd, H, W, torch = env
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "block_table_example.json")) as fh:
        ex = json.load(fh)
    rows = [ex["tables"][k] for k in sorted(ex["tables"])]
    mb = max(len(r) for r in rows)
    table = np.full((len(rows), mb), -1, dtype=np.int32)
    for i, r in enumerate(rows):
        table[i, :len(r)] = r
    rng = np.random.default_rng(91)
    lens = np.array([16 * len(r) - int(rng.integers(0, 16)) for r in rows], dtype=np.int32)
    cases = [(table, lens, None)]
    b, mb = 37, 50
    table = rng.permutation(b * mb).astype(np.int32).reshape(b, mb)
    table[rng.random((b, mb)) < 0.1] = -1
    lens = rng.integers(0, 16 * mb + 1, size=b).astype(np.int32)
    lens[:3] = [0, 1, 16 * mb]
    first = (lens * rng.random(b)).astype(np.int32)
    cases += [(table, lens, None), (table, lens, first), (table, lens, np.maximum(lens - 1, 0))]
    for table, lens, first in cases:
        f = np.zeros_like(lens) if first is None else first
        want = []
        for i in range(len(lens)):
            for t in range(int(f[i]), int(lens[i])):
                e = int(table[i, t // 16])
                want.append(-1 if e < 0 else e * 16 + t % 16)
        got = kvd.kvd_slot_mapping(torch.from_numpy(table).cuda(), torch.from_numpy(lens).cuda(),
                                   None if first is None else torch.from_numpy(first).cuda())
        assert np.array_equal(got.cpu().numpy(), np.array(want, dtype=np.int32))


def test_workspace_reused_across_shapes(env):
    """One workspace serves calls of different shapes in turn (batch, heads,
    chunking, scores), twice round: each call's outputs, lse and scores equal
    those of the same call on a fresh workspace, bit for bit -- nothing a call
    leaves in the workspace reaches a later call."""
    kvd, H, W, torch = env
    shapes = [  # (b, n_q, n_kv, d, length range, chunk, score)
        (6, 16, 4, 128, (100, 3000), 128, False),
        (20, 8, 2, 64, (1, 900), 32, True),
        (2, 32, 8, 128, (2000, 4000), 256, False),
        (40, 8, 4, 128, (0, 700), 64, False),
        (3, 8, 2, 64, (1, 300), 32, True),
    ]
    cases = []
    for k, (b, n_q, n_kv, d, span, chunk, with_score) in enumerate(shapes):
        w = W.DecodeWorkload(f"ws-reuse-{k}", seed=500 + k, b=b, layers=1, n_q=n_q, n_kv=n_kv, head_dim=d,
                             ctx=("uniform", span[0], span[1]))
        cases.append((H.PagedCase(w), chunk, with_score))
    need = 0
    for case, chunk, with_score in cases:
        score = torch.zeros((case.w.b, case.max_ctx), device="cuda") if with_score else None
        a = kvd.make_args(case.q[0], case.table_t, case.lens_t, case.max_ctx, torch.empty_like(case.q[0]),
                          chunk_tokens=chunk, score=score, score_weight=0.5, pool=case.pool)
        need = max(need, kvd.kvd_decode_workspace_bytes(case.pool, a))
    shared = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    for rnd in range(2):
        for k, (case, chunk, with_score) in enumerate(cases):
            res = []
            for ws in (shared, None):
                q = case.q[0]
                out = torch.full_like(q, float("nan"))
                lse = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device="cuda")
                score = torch.ones((case.w.b, case.max_ctx), device="cuda") if with_score else None
                kvd.decode(case.pool, 0, q, case.table_t, case.lens_t, case.max_ctx, out=out, lse_out=lse,
                           chunk_tokens=chunk, score=score, score_weight=0.5, workspace=ws)
                res.append((out, lse, score))
            torch.cuda.synchronize()
            (o1, l1, s1), (o2, l2, s2) = res
            assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), (rnd, k)
            assert torch.equal(l1, l2), (rnd, k)
            if with_score:
                assert torch.equal(s1, s2), (rnd, k)
            assert not torch.isnan(o1.float()).any(), (rnd, k)
