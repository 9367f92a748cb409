"""Parity at the full workload sizes, in the launch configuration the benchmark times.

The per-layer launch (grid, chunking, workspace) is the benchmark's, and so
is the pool: the ragged 8B batch keeps all 32 layers and the 70B-shaped step
all 80 (172 GB, every layer base beyond the first 4 GiB addressed with 64-bit
offsets).  Every sequence is checked against the oracle at the first layer,
the last layer and one seeded layer between them.  The FP8 + score workload
runs all 32 layers (its cumulative score needs every one) and samples
sequences.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import decode_attention_paged_04_amd as kvd
    import gpu_harness as H
    import workloads as W
    return kvd, H, W, torch


def _check(H, torch, case, layer, seqs=None, rel_tol=None):
    out, lse = case.run(layer)
    torch.cuda.synchronize()
    ref_o, ref_lse = case.oracle(layer, seqs)
    seqs = list(range(len(case.lens))) if seqs is None else list(seqs)
    for i in seqs:
        mx, rel = H.assert_bf16_close(out[i], ref_o[i], rel_tol=rel_tol or H.TOL_REL_L2,
                                      what=f"{case.w.name} layer {layer} seq {i}")
        H.say(f"{case.w.name} layer {layer} seq {i}: max-abs {mx:.2e} rel-L2 {rel:.2e}")
    H.assert_lse_close(lse[seqs], ref_lse[seqs])


def test_full_8b_single_layer(env):
    kvd, H, W, torch = env
    case = H.PagedCase(W.WORKLOADS["8b_layer"])
    _check(H, torch, case, 0)


def _checked_layers(w):
    """First, last and one seeded layer between them."""
    r = int(np.random.default_rng(w.seed + 99).integers(1, w.layers - 1))
    return [0, r, w.layers - 1]


def test_full_8b_ragged_batch(env):
    kvd, H, W, torch = env
    w = W.WORKLOADS["8b_ragged"]
    layers = _checked_layers(w)
    H.say(f"8b_ragged: {w.layers}-layer pool, all {w.b} sequences at layers {layers}")
    case = H.PagedCase(w, keep_layers=layers)
    for layer in layers:
        _check(H, torch, case, layer)


@pytest.mark.timeout(900)
def test_full_70b_long_context(env):
    kvd, H, W, torch = env
    w = W.WORKLOADS["70b_long"]
    layers = _checked_layers(w)
    H.say(f"70b_long: {w.layers}-layer pool (171.8 GB), all {w.b} sequences at layers {layers}")
    case = H.PagedCase(w, keep_layers=layers)
    assert case.pool.kv.numel() == 171_798_691_840
    for layer in layers:
        _check(H, torch, case, layer)
        case.kv.pop(layer, None)                     # host copies: one layer at a time


def test_full_8b_fp8_with_scores(env):
    kvd, H, W, torch = env
    from oracle import e4m3, paged
    w = W.WORKLOADS["8b_fp8_scores"]
    lens = W.context_lengths(w)
    rng = np.random.default_rng(w.seed + 77)
    seqs = sorted({int(np.argmin(lens)), int(rng.integers(0, w.b))})
    H.say(f"fp8+scores: sampled sequences {seqs} of lengths {[int(lens[i]) for i in seqs]}")
    case = H.PagedCase(w, keep_seqs=seqs)
    stride = case.max_ctx
    init = W.initial_scores(w, stride, "cuda")
    score = init.clone()
    init_np = init.cpu().numpy()
    outs = {}
    for layer in range(w.layers):
        out, lse = case.run(layer, score=score, weight=1.0 / w.layers)
        if layer in (0, w.layers - 1):
            outs[layer] = (out.clone(), lse.clone())
    torch.cuda.synchronize()
    for layer, (out, lse) in outs.items():
        ref_o, ref_lse = case.oracle(layer, seqs)
        for i in seqs:
            mx, rel = H.assert_bf16_close(out[i], ref_o[i], rel_tol=H.TOL_FP8_REL_L2,
                                          what=f"fp8 layer {layer} seq {i}")
            H.say(f"fp8 layer {layer} seq {i}: max-abs {mx:.2e} rel-L2 {rel:.2e}")
        H.assert_lse_close(lse[seqs], ref_lse[seqs])
    # the stored codes and scales of the sampled sequences, layer 5
    lay = case.layout()
    for i in seqs:
        s = int(lens[i])
        k_idx, v_idx = paged.gather_indices(lay, 5, case.table[i], s)
        Ks, Vs = case.kv_seq[(5, i)]
        ck, sk = e4m3.quantize_sequence(Ks.float().numpy())
        cv, sv = e4m3.quantize_sequence(Vs.float().numpy())
        kv = case.pool.kv
        got_k = kv[torch.from_numpy(k_idx).cuda()].cpu().numpy()
        got_v = kv[torch.from_numpy(v_idx).cuda()].cpu().numpy()
        assert np.array_equal(got_k, ck) and np.array_equal(got_v, cv)
        nb = sk.shape[0]
        sc_idx = np.array([[lay.scale_index(5, int(case.table[i, b]), j, 0) for j in range(w.n_kv)]
                           for b in range(nb)])
        got_sk = case.pool.scales[torch.from_numpy(sc_idx).cuda()].cpu().numpy()
        got_sv = case.pool.scales[torch.from_numpy(sc_idx + 1).cuda()].cpu().numpy()
        assert np.array_equal(got_sk, sk) and np.array_equal(got_sv, sv)
    got = score.cpu().double().numpy()
    ref = case.oracle_scores(init_np, seqs, 1.0 / w.layers)
    for i in seqs:
        err = H.score_rel_error(got[i], ref[i])
        H.say(f"scores seq {i}: max rel error {err:.2e}")
        assert err <= H.TOL_SCORE_REL


@pytest.mark.parametrize("name,chunks", [("8b_prefix", (0,)), ("8b_prefix1024", (0, 512))])
def test_full_shared_prefix_batch(env, name, chunks):
    """The shared-prefix workloads the benchmark times (32 requests behind one
    16,384-token prompt, 1,024 behind one 4,096-token prompt; the prompt stored
    once, each request's own tokens after it; one layer): sampled sequences
    against the oracle over each one's logical K/V -- the prompt's rows as
    stored by request 0, then its own -- with the library's chunking and, for
    the 1,024 requests, 512-token chunks (nine per request, chunk-major over
    sixteen sequences per lane)."""
    kvd, H, W, torch = env
    from oracle import attention
    w = W.WORKLOADS[name].with_(layers=1)
    lens = W.context_lengths(w)
    table, nb = W.block_tables(w, lens)
    first, start, n = W.stored_rows(w, lens)
    table_t, lens_t = torch.from_numpy(table).cuda(), torch.from_numpy(lens).cuda()
    slots = kvd.kvd_slot_mapping(table_t, lens_t, first_token=torch.from_numpy(first).cuda())
    assert slots.numel() == n
    pool = kvd.allocate_pool(1, nb, w.n_kv, w.head_dim, kvd.KVD_BF16)
    K, V = W.keys_values(w, 0, n, "cuda")
    kvd.kvd_write_kv(pool, 0, K, V, slots)
    q = W.query(w, 0, "cuda")
    qf = H.bf16_to_f64(q)
    Kc, Vc = K.cpu(), V.cpu()
    del K, V
    P = w.shared_prefix
    rng = np.random.default_rng(w.seed + 5)
    sample = sorted({0, 13, w.b - 1, int(rng.integers(1, w.b - 1))})
    refs = {}
    for i in sample:
        a = int(start[i])
        e = a + int(lens[i]) - (P if i else 0)
        Ki = torch.cat([Kc[:P], Kc[a:e]]) if i else Kc[a:e]
        Vi = torch.cat([Vc[:P], Vc[a:e]]) if i else Vc[a:e]
        refs[i] = attention.decode_sequence(qf[i], H.bf16_to_f64(Ki), H.bf16_to_f64(Vi))
    # the automatic split as the benchmark runs it (even chunks: the batch shares
    # its prompt) and with the default uneven chunk pairs
    for chunk, even in [(c, e) for c in chunks for e in ((True, False) if c == 0 else (False,))]:
        out = torch.empty_like(q)
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
        kvd.decode(pool, 0, q, table_t, lens_t, int(lens.max()), out=out, lse_out=lse, chunk_tokens=chunk,
                   even_chunks=even)
        torch.cuda.synchronize()
        for i in sample:
            ref_o, ref_l = refs[i]
            mx, rel = H.assert_bf16_close(out[i], ref_o, what=f"{name} chunk {chunk} even {even} seq {i}")
            H.say(f"{name} chunk {chunk} even {even} seq {i}: max-abs {mx:.2e} rel-L2 {rel:.2e}")
            H.assert_lse_close(lse[i:i + 1], ref_l[None])
        assert not torch.isnan(out.float()).any()
