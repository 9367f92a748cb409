"""Closed-form cases of the decode step on the GPU, checked against the
mathematics directly rather than against the oracle.

The step is softmax(q K^T / sqrt(d_h)) V per query head over the cached rows of
its sequence (froggydisk, "LLM에서 KV 캐시는 얼마나 생길까", the attention
walk-through; GQA: the query heads of a group share one KV head).  So:

* one cached token: its weight is 1 -- the output is that token's V row bit for
  bit and lse is the scaled logit; with an FP8 pool whose V row lies on the
  E4M3 grid under a power-of-two scale the stored row decodes exactly, so the
  output is again the row bit for bit;
* q = 0: every weight is 1/s, the output is the mean of V and lse = ln s;
* all V rows equal: the weights sum to 1, the output is that row bit for bit;
* one logit 40 above every other: the other weights are below e^-40, the output
  is that token's V row bit for bit;
* the fused score (gist.science summary of "Not all thinking needs HBM",
  methodology 2): one call adds weight / n_q * sum over heads of alpha, and
  alpha sums to 1 over the tokens of each head, so every sequence's score total
  grows by exactly the weight (in fp32: within 1e-5), and positions past s_i
  stay untouched.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

N_KV, G, NB = 2, 4, 160


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import decode_attention_paged_04_amd as kvd
    import gpu_harness as H
    return kvd, H, torch


def _store(kvd, torch, pool, K, V, lens, seed):
    """Write the sequences' rows (K, V [sum(lens)][n_kv][d], bf16) into
    seeded, scattered blocks; returns the block table (cuda int32)."""
    rng = np.random.default_rng(seed)
    need = [-(-int(s) // 16) for s in lens]
    perm = rng.permutation(NB)[:sum(need)]
    mb = max(max(need), 1)
    table = np.full((len(lens), mb), -1, dtype=np.int32)
    slots, k = [], 0
    for i, n in enumerate(need):
        table[i, :n] = perm[k:k + n]
        k += n
        slots += [int(table[i, t // 16]) * 16 + t % 16 for t in range(int(lens[i]))]
    if slots:
        kvd.kvd_write_kv(pool, 0, K.cuda(), V.cuda(), torch.tensor(slots, dtype=torch.int32, device="cuda"))
    return torch.from_numpy(table).cuda()


def _run(kvd, torch, pool, q, table, lens, chunk=0, score=None, weight=0.0):
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    lens_t = torch.tensor(lens, dtype=torch.int32, device="cuda")
    kvd.decode(pool, 0, q, table, lens_t, max(max(lens), 1), out=out, lse_out=lse, chunk_tokens=chunk,
               score=score, score_weight=weight)
    torch.cuda.synchronize()
    return out, lse


def _bits(t):
    import torch
    return t.detach().cpu().contiguous().view(torch.int16)


@pytest.mark.parametrize("d", [64, 128])
def test_one_token_gives_its_value_row(env, d):
    kvd, H, torch = env
    g = torch.Generator().manual_seed(900 + d)
    lens = [1] * 6
    K = torch.randn((6, N_KV, d), generator=g).to(torch.bfloat16)
    V = torch.randn((6, N_KV, d), generator=g).to(torch.bfloat16)
    q = torch.randn((6, N_KV * G, d), generator=g).to(torch.bfloat16).cuda()
    pool = kvd.allocate_pool(1, NB, N_KV, d, kvd.KVD_BF16)
    table = _store(kvd, torch, pool, K, V, lens, 1)
    out, lse = _run(kvd, torch, pool, q, table, lens)
    want = V.repeat_interleave(G, dim=1)                     # head h reads KV head h // G
    assert torch.equal(_bits(out), _bits(want))
    qf, kf = H.bf16_to_f64(q), H.bf16_to_f64(K)
    ref_lse = np.einsum("ihc,ihc->ih", qf, np.repeat(kf, G, axis=1)) / np.sqrt(d)
    H.assert_lse_close(lse, ref_lse)


def test_one_token_fp8_on_the_grid_is_exact(env):
    """An E4M3 row times 2^-4, with 448 * 2^-4 as its largest magnitude: the
    block's scale is absmax / 448 = 2^-4 exactly, every element is a code times
    the scale, and the decoded row equals the written one."""
    kvd, H, torch = env
    d = 128
    rng = np.random.default_rng(5)
    mant = 1.0 + rng.integers(0, 8, (5, N_KV, d)) / 8.0
    expo = rng.integers(-6, 8, (5, N_KV, d)).astype(np.float64)
    sign = np.where(rng.random((5, N_KV, d)) < 0.5, -1.0, 1.0)
    vals = sign * mant * np.exp2(expo)                       # normal E4M3 values, |v| < 448
    vals[:, :, 0] = 448.0
    Vf = torch.from_numpy(vals * 2.0 ** -4).float()
    V = Vf.to(torch.bfloat16)
    assert torch.equal(V.float(), Vf)                        # 4 significant bits: bf16-exact
    g = torch.Generator().manual_seed(6)
    K = torch.randn((5, N_KV, d), generator=g).to(torch.bfloat16)
    q = torch.randn((5, N_KV * G, d), generator=g).to(torch.bfloat16).cuda()
    pool = kvd.allocate_pool(1, NB, N_KV, d, kvd.KVD_FP8_E4M3)
    lens = [1] * 5
    table = _store(kvd, torch, pool, K, V, lens, 2)
    out, _ = _run(kvd, torch, pool, q, table, lens)
    assert torch.equal(_bits(out), _bits(V.repeat_interleave(G, dim=1)))


@pytest.mark.parametrize("chunk", [0, 64])
def test_zero_query_averages_the_values(env, chunk):
    kvd, H, torch = env
    d = 128
    lens = [1, 17, 100, 1000]
    g = torch.Generator().manual_seed(7)
    n = sum(lens)
    K = torch.randn((n, N_KV, d), generator=g).to(torch.bfloat16)
    V = torch.randn((n, N_KV, d), generator=g).to(torch.bfloat16)
    q = torch.zeros((len(lens), N_KV * G, d), dtype=torch.bfloat16, device="cuda")
    pool = kvd.allocate_pool(1, NB, N_KV, d, kvd.KVD_BF16)
    table = _store(kvd, torch, pool, K, V, lens, 3)
    out, lse = _run(kvd, torch, pool, q, table, lens, chunk=chunk)
    Vf = H.bf16_to_f64(V)
    ref = np.zeros((len(lens), N_KV * G, d))
    a = 0
    for i, s in enumerate(lens):
        ref[i] = np.repeat(Vf[a:a + s].mean(axis=0), G, axis=0)
        a += s
    H.assert_bf16_close(out, ref, what=f"q = 0, chunk {chunk}")
    H.assert_lse_close(lse, np.repeat(np.log(np.array(lens, dtype=np.float64))[:, None], N_KV * G, axis=1))


@pytest.mark.parametrize("chunk", [0, 64])
def test_equal_value_rows_give_that_row(env, chunk):
    kvd, H, torch = env
    d = 128
    lens = [3, 16, 33, 700]
    g = torch.Generator().manual_seed(8)
    n = sum(lens)
    K = torch.randn((n, N_KV, d), generator=g).to(torch.bfloat16)
    rows = torch.randn((len(lens), N_KV, d), generator=g).to(torch.bfloat16)
    V = torch.cat([rows[i:i + 1].expand(s, N_KV, d) for i, s in enumerate(lens)]).contiguous()
    q = (3.0 * torch.randn((len(lens), N_KV * G, d), generator=g)).to(torch.bfloat16).cuda()
    pool = kvd.allocate_pool(1, NB, N_KV, d, kvd.KVD_BF16)
    table = _store(kvd, torch, pool, K, V, lens, 4)
    out, _ = _run(kvd, torch, pool, q, table, lens, chunk=chunk)
    assert torch.equal(_bits(out), _bits(rows.repeat_interleave(G, dim=1)))


def test_dominant_logit_selects_its_row(env):
    kvd, H, torch = env
    d = 128
    lens = [50, 300]
    picks = [17, 233]
    g = torch.Generator().manual_seed(9)
    n = sum(lens)
    u = torch.randn((len(lens), N_KV, d), generator=g)
    u = u / u.norm(dim=-1, keepdim=True)
    q = u.repeat_interleave(G, dim=1).to(torch.bfloat16)     # every head of a group: the same u
    K = (0.1 * torch.randn((n, N_KV, d), generator=g)).to(torch.bfloat16)
    V = torch.randn((n, N_KV, d), generator=g).to(torch.bfloat16)
    a = 0
    for i, s in enumerate(lens):
        # logit of the picked row: u . (c u) / sqrt(d) = c / sqrt(d); the others stay near 0
        K[a + picks[i]] = (80.0 * np.sqrt(d) * u[i]).to(torch.bfloat16)
        a += s
    qf, kf = H.bf16_to_f64(q), H.bf16_to_f64(K)
    a = 0
    for i, s in enumerate(lens):
        lg = np.einsum("hc,thc->ht", qf[i], np.repeat(kf[a:a + s], G, axis=1)) / np.sqrt(d)
        others = np.delete(lg, picks[i], axis=1)
        assert np.all(lg[:, picks[i]] - others.max(axis=1) > 40.0)
        a += s
    pool = kvd.allocate_pool(1, NB, N_KV, d, kvd.KVD_BF16)
    table = _store(kvd, torch, pool, K, V, lens, 5)
    out, _ = _run(kvd, torch, pool, q.cuda(), table, lens, chunk=64)
    a = 0
    for i, s in enumerate(lens):
        want = V[a + picks[i]].repeat_interleave(G, dim=0)
        assert torch.equal(_bits(out[i]), _bits(want))
        a += s


@pytest.mark.parametrize("fp8", [False, True])
def test_score_total_grows_by_the_weight(env, fp8):
    kvd, H, torch = env
    d = 128
    lens = [1, 40, 257, 900]
    g = torch.Generator().manual_seed(10)
    n = sum(lens)
    K = torch.randn((n, N_KV, d), generator=g).to(torch.bfloat16)
    V = torch.randn((n, N_KV, d), generator=g).to(torch.bfloat16)
    pool = kvd.allocate_pool(1, NB, N_KV, d, kvd.KVD_FP8_E4M3 if fp8 else kvd.KVD_BF16)
    table = _store(kvd, torch, pool, K, V, lens, 6)
    stride = max(lens) + 7
    score = torch.zeros((len(lens), stride), dtype=torch.float32, device="cuda")
    for call, w in enumerate((1.0, 0.25)):
        q = torch.randn((len(lens), N_KV * G, d), generator=g).to(torch.bfloat16).cuda()
        _run(kvd, torch, pool, q, table, lens, chunk=64, score=score, weight=w)
        got = score.cpu().double().numpy()
        total = 1.0 if call == 0 else 1.25
        for i, s in enumerate(lens):
            assert abs(got[i, :s].sum() - total) <= 1e-5 * total, (i, got[i, :s].sum())
            assert np.all(got[i, :s] > 0) and np.all(got[i, s:] == 0)
