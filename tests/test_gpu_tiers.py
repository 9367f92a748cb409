"""Tier-restricted decode on the GPU against the oracle.

A block-table entry of -1 inside a sequence's context marks a block that is
not attended; the decode then covers the remaining blocks only (the T0 and T1
tiers of "Not all thinking needs HBM").  Checked: the restricted decode
against the oracle for bf16 and FP8 pools and several chunkings; Proposition
1 -- moving the T1 blocks to other physical blocks (where a prefetch would put
them) leaves the result bit for bit unchanged; fused scores over a restricted
step; and a loop that re-plans the tiers from the fused scores every 64 steps
with the native planner.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

LENS = [40, 1, 100, 257, 33, 70]


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import decode_attention_paged_04_amd as kvd
    import gpu_harness as H
    import workloads as W
    return kvd, H, W, torch


def _case(H, W, fp8, d=128, lens=LENS, layers=1, seed=600, spare=0):
    w = W.DecodeWorkload(f"tiers-d{d}", seed=seed, b=len(lens), layers=layers, n_q=16, n_kv=4, head_dim=d,
                         ctx=("fixed", 0), kv_dtype="fp8" if fp8 else "bf16")
    lens = np.array(lens, dtype=np.int32)
    table, nb = W.block_tables(w, lens)
    return H.PagedCase(w, lens=lens, table=table, num_blocks=nb + spare)


def _drop_pattern(table, lens, rng):
    """A copy of the table with some blocks marked -1: random ones, plus a
    sequence's first block, another's partial last block, and all of one."""
    t = table.copy()
    for i, s in enumerate(lens):
        nb = -(-int(s) // 16)
        for b in range(nb):
            if rng.random() < 0.4:
                t[i, b] = -1
    t[0, 0] = -1
    t[2, -(-int(lens[2]) // 16) - 1] = -1
    t[4, :3] = -1                                # every block of sequence 4
    return t


def _oracle(case, layer, table, H):
    from oracle import tiers
    qf = H.bf16_to_f64(case.q[layer])
    o = np.zeros(qf.shape)
    lse = np.zeros(qf.shape[:2])
    for i, s in enumerate(case.lens):
        s = int(s)
        K, V = case.logical(layer, i)
        keep = np.array([table[i, t // 16] >= 0 for t in range(s)], dtype=bool)
        o[i], lse[i] = tiers.restricted_decode(qf[i], K, V, keep)
    return o, lse


@pytest.mark.parametrize("fp8", [False, True])
def test_restricted_decode_matches_oracle(env, fp8):
    kvd, H, W, torch = env
    case = _case(H, W, fp8)
    rt = _drop_pattern(case.table, case.lens, np.random.default_rng(1))
    ref_o, ref_l = _oracle(case, 0, rt, H)
    rt_t = torch.from_numpy(rt).cuda()
    for chunk in (0, 16, 48, 256):
        H.say(f"restricted fp8={fp8} chunk={chunk}")
        out = torch.empty_like(case.q[0])
        lse = torch.empty(case.q[0].shape[:2], dtype=torch.float32, device="cuda")
        kvd.decode(case.pool, 0, case.q[0], rt_t, case.lens_t, case.max_ctx, out=out, lse_out=lse,
                   chunk_tokens=chunk)
        torch.cuda.synchronize()
        H.assert_bf16_close(out, ref_o, what=f"restricted fp8={fp8} chunk={chunk}")
        H.assert_lse_close(lse, ref_l)
        assert torch.all(out[4] == 0) and torch.all(torch.isneginf(lse[4]))


@pytest.mark.parametrize("fp8", [False, True])
def test_t1_placement_does_not_change_the_result(env, fp8):
    """Proposition 1: the split between T0 and T1 -- and where the T1 blocks sit
    once prefetched -- does not change the result, bit for bit."""
    kvd, H, W, torch = env
    spare = 64
    case = _case(H, W, fp8, spare=spare)
    rng = np.random.default_rng(2)
    plans = []
    for i, s in enumerate(case.lens):
        nb = -(-int(s) // 16)
        sc = rng.random(nb)
        plans.append(kvd.tier_plan(sc, 1, 1, max(nb // 3, 0), max(nb // 3, 0)))
    rt = case.table.copy()
    for i, p in enumerate(plans):
        rt[i, :len(p)] = kvd.tier_restrict(case.table[i, :len(p)], p)
    # the same evicted set, the T1 blocks copied to spare physical blocks
    moved = rt.copy()
    lay = case.layout()
    w_bytes = 1 if fp8 else 2
    block_bytes = lay.n_kv * lay.tile_pair_elems * w_bytes
    nxt = case.num_blocks - spare
    for i, p in enumerate(plans):
        for b, tier in enumerate(p):
            if tier == kvd.KVD_TIER_T1:
                src = int(case.table[i, b])
                a, z = src * block_bytes, nxt * block_bytes
                case.pool.kv[z:z + block_bytes] = case.pool.kv[a:a + block_bytes]
                if fp8:
                    for j in range(lay.n_kv):
                        d0, s0 = lay.scale_index(0, nxt, j, 0), lay.scale_index(0, src, j, 0)
                        case.pool.scales[d0:d0 + 2] = case.pool.scales[s0:s0 + 2]
                moved[i, b] = nxt
                nxt += 1
    assert nxt > case.num_blocks - spare                 # some T1 blocks were moved
    outs = []
    for table in (rt, moved):
        out = torch.empty_like(case.q[0])
        lse = torch.empty(case.q[0].shape[:2], dtype=torch.float32, device="cuda")
        kvd.decode(case.pool, 0, case.q[0], torch.from_numpy(table).cuda(), case.lens_t, case.max_ctx,
                   out=out, lse_out=lse)
        torch.cuda.synchronize()
        outs.append((out.cpu(), lse.cpu()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    ref_o, ref_l = _oracle(case, 0, rt, H)
    H.assert_bf16_close(outs[0][0], ref_o, what=f"prop1 fp8={fp8}")
    H.assert_lse_close(outs[0][1], ref_l)


@pytest.mark.parametrize("fp8", [False, True])
def test_restricted_step_scores(env, fp8):
    kvd, H, W, torch = env
    from oracle import scores, tiers
    case = _case(H, W, fp8, layers=2)
    rt = _drop_pattern(case.table, case.lens, np.random.default_rng(3))
    rt_t = torch.from_numpy(rt).cuda()
    stride = case.max_ctx + 5
    init = np.random.default_rng(4).random((len(case.lens), stride)).astype(np.float32)
    score = torch.from_numpy(init).cuda()
    for layer in range(2):
        out = torch.empty_like(case.q[layer])
        kvd.decode(case.pool, layer, case.q[layer], rt_t, case.lens_t, case.max_ctx, out=out,
                   score=score, score_weight=0.5)
    torch.cuda.synchronize()
    got = score.cpu().numpy().astype(np.float64)
    ref = init.astype(np.float64).copy()
    for i, s in enumerate(case.lens):
        s = int(s)
        keep = np.array([rt[i, t // 16] >= 0 for t in range(s)], dtype=bool)
        for layer in range(2):
            K, _ = case.logical(layer, i)
            a = tiers.restricted_weights(H.bf16_to_f64(case.q[layer])[i], K, keep)
            ref[i, :s] += scores.layer_increment(a, 0.5)
    assert np.all(np.isfinite(got))
    err = H.score_rel_error(got, ref)
    assert err <= H.TOL_SCORE_REL, err
    # tokens outside the kept set, and the whole of sequence 4, are untouched
    assert np.array_equal(got[4], init[4].astype(np.float64))


def test_retiering_loop(env):
    """130 decode steps with fused scores; the tiers are re-planned from the
    scores every 64 steps (native planner) and the steps between use the
    restricted table; every step matches the oracle over the same kept set."""
    kvd, H, W, torch = env
    from oracle import tiers
    case = _case(H, W, False, lens=[300, 190], seed=610)
    stride = case.max_ctx
    score = torch.zeros((2, stride), dtype=torch.float32, device="cuda")
    K0, V0 = case.logical(0, 0)
    K1, V1 = case.logical(0, 1)
    logical = [(K0, V0), (K1, V1)]
    rt = case.table.copy()
    g = torch.Generator().manual_seed(5)
    retiered = 0
    for step in range(130):
        if tiers.retier_due(step):
            host = score.cpu().numpy()
            rt = case.table.copy()
            for i, s in enumerate(case.lens):
                bs = kvd.tier_block_scores(host[i, :int(s)])
                nb = len(bs)
                p = kvd.tier_plan(bs, 1, 2, nb // 4, nb // 4)
                assert np.array_equal(p, tiers.plan_tiers(bs, 1, 2, nb // 4, nb // 4))
                rt[i, :nb] = kvd.tier_restrict(case.table[i, :nb], p)
            retiered += 1
        q = torch.randn(case.q[0].shape, generator=g).to(torch.bfloat16).cuda()
        out = torch.empty_like(q)
        kvd.decode(case.pool, 0, q, torch.from_numpy(rt).cuda(), case.lens_t, case.max_ctx, out=out,
                   score=score, score_weight=1.0)
        torch.cuda.synchronize()
        if step % 13 == 0 or step in (63, 64, 65, 129):
            qf = H.bf16_to_f64(q)
            ref = np.zeros(qf.shape)
            for i, s in enumerate(case.lens):
                keep = np.array([rt[i, t // 16] >= 0 for t in range(int(s))], dtype=bool)
                ref[i], _ = tiers.restricted_decode(qf[i], *logical[i], keep)
            H.assert_bf16_close(out, ref, what=f"retier step {step}")
    assert retiered == 3
