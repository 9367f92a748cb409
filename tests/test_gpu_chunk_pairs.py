"""Uneven chunk pairs of the automatic split, on the GPU against the oracle.

With an automatic split, an even number of KV heads, two or more chunks and no
score, the chunks come in pairs of C + d and C - d tokens whose order depends
on the KV head's parity (kvd_decode_plan documents the spans).  The per-chunk
partials must equal the oracle's attention over exactly those spans, their
merge the one-call step bit for bit and the oracle's step within tolerance; a
fused append whose token lies where the two parities' spans differ must store
it once, before it is read, exactly as kvd_write_kv does; dropped blocks at the
pair boundaries must leave exactly the kept tokens attended; and a last chunk
without a partner keeps its even span.  (The mixed-precision decode over such
pairs is checked with the other mixed tests.)
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

# At a 5,000-token bound with 2 KV heads the automatic split takes 5 chunks of
# 1,024 tokens and d = 32: pairs (0, 1) and (2, 3), chunk 4 alone.  Token
# s - 1 of each sequence: 4999 in the lone chunk; 3049 in chunk 2 of an even
# head ([2048, 3104)) but chunk 3 of an odd one ([3040, 4096)); 1024 in chunk 0
# of an even head ([0, 1056)) but chunk 1 of an odd one ([992, 2048)); none;
# 2048 at the start of pair (2, 3) for both.
LENS = [5000, 3050, 1025, 0, 2049]
N_KV, G, D = 2, 4, 128


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import decode_attention_paged_04_amd as kvd
    import gpu_harness as H
    import workloads as W
    return kvd, H, W, torch


def _skew(C):
    return 32 * ((45 * C + 16000) // 32000)


def _span(j, c, C, nc, d):
    """Tokens [lo, hi) of chunk c of KV head j, as the plan's documentation states."""
    if d and (c | 1) < nc:
        base = (c & ~1) * C
        mid = base + C + (d if j % 2 == 0 else -d)
        return (base, mid) if c % 2 == 0 else (mid, base + 2 * C)
    return c * C, (c + 1) * C


def _case(H, W, fp8, seed):
    w = W.DecodeWorkload(f"pairs-{'fp8' if fp8 else 'bf16'}", seed=seed, b=len(LENS), layers=1,
                         n_q=G * N_KV, n_kv=N_KV, head_dim=D, ctx=("fixed", 0),
                         kv_dtype="fp8" if fp8 else "bf16")
    lens = np.array(LENS, dtype=np.int32)
    table, nb = W.block_tables(w, lens, pad_value=-1)
    return H.PagedCase(w, lens=lens, table=table, num_blocks=nb)


@pytest.mark.parametrize("fp8", [False, True])
def test_partials_follow_the_uneven_spans(env, fp8):
    kvd, H, W, torch = env
    from oracle import attention
    case = _case(H, W, fp8, 90 + int(fp8))
    part_o, part_lse, C, nc = kvd.kvd_decode_partials(case.pool, 0, case.q[0], case.table_t, case.lens_t,
                                                      case.max_ctx, chunk_tokens=0)
    torch.cuda.synchronize()
    assert (C, nc) == (1024, 5)
    d = _skew(C)
    assert d == 32
    po, pl = part_o.cpu().double().numpy(), part_lse.cpu().double().numpy()
    qf = H.bf16_to_f64(case.q[0])
    for i, s in enumerate(LENS):
        K, V = case.logical(0, i)
        for h in range(G * N_KV):
            j = h // G
            for c in range(nc):
                lo, hi = _span(j, c, C, nc, d)
                hi = min(hi, s)
                if lo >= hi:
                    assert pl[i, h, c] == -np.inf, (i, h, c)
                    continue
                o, lse = attention.decode_head(qf[i, h], K[lo:hi, j, :], V[lo:hi, j, :])
                err = np.abs(po[i, h, c] - o).max() / max(1.0, np.abs(o).max())
                assert err <= 1e-5, (i, h, c, err)
                assert abs(pl[i, h, c] - lse) <= 1e-5 * max(1.0, abs(lse)), (i, h, c)
    # the merge of these partials is the one-call step, bit for bit
    out = torch.empty_like(case.q[0])
    lse = torch.empty(case.q[0].shape[:2], dtype=torch.float32, device="cuda")
    kvd.kvd_merge_partials(part_o, part_lse, out, lse)
    ref_out, ref_lse = case.run(0)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
    assert torch.equal(lse, ref_lse)
    # and the step matches the oracle's
    ref_o, ref_l = case.oracle(0)
    for i in range(len(LENS)):
        H.assert_bf16_close(ref_out[i], ref_o[i], what=f"uneven pairs fp8={fp8} seq {i}")
    H.assert_lse_close(ref_lse, ref_l)


def _twin(kvd, case):
    d = case.pool.desc
    twin = kvd.allocate_pool(d.num_layers, d.num_blocks, d.n_kv, d.head_dim, d.dtype)
    twin.kv.copy_(case.pool.kv)
    if case.fp8:
        twin.scales.copy_(case.pool.scales)
    return twin


@pytest.mark.parametrize("fp8", [False, True])
def test_fused_append_into_uneven_pairs(env, fp8):
    kvd, H, W, torch = env
    case = _case(H, W, fp8, 95 + int(fp8))
    g = torch.Generator(device="cuda").manual_seed(97 + int(fp8))
    new_k = torch.randn((len(LENS), N_KV, D), generator=g, device="cuda").to(torch.bfloat16)
    new_v = torch.randn((len(LENS), N_KV, D), generator=g, device="cuda").to(torch.bfloat16)
    slots = [int(case.table[i, (s - 1) // 16]) * 16 + (s - 1) % 16 if s > 0 else -1
             for i, s in enumerate(LENS)]
    slots_t = torch.tensor(slots, dtype=torch.int32, device="cuda")
    ref_pool, fused_pool = _twin(kvd, case), _twin(kvd, case)
    kvd.kvd_write_kv(ref_pool, 0, new_k, new_v, slots_t)
    outs = []
    for pool, fused in ((ref_pool, False), (fused_pool, True)):
        out = torch.empty_like(case.q[0])
        lse = torch.empty(case.q[0].shape[:2], dtype=torch.float32, device="cuda")
        kvd.decode(pool, 0, case.q[0], case.table_t, case.lens_t, case.max_ctx, out=out, lse_out=lse,
                   chunk_tokens=0, new_k=new_k if fused else None, new_v=new_v if fused else None)
        outs.append((out, lse))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1], outs[1][1])
    assert torch.equal(ref_pool.kv, fused_pool.kv)
    if fp8:
        assert torch.equal(ref_pool.scales.view(torch.int32), fused_pool.scales.view(torch.int32))
    assert not torch.equal(case.pool.kv, fused_pool.kv)


@pytest.mark.parametrize("fp8", [False, True])
def test_restricted_decode_over_uneven_pairs(env, fp8):
    """Dropped blocks (negative table entries) inside chunks of uneven length:
    the step attends to exactly the kept tokens, as the oracle's restricted step."""
    kvd, H, W, torch = env
    from oracle import tiers
    case = _case(H, W, fp8, 98 + int(fp8))
    rng = np.random.default_rng(99)
    table = case.table.copy()
    for i, s in enumerate(LENS):
        nb = -(-s // 16)
        for b in range(nb):
            if rng.random() < 0.3:
                table[i, b] = -1
    # blocks at the pair boundaries of both head parities (tokens 992-1055 and 3040-3103)
    table[0, 62:66] = -1
    table[1, 190:194] = -1
    qf = H.bf16_to_f64(case.q[0])
    ref_o = np.zeros(qf.shape)
    ref_l = np.zeros(qf.shape[:2])
    for i, s in enumerate(LENS):
        K, V = case.logical(0, i)
        keep = np.array([table[i, t // 16] >= 0 for t in range(s)], dtype=bool)
        ref_o[i], ref_l[i] = tiers.restricted_decode(qf[i], K, V, keep)
    out = torch.empty_like(case.q[0])
    lse = torch.empty(case.q[0].shape[:2], dtype=torch.float32, device="cuda")
    kvd.decode(case.pool, 0, case.q[0], torch.from_numpy(table).cuda(), case.lens_t, case.max_ctx,
               out=out, lse_out=lse, chunk_tokens=0)
    torch.cuda.synchronize()
    H.assert_bf16_close(out, ref_o, what=f"restricted over uneven pairs fp8={fp8}")
    H.assert_lse_close(lse, ref_l)
