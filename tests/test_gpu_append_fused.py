"""The fused append (kvd_decode_attn_append) on the GPU.

One launch stores token s_i - 1 of every sequence and decodes.  It must leave
exactly what kvd_write_kv of those tokens followed by the decode call leaves:
the same pool bytes (codes and scales for FP8, including a re-quantised tile
whose scale grows), the same outputs, lse and fused scores, bit for bit --
for ragged lengths whose last token opens a block, fills one, or ends a chunk,
for sequences with no tokens, and for a sequence whose last block is marked
not attended (nothing is stored for it).
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

LENS = [0, 1, 16, 17, 33, 47, 48, 100, 257, 49, 96, 97]


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import decode_attention_paged_04_amd as kvd
    import gpu_harness as H
    import workloads as W
    return kvd, H, W, torch


def _twin(kvd, torch, case):
    """A second pool with the same bytes as the case's pool."""
    d = case.pool.desc
    twin = kvd.allocate_pool(d.num_layers, d.num_blocks, d.n_kv, d.head_dim, d.dtype)
    twin.kv.copy_(case.pool.kv)
    if case.fp8:
        twin.scales.copy_(case.pool.scales)
    return twin


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_fused_append_equals_write_then_decode(env, fp8, d):
    kvd, H, W, torch = env
    w = W.DecodeWorkload(f"append-fused-d{d}", seed=60 + d, b=len(LENS), layers=1, n_q=8, n_kv=2,
                         head_dim=d, ctx=("fixed", 0), kv_dtype="fp8" if fp8 else "bf16")
    lens = np.array(LENS, dtype=np.int32)
    table, nb = W.block_tables(w, lens, pad_value=-1)
    case = H.PagedCase(w, lens=lens, table=table, num_blocks=nb)
    g = torch.Generator(device="cuda").manual_seed(61 + d)
    new_k = torch.randn((len(LENS), 2, d), generator=g, device="cuda").to(torch.bfloat16)
    new_v = torch.randn((len(LENS), 2, d), generator=g, device="cuda").to(torch.bfloat16)
    new_k[4] *= 40.0                                   # its FP8 tile's scale grows: old rows re-encoded
    run_table = case.table.copy()
    run_table[7, (int(lens[7]) - 1) // 16] = -1        # last block not attended: nothing stored
    table_t = torch.from_numpy(run_table).cuda()
    slots = []
    for i, s in enumerate(LENS):
        p = int(run_table[i, (s - 1) // 16]) if s > 0 else -1
        slots.append(p * 16 + (s - 1) % 16 if s > 0 and p >= 0 else -1)
    slots_t = torch.tensor(slots, dtype=torch.int32, device="cuda")
    for chunk in (0, 16, 48):
        H.say(f"fused append fp8={fp8} d={d} chunk={chunk}")
        ref_pool = _twin(kvd, torch, case)
        fused_pool = _twin(kvd, torch, case)
        kvd.kvd_write_kv(ref_pool, 0, new_k, new_v, slots_t)
        outs = []
        for pool, fused in ((ref_pool, False), (fused_pool, True)):
            out = torch.empty_like(case.q[0])
            lse = torch.empty(case.q[0].shape[:2], dtype=torch.float32, device="cuda")
            kvd.decode(pool, 0, case.q[0], table_t, case.lens_t, case.max_ctx, out=out, lse_out=lse,
                       chunk_tokens=chunk, new_k=new_k if fused else None, new_v=new_v if fused else None)
            outs.append((out, lse))
        torch.cuda.synchronize()
        assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16)), chunk
        assert torch.equal(outs[0][1], outs[1][1]), chunk
        assert torch.equal(ref_pool.kv, fused_pool.kv), chunk
        if fp8:
            assert torch.equal(ref_pool.scales.view(torch.int32), fused_pool.scales.view(torch.int32)), chunk
        # the append did change the pool (it is not a no-op on both sides)
        assert not torch.equal(case.pool.kv, fused_pool.kv)


@pytest.mark.parametrize("fp8", [False, True])
def test_fused_append_with_scores(env, fp8):
    kvd, H, W, torch = env
    d = 128
    w = W.DecodeWorkload("append-fused-scores", seed=70, b=len(LENS), layers=1, n_q=8, n_kv=2,
                         head_dim=d, ctx=("fixed", 0), kv_dtype="fp8" if fp8 else "bf16")
    lens = np.array(LENS, dtype=np.int32)
    table, nb = W.block_tables(w, lens, pad_value=-1)
    case = H.PagedCase(w, lens=lens, table=table, num_blocks=nb)
    g = torch.Generator(device="cuda").manual_seed(71)
    new_k = torch.randn((len(LENS), 2, d), generator=g, device="cuda").to(torch.bfloat16)
    new_v = torch.randn((len(LENS), 2, d), generator=g, device="cuda").to(torch.bfloat16)
    slots = [int(case.table[i, (s - 1) // 16]) * 16 + (s - 1) % 16 if s > 0 else -1 for i, s in enumerate(LENS)]
    slots_t = torch.tensor(slots, dtype=torch.int32, device="cuda")
    stride = case.max_ctx + 3
    init = torch.rand((len(LENS), stride), generator=g, device="cuda")
    for chunk in (0, 32):
        ref_pool, fused_pool = _twin(kvd, torch, case), _twin(kvd, torch, case)
        kvd.kvd_write_kv(ref_pool, 0, new_k, new_v, slots_t)
        res = []
        for pool, fused in ((ref_pool, False), (fused_pool, True)):
            score = init.clone()
            out = torch.empty_like(case.q[0])
            kvd.decode(pool, 0, case.q[0], case.table_t, case.lens_t, case.max_ctx, out=out, chunk_tokens=chunk,
                       score=score, score_weight=0.5, new_k=new_k if fused else None,
                       new_v=new_v if fused else None)
            res.append((out, score))
        torch.cuda.synchronize()
        assert torch.equal(res[0][0].view(torch.int16), res[1][0].view(torch.int16))
        assert torch.equal(res[0][1], res[1][1])
        assert torch.equal(ref_pool.kv, fused_pool.kv)


@pytest.mark.parametrize("fp8", [False, True])
def test_fused_append_past_the_bound_stores_nothing(env, fp8):
    """A context length above min(max_context_len, 16 * max_blocks_per_seq)
    has no slot for its new token inside the bound: the call stores nothing
    (every cached row keeps its bytes) and attends to the clamped context,
    exactly as the plain decode call with the same arguments."""
    kvd, H, W, torch = env
    d = 64
    lens = np.array([40, 64, 100], dtype=np.int32)
    w = W.DecodeWorkload("append-fused-bound", seed=75, b=3, layers=1, n_q=4, n_kv=2, head_dim=d,
                         ctx=("fixed", 0), kv_dtype="fp8" if fp8 else "bf16")
    table, nb = W.block_tables(w, lens, pad_value=-1)
    case = H.PagedCase(w, lens=lens, table=table, num_blocks=nb)
    g = torch.Generator(device="cuda").manual_seed(76)
    new_k = torch.randn((3, 2, d), generator=g, device="cuda").to(torch.bfloat16)
    new_v = torch.randn((3, 2, d), generator=g, device="cuda").to(torch.bfloat16)
    # bound 48: sequence 0 (40 tokens) appends at row 39; 1 and 2 lie past the bound
    bound = 48
    ref_pool, fused_pool = _twin(kvd, torch, case), _twin(kvd, torch, case)
    first = torch.tensor([39, 0, 0], dtype=torch.int32, device="cuda")
    only0 = torch.tensor([40, 0, 0], dtype=torch.int32, device="cuda")
    slots = kvd.kvd_slot_mapping(case.table_t, only0, first_token=first)      # sequence 0's token 39 only
    assert slots.numel() == 1
    kvd.kvd_write_kv(ref_pool, 0, new_k[:1], new_v[:1], slots)
    outs = []
    for pool, fused in ((ref_pool, False), (fused_pool, True)):
        out = torch.empty_like(case.q[0])
        lse = torch.empty(case.q[0].shape[:2], dtype=torch.float32, device="cuda")
        kvd.decode(pool, 0, case.q[0], case.table_t, case.lens_t, bound, out=out, lse_out=lse, chunk_tokens=16,
                   new_k=new_k if fused else None, new_v=new_v if fused else None)
        outs.append((out, lse))
    torch.cuda.synchronize()
    assert torch.equal(ref_pool.kv, fused_pool.kv)
    if fp8:
        assert torch.equal(ref_pool.scales.view(torch.int32), fused_pool.scales.view(torch.int32))
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1], outs[1][1])
    # the oracle over the clamped contexts (the stored rows of sequences 1 and 2 unchanged)
    from oracle import attention
    qf = H.bf16_to_f64(case.q[0])
    for i in (1, 2):
        Ki, Vi = case.logical(0, i)
        o, _ = attention.decode_sequence(qf[i], Ki[:bound], Vi[:bound])
        H.assert_bf16_close(outs[1][0][i], o, rel_tol=H.TOL_FP8_REL_L2 if fp8 else H.TOL_REL_L2,
                            what=f"clamped sequence {i}")
