"""kvd_decode_attn_no_alloc: the decode step with the library's fixed
per-device scratch instead of a caller workspace, for callers that cannot
allocate.

Through the C ABI it must give, bit for bit, what kvd_decode_attn /
kvd_decode_attn_fp8 give with a workspace -- outputs, lse and fused scores --
on two calls in a row, the second with a smaller input (the scratch keeps the
first call's contents, which must not leak into the second), and both must
meet the oracle's tolerance.  A call whose scratch need exceeds the fixed
size is refused before any launch.
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


def _both(kvd, torch, case, chunk, score_init=None):
    """(out, lse, score) from kvd_decode_attn[_fp8] with a workspace and from
    kvd_decode_attn_no_alloc, same arguments."""
    q = case.q[0]
    res = []
    for no_alloc in (False, True):
        out = torch.full_like(q, float("nan"))
        lse = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device="cuda")
        score = None if score_init is None else score_init.clone()
        args = kvd.make_args(q, case.table_t, case.lens_t, case.max_ctx, out, lse, chunk, None, score,
                             0.25, pool=case.pool)
        if no_alloc:
            kvd.kvd_decode_attn_no_alloc(case.pool, 0, args)
        else:
            ws = kvd.allocate_workspace(case.pool, args)
            (kvd.kvd_decode_attn_fp8 if case.fp8 else kvd.kvd_decode_attn)(case.pool, 0, args)
        torch.cuda.synchronize()
        res.append((out, lse, score))
    return res


def torch_equal_bits(x, y):
    import torch
    return torch.equal(x.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("fp8", [False, True])
def test_no_alloc_equals_workspace_call_twice(env, fp8):
    kvd, H, W, torch = env
    runs = [
        # (b, length range, n_q, n_kv, d, chunk, score): the second call is smaller
        (8, (1, 3000), 16, 4, 128, 256, False),
        (3, (0, 500), 8, 2, 64, 64, False),
        (6, (1, 2500), 16, 4, 128, 128, True),
        (2, (1, 300), 8, 2, 128, 32, True),
        (5, (1, 200), 8, 2, 64, 0, False),           # one chunk: no scratch used
    ]
    for k, (b, span, n_q, n_kv, d, chunk, with_score) in enumerate(runs):
        w = W.DecodeWorkload(f"no-alloc-{k}", seed=300 + k, b=b, layers=1, n_q=n_q, n_kv=n_kv, head_dim=d,
                             ctx=("uniform", span[0], span[1]), kv_dtype="fp8" if fp8 else "bf16")
        lens = W.context_lengths(w)
        case = H.PagedCase(w, lens=lens)
        init = None
        if with_score:
            init = torch.rand((b, case.max_ctx + 5), generator=torch.Generator(device="cuda").manual_seed(k),
                              device="cuda")
        (o1, l1, s1), (o2, l2, s2) = _both(kvd, torch, case, chunk, init)
        H.say(f"no-alloc call {k}: fp8={fp8} b={b} lens {int(lens.min())}..{int(lens.max())} chunk {chunk}")
        assert torch_equal_bits(o1, o2), k
        assert torch.equal(l1, l2), k
        if with_score:
            assert torch.equal(s1, s2), k
        ref_o, ref_lse = case.oracle(0)
        for i in range(b):
            H.assert_bf16_close(o2[i], ref_o[i], rel_tol=H.TOL_FP8_REL_L2 if fp8 else H.TOL_REL_L2,
                                what=f"no-alloc call {k} seq {i}")
        H.assert_lse_close(l2, ref_lse)


def test_no_alloc_refuses_more_than_its_scratch(env):
    kvd, H, W, torch = env
    import ctypes
    b, n_q, d, s = 32, 32, 128, 32768                 # score scratch of 32*32*32800*4 B > 32 MiB
    pool = kvd.allocate_pool(1, 16, 8, d)
    q = torch.zeros((b, n_q, d), dtype=torch.bfloat16, device="cuda")
    table = torch.zeros((b, s // 16), dtype=torch.int32, device="cuda")
    lens = torch.full((b,), s, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    score = torch.zeros((b, s), dtype=torch.float32, device="cuda")
    args = kvd.make_args(q, table, lens, s, out, score=score, score_weight=1.0, pool=pool)
    assert kvd.kvd_decode_workspace_bytes(pool, args) > 32 << 20
    st = kvd.lib.kvd_decode_attn_no_alloc(pool.handle, 0, ctypes.byref(args), None)
    assert st == 4, kvd.kvd_status_string(st)          # KVD_ERR_WORKSPACE, nothing launched
    torch.cuda.synchronize()
    assert bool((score == 0).all())
