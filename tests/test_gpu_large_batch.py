"""Decode against the oracle where the work decomposition takes its rarer
branches: more than 512 sequences (several, then more than 64, sequences per
lane of the unit-locating wave) and batches whose context splits into more
than 64 chunks (sequence-major order of the full chunks).  bf16 and FP8 pools,
with an empty and a one-token sequence in every batch.  The outputs are
filled with NaN bytes first, so a head whose chunks were not all computed and
merged would keep NaN; the call runs twice on one workspace.
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


CASES = [
    # (name, b, length range, kv dtype, chunk tokens, n_q, n_kv, d)
    ("b600-bf16", 600, (0, 400), "bf16", 16, 8, 2, 64),
    ("b600-fp8", 600, (0, 400), "fp8", 32, 8, 2, 64),
    ("b4200-bf16", 4200, (0, 160), "bf16", 16, 4, 1, 64),
    ("b4200-fp8", 4200, (0, 160), "fp8", 32, 4, 1, 64),
    ("b3-s1100-chunk16-bf16", 3, (1090, 1100), "bf16", 16, 32, 8, 128),
    ("b3-s1100-chunk16-fp8", 3, (1090, 1100), "fp8", 16, 32, 8, 128),
    ("b40-69chunks-bf16", 40, (0, 1100), "bf16", 16, 8, 2, 128),
]


@pytest.mark.parametrize("name,b,span,dt,chunk,n_q,n_kv,d", CASES, ids=[c[0] for c in CASES])
def test_decode_rare_decompositions(env, name, b, span, dt, chunk, n_q, n_kv, d):
    kvd, H, W, torch = env
    w = W.DecodeWorkload(f"rare-{name}", seed=4000 + b, b=b, layers=1, n_q=n_q, n_kv=n_kv, head_dim=d,
                         ctx=("uniform", span[0], span[1]), kv_dtype=dt)
    lens = W.context_lengths(w)
    lens[0], lens[min(1, b - 1)] = 0, 1
    H.say(f"{name}: b={b} lengths {int(lens.min())}..{int(lens.max())} chunk {chunk}")
    case = H.PagedCase(w, lens=lens)
    q = case.q[0]
    ref_o, ref_lse = case.oracle(0)
    tol = H.TOL_FP8_REL_L2 if case.fp8 else H.TOL_REL_L2
    ws = None
    for run in range(2):
        out = torch.full_like(q, float("nan"))
        lse = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device="cuda")
        args = kvd.make_args(q, case.table_t, case.lens_t, case.max_ctx, out, lse, chunk, pool=case.pool)
        ch, nc = kvd.kvd_decode_plan(case.pool, args)
        assert ch == chunk and nc == -(-case.max_ctx // chunk)
        if ws is None:
            ws = kvd.allocate_workspace(case.pool, args)
        else:
            args.workspace, args.workspace_bytes = ws.data_ptr(), kvd.kvd_decode_workspace_bytes(case.pool, args)
        (kvd.kvd_decode_attn_fp8 if case.fp8 else kvd.kvd_decode_attn)(case.pool, 0, args)
        torch.cuda.synchronize()
        worst = (0.0, 0.0)
        for i in range(b):
            mx, rel = H.assert_bf16_close(out[i], ref_o[i], rel_tol=tol, what=f"{name} run {run} seq {i} (s={lens[i]})")
            worst = (max(worst[0], mx), max(worst[1], rel))
        H.assert_lse_close(lse, ref_lse)
        H.say(f"{name} run {run}: {nc} chunks, worst max-abs {worst[0]:.2e} rel-L2 {worst[1]:.2e}")
