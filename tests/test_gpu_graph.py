"""Decode calls captured in a HIP graph and replayed.

A serving loop captures its per-layer decode calls once and replays them every
step with new queries (and, with scores, a growing score array).  Every replay
must equal the eager call on the same inputs, bit for bit: the calls record
only kernel launches (no memset or copy nodes), and no launch depends on
scratch memory left by an earlier one.  Eager work and synchronisations run
between the replays.
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


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("scores", [False, True])
def test_graph_replays_equal_eager_calls(env, fp8, scores):
    kvd, H, W, torch = env
    lens = np.array([1, 40, 300, 77, 0, 513], dtype=np.int32)
    w = W.DecodeWorkload("graph", seed=80, b=len(lens), layers=2, n_q=16, n_kv=4, head_dim=128,
                         ctx=("fixed", 0), kv_dtype="fp8" if fp8 else "bf16")
    table, nb = W.block_tables(w, lens, pad_value=-1)
    case = H.PagedCase(w, lens=lens, table=table, num_blocks=nb)
    chunk = 64
    q = [case.q[layer].clone() for layer in range(2)]
    out = [torch.empty_like(q[0]) for _ in range(2)]
    lse = [torch.empty(q[0].shape[:2], dtype=torch.float32, device="cuda") for _ in range(2)]
    stride = case.max_ctx + 5
    score = torch.zeros((len(lens), stride), dtype=torch.float32, device="cuda") if scores else None
    args = [kvd.make_args(q[layer], case.table_t, case.lens_t, case.max_ctx, out[layer], lse[layer], chunk,
                          None, score, 0.5 if scores else 0.0, pool=case.pool) for layer in range(2)]
    ws = [kvd.allocate_workspace(case.pool, a) for a in args]
    fn = kvd.kvd_decode_attn_fp8 if fp8 else kvd.kvd_decode_attn

    def step():
        for layer in range(2):
            fn(case.pool, layer, args[layer])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                   # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    g = torch.Generator(device="cuda").manual_seed(81)
    for rep in range(4):
        new_q = [torch.randn(q[0].shape, generator=g, device="cuda").to(torch.bfloat16) for _ in range(2)]
        for layer in range(2):
            q[layer].copy_(new_q[layer])
        start = score.clone() if scores else None
        graph.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in out] + [x.clone() for x in lse] + ([score.clone()] if scores else [])
        # eager, same inputs
        if scores:
            score.copy_(start)
        torch.randn(1 << 20, device="cuda").sum()  # unrelated eager work between
        step()
        torch.cuda.synchronize()
        want = [o.clone() for o in out] + [x.clone() for x in lse] + ([score.clone()] if scores else [])
        for a, b in zip(got, want):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b), rep
        if rep == 0:                             # and the replay is right: the oracle on its inputs
            case.q[0] = new_q[0]
            ref_o, ref_l = case.oracle(0)
            H.assert_bf16_close(got[0], ref_o, what=f"graph replay fp8={fp8} scores={scores}")
            H.assert_lse_close(got[2], ref_l)
