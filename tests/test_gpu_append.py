"""GPU parity of the decode-step append path against the float64 oracle.

A prompt is stored, then tokens are appended a few at a time -- mostly one per
sequence per call, the way a decode step adds its token -- into partly filled
blocks.  FP8 pools re-quantise the touched tiles; their codes and scales must
match the oracle's append step bit for bit, and the decode over the result must
match the oracle's attention over the values as they read back.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

FINAL = [1, 15, 16, 17, 33, 40, 70, 5]
PREFIX = [0, 3, 16, 10, 1, 32, 45, 5]
# tokens appended per call (cycled); 3 lets a run cross a block boundary
STRIDE = [1, 1, 3, 1, 2]


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import decode_attention_paged_04_amd as kvd
    import gpu_harness as H
    import workloads as W
    return kvd, H, W, torch


def _slots(table, i, lo, hi):
    return [int(table[i, t // 16]) * 16 + t % 16 for t in range(lo, hi)]


def _append_schedule():
    """Calls of the append phase: for each call, the (sequence, first, end) token ranges."""
    done = list(PREFIX)
    calls, k = [], 0
    while any(d < f for d, f in zip(done, FINAL)):
        m = STRIDE[k % len(STRIDE)]
        call = []
        for i, (d, f) in enumerate(zip(done, FINAL)):
            if d < f:
                e = min(f, d + m)
                call.append((i, d, e))
                done[i] = e
        calls.append(call)
        k += 1
    return calls


@pytest.mark.parametrize("fp8", [True, False])
@pytest.mark.parametrize("d", [64, 128])
def test_append_matches_oracle(env, fp8, d):
    kvd, H, W, torch = env
    from oracle import attention, e4m3, paged
    lens = np.array(FINAL, dtype=np.int32)
    w = W.DecodeWorkload(f"append-d{d}", seed=300 + d, b=len(FINAL), layers=1, n_q=8, n_kv=2,
                         head_dim=d, ctx=("fixed", 0), kv_dtype="fp8" if fp8 else "bf16")
    table, nb = W.block_tables(w, lens)
    offs = W.offsets(lens)
    n = int(offs[-1])
    K, V = W.keys_values(w, 0, n, "cuda")
    # a late, large element forces a scale change (and a re-encode) mid-block
    K[int(offs[6]) + 50, 1, 7] = 40.0
    V[int(offs[5]) + 35, 0, 3] = -25.0
    q = W.query(w, 0, "cuda")
    dt = kvd.KVD_FP8_E4M3 if fp8 else kvd.KVD_BF16
    pool = kvd.allocate_pool(1, nb, w.n_kv, d, dt)
    pool.kv.fill_(0xFF)
    Kc, Vc = K.cpu(), V.cpu()
    Kf, Vf = H.bf16_to_f64(Kc).astype(np.float32), H.bf16_to_f64(Vc).astype(np.float32)

    def write(ranges):
        idx, slots = [], []
        for i, lo, hi in ranges:
            idx += [int(offs[i]) + t for t in range(lo, hi)]
            slots += _slots(table, i, lo, hi)
        if not idx:
            return
        it = torch.tensor(idx, dtype=torch.long, device="cuda")
        st = torch.tensor(slots, dtype=torch.int32, device="cuda")
        kvd.kvd_write_kv(pool, 0, K[it].contiguous(), V[it].contiguous(), st)

    # the oracle's view: codes and scales per sequence, advanced call by call
    state = {}
    if fp8:
        for i in range(len(FINAL)):
            state[i] = [np.zeros((0, w.n_kv, d), np.uint8), np.zeros((0, w.n_kv), np.float32),
                        np.zeros((0, w.n_kv, d), np.uint8), np.zeros((0, w.n_kv), np.float32)]

    def oracle_write(ranges):
        if not fp8:
            return
        for i, lo, hi in ranges:
            a = int(offs[i])
            ck, sk, cv, sv = state[i]
            ck, sk = e4m3.append_sequence(ck, sk, Kf[a + lo:a + hi])
            cv, sv = e4m3.append_sequence(cv, sv, Vf[a + lo:a + hi])
            state[i] = [ck, sk, cv, sv]

    prefill = [(i, 0, p) for i, p in enumerate(PREFIX) if p > 0]
    H.say(f"append d={d} fp8={fp8}: prefill")
    write(prefill)
    oracle_write(prefill)
    calls = _append_schedule()
    for c, ranges in enumerate(calls):
        H.say(f"  call {c}: {ranges}")
        write(ranges)
        oracle_write(ranges)
    torch.cuda.synchronize()
    H.say(f"append d={d} fp8={fp8}: {len(calls)} append calls done")

    lay = paged.PoolLayout(1, nb, w.n_kv, d, elem_bytes=1 if fp8 else 2)
    got = pool.kv.cpu().numpy()
    logical = {}
    for i, s in enumerate(FINAL):
        a = int(offs[i])
        if fp8:
            ck, sk, cv, sv = state[i]
            k_idx, v_idx = paged.gather_indices(lay, 0, table[i], s)
            assert np.array_equal(got[k_idx], ck), f"K codes of sequence {i}: {np.count_nonzero(got[k_idx] != ck)} differ"
            assert np.array_equal(got[v_idx], cv), f"V codes of sequence {i}: {np.count_nonzero(got[v_idx] != cv)} differ"
            got_sc = pool.scales.cpu().numpy()
            for b in range(sk.shape[0]):
                p = int(table[i, b])
                for j in range(w.n_kv):
                    assert got_sc[lay.scale_index(0, p, j, 0)].view(np.uint32) == sk[b, j].view(np.uint32)
                    assert got_sc[lay.scale_index(0, p, j, 1)].view(np.uint32) == sv[b, j].view(np.uint32)
            logical[i] = (e4m3.dequantize_sequence(ck, sk), e4m3.dequantize_sequence(cv, sv))
        else:
            logical[i] = (Kf[a:a + s].astype(np.float64), Vf[a:a + s].astype(np.float64))

    # the re-encode must actually have happened for the planted values
    if fp8:
        blk = 50 // 16
        assert state[6][1][blk, 1] == np.float32(np.float32(40.0) / np.float32(448.0))

    lens_t = torch.from_numpy(lens).cuda()
    table_t = torch.from_numpy(table).cuda()
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    kvd.decode(pool, 0, q, table_t, lens_t, int(lens.max()), out=out, lse_out=lse, chunk_tokens=32)
    torch.cuda.synchronize()
    qf = H.bf16_to_f64(q)
    ref_o = np.zeros(qf.shape)
    ref_l = np.zeros(qf.shape[:2])
    for i in range(len(FINAL)):
        ref_o[i], ref_l[i] = attention.decode_sequence(qf[i], *logical[i])
    H.assert_bf16_close(out, ref_o, what=f"append d{d} fp8={fp8}")
    H.assert_lse_close(lse, ref_l)
