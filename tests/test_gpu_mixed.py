"""Mixed-precision decode on the GPU against the oracle.

Each sequence's blocks are split at random between a bf16 pool and an FP8
pool; its table row (native kvd_mixed_row) lists one precision's blocks, a -1
if that run is odd, then the other's, FP8 entries carrying bit 30.  The decode
must match the oracle's step over the blocks as stored; rows of one precision
must give exactly the single-precision kernels' results.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

LENS = [40, 16, 1, 100, 257, 33, 0, 75]
N_KV, G = 2, 4


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import decode_attention_paged_04_amd as kvd
    import gpu_harness as H
    return kvd, H, torch


class MixedCase:
    """Two pools, the sequences' data, and the oracle's view of every block."""

    def __init__(self, kvd, H, torch, d, seed, mode="random", lens=LENS):
        rng = np.random.default_rng(seed)
        g = torch.Generator().manual_seed(seed)
        self.d = d
        self.lens = lens = list(lens)
        blocks16, blocks8 = [], []                       # (seq, logical block)
        self.prec = []
        for i, s in enumerate(lens):
            nb = -(-s // 16)
            if mode == "bf16":
                p = [0] * nb
            elif mode == "fp8":
                p = [1] * nb
            else:
                p = list(rng.integers(0, 2, nb))
            self.prec.append(p)
            for b in range(nb):
                (blocks8 if p[b] else blocks16).append((i, b))
        self.nb16, self.nb8 = max(len(blocks16), 1) + 3, max(len(blocks8), 1) + 3
        self.pool16 = kvd.allocate_pool(1, self.nb16, N_KV, d, kvd.KVD_BF16)
        self.pool8 = kvd.allocate_pool(1, self.nb8, N_KV, d, kvd.KVD_FP8_E4M3)
        self.pool16.kv.fill_(0xFF)
        self.pool8.kv.fill_(0xFF)
        phys16 = rng.permutation(self.nb16)
        phys8 = rng.permutation(self.nb8)
        self.phys = {}
        for k, key in enumerate(blocks16):
            self.phys[key] = int(phys16[k])
        for k, key in enumerate(blocks8):
            self.phys[key] = int(phys8[k])
        self.K = [torch.randn((s, N_KV, d), generator=g).to(torch.bfloat16) for s in lens]
        self.V = [torch.randn((s, N_KV, d), generator=g).to(torch.bfloat16) for s in lens]
        self.q = torch.randn((len(lens), N_KV * G, d), generator=g).to(torch.bfloat16)
        for pool, which in ((self.pool16, 0), (self.pool8, 1)):
            Ks, Vs, slots = [], [], []
            for i, s in enumerate(lens):
                for b in range(-(-s // 16)):
                    if self.prec[i][b] != which:
                        continue
                    lo, hi = 16 * b, min(s, 16 * b + 16)
                    Ks.append(self.K[i][lo:hi])
                    Vs.append(self.V[i][lo:hi])
                    slots += [self.phys[(i, b)] * 16 + r for r in range(hi - lo)]
            if slots:
                kvd.kvd_write_kv(pool, 0, torch.cat(Ks).cuda(), torch.cat(Vs).cuda(),
                                 torch.tensor(slots, dtype=torch.int32, device="cuda"))
        # rows (the partial last block, if any, is the last of its run)
        rows, self.ctx = [], []
        for i, s in enumerate(lens):
            nb = -(-s // 16)
            ids16 = [self.phys[(i, b)] for b in range(nb) if not self.prec[i][b]]
            ids8 = [self.phys[(i, b)] for b in range(nb) if self.prec[i][b]]
            fp8_last = bool(self.prec[i][nb - 1]) if nb else True
            tail = s - 16 * (nb - 1) if nb else 16
            row, c = kvd.mixed_row(ids16, ids8, fp8_last, tail)
            rows.append(row)
            self.ctx.append(c)
        self.mb = max(max(len(r) for r in rows), 1)
        self.table = np.full((len(lens), self.mb), -1, dtype=np.int32)
        for i, r in enumerate(rows):
            self.table[i, :len(r)] = r
        self.H = H

    def stored_blocks(self, i):
        """(K, V) float64 of every block of sequence i as its pool holds it."""
        from oracle import e4m3
        out = []
        s = self.lens[i]
        for b in range(-(-s // 16)):
            lo, hi = 16 * b, min(s, 16 * b + 16)
            K = self.H.bf16_to_f64(self.K[i][lo:hi])
            V = self.H.bf16_to_f64(self.V[i][lo:hi])
            if self.prec[i][b]:
                ck, sk = e4m3.quantize_sequence(K.astype(np.float32))
                cv, sv = e4m3.quantize_sequence(V.astype(np.float32))
                K, V = e4m3.dequantize_sequence(ck, sk), e4m3.dequantize_sequence(cv, sv)
            out.append((K, V, b))
        return out

    def run(self, kvd, torch, table, chunk=0):
        out = torch.empty_like(self.q).cuda()
        lse = torch.empty(self.q.shape[:2], dtype=torch.float32, device="cuda")
        lens = torch.tensor(self.ctx, dtype=torch.int32, device="cuda")
        kvd.decode_mixed(self.pool16, self.pool8, 0, self.q.cuda(), torch.from_numpy(table).cuda(), lens,
                         max(max(self.ctx), 1), out=out, lse_out=lse, chunk_tokens=chunk)
        torch.cuda.synchronize()
        return out, lse


# Lengths whose automatic split at a 5,000-token bound is five 1,024-token
# chunks with uneven pairs (d = 32): the two passes then step over the spans of
# chunks whose boundaries depend on the KV head's parity.
PAIR_LENS = [5000, 3050, 1025, 0, 2049]


def test_mixed_decode_over_uneven_chunk_pairs(env):
    kvd, H, torch = env
    from oracle import mixed
    case = MixedCase(kvd, H, torch, 128, seed=760, lens=PAIR_LENS)
    args = kvd.make_args(case.q.cuda(), torch.from_numpy(case.table).cuda(),
                         torch.tensor(case.ctx, dtype=torch.int32, device="cuda"), max(case.ctx),
                         torch.empty_like(case.q).cuda(), pool=case.pool16)
    assert kvd.kvd_decode_plan(case.pool16, args) == (1024, 5)
    qf = H.bf16_to_f64(case.q)
    ref_o = np.zeros(qf.shape)
    ref_l = np.zeros(qf.shape[:2])
    for i in range(len(PAIR_LENS)):
        ref_o[i], ref_l[i] = mixed.decode_mixed(qf[i], [(k, v) for k, v, _ in case.stored_blocks(i)])
    out, lse = case.run(kvd, torch, case.table, 0)
    H.assert_bf16_close(out, ref_o, what="mixed over uneven chunk pairs")
    H.assert_lse_close(lse, ref_l)


@pytest.mark.parametrize("d", [64, 128])
def test_mixed_decode_matches_oracle(env, d):
    kvd, H, torch = env
    from oracle import mixed
    case = MixedCase(kvd, H, torch, d, seed=700 + d)
    qf = H.bf16_to_f64(case.q)
    ref_o = np.zeros(qf.shape)
    ref_l = np.zeros(qf.shape[:2])
    for i in range(len(LENS)):
        ref_o[i], ref_l[i] = mixed.decode_mixed(qf[i], [(k, v) for k, v, _ in case.stored_blocks(i)])
    for chunk in (0, 16, 48, 256):
        H.say(f"mixed d={d} chunk={chunk}")
        out, lse = case.run(kvd, torch, case.table, chunk)
        H.assert_bf16_close(out, ref_o, what=f"mixed d{d} chunk{chunk}")
        H.assert_lse_close(lse, ref_l)
    # a keep mask on top: drop the first block of every row that has more than one
    t2 = case.table.copy()
    dropped = {}
    for i, s in enumerate(LENS):
        if -(-s // 16) > 1 and t2[i, 0] >= 0:
            e = int(t2[i, 0])
            t2[i, 0] = -1
            dropped[i] = (e, bool(e & kvd.PRECISION_BIT))
    out, lse = case.run(kvd, torch, t2)
    for i in range(len(LENS)):
        blocks = case.stored_blocks(i)
        if i in dropped:
            e, is8 = dropped[i]
            phys = e & ~kvd.PRECISION_BIT
            blocks = [x for x in blocks if not (bool(case.prec[i][x[2]]) == is8 and case.phys[(i, x[2])] == phys)]
        ref_o[i], ref_l[i] = mixed.decode_mixed(qf[i], [(k, v) for k, v, _ in blocks])
    H.assert_bf16_close(out, ref_o, what=f"mixed d{d} with drops")
    H.assert_lse_close(lse, ref_l)


@pytest.mark.parametrize("mode", ["bf16", "fp8"])
def test_one_precision_rows_equal_the_plain_kernels(env, mode):
    kvd, H, torch = env
    case = MixedCase(kvd, H, torch, 128, seed=710, mode=mode)
    plain = case.table & ~kvd.PRECISION_BIT
    plain[case.table < 0] = -1
    pool = case.pool16 if mode == "bf16" else case.pool8
    for chunk in (0, 48):
        out_m, lse_m = case.run(kvd, torch, case.table, chunk)
        out = torch.empty_like(out_m)
        lse = torch.empty_like(lse_m)
        kvd.decode(pool, 0, case.q.cuda(), torch.from_numpy(plain).cuda(),
                   torch.tensor(case.ctx, dtype=torch.int32, device="cuda"), max(case.ctx), out=out,
                   lse_out=lse, chunk_tokens=chunk)
        torch.cuda.synchronize()
        assert torch.equal(out, out_m) and torch.equal(lse, lse_m), (mode, chunk)


@pytest.mark.parametrize("d", [64, 128])
def test_rows_in_logical_order(env, d):
    """A row may also list the blocks in their logical order, precisions
    alternating (each entry names its own pool): the step over the same stored
    tokens, for the library's chunking and for chunks that start mid-page."""
    kvd, H, torch = env
    from oracle import mixed
    case = MixedCase(kvd, H, torch, d, seed=720 + d)
    table = np.full((len(LENS), case.mb), -1, dtype=np.int32)
    for i, s in enumerate(LENS):
        for b in range(-(-s // 16)):
            table[i, b] = case.phys[(i, b)] | (kvd.PRECISION_BIT if case.prec[i][b] else 0)
    case.ctx = list(LENS)
    qf = H.bf16_to_f64(case.q)
    ref_o = np.zeros(qf.shape)
    ref_l = np.zeros(qf.shape[:2])
    for i in range(len(LENS)):
        ref_o[i], ref_l[i] = mixed.decode_mixed(qf[i], [(k, v) for k, v, _ in case.stored_blocks(i)])
    for chunk in (0, 16, 48, 96):
        H.say(f"mixed logical order d={d} chunk={chunk}")
        out, lse = case.run(kvd, torch, table, chunk)
        H.assert_bf16_close(out, ref_o, what=f"mixed logical order d{d} chunk{chunk}")
        H.assert_lse_close(lse, ref_l)
