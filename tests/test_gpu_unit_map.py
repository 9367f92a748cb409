"""The decode grid's work decomposition, read back from the device.

kvd_debug_unit_map runs the decode kernels' own unit-location code and reports
the (sequence, chunk) unit of every workgroup.  For each KV head the units
must cover every (sequence, chunk) pair of the launch exactly once, in the
order the kernels promise: the chunks a sequence fills completely first, then
each sequence's partly filled last chunk, then the empty chunks; the full
chunks chunk-major (chunk c of every sequence that has it, then chunk c + 1),
the other two runs sequence by sequence.  The order only decides which
workgroup computes a unit; the batch sizes here reach every branch of the
location code (one sequence per lane, up to eight, more than eight, more than
64 per lane; more than 64 chunks).

Each workgroup also reports its KV head and token span.  They must follow the
documented split: head x % n_kv and span [c*C, (c+1)*C), or, for an automatic
split with an even n_kv and two or more chunks, the uneven pairs (C + d on the
workgroups with x even, C - d on their neighbours, d = 32 * floor((45 C +
16000) / 32000)); and for every sequence and head the spans of its chunks
must tile [0, n_chunks * C) exactly.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import decode_attention_paged_04_amd as kvd
    return kvd, torch


def expected_order(lens, chunk, n_chunks, bound):
    """Units (sequence, chunk) in grid order, written from the rule above."""
    s = np.clip(np.asarray(lens, dtype=np.int64), 0, bound)
    b = len(s)
    full = [(i, c) for i in range(b) for c in range(n_chunks) if (c + 1) * chunk <= s[i]]
    full.sort(key=lambda u: (u[1], u[0]))
    part = [(i, int(s[i] // chunk)) for i in range(b) if s[i] % chunk]
    empty = [(i, c) for i in range(b) for c in range(n_chunks) if c * chunk >= s[i]]
    return full + part + empty, s


def expected_span(x, c, n_kv, C, nc, skew):
    """(head, first token, end token) of chunk c for workgroup x, from the rule above."""
    j = x % n_kv
    if skew and (c | 1) < nc:
        j ^= c & 1
        base = (c & ~1) * C
        mid = base + C + (skew if j % 2 == 0 else -skew)
        return (j, mid, base + 2 * C) if c & 1 else (j, base, mid)
    return j, c * C, (c + 1) * C


def expected_skew(chunk_arg, C, nc, n_kv):
    if chunk_arg != 0 or nc < 2 or n_kv % 2 or C % 32:
        return 0
    d = 32 * ((45 * C + 16000) // 32000)
    return d if d > 0 and C - d >= 32 else 0


def _check_spans(units, n_kv, C, nc, skew):
    b_units = units.shape[0]
    for x in range(b_units):
        i, c, s, j, lo, hi = (int(v) for v in units[x])
        assert (j, lo, hi) == expected_span(x, c, n_kv, C, nc, skew), (x, units[x])
        if skew and (c | 1) < nc:
            assert hi - lo == (C + skew if x % 2 == 0 else C - skew), (x, units[x])
    # per (sequence, head): the spans tile [0, nc * C)
    spans = {}
    for i, c, s, j, lo, hi in units.tolist():
        spans.setdefault((i, j), []).append((c, lo, hi))
    for key, v in spans.items():
        v.sort()
        assert [c for c, _, _ in v] == list(range(nc)), key
        assert v[0][1] == 0 and v[-1][2] == nc * C, key
        assert all(v[k][2] == v[k + 1][1] for k in range(nc - 1)), key


def _case(kvd, torch, lens, n_kv, chunk, max_ctx, g=2, d=64, even=False):
    b = len(lens)
    pool = kvd.allocate_pool(1, 1, n_kv, d)
    mb = max(1, -(-max_ctx // 16))
    q = torch.zeros((b, g * n_kv, d), dtype=torch.bfloat16, device="cuda")
    table = torch.zeros((b, mb), dtype=torch.int32, device="cuda")
    lens_t = torch.tensor(np.asarray(lens, dtype=np.int32), device="cuda")
    out = torch.empty_like(q)
    args = kvd.make_args(q, table, lens_t, max_ctx, out, chunk_tokens=chunk, pool=pool, even_chunks=even)
    ch, nc = kvd.kvd_decode_plan(pool, args)
    units = kvd.kvd_debug_unit_map(pool, args).cpu().numpy()
    return units, ch, nc


def _check(units, lens, n_kv, chunk, n_chunks, bound):
    order, s = expected_order(lens, chunk, n_chunks, bound)
    assert units.shape == (len(lens) * n_kv * n_chunks, 6)
    for j in range(n_kv):
        got = units[j::n_kv, :3]
        assert got.shape[0] == len(order)
        exp = np.array(order, dtype=np.int64).reshape(-1, 2)
        bad = np.nonzero((got[:, 0] != exp[:, 0]) | (got[:, 1] != exp[:, 1]))[0]
        assert bad.size == 0, f"head {j}: first mismatch at unit {bad[0]}: got {got[bad[0]]}, want {exp[bad[0]]}"
        assert np.array_equal(got[:, 2], s[exp[:, 0]])


CASES = [
    # (name, b, length range, n_kv, chunk, max_ctx)
    ("one sequence", 1, (0, 40000), 8, 0, 40000),
    ("one sequence, 80 chunks", 1, (1280, 1280), 2, 16, 1280),
    ("3 seqs, 69 chunks", 3, (1000, 1100), 2, 16, 1100),
    ("40 seqs, 69 chunks", 40, (0, 1100), 1, 16, 1100),
    ("64 seqs (one per lane)", 64, (0, 700), 2, 48, 700),
    ("65 seqs (two per lane)", 65, (0, 700), 2, 48, 700),
    ("512 seqs (eight per lane)", 512, (0, 300), 1, 16, 300),
    ("513 seqs (nine per lane)", 513, (0, 300), 1, 16, 300),
    ("600 seqs", 600, (0, 400), 2, 16, 400),
    ("600 seqs, 70 chunks", 600, (0, 1120), 1, 16, 1120),
    ("4095 seqs", 4095, (0, 200), 1, 16, 200),
    ("4200 seqs (more than 64 per lane)", 4200, (0, 200), 2, 16, 200),
    ("9000 seqs", 9000, (0, 100), 1, 32, 100),
    ("lengths above the bound", 100, (0, 5000), 1, 256, 3000),
    # automatic splits: uneven pairs (32 chunks; 2 chunks; 5 chunks, the last
    # without a partner), and none with an odd n_kv
    ("auto, one sequence, 8 heads", 1, (40000, 40000), 8, 0, 40000),
    ("auto, 64 seqs", 64, (0, 5000), 2, 0, 5000),
    ("auto, odd chunk count", 3, (1000, 5000), 2, 0, 5000),
    ("auto, one KV head", 2, (1000, 5000), 1, 0, 5000),
]


@pytest.mark.parametrize("name,b,rng_lens,n_kv,chunk,max_ctx", CASES, ids=[c[0] for c in CASES])
def test_unit_map_is_the_promised_order(env, name, b, rng_lens, n_kv, chunk, max_ctx):
    kvd, torch = env
    rng = np.random.default_rng(b * 7919 + max_ctx)
    lens = rng.integers(rng_lens[0], rng_lens[1] + 1, size=b)
    # empty, one-token and exactly-full sequences among them
    if b >= 4:
        lens[0], lens[1], lens[2] = 0, 1, min(max_ctx, 16 * (max(chunk, 16) // 16) * 2)
    units, ch, nc = _case(kvd, torch, lens, n_kv, chunk, max_ctx)
    _check(units, lens, n_kv, ch, nc, min(max_ctx, 16 * max(1, -(-max_ctx // 16))))
    _check_spans(units, n_kv, ch, nc, expected_skew(chunk, ch, nc, n_kv))


def test_even_chunks_flag_keeps_even_spans(env):
    """KVD_FLAG_EVEN_CHUNKS: an automatic split that would pair its chunks
    unevenly keeps [c*C, (c+1)*C) and head x % n_kv for every workgroup."""
    kvd, torch = env
    lens = np.full(3, 5000)
    units, ch, nc = _case(kvd, torch, lens, 2, 0, 5000, even=True)
    assert nc == 5 and expected_skew(0, ch, nc, 2) > 0          # uneven without the flag
    _check(units, lens, 2, ch, nc, 5000)
    _check_spans(units, 2, ch, nc, 0)
