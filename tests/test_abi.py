"""The C ABI on the host: exports, pool sizing, validation and planning (no GPU).

None of these calls reach a kernel launch: every argument error is detected on
the host first, and the pool / plan functions are pure host code.  Device
pointers are stand-in integers that are never dereferenced.
"""
import ctypes
import os
import re

import pytest

import decode_attention_paged_04_amd as kvd
from oracle import footprint

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 1 << 24            # 16-byte aligned stand-in for a device pointer


def header_symbols():
    inc = os.path.join(ROOT, "include")
    hdr = "".join(open(os.path.join(inc, f)).read() for f in sorted(os.listdir(inc)) if f.endswith(".h"))
    hdr = re.sub(r"/\*.*?\*/", "", hdr, flags=re.S)
    return sorted(set(re.findall(r"\b(kvd_[a-z0-9_]+)\s*\(", hdr)))


def test_every_declared_symbol_is_exported():
    syms = header_symbols()
    assert "kvd_decode_attn" in syms and "kvd_merge_partials" in syms
    lib = ctypes.CDLL(kvd.LIB_PATH)
    for s in syms:
        assert hasattr(lib, s), s
    assert set(syms) == set(kvd.EXPORTS), "binding and header disagree"


@pytest.mark.parametrize("layers,n_kv,d,dtype,per_token", [
    (32, 8, 128, kvd.KVD_BF16, 131072),        # Llama-3.1-8B, BF16
    (80, 8, 128, kvd.KVD_BF16, 327680),        # Llama-3(.1)-70B, BF16
    (32, 8, 128, kvd.KVD_FP8_E4M3, 65536),     # 8B with FP8 KV
])
def test_pool_bytes_per_token(layers, n_kv, d, dtype, per_token):
    kv, sc = kvd.kvd_pool_bytes(layers, 100, n_kv, d, dtype)
    assert kv / (100 * 16) == per_token
    w = 2 if dtype == kvd.KVD_BF16 else 1
    assert kv / (100 * 16) == footprint.kv_bytes_per_token(layers, n_kv, d, w)
    assert sc == (layers * 100 * n_kv * 2 * 4 if dtype == kvd.KVD_FP8_E4M3 else 0)


def _status(fn, *args):
    return getattr(kvd.lib, fn)(*args)


def _desc(**kw):
    base = dict(num_layers=2, num_blocks=64, block_size=16, n_kv=2, head_dim=128, dtype=kvd.KVD_BF16)
    base.update(kw)
    return kvd.PoolDesc(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(block_size=32), 2), (dict(head_dim=96), 2), (dict(head_dim=256), 2),
    (dict(num_layers=0), 1), (dict(num_blocks=0), 1), (dict(n_kv=0), 1), (dict(dtype=7), 1),
    (dict(num_blocks=1 << 18, n_kv=8), 2),         # one layer >= 4 GiB
])
def test_pool_desc_errors(kw, status):
    d = _desc(**kw)
    h = ctypes.c_void_p(0)
    assert _status("kvd_create_pool", ctypes.byref(d), FAKE, None, ctypes.byref(h)) == status
    assert not h.value


def test_create_pool_pointer_rules():
    h = ctypes.c_void_p(0)
    d = _desc()
    assert _status("kvd_create_pool", ctypes.byref(d), None, None, ctypes.byref(h)) == 1
    assert _status("kvd_create_pool", ctypes.byref(d), FAKE + 8, None, ctypes.byref(h)) == 1
    assert _status("kvd_create_pool", ctypes.byref(d), FAKE, FAKE, ctypes.byref(h)) == 1   # bf16 + scales
    d8 = _desc(dtype=kvd.KVD_FP8_E4M3)
    assert _status("kvd_create_pool", ctypes.byref(d8), FAKE, None, ctypes.byref(h)) == 1  # fp8, no scales
    assert _status("kvd_create_pool", ctypes.byref(d8), FAKE, FAKE, None) == 1
    assert _status("kvd_create_pool", ctypes.byref(d8), FAKE, FAKE, ctypes.byref(h)) == 0
    assert _status("kvd_destroy_pool", h) == 0
    assert _status("kvd_destroy_pool", None) == 1


def _pool(dtype=kvd.KVD_BF16, head_dim=128, n_kv=2):
    d = _desc(dtype=dtype, head_dim=head_dim, n_kv=n_kv)
    h = ctypes.c_void_p(0)
    assert _status("kvd_create_pool", ctypes.byref(d), FAKE,
                   FAKE if dtype == kvd.KVD_FP8_E4M3 else None, ctypes.byref(h)) == 0
    return kvd.Pool(d, None, None, h.value)


def _args(**kw):
    base = dict(b=2, n_q=8, max_blocks_per_seq=8, max_context_len=100, q=FAKE, block_table=FAKE,
                context_lens=FAKE, out=FAKE, lse_out=None, chunk_tokens=0, workspace=None,
                workspace_bytes=0, score=None, score_stride=0, score_weight=0.0)
    base.update(kw)
    return kvd.DecodeArgs(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(n_q=7), 1),                      # n_q not a multiple of n_kv
    (dict(n_q=34), 2),                     # g = 17 > 16
    (dict(chunk_tokens=24), 1),            # not a multiple of 16
    (dict(chunk_tokens=-16), 1),
    (dict(b=-1), 1), (dict(max_blocks_per_seq=0), 1), (dict(max_context_len=-5), 1),
    (dict(q=None), 1), (dict(block_table=None), 1), (dict(context_lens=None), 1), (dict(out=None), 1),
    (dict(score=FAKE, score_stride=50), 1),      # stride shorter than the context bound
    (dict(score=FAKE, score_stride=100, chunk_tokens=48), 1),   # scores need whole 32-token pairs
    (dict(chunk_tokens=16), 4),            # needs a workspace, none given
    (dict(chunk_tokens=16, workspace=FAKE, workspace_bytes=16), 4),
    (dict(chunk_tokens=16, workspace=FAKE + 16, workspace_bytes=1 << 30), 4),   # misaligned
    (dict(q=FAKE + 8), 1), (dict(out=FAKE + 4), 1),                            # misaligned vectors
    (dict(lse_out=FAKE + 2), 1), (dict(score=FAKE + 2, score_stride=100), 1),
    (dict(flags=2), 1), (dict(flags=1 << 31), 1),                            # unknown flag bits
])
def test_decode_argument_errors(kw, status):
    pool = _pool()
    a = _args(**kw)
    assert _status("kvd_decode_attn", pool.handle, 0, ctypes.byref(a), None) == status


def test_decode_dtype_and_layer_errors():
    bf, f8 = _pool(), _pool(kvd.KVD_FP8_E4M3)
    a = _args()
    assert _status("kvd_decode_attn_fp8", bf.handle, 0, ctypes.byref(a), None) == 3
    assert _status("kvd_decode_attn", f8.handle, 0, ctypes.byref(a), None) == 3
    assert _status("kvd_decode_attn", bf.handle, 2, ctypes.byref(a), None) == 1
    assert _status("kvd_decode_attn", bf.handle, -1, ctypes.byref(a), None) == 1
    assert _status("kvd_decode_attn", None, 0, ctypes.byref(a), None) == 1
    assert _status("kvd_decode_attn", bf.handle, 0, None, None) == 1
    # an empty batch is a valid no-op
    a0 = _args(b=0)
    assert _status("kvd_decode_attn", bf.handle, 0, ctypes.byref(a0), None) == 0


def test_partials_argument_errors():
    pool = _pool()
    a = _args()
    assert _status("kvd_decode_partials", pool.handle, 0, ctypes.byref(a), None, FAKE, None) == 1
    assert _status("kvd_decode_partials", pool.handle, 0, ctypes.byref(a), FAKE, None, None) == 1
    assert _status("kvd_decode_partials", pool.handle, 0, ctypes.byref(a), FAKE + 4, FAKE, None) == 1
    sa = _args(score=FAKE, score_stride=100)
    assert _status("kvd_decode_partials", pool.handle, 0, ctypes.byref(sa), FAKE, FAKE, None) == 1
    # works on either dtype; an empty batch is a no-op
    a0 = _args(b=0)
    assert _status("kvd_decode_partials", _pool(kvd.KVD_FP8_E4M3).handle, 0, ctypes.byref(a0), FAKE, FAKE, None) == 0


def test_binding_checks_shapes_before_any_call():
    import torch
    b, n_q, d = 2, 8, 128
    q = torch.zeros((b, n_q, d), dtype=torch.bfloat16)
    bt = torch.zeros((b, 4), dtype=torch.int32)
    lens = torch.zeros((b,), dtype=torch.int32)
    out = torch.zeros_like(q)
    with pytest.raises(ValueError, match="block_table"):
        kvd.make_args(q, torch.zeros((3, 4), dtype=torch.int32), lens, 64, out)
    with pytest.raises(ValueError, match="context_lens"):
        kvd.make_args(q, bt, torch.zeros((3,), dtype=torch.int32), 64, out)
    with pytest.raises(ValueError, match="out"):
        kvd.make_args(q, bt, lens, 64, torch.zeros((b, n_q, 64), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="q must be"):
        kvd.make_args(q.float(), bt, lens, 64, out)
    with pytest.raises(ValueError, match="lse_out"):
        kvd.make_args(q, bt, lens, 64, out, lse_out=torch.zeros((b, n_q + 1)))
    with pytest.raises(ValueError, match="score"):
        kvd.make_args(q, bt, lens, 64, out, score=torch.zeros((b + 1, 64)))
    with pytest.raises(ValueError, match="GPU"):         # host tensors never reach the library
        kvd.make_args(q, bt, lens, 64, out)
    with pytest.raises(ValueError, match="GPU"):         # the slot mapping is computed on the device
        kvd.kvd_slot_mapping(bt, lens)
    with pytest.raises(ValueError, match="block_table"):
        kvd.kvd_slot_mapping(bt[0], lens)


def test_slot_mapping_argument_errors():
    # (block_table, max_blocks, b, lens, first, out_start, max_tokens, slots, n_slots, stream)
    assert _status("kvd_slot_mapping", FAKE, 4, -1, FAKE, None, FAKE, 64, FAKE, 64, None) == 1
    assert _status("kvd_slot_mapping", FAKE, 0, 2, FAKE, None, FAKE, 64, FAKE, 64, None) == 1
    assert _status("kvd_slot_mapping", FAKE, 4, 2, FAKE, None, FAKE, -1, FAKE, 64, None) == 1
    assert _status("kvd_slot_mapping", FAKE, 4, 2, FAKE, None, FAKE, 64, FAKE, -1, None) == 1
    assert _status("kvd_slot_mapping", FAKE, 1 << 27, 2, FAKE, None, FAKE, 64, FAKE, 64, None) == 2
    assert _status("kvd_slot_mapping", FAKE, 1 << 20, 1 << 16, FAKE, None, FAKE, 1 << 16, FAKE, 64, None) == 2
    assert _status("kvd_slot_mapping", None, 4, 2, FAKE, None, FAKE, 64, FAKE, 64, None) == 1
    assert _status("kvd_slot_mapping", FAKE, 4, 2, None, None, FAKE, 64, FAKE, 64, None) == 1
    assert _status("kvd_slot_mapping", FAKE, 4, 2, FAKE, None, None, 64, FAKE, 64, None) == 1
    assert _status("kvd_slot_mapping", FAKE, 4, 2, FAKE, None, FAKE, 64, None, 64, None) == 1
    # nothing to do: no pointer is needed
    assert _status("kvd_slot_mapping", None, 4, 0, None, None, None, 64, None, 0, None) == 0
    assert _status("kvd_slot_mapping", None, 4, 2, None, None, None, 0, None, 0, None) == 0


def test_unit_map_argument_errors():
    pool = _pool()
    args = kvd.DecodeArgs(2, 8, 4, 64, FAKE, FAKE, FAKE, FAKE, None, 0, None, 0, None, 0, 0.0)
    assert _status("kvd_debug_unit_map", None, ctypes.byref(args), FAKE, None) == 1
    assert _status("kvd_debug_unit_map", pool.handle, None, FAKE, None) == 1
    assert _status("kvd_debug_unit_map", pool.handle, ctypes.byref(args), None, None) == 1
    bad = kvd.DecodeArgs(2, 7, 4, 64, FAKE, FAKE, FAKE, FAKE, None, 0, None, 0, None, 0, 0.0)
    assert _status("kvd_debug_unit_map", pool.handle, ctypes.byref(bad), FAKE, None) == 1
    empty = kvd.DecodeArgs(0, 8, 4, 64, None, None, None, None, None, 0, None, 0, None, 0, 0.0)
    assert _status("kvd_debug_unit_map", pool.handle, ctypes.byref(empty), None, None) == 0


def test_write_and_merge_argument_errors():
    pool = _pool()
    assert _status("kvd_write_kv", pool.handle, 5, FAKE, FAKE, FAKE, 4, None) == 1
    assert _status("kvd_write_kv", pool.handle, 0, FAKE, FAKE, FAKE, -1, None) == 1
    assert _status("kvd_write_kv", pool.handle, 0, None, FAKE, FAKE, 4, None) == 1
    assert _status("kvd_write_kv", pool.handle, 0, None, None, None, 0, None) == 0
    assert _status("kvd_merge_partials", FAKE, FAKE, 1, 4, 2, 96, FAKE, None, None) == 2
    assert _status("kvd_merge_partials", FAKE, FAKE, 1, 4, 0, 128, FAKE, None, None) == 1
    assert _status("kvd_merge_partials", None, FAKE, 1, 4, 2, 128, FAKE, None, None) == 1
    assert _status("kvd_merge_partials", None, None, 0, 4, 2, 128, None, None, None) == 0
    # misaligned: part_o (16 bytes), part_lse (4), out (8), lse_out (4)
    assert _status("kvd_merge_partials", FAKE + 4, FAKE, 1, 4, 2, 128, FAKE, None, None) == 1
    assert _status("kvd_merge_partials", FAKE, FAKE + 2, 1, 4, 2, 128, FAKE, None, None) == 1
    assert _status("kvd_merge_partials", FAKE, FAKE, 1, 4, 2, 128, FAKE + 2, None, None) == 1
    assert _status("kvd_merge_partials", FAKE, FAKE, 1, 4, 2, 128, FAKE, FAKE + 1, None) == 1
    assert _status("kvd_debug_fp8_decode", None, -1, None, None) == 1
    assert _status("kvd_debug_gather_offsets", pool.handle, 0, FAKE, 2, 1, 33, FAKE, FAKE, None) == 1


def _plan(pool, **kw):
    a = _args(**kw)
    c, n = kvd.kvd_decode_plan(pool, a)
    ws = kvd.kvd_decode_workspace_bytes(pool, a)
    return c, n, ws


def test_plan_and_workspace():
    pool = _pool()
    # forced chunks: ceil(100 / 32) = 4 chunks; partials b*n_q*4*(128+1) fp32,
    # each region 256-aligned
    c, n, ws = _plan(pool, chunk_tokens=32)
    assert (c, n) == (32, 4)
    po = 2 * 8 * 4 * 128 * 4
    pl = -(-(2 * 8 * 4 * 4) // 256) * 256
    assert ws == po + pl
    # one chunk and no score: no workspace
    c, n, ws = _plan(pool, chunk_tokens=0, max_context_len=100)
    assert n == 1 and ws == 0 and c >= 100
    # scores add the logit scratch and the lse buffer
    c, n, ws = _plan(pool, score=FAKE, score_stride=100)
    stride = (100 + 31) // 32 * 32 + 32
    assert ws == -(-(2 * 8 * stride * 4) // 256) * 256 + 256
    # the context bound is clamped by the block table width
    c, n, _ = _plan(pool, chunk_tokens=16, max_context_len=1000)
    assert n == 8


@pytest.mark.parametrize("b,n_kv,n_q,s,chunk", [(1, 8, 32, 32768, 1024), (4, 8, 64, 131072, 16384),
                                                 (32, 8, 32, 16384, 1024), (32, 8, 32, 32768, 2048)])
def test_auto_plan_fills_the_chip(b, n_kv, n_q, s, chunk):
    d = _desc(n_kv=n_kv, num_blocks=1024)
    h = ctypes.c_void_p(0)
    assert _status("kvd_create_pool", ctypes.byref(d), FAKE, None, ctypes.byref(h)) == 0
    pool = kvd.Pool(d, None, None, h.value)
    a = _args(b=b, n_q=n_q, max_context_len=s, max_blocks_per_seq=s // 16)
    c, n = kvd.kvd_decode_plan(pool, a)
    assert c % 16 == 0 and n == -(-s // c)
    assert c == chunk                   # the split measured best for these shapes
    assert b * n_kv * n >= 256          # at least one workgroup per compute unit


def test_mixed_decode_errors():
    p16, p8 = _pool(), _pool(kvd.KVD_FP8_E4M3)
    a = _args()
    f = kvd.lib.kvd_decode_attn_mixed
    assert f(p16.handle, p8.handle, 0, ctypes.byref(_args(score=FAKE, score_stride=100)), None) == 2   # no score
    assert f(p8.handle, p8.handle, 0, ctypes.byref(a), None) == 3          # first pool must be bf16
    assert f(p16.handle, p16.handle, 0, ctypes.byref(a), None) == 3        # second pool must be FP8
    assert f(p16.handle, _pool(kvd.KVD_FP8_E4M3, head_dim=64).handle, 0, ctypes.byref(a), None) == 1
    assert f(p16.handle, _pool(kvd.KVD_FP8_E4M3, n_kv=4).handle, 0, ctypes.byref(a), None) == 1
    assert f(p16.handle, None, 0, ctypes.byref(a), None) == 1
    assert f(p16.handle, p8.handle, 5, ctypes.byref(a), None) == 1         # layer out of range


def test_fused_append_errors():
    p16, p8 = _pool(), _pool(kvd.KVD_FP8_E4M3)
    a = _args()
    f = kvd.lib.kvd_decode_attn_append
    assert f(p16.handle, 0, ctypes.byref(a), None, FAKE, None) == 1        # new_k missing
    assert f(p8.handle, 0, ctypes.byref(a), FAKE, None, None) == 1         # new_v missing
    assert f(None, 0, ctypes.byref(a), FAKE, FAKE, None) == 1
    assert f(p16.handle, 5, ctypes.byref(a), FAKE, FAKE, None) == 1        # layer out of range
    assert f(p16.handle, 0, ctypes.byref(_args(chunk_tokens=8)), FAKE, FAKE, None) == 1


def test_launch_size_limits():
    """Grids of 256-work-item workgroups hold fewer than 2^32 work-items."""
    pool = _pool()                                   # n_kv = 2, d_h = 128
    big = _args(b=1 << 20, max_context_len=128, max_blocks_per_seq=8, chunk_tokens=16,
                workspace=FAKE, workspace_bytes=1 << 62)
    assert _status("kvd_decode_attn", pool.handle, 0, ctypes.byref(big), None) == 2    # 2^24 workgroups
    ok = _args(b=(1 << 20) - 1, max_context_len=128, max_blocks_per_seq=8, chunk_tokens=16)
    c, n = ctypes.c_int32(0), ctypes.c_int32(0)
    assert _status("kvd_decode_plan", pool.handle, ctypes.byref(ok), ctypes.byref(c), ctypes.byref(n)) == 0
    heads = _args(b=1 << 21, max_context_len=16, max_blocks_per_seq=1)              # b * n_q = 2^24
    assert _status("kvd_decode_attn", pool.handle, 0, ctypes.byref(heads), None) == 2
    assert _status("kvd_write_kv", pool.handle, 0, FAKE, FAKE, FAKE, 1 << 24, None) == 2   # 2^32 elements
    assert _status("kvd_merge_partials", FAKE, FAKE, 1 << 21, 8, 4, 128, FAKE, None, None) == 2


def test_stream_read_argument_errors():
    f = "kvd_debug_stream_read"
    assert _status(f, None, 1 << 20, FAKE, 512, None) == 1            # no data
    assert _status(f, FAKE, 1 << 20, None, 512, None) == 1            # no sink
    assert _status(f, FAKE, 1000, FAKE, 512, None) == 1               # not a multiple of 16
    assert _status(f, FAKE, 0, FAKE, 512, None) == 1                  # empty
    assert _status(f, FAKE + 8, 1 << 20, FAKE, 512, None) == 1        # misaligned
    assert _status(f, FAKE, 1 << 20, FAKE, 0, None) == 1              # no workgroups
    assert _status(f, FAKE, 1 << 20, FAKE, 65537, None) == 1          # too many
    assert _status(f, FAKE, 1 << 32, FAKE, 512, None) == 2            # beyond one buffer resource


def test_binding_refuses_host_tensors():
    """Every wrapper of a device-side call refuses host tensors before the
    library sees a pointer (a host address read by a kernel would fault)."""
    import torch
    pool = _pool()                                   # host handle over a stand-in address
    pool_t = kvd.Pool(pool.desc, torch.zeros(16, dtype=torch.uint8), None, None)
    k = torch.zeros((4, pool.desc.n_kv, pool.desc.head_dim), dtype=torch.bfloat16)
    slots = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU"):
        kvd.kvd_write_kv(pool_t, 0, k, k.clone(), slots)
    part_o = torch.zeros((1, 2, 3, 128))
    with pytest.raises(ValueError, match="GPU"):
        kvd.kvd_merge_partials(part_o, torch.zeros((1, 2, 3)), torch.zeros((1, 2, 128), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="GPU"):
        kvd.kvd_debug_fp8_decode(torch.zeros(8, dtype=torch.uint8), torch.zeros(8))
    with pytest.raises(ValueError, match="GPU"):
        kvd.kvd_debug_gather_offsets(pool_t, 0, torch.zeros((1, 2), dtype=torch.int32), 32,
                                     torch.zeros((1, pool.desc.n_kv, 32), dtype=torch.int64),
                                     torch.zeros((1, pool.desc.n_kv, 32), dtype=torch.int64))
    with pytest.raises(ValueError, match="GPU"):
        kvd.kvd_debug_stream_read(torch.zeros(64, dtype=torch.uint8), torch.zeros(256, dtype=torch.int32), 1)
