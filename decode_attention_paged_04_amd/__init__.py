"""Python binding of libkvdecode (paged GQA decode attention for MI355X).

Argument marshalling only: every step of the decode path runs in the HIP
kernels of ``libkvdecode.so``.  PyTorch supplies device memory and streams.
The functions keep the C names; see ``include/kvdecode.h`` for the layout,
ownership and error rules.  Importing this package fails if the library has
not been built (``python decode_attention_paged_04_amd/build.py``).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvdecode.so")

BLOCK_SIZE = 16
KVD_BF16, KVD_FP8_E4M3 = 0, 1
KVD_FLAG_EVEN_CHUNKS = 1
STATUS = {0: "KVD_OK", 1: "KVD_ERR_INVALID_ARG", 2: "KVD_ERR_UNSUPPORTED", 3: "KVD_ERR_DTYPE",
          4: "KVD_ERR_WORKSPACE", 5: "KVD_ERR_HIP", 6: "KVD_ERR_CAPACITY"}
KVD_ERR_CAPACITY = 6


class KvdError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        super().__init__(f"{where}: {STATUS.get(status, status)}" + (f" ({detail})" if detail else ""))
        self.status = status


class PoolDesc(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("n_kv", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int)]


class DecodeArgs(ctypes.Structure):
    _fields_ = [("b", ctypes.c_int32), ("n_q", ctypes.c_int32),
                ("max_blocks_per_seq", ctypes.c_int32), ("max_context_len", ctypes.c_int32),
                ("q", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("context_lens", ctypes.c_void_p), ("out", ctypes.c_void_p),
                ("lse_out", ctypes.c_void_p), ("chunk_tokens", ctypes.c_int32),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("score", ctypes.c_void_p), ("score_stride", ctypes.c_int32),
                ("score_weight", ctypes.c_float), ("flags", ctypes.c_uint32)]


EXPORTS = {
    "kvd_pool_bytes": (ctypes.POINTER(PoolDesc), ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)),
    "kvd_create_pool": (ctypes.POINTER(PoolDesc), ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p)),
    "kvd_destroy_pool": (ctypes.c_void_p,),
    "kvd_write_kv": (ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                     ctypes.c_int32, ctypes.c_void_p),
    "kvd_slot_mapping": (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                         ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p),
    "kvd_decode_plan": (ctypes.c_void_p, ctypes.POINTER(DecodeArgs), ctypes.POINTER(ctypes.c_int32),
                        ctypes.POINTER(ctypes.c_int32)),
    "kvd_decode_workspace_bytes": (ctypes.c_void_p, ctypes.POINTER(DecodeArgs), ctypes.POINTER(ctypes.c_size_t)),
    "kvd_decode_attn": (ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(DecodeArgs), ctypes.c_void_p),
    "kvd_decode_attn_fp8": (ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(DecodeArgs), ctypes.c_void_p),
    "kvd_decode_attn_mixed": (ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(DecodeArgs),
                              ctypes.c_void_p),
    "kvd_decode_attn_append": (ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(DecodeArgs), ctypes.c_void_p,
                               ctypes.c_void_p, ctypes.c_void_p),
    "kvd_decode_attn_no_alloc": (ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(DecodeArgs), ctypes.c_void_p),
    "kvd_decode_partials": (ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(DecodeArgs), ctypes.c_void_p,
                            ctypes.c_void_p, ctypes.c_void_p),
    "kvd_merge_partials": (ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                           ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p),
    "kvd_status_string": (ctypes.c_int,),
    "kvd_last_hip_error": (),
    "kvd_debug_gather_offsets": (ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                                 ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_void_p),
    "kvd_debug_unit_map": (ctypes.c_void_p, ctypes.POINTER(DecodeArgs), ctypes.c_void_p, ctypes.c_void_p),
    "kvd_debug_fp8_decode": (ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p),
    "kvd_debug_stream_read": (ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p),
    # host block bookkeeping (kvblocks.h)
    "kvd_bm_create": (ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_void_p)),
    "kvd_bm_destroy": (ctypes.c_void_p,),
    "kvd_bm_add_sequence": (ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_int64),
                            ctypes.POINTER(ctypes.c_int32)),
    "kvd_bm_append": (ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p),
    "kvd_bm_slots": (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p),
    "kvd_bm_length": (ctypes.c_void_p, ctypes.c_int64, ctypes.POINTER(ctypes.c_int32)),
    "kvd_bm_block_table": (ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32,
                           ctypes.POINTER(ctypes.c_int32)),
    "kvd_bm_fill_tables": (ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                           ctypes.c_void_p),
    "kvd_bm_free_sequence": (ctypes.c_void_p, ctypes.c_int64),
    "kvd_bm_counts": (ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32),
                      ctypes.POINTER(ctypes.c_int32)),
    "kvd_bm_refcount": (ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)),
    "kvd_tier_block_scores": (ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p),
    "kvd_tier_plan": (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                      ctypes.c_int32, ctypes.c_void_p),
    "kvd_tier_restrict": (ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p),
    "kvd_mixed_row": (ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                      ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32),
                      ctypes.POINTER(ctypes.c_int32)),
}


def _load():
    # PyTorch's ROCm build carries its own HIP runtime (libamdhip64.so, same
    # soname as the system's).  Importing torch first makes the library's
    # libamdhip64.so.7 dependency resolve to that already-loaded runtime, so
    # the process holds one HIP runtime; loading the library first would map a
    # second one beside torch's, and the second runtime to touch the device can
    # fail with hipErrorNoDevice.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python decode_attention_paged_04_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, argtypes in EXPORTS.items():
        fn = getattr(lib, name)
        fn.argtypes = list(argtypes)
        fn.restype = ctypes.c_char_p if name in ("kvd_status_string", "kvd_last_hip_error") else ctypes.c_int
    return lib


lib = _load()


def _check(st: int, where: str):
    if st != 0:
        detail = lib.kvd_last_hip_error().decode() if st == 5 else ""
        raise KvdError(st, where, detail)


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return int(stream)
    import torch
    if torch.cuda.is_available():
        return int(torch.cuda.current_stream().cuda_stream)
    return None


def kvd_pool_bytes(num_layers: int, num_blocks: int, n_kv: int, head_dim: int,
                   dtype: int = KVD_BF16, block_size: int = BLOCK_SIZE):
    d = PoolDesc(num_layers, num_blocks, block_size, n_kv, head_dim, dtype)
    kv, sc = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(lib.kvd_pool_bytes(ctypes.byref(d), ctypes.byref(kv), ctypes.byref(sc)), "kvd_pool_bytes")
    return kv.value, sc.value


class Pool:
    """Host handle over a caller-owned pool (``kv`` and, for FP8, ``scales``)."""

    def __init__(self, desc: PoolDesc, kv, scales, handle: int):
        self.desc, self.kv, self.scales, self.handle = desc, kv, scales, handle

    @property
    def fp8(self) -> bool:
        return self.desc.dtype == KVD_FP8_E4M3

    def __del__(self):
        h = getattr(self, "handle", None)
        if h and lib is not None:          # at interpreter exit the module may be gone
            lib.kvd_destroy_pool(h)
            self.handle = None


def kvd_create_pool(num_layers: int, num_blocks: int, n_kv: int, head_dim: int, kv, scales=None,
                    dtype: int = KVD_BF16, block_size: int = BLOCK_SIZE) -> Pool:
    """Wrap device buffers ``kv`` (and ``scales`` for FP8) as a pool."""
    d = PoolDesc(num_layers, num_blocks, block_size, n_kv, head_dim, dtype)
    h = ctypes.c_void_p(0)
    _check(lib.kvd_create_pool(ctypes.byref(d), _ptr(kv), _ptr(scales), ctypes.byref(h)), "kvd_create_pool")
    return Pool(d, kv, scales, h.value)


def allocate_pool(num_layers: int, num_blocks: int, n_kv: int, head_dim: int,
                  dtype: int = KVD_BF16, device="cuda") -> Pool:
    """Allocate the pool's memory with torch and create the handle."""
    import torch
    kv_bytes, sc_bytes = kvd_pool_bytes(num_layers, num_blocks, n_kv, head_dim, dtype)
    kv = torch.empty(kv_bytes, dtype=torch.uint8, device=device)
    sc = torch.zeros(sc_bytes // 4, dtype=torch.float32, device=device) if sc_bytes else None
    return kvd_create_pool(num_layers, num_blocks, n_kv, head_dim, kv, sc, dtype)


def kvd_write_kv(pool: Pool, layer: int, k, v, slot_mapping, stream=None):
    """Store bf16 ``k``/``v`` ``[n_tok][n_kv][head_dim]`` at ``slot_mapping`` (int32)."""
    import torch
    n = int(slot_mapping.numel())
    shape = (n, pool.desc.n_kv, pool.desc.head_dim)
    _check_tensor(slot_mapping, "slot_mapping", (n,), torch.int32)
    _check_tensor(k, "k", shape, torch.bfloat16, slot_mapping.device)
    _check_tensor(v, "v", shape, torch.bfloat16, slot_mapping.device)
    _require_gpu(slot_mapping, "slot_mapping")
    _require(pool.kv.device == slot_mapping.device, "the pool and the new rows must share a device")
    _check(lib.kvd_write_kv(pool.handle, layer, _ptr(k), _ptr(v), _ptr(slot_mapping), n, _stream(stream)),
           "kvd_write_kv")


def kvd_slot_mapping(block_table, context_lens, first_token=None, stream=None):
    """Slot mapping of kvd_write_kv for tokens ``first_token[i] .. context_lens[i] - 1``
    of every sequence (all tokens when ``first_token`` is None), packed in
    sequence order; computed on the device by the library.  ``block_table``
    int32 ``[b][max_blocks]``, ``context_lens`` and ``first_token`` int32 ``[b]``,
    all on one GPU.  Returns int32 ``[n]`` on that device."""
    import torch
    _require(block_table is not None and block_table.dim() == 2, "block_table must be [b][max_blocks]")
    b, mb = (int(x) for x in block_table.shape)
    dev = block_table.device
    _check_tensor(block_table, "block_table", (b, mb), torch.int32)
    _require_gpu(block_table, "block_table")
    _check_tensor(context_lens, "context_lens", (b,), torch.int32, dev)
    if first_token is not None:
        _check_tensor(first_token, "first_token", (b,), torch.int32, dev)
    lens = context_lens.to(torch.int64)
    first = first_token.to(torch.int64) if first_token is not None else torch.zeros_like(lens)
    lh, fh = lens.cpu(), first.cpu()
    _require(bool(((lh >= 0) & (lh <= BLOCK_SIZE * mb)).all()), "context longer than its block-table row")
    _require(bool(((fh >= 0) & (fh <= lh)).all()), "first_token must lie in [0, context_lens]")
    counts = lens - first
    start = torch.cumsum(counts, 0) - counts if b else counts
    n = int((lh - fh).sum())
    slots = torch.empty(n, dtype=torch.int32, device=dev)
    max_tok = int((lh - fh).max()) if b else 0
    _check(lib.kvd_slot_mapping(_ptr(block_table), mb, b, _ptr(context_lens),
                                _ptr(first_token), _ptr(start), max_tok, _ptr(slots), n, _stream(stream)),
           "kvd_slot_mapping")
    return slots


def _require(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _require_gpu(t, name: str):
    """The library takes device pointers only: a host tensor never reaches it."""
    _require(t.is_cuda, f"{name} must be on a GPU (the library reads device memory only)")


def _check_tensor(t, name: str, shape, dtype, device=None):
    import torch
    _require(t is not None, f"{name} is required")
    _require(isinstance(t, torch.Tensor), f"{name} must be a torch tensor")
    _require(t.dtype == dtype, f"{name} must be {dtype}, got {t.dtype}")
    _require(t.is_contiguous(), f"{name} must be contiguous")
    _require(tuple(t.shape) == tuple(shape), f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if device is not None:
        _require(t.device == device, f"{name} must be on {device}, got {t.device}")


def make_args(q, block_table, context_lens, max_context_len: int, out, lse_out=None,
              chunk_tokens: int = 0, workspace=None, score=None, score_weight: float = 0.0,
              pool: Optional["Pool"] = None, need_out: bool = True, even_chunks: bool = False) -> DecodeArgs:
    """Check every tensor against the others (and the pool) and pack the C struct.

    The C library sees raw pointers only, so this is where sizes are enforced:
    q ``[b][n_q][d]`` bf16, block_table ``[b][max_blocks]`` int32, context_lens
    ``[b]`` int32, out like q, lse_out ``[b][n_q]`` fp32, score ``[b][stride]`` fp32,
    all contiguous and on q's device.  ``even_chunks`` sets KVD_FLAG_EVEN_CHUNKS.
    """
    import torch
    _require(q is not None and q.dim() == 3, "q must be [b][n_q][head_dim]")
    b, n_q, d = (int(x) for x in q.shape)
    dev = q.device
    _check_tensor(q, "q", (b, n_q, d), torch.bfloat16)
    _require(block_table is not None and block_table.dim() == 2, "block_table must be [b][max_blocks]")
    _check_tensor(block_table, "block_table", (b, int(block_table.shape[1])), torch.int32, dev)
    _check_tensor(context_lens, "context_lens", (b,), torch.int32, dev)
    if need_out or out is not None:
        _check_tensor(out, "out", (b, n_q, d), torch.bfloat16, dev)
    if lse_out is not None:
        _check_tensor(lse_out, "lse_out", (b, n_q), torch.float32, dev)
    if score is not None:
        _require(score.dim() == 2, "score must be [b][stride]")
        _check_tensor(score, "score", (b, int(score.shape[1])), torch.float32, dev)
    if workspace is not None:
        _require(workspace.is_contiguous() and workspace.device == dev, "workspace must be contiguous on q's device")
    if pool is not None:
        _require(d == pool.desc.head_dim, f"q head_dim {d} != pool head_dim {pool.desc.head_dim}")
        _require(pool.kv.device == dev, "pool and q must share a device")
    _require(dev.type == "cuda", "tensors must be on a GPU")
    return DecodeArgs(
        b, n_q, int(block_table.shape[1]), int(max_context_len),
        _ptr(q), _ptr(block_table), _ptr(context_lens), _ptr(out), _ptr(lse_out), int(chunk_tokens),
        _ptr(workspace), int(workspace.numel() * workspace.element_size()) if workspace is not None else 0,
        _ptr(score), int(score.shape[1]) if score is not None else 0, float(score_weight),
        KVD_FLAG_EVEN_CHUNKS if even_chunks else 0)


def kvd_decode_plan(pool: Pool, args: DecodeArgs):
    c, n = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(lib.kvd_decode_plan(pool.handle, ctypes.byref(args), ctypes.byref(c), ctypes.byref(n)),
           "kvd_decode_plan")
    return c.value, n.value


def kvd_decode_workspace_bytes(pool: Pool, args: DecodeArgs) -> int:
    n = ctypes.c_size_t(0)
    _check(lib.kvd_decode_workspace_bytes(pool.handle, ctypes.byref(args), ctypes.byref(n)),
           "kvd_decode_workspace_bytes")
    return n.value


def allocate_workspace(pool: Pool, args: DecodeArgs, device="cuda"):
    import torch
    n = kvd_decode_workspace_bytes(pool, args)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device=device) if n else None
    if ws is not None:
        args.workspace, args.workspace_bytes = _ptr(ws), n
    return ws


def kvd_decode_attn(pool: Pool, layer: int, args: DecodeArgs, stream=None):
    _check(lib.kvd_decode_attn(pool.handle, layer, ctypes.byref(args), _stream(stream)), "kvd_decode_attn")


def kvd_decode_attn_fp8(pool: Pool, layer: int, args: DecodeArgs, stream=None):
    _check(lib.kvd_decode_attn_fp8(pool.handle, layer, ctypes.byref(args), _stream(stream)),
           "kvd_decode_attn_fp8")


def kvd_decode_attn_append(pool: Pool, layer: int, args: DecodeArgs, new_k, new_v, stream=None):
    """Store token s_i - 1 of every sequence (bf16 ``new_k``/``new_v``
    ``[b][n_kv][head_dim]``) and decode, in one launch (bf16 or FP8 pool)."""
    import torch
    shape = (int(args.b), pool.desc.n_kv, pool.desc.head_dim)
    _check_tensor(new_k, "new_k", shape, torch.bfloat16)
    _require(new_k.is_cuda, "new_k must be on the GPU")
    _check_tensor(new_v, "new_v", shape, torch.bfloat16, new_k.device)
    _check(lib.kvd_decode_attn_append(pool.handle, layer, ctypes.byref(args), _ptr(new_k), _ptr(new_v),
                                      _stream(stream)), "kvd_decode_attn_append")


def kvd_decode_attn_no_alloc(pool: Pool, layer: int, args: DecodeArgs, stream=None):
    """kvd_decode_attn (bf16 or FP8 pool) with the library's fixed per-device
    scratch instead of ``args.workspace``: allocates nothing."""
    _check(lib.kvd_decode_attn_no_alloc(pool.handle, layer, ctypes.byref(args), _stream(stream)),
           "kvd_decode_attn_no_alloc")


def kvd_decode_attn_mixed(pool_bf16: Pool, pool_fp8: Pool, layer: int, args: DecodeArgs, stream=None):
    """Decode over bf16 blocks of ``pool_bf16`` and FP8 blocks of ``pool_fp8``
    (table entries of FP8 blocks carry bit 30; see kvd_mixed_row)."""
    _require(pool_fp8.desc.n_kv == pool_bf16.desc.n_kv and pool_fp8.desc.head_dim == pool_bf16.desc.head_dim,
             "the two pools differ in shape")
    _require(pool_fp8.kv.device == pool_bf16.kv.device, "the two pools must share a device")
    _check(lib.kvd_decode_attn_mixed(pool_bf16.handle, pool_fp8.handle, layer, ctypes.byref(args),
                                     _stream(stream)), "kvd_decode_attn_mixed")


def decode_mixed(pool_bf16: Pool, pool_fp8: Pool, layer: int, q, block_table, context_lens,
                 max_context_len: int, out=None, lse_out=None, chunk_tokens: int = 0, workspace=None,
                 stream=None, even_chunks: bool = False):
    """Convenience: allocate out/workspace as needed and run one mixed-precision decode."""
    import torch
    if out is None:
        out = torch.empty_like(q)
    args = make_args(q, block_table, context_lens, max_context_len, out, lse_out, chunk_tokens,
                     workspace, pool=pool_bf16, even_chunks=even_chunks)
    ws = workspace if workspace is not None else allocate_workspace(pool_bf16, args, device=q.device)
    kvd_decode_attn_mixed(pool_bf16, pool_fp8, layer, args, stream)
    return out, ws


def kvd_decode_partials(pool: Pool, layer: int, q, block_table, context_lens, max_context_len: int,
                        part_o=None, part_lse=None, chunk_tokens: int = 0, stream=None,
                        even_chunks: bool = False):
    """Per-chunk partials (fp32 o_c ``[b][n_q][n_chunks][d]``, lse_c ``[b][n_q][n_chunks]``).

    Allocates the partial buffers when not given; returns ``(part_o, part_lse, chunk, n_chunks)``.
    """
    import torch
    b, n_q, d = (int(x) for x in q.shape)
    args = make_args(q, block_table, context_lens, max_context_len, None, chunk_tokens=chunk_tokens,
                     pool=pool, need_out=False, even_chunks=even_chunks)
    chunk, nc = kvd_decode_plan(pool, args)
    if part_o is None:
        part_o = torch.empty((b, n_q, nc, d), dtype=torch.float32, device=q.device)
    if part_lse is None:
        part_lse = torch.empty((b, n_q, nc), dtype=torch.float32, device=q.device)
    _check_tensor(part_o, "part_o", (b, n_q, nc, d), torch.float32, q.device)
    _check_tensor(part_lse, "part_lse", (b, n_q, nc), torch.float32, q.device)
    _check(lib.kvd_decode_partials(pool.handle, layer, ctypes.byref(args), _ptr(part_o), _ptr(part_lse),
                                   _stream(stream)), "kvd_decode_partials")
    return part_o, part_lse, chunk, nc


def kvd_merge_partials(part_o, part_lse, out, lse_out=None, stream=None):
    """part_o fp32 ``[b][n_q][n_chunks][d]``, part_lse ``[b][n_q][n_chunks]`` -> out bf16."""
    import torch
    b, n_q, nc, d = (int(x) for x in part_o.shape)
    _check_tensor(part_o, "part_o", (b, n_q, nc, d), torch.float32)
    _check_tensor(part_lse, "part_lse", (b, n_q, nc), torch.float32, part_o.device)
    _check_tensor(out, "out", (b, n_q, d), torch.bfloat16, part_o.device)
    _require_gpu(part_o, "part_o")
    if lse_out is not None:
        _check_tensor(lse_out, "lse_out", (b, n_q), torch.float32, part_o.device)
    _check(lib.kvd_merge_partials(_ptr(part_o), _ptr(part_lse), b, n_q, nc, d, _ptr(out), _ptr(lse_out),
                                  _stream(stream)), "kvd_merge_partials")


def kvd_status_string(status: int) -> str:
    return lib.kvd_status_string(status).decode()


def kvd_debug_gather_offsets(pool: Pool, layer: int, block_table, n_tok: int, out_k, out_v, stream=None):
    import torch
    b, mb = (int(x) for x in block_table.shape)
    _check_tensor(block_table, "block_table", (b, mb), torch.int32)
    _check_tensor(out_k, "out_k", (b, pool.desc.n_kv, n_tok), torch.int64, block_table.device)
    _check_tensor(out_v, "out_v", (b, pool.desc.n_kv, n_tok), torch.int64, block_table.device)
    _require_gpu(block_table, "block_table")
    _check(lib.kvd_debug_gather_offsets(pool.handle, layer, _ptr(block_table), mb, b, n_tok, _ptr(out_k),
                                        _ptr(out_v), _stream(stream)), "kvd_debug_gather_offsets")


def kvd_debug_unit_map(pool: Pool, args: DecodeArgs, device="cuda", stream=None):
    """(sequence, chunk, clamped length, KV head, first token, end token) of
    every workgroup of a decode launch with ``args``, int32 ``[grid][6]``."""
    import torch
    _, nc = kvd_decode_plan(pool, args)
    units = torch.full((int(args.b) * pool.desc.n_kv * nc, 6), -7, dtype=torch.int32, device=device)
    _check(lib.kvd_debug_unit_map(pool.handle, ctypes.byref(args), _ptr(units), _stream(stream)),
           "kvd_debug_unit_map")
    return units


def kvd_debug_fp8_decode(codes, out, stream=None):
    import torch
    _check_tensor(codes, "codes", (int(codes.numel()),), torch.uint8)
    _check_tensor(out, "out", (int(codes.numel()),), torch.float32, codes.device)
    _require_gpu(codes, "codes")
    _check(lib.kvd_debug_fp8_decode(_ptr(codes), int(codes.numel()), _ptr(out), _stream(stream)),
           "kvd_debug_fp8_decode")


def kvd_debug_stream_read(data, sink, grid: int, stream=None):
    """Stream-read every byte of ``data`` (a contiguous device tensor, a
    multiple of 16 bytes) with the decode kernels' loads; ``sink``: uint32
    ``[grid * 256]``, the per-work-item XOR of the words read."""
    import torch
    nbytes = int(data.numel()) * data.element_size()
    _require(data.is_contiguous(), "data must be contiguous")
    _require_gpu(data, "data")
    _check_tensor(sink, "sink", (int(grid) * 256,), torch.int32, data.device)
    _check(lib.kvd_debug_stream_read(_ptr(data), nbytes, _ptr(sink), int(grid), _stream(stream)),
           "kvd_debug_stream_read")


def decode(pool: Pool, layer: int, q, block_table, context_lens, max_context_len: int, out=None,
           lse_out=None, chunk_tokens: int = 0, score=None, score_weight: float = 0.0,
           workspace=None, stream=None, new_k=None, new_v=None, even_chunks: bool = False):
    """Convenience: allocate out/workspace as needed and run one decode call
    (with ``new_k``/``new_v``: the fused append of token s_i - 1 first)."""
    import torch
    if out is None:
        out = torch.empty_like(q)
    args = make_args(q, block_table, context_lens, max_context_len, out, lse_out, chunk_tokens,
                     workspace, score, score_weight, pool=pool, even_chunks=even_chunks)
    ws = workspace
    if ws is None:
        ws = allocate_workspace(pool, args, device=q.device)
    if new_k is not None or new_v is not None:
        _require(new_k is not None and new_v is not None, "new_k and new_v go together")
        kvd_decode_attn_append(pool, layer, args, new_k, new_v, stream)
    else:
        (kvd_decode_attn_fp8 if pool.fp8 else kvd_decode_attn)(pool, layer, args, stream)
    return out, ws


# ---------------------------------------------------------------- block bookkeeping
def _i32(values):
    """Host int32 array (numpy) and its address."""
    import numpy as np
    a = np.ascontiguousarray(np.asarray(values, dtype=np.int32))
    return a, a.ctypes.data


class BlockManager:
    """Host block bookkeeping of a paged pool (kvblocks.h): free list, reference
    counts, on-demand growth and, optionally, the prefix cache.  Marshalling
    only; every decision is made by the native library."""

    def __init__(self, num_blocks: int, prefix_cache: bool = False):
        h = ctypes.c_void_p()
        _check(lib.kvd_bm_create(int(num_blocks), 1 if prefix_cache else 0, ctypes.byref(h)), "kvd_bm_create")
        self.handle = h.value
        self.num_blocks = int(num_blocks)

    def __del__(self):
        if getattr(self, "handle", None) and lib is not None:
            lib.kvd_bm_destroy(self.handle)
            self.handle = None

    def add_sequence(self, n_tokens: int, tokens=None):
        """Returns (sequence id, number of leading prompt tokens already cached)."""
        sid, cached = ctypes.c_int64(), ctypes.c_int32()
        if tokens is not None:
            arr, ptr = _i32(tokens)
            _require(arr.shape == (n_tokens,), "tokens must hold n_tokens ids")
        else:
            arr, ptr = None, None
        _check(lib.kvd_bm_add_sequence(self.handle, ptr, int(n_tokens), ctypes.byref(sid), ctypes.byref(cached)),
               "kvd_bm_add_sequence")
        return sid.value, cached.value

    def append(self, seq_id: int, n: int = 1, tokens=None):
        """Append n tokens; returns their slots (the slot mapping of kvd_write_kv)."""
        import numpy as np
        slots = np.zeros(max(n, 1), dtype=np.int32)
        if tokens is not None:
            arr, ptr = _i32(tokens)
            _require(arr.shape == (n,), "tokens must hold n ids")
        else:
            arr, ptr = None, None
        _check(lib.kvd_bm_append(self.handle, int(seq_id), ptr, int(n), slots.ctypes.data), "kvd_bm_append")
        return [int(x) for x in slots[:n]]

    def slots(self, seq_id: int, first: int, n: int):
        import numpy as np
        out = np.zeros(max(n, 1), dtype=np.int32)
        _check(lib.kvd_bm_slots(self.handle, int(seq_id), int(first), int(n), out.ctypes.data), "kvd_bm_slots")
        return [int(x) for x in out[:n]]

    def length(self, seq_id: int) -> int:
        n = ctypes.c_int32()
        _check(lib.kvd_bm_length(self.handle, int(seq_id), ctypes.byref(n)), "kvd_bm_length")
        return n.value

    def table(self, seq_id: int):
        import numpy as np
        n = ctypes.c_int32()
        cap = -(-self.length(seq_id) // BLOCK_SIZE)
        out = np.zeros(max(cap, 1), dtype=np.int32)
        _check(lib.kvd_bm_block_table(self.handle, int(seq_id), out.ctypes.data, cap, ctypes.byref(n)),
               "kvd_bm_block_table")
        return [int(x) for x in out[:n.value]]

    def fill_tables(self, seq_ids, max_blocks: int):
        """(block table int32 [b][max_blocks] padded with -1, context lengths int32 [b]) as numpy."""
        import numpy as np
        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64))
        b = int(ids.shape[0])
        table = np.full((max(b, 1), max_blocks), -1, dtype=np.int32)
        lens = np.zeros(max(b, 1), dtype=np.int32)
        _check(lib.kvd_bm_fill_tables(self.handle, ids.ctypes.data, b, table.ctypes.data, int(max_blocks),
                                      lens.ctypes.data), "kvd_bm_fill_tables")
        return table[:b], lens[:b]

    def free_sequence(self, seq_id: int):
        _check(lib.kvd_bm_free_sequence(self.handle, int(seq_id)), "kvd_bm_free_sequence")

    def counts(self):
        """(free, cached but unused, used) block counts."""
        f, c, u = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check(lib.kvd_bm_counts(self.handle, ctypes.byref(f), ctypes.byref(c), ctypes.byref(u)), "kvd_bm_counts")
        return f.value, c.value, u.value

    def refcount(self, block: int) -> int:
        r = ctypes.c_int32()
        _check(lib.kvd_bm_refcount(self.handle, int(block), ctypes.byref(r)), "kvd_bm_refcount")
        return r.value


# ---------------------------------------------------------------- tiers
KVD_TIER_T0, KVD_TIER_T1, KVD_TIER_T3 = 0, 1, 3


def tier_block_scores(token_scores):
    """Per-block sums (float64 numpy) of one sequence's token scores (host fp32)."""
    import numpy as np
    ts = np.ascontiguousarray(np.asarray(token_scores, dtype=np.float32))
    n = int(ts.shape[0])
    out = np.zeros(max(-(-n // BLOCK_SIZE), 1), dtype=np.float64)
    _check(lib.kvd_tier_block_scores(ts.ctypes.data, n, out.ctypes.data), "kvd_tier_block_scores")
    return out[:-(-n // BLOCK_SIZE)]


def tier_plan(block_scores, protect_first: int, protect_last: int, t0_blocks: int, t1_blocks: int):
    """Tier (KVD_TIER_*) of every block, int8 numpy."""
    import numpy as np
    sc = np.ascontiguousarray(np.asarray(block_scores, dtype=np.float64))
    nb = int(sc.shape[0])
    out = np.zeros(max(nb, 1), dtype=np.int8)
    _check(lib.kvd_tier_plan(sc.ctypes.data, nb, int(protect_first), int(protect_last), int(t0_blocks),
                             int(t1_blocks), out.ctypes.data), "kvd_tier_plan")
    return out[:nb]


def tier_restrict(table_row, tiers):
    """The block-table row of a decode over T0 and T1 (T3 entries become -1)."""
    import numpy as np
    row = np.ascontiguousarray(np.asarray(table_row, dtype=np.int32))
    t = np.ascontiguousarray(np.asarray(tiers, dtype=np.int8))
    _require(row.shape == t.shape, "table row and tiers differ in length")
    out = np.zeros(max(row.shape[0], 1), dtype=np.int32)
    _check(lib.kvd_tier_restrict(row.ctypes.data, t.ctypes.data, int(row.shape[0]), out.ctypes.data),
           "kvd_tier_restrict")
    return out[:row.shape[0]]


# ---------------------------------------------------------------- mixed precision
PRECISION_BIT = 1 << 30


def mixed_row(ids_bf16, ids_fp8, fp8_last: bool, tail_tokens: int):
    """(row int32 numpy, context length) of one sequence for kvd_decode_attn_mixed."""
    import numpy as np
    a = np.ascontiguousarray(np.asarray(ids_bf16, dtype=np.int32))
    b = np.ascontiguousarray(np.asarray(ids_fp8, dtype=np.int32))
    cap = int(a.shape[0] + b.shape[0] + 1)
    row = np.zeros(cap, dtype=np.int32)
    n, s = ctypes.c_int32(), ctypes.c_int32()
    _check(lib.kvd_mixed_row(a.ctypes.data, int(a.shape[0]), b.ctypes.data, int(b.shape[0]), 1 if fp8_last else 0,
                             int(tail_tokens), row.ctypes.data, cap, ctypes.byref(n), ctypes.byref(s)),
           "kvd_mixed_row")
    return row[:n.value], s.value
