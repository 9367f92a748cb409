// C ABI of libkvdecode: validation, pool layout, launch planning, workspace.
#include <atomic>
#include <cstdio>
#include <mutex>
#include <new>

#include "kvd_internal.h"

struct kvd_pool {
  kvd::PoolView v;
};

namespace {

using kvd::DecodePlan;
using kvd::PoolView;

// Automatic split of the context into chunks (one workgroup per (sequence, KV
// head, chunk)).  With few (sequence, KV head) units -- one long request, or
// a handful of them -- about one workgroup per compute unit of a 256-CU part
// streams best: each workgroup keeps its four waves busy on one long run of
// blocks and the merge has few chunks to combine.  With many units the
// lengths of a batch usually differ (the host only knows their maximum), so
// the split aims at about sixteen workgroups per compute unit, sized on the
// maximum, which evens out short and long sequences.  Chunks are at least
// kMinChunk tokens and a multiple of kChunkQuantum.  (Measured on MI355X:
// 8B-shaped single sequence best at 1024 tokens, 70B-shaped 4 x 131k at
// 16384, 32 ragged 4k..16k sequences at 1024.)
constexpr int64_t kComputeUnits = 256;
constexpr int64_t kManyUnits = 256;
constexpr int32_t kMinChunk = 1024;
constexpr int32_t kChunkQuantum = 128;

// Uneven chunk pairs.  Workgroup x runs on XCD x % 8, and on MI355X the odd
// XCDs stream a few per cent slower than the even ones (per-workgroup
// timestamps: mean finish 5-7 % later on long launches, the same XCDs on
// every run and device measured).  An automatic split with an even number of
// KV heads therefore pairs its chunks: in chunks 2p and 2p + 1 the heads of a
// pair trade places, so the workgroup on the even XCD always takes the longer
// chunk, C + d, and its neighbour on the odd XCD the shorter, C - d, with d
// about 4.5 % of C in whole 32-token pairs (measured: 70B-shaped layer call
// 320 -> 316 us, 256-request batch 421 -> 415 us, ragged batch 207 -> 205 us;
// 8 % and more was slower again; a fused score was slower with it, so a call
// with a score keeps even chunks, and so does a call with
// KVD_FLAG_EVEN_CHUNKS, for batches whose shared blocks the L2 serves).  Unit boundaries stay fixed for given
// arguments, so results stay deterministic.
constexpr int32_t kSkewPermille = 45;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Launch status is read back with hipGetLastError, which also reports an error
// left behind by an earlier, unrelated runtime call in this thread; clear that
// first so that only this call's launches are checked.
void clear_stale_error() { (void)hipGetLastError(); }

// HIP error behind the calling thread's most recent KVD_ERR_HIP (errno-like).
thread_local hipError_t t_last_hip = hipSuccess;

#define KVD_TRY_HIP(call)         \
  do {                            \
    const hipError_t e_ = (call); \
    if (e_ != hipSuccess) {       \
      t_last_hip = e_;            \
      return KVD_ERR_HIP;         \
    }                             \
  } while (0)

kvd_status check_desc(const kvd_pool_desc* d) {
  if (!d) return KVD_ERR_INVALID_ARG;
  if (d->num_layers < 1 || d->num_blocks < 1 || d->n_kv < 1) return KVD_ERR_INVALID_ARG;
  if (d->dtype != KVD_BF16 && d->dtype != KVD_FP8_E4M3) return KVD_ERR_INVALID_ARG;
  if (d->block_size != kvd::kBlock) return KVD_ERR_UNSUPPORTED;
  if (d->head_dim != 64 && d->head_dim != 128) return KVD_ERR_UNSUPPORTED;
  const int64_t eb = d->dtype == KVD_BF16 ? 2 : 1;
  const int64_t layer = (int64_t)d->num_blocks * d->n_kv * 2 * kvd::kBlock * d->head_dim * eb;
  if (layer >= ((int64_t)1 << 32)) return KVD_ERR_UNSUPPORTED;
  return KVD_OK;
}

kvd_status plan_decode(const PoolView& p, const kvd_decode_args* a, DecodePlan* out) {
  if (!a) return KVD_ERR_INVALID_ARG;
  if (a->b < 0 || a->n_q < 1 || a->max_blocks_per_seq < 1 || a->max_context_len < 0)
    return KVD_ERR_INVALID_ARG;
  if (a->n_q % p.n_kv != 0) return KVD_ERR_INVALID_ARG;
  if (a->n_q / p.n_kv > 16) return KVD_ERR_UNSUPPORTED;
  if (a->chunk_tokens < 0 || a->chunk_tokens % kvd::kBlock != 0) return KVD_ERR_INVALID_ARG;
  if ((a->flags & ~KVD_FLAG_EVEN_CHUNKS) != 0) return KVD_ERR_INVALID_ARG;
  if (a->score && (a->score_stride < 1 || a->score_stride < a->max_context_len))
    return KVD_ERR_INVALID_ARG;
  // With a score every chunk must cover whole 32-token pairs: a pair's score
  // slots must not reach into the next chunk's.
  if (a->score && a->chunk_tokens % 32 != 0) return KVD_ERR_INVALID_ARG;
  DecodePlan pl{};
  const int64_t bound64 = std::min<int64_t>(a->max_context_len, (int64_t)kvd::kBlock * a->max_blocks_per_seq);
  if (bound64 > (int64_t)1 << 30) return KVD_ERR_UNSUPPORTED;
  pl.ctx_bound = (int32_t)bound64;
  int64_t chunk = a->chunk_tokens;
  if (chunk == 0) {
    const int64_t units = (int64_t)std::max(a->b, 1) * p.n_kv;
    const int64_t target = units >= kManyUnits ? 16 * kComputeUnits : kComputeUnits;
    const int64_t total = units * std::max(pl.ctx_bound, 1);
    chunk = (total + target - 1) / target;
    chunk = (chunk + kChunkQuantum - 1) / kChunkQuantum * kChunkQuantum;
    chunk = std::max<int64_t>(chunk, kMinChunk);
  }
  const int64_t whole = std::max<int64_t>(kvd::kBlock, (pl.ctx_bound + 15) / 16 * 16);
  if (chunk > whole) chunk = whole;
  pl.chunk = (int32_t)chunk;
  pl.n_chunks = (int32_t)std::max<int64_t>(1, (pl.ctx_bound + chunk - 1) / chunk);
  pl.chunk_skew = 0;
  if (a->chunk_tokens == 0 && pl.n_chunks >= 2 && p.n_kv % 2 == 0 && !a->score && pl.chunk % 32 == 0 &&
      (a->flags & KVD_FLAG_EVEN_CHUNKS) == 0) {
    const int32_t d = (int32_t)(((int64_t)pl.chunk * kSkewPermille + 16000) / 32000) * 32;
    if (d > 0 && pl.chunk - d >= 32) pl.chunk_skew = d;
  }
  // grids of 256-work-item workgroups: fewer than 2^32 work-items per launch
  if ((int64_t)pl.n_chunks * std::max(a->b, 1) * p.n_kv >= ((int64_t)1 << 24)) return KVD_ERR_UNSUPPORTED;
  if ((int64_t)a->b * a->n_q >= ((int64_t)1 << 24)) return KVD_ERR_UNSUPPORTED;
  pl.final_direct = pl.n_chunks == 1;
  pl.scores = a->score != nullptr;
  pl.logit_stride = (pl.ctx_bound + 31) / 32 * 32 + 32;
  size_t off = 0;
  const size_t bq = (size_t)a->b * a->n_q;
  if (!pl.final_direct) {
    pl.off_part_o = off;
    off = align256(off + bq * pl.n_chunks * p.head_dim * sizeof(float));
    pl.off_part_lse = off;
    off = align256(off + bq * pl.n_chunks * sizeof(float));
  }
  if (pl.scores) {
    pl.off_logits = off;
    off = align256(off + bq * pl.logit_stride * sizeof(float));
    pl.off_lse2 = off;
    off = align256(off + bq * sizeof(float));
  }
  pl.total = off;
  *out = pl;
  return KVD_OK;
}

// Scratch of kvd_decode_attn_no_alloc, for callers that cannot allocate: one
// array per device, held from the library's first use on a device until the
// process ends.  Host code never uses the array's name as an address (on the
// host it is a stand-in, not device memory); it uses the address
// hipGetSymbolAddress returns for the current device, looked up once per
// device and kept in g_scratch.
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the calling thread's current device.
kvd_status static_scratch(char** out) {
  int dev = -1;
  KVD_TRY_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return KVD_ERR_UNSUPPORTED;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      KVD_TRY_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
      if (!p) return KVD_ERR_HIP;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = static_cast<char*>(p);
  return KVD_OK;
}

// One decode call.  ext_part_o / ext_part_lse (both or neither): write the
// per-chunk partials there and stop, instead of producing the merged output.
// pool8 (mixed precision only): the FP8 pool beside the bf16 pool `pool`.
// new_k / new_v (both or neither): the fused append of token s_i - 1.
// fixed_ws (with capacity fixed_cap): scratch to use instead of the caller's
// workspace (args->workspace is then ignored).
kvd_status decode_common(const kvd_pool* pool, int32_t layer, const kvd_decode_args* a,
                         void* stream, bool any_dtype, kvd_dtype want, float* ext_part_o,
                         float* ext_part_lse, const kvd_pool* pool8 = nullptr,
                         const void* new_k = nullptr, const void* new_v = nullptr,
                         char* fixed_ws = nullptr, size_t fixed_cap = 0) {
  if (!pool || !a) return KVD_ERR_INVALID_ARG;
  const PoolView& p = pool->v;
  if (!any_dtype && p.dtype != want) return KVD_ERR_DTYPE;
  if (layer < 0 || layer >= p.num_layers) return KVD_ERR_INVALID_ARG;
  if (pool8) {
    const PoolView& p8 = pool8->v;
    if (p8.dtype != KVD_FP8_E4M3) return KVD_ERR_DTYPE;
    if (p8.num_layers != p.num_layers || p8.n_kv != p.n_kv || p8.head_dim != p.head_dim)
      return KVD_ERR_INVALID_ARG;
    if (p.num_blocks >= kvd::kPrecisionBit || p8.num_blocks >= kvd::kPrecisionBit) return KVD_ERR_UNSUPPORTED;
    if (a->score) return KVD_ERR_UNSUPPORTED;
  }
  const bool external = ext_part_o != nullptr || ext_part_lse != nullptr;
  if (external && (a->score || !ext_part_o || !ext_part_lse)) return KVD_ERR_INVALID_ARG;
  DecodePlan pl;
  kvd_status st = plan_decode(p, a, &pl);
  if (st != KVD_OK) return st;
  if (a->b == 0) return KVD_OK;
  if (!a->q || !a->block_table || !a->context_lens) return KVD_ERR_INVALID_ARG;
  if (!external && !a->out) return KVD_ERR_INVALID_ARG;
  // the kernels' vector accesses: q in 16-byte loads, out in 8-byte stores
  if (((uintptr_t)a->q & 15) != 0 || (!external && ((uintptr_t)a->out & 7) != 0)) return KVD_ERR_INVALID_ARG;
  if (((uintptr_t)a->lse_out & 3) != 0 || ((uintptr_t)a->score & 3) != 0) return KVD_ERR_INVALID_ARG;
  if (fixed_ws) {
    if (pl.total > fixed_cap) return KVD_ERR_WORKSPACE;
  } else if (!external && pl.total > 0) {
    if (!a->workspace || a->workspace_bytes < pl.total) return KVD_ERR_WORKSPACE;
    if (((uintptr_t)a->workspace & 255) != 0) return KVD_ERR_WORKSPACE;
  }
  if (external && ((((uintptr_t)ext_part_o) & 15) != 0 || (((uintptr_t)ext_part_lse) & 3) != 0))
    return KVD_ERR_INVALID_ARG;
  char* ws = fixed_ws ? fixed_ws : static_cast<char*>(a->workspace);
  const bool final_direct = !external && pl.final_direct;
  kvd::DecodeLaunch L{};
  L.layer_base = p.kv_base + (size_t)layer * (size_t)p.layer_bytes;
  L.new_k = static_cast<const uint16_t*>(new_k);
  L.new_v = static_cast<const uint16_t*>(new_v);
  L.layer_bytes = (uint32_t)p.layer_bytes;
  L.layer_scales = p.scale_base ? p.scale_base + (size_t)layer * p.num_blocks * p.n_kv * 2 : nullptr;
  L.q = static_cast<const uint16_t*>(a->q);
  L.block_table = a->block_table;
  L.context_lens = a->context_lens;
  L.b = a->b;
  L.n_q = a->n_q;
  L.n_kv = p.n_kv;
  L.g = a->n_q / p.n_kv;
  L.max_blocks = a->max_blocks_per_seq;
  L.num_blocks = p.num_blocks;
  L.ctx_bound = pl.ctx_bound;
  L.chunk = pl.chunk;
  L.n_chunks = pl.n_chunks;
  L.chunk_skew = pl.chunk_skew;
  L.out = static_cast<uint16_t*>(a->out);
  L.lse_out = a->lse_out;
  if (external) {
    L.part_o = ext_part_o;
    L.part_lse = ext_part_lse;
  } else if (!final_direct) {
    L.part_o = reinterpret_cast<float*>(ws + pl.off_part_o);
    L.part_lse = reinterpret_cast<float*>(ws + pl.off_part_lse);
  }
  const bool scores = !external && pl.scores;
  L.logits = scores ? reinterpret_cast<float*>(ws + pl.off_logits) : nullptr;
  L.lse2 = scores ? reinterpret_cast<float*>(ws + pl.off_lse2) : nullptr;
  L.logit_stride = pl.logit_stride;
  hipStream_t s = static_cast<hipStream_t>(stream);
  clear_stale_error();
  int kind = p.dtype == KVD_FP8_E4M3 ? kvd::kFp8 : kvd::kBf16;
  if (pool8) {
    const PoolView& p8 = pool8->v;
    kind = kvd::kMixed;
    L.layer_base8 = p8.kv_base + (size_t)layer * (size_t)p8.layer_bytes;
    L.layer_bytes8 = (uint32_t)p8.layer_bytes;
    L.layer_scales8 = p8.scale_base + (size_t)layer * p8.num_blocks * p8.n_kv * 2;
    L.num_blocks8 = p8.num_blocks;
  }
  KVD_TRY_HIP(kvd::launch_decode(L, p.head_dim, kind, final_direct, scores, s));
  if (external) return KVD_OK;
  if (!final_direct) {
    KVD_TRY_HIP(kvd::launch_merge(L.part_o, L.part_lse, a->b, a->n_q, pl.n_chunks, p.head_dim, L.out,
                                  a->lse_out, L.lse2, s));
  }
  if (scores) {
    KVD_TRY_HIP(kvd::launch_score(L.logits, L.lse2, a->context_lens, pl.ctx_bound, a->b, a->n_q,
                          pl.logit_stride, a->score, a->score_stride, a->score_weight, s));
  }
  return KVD_OK;
}

}  // namespace

extern "C" {

kvd_status kvd_pool_bytes(const kvd_pool_desc* d, size_t* kv_bytes, size_t* scale_bytes) {
  kvd_status st = check_desc(d);
  if (st != KVD_OK) return st;
  const size_t eb = d->dtype == KVD_BF16 ? 2 : 1;
  const size_t tiles = (size_t)d->num_layers * d->num_blocks * d->n_kv;
  if (kv_bytes) *kv_bytes = tiles * 2 * kvd::kBlock * d->head_dim * eb;
  if (scale_bytes) *scale_bytes = d->dtype == KVD_FP8_E4M3 ? tiles * 2 * sizeof(float) : 0;
  return KVD_OK;
}

kvd_status kvd_create_pool(const kvd_pool_desc* d, void* kv_base, float* scale_base, kvd_pool** out) {
  if (!out) return KVD_ERR_INVALID_ARG;
  kvd_status st = check_desc(d);
  if (st != KVD_OK) return st;
  if (!kv_base || ((uintptr_t)kv_base & 15) != 0) return KVD_ERR_INVALID_ARG;
  if (d->dtype == KVD_FP8_E4M3) {
    if (!scale_base || ((uintptr_t)scale_base & 3) != 0) return KVD_ERR_INVALID_ARG;
  } else if (scale_base) {
    return KVD_ERR_INVALID_ARG;
  }
  kvd_pool* p = new (std::nothrow) kvd_pool;
  if (!p) return KVD_ERR_CAPACITY;                  // host memory
  PoolView& v = p->v;
  v.num_layers = d->num_layers;
  v.num_blocks = d->num_blocks;
  v.n_kv = d->n_kv;
  v.head_dim = d->head_dim;
  v.dtype = d->dtype;
  v.kv_base = static_cast<char*>(kv_base);
  v.scale_base = scale_base;
  v.elem_bytes = d->dtype == KVD_BF16 ? 2 : 1;
  v.tile_pair_bytes = 2LL * kvd::kBlock * d->head_dim * v.elem_bytes;
  v.layer_bytes = (int64_t)d->num_blocks * d->n_kv * v.tile_pair_bytes;
  *out = p;
  return KVD_OK;
}

kvd_status kvd_destroy_pool(kvd_pool* pool) {
  if (!pool) return KVD_ERR_INVALID_ARG;
  delete pool;
  return KVD_OK;
}

kvd_status kvd_write_kv(const kvd_pool* pool, int32_t layer, const void* k, const void* v,
                        const int32_t* slot_mapping, int32_t n_tok, void* hip_stream) {
  if (!pool) return KVD_ERR_INVALID_ARG;
  if (layer < 0 || layer >= pool->v.num_layers || n_tok < 0) return KVD_ERR_INVALID_ARG;
  if (n_tok == 0) return KVD_OK;
  if (!k || !v || !slot_mapping) return KVD_ERR_INVALID_ARG;
  // the bf16 store runs one work-item per element: fewer than 2^32 per launch
  if (pool->v.dtype == KVD_BF16 && (int64_t)n_tok * pool->v.n_kv * pool->v.head_dim >= ((int64_t)1 << 32))
    return KVD_ERR_UNSUPPORTED;
  clear_stale_error();
  KVD_TRY_HIP(kvd::launch_write(pool->v, layer, static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                        slot_mapping, n_tok, static_cast<hipStream_t>(hip_stream)));
  return KVD_OK;
}

kvd_status kvd_slot_mapping(const int32_t* block_table, int32_t max_blocks_per_seq, int32_t b,
                            const int32_t* context_lens, const int32_t* first_token, const int64_t* out_start,
                            int32_t max_tokens_per_seq, int32_t* slots, int64_t n_slots, void* hip_stream) {
  if (b < 0 || max_blocks_per_seq < 1 || max_tokens_per_seq < 0 || n_slots < 0) return KVD_ERR_INVALID_ARG;
  if ((int64_t)max_blocks_per_seq * kvd::kBlock >= ((int64_t)1 << 31)) return KVD_ERR_UNSUPPORTED;
  // 256-work-item workgroups: fewer than 2^32 work-items per launch
  if ((int64_t)b * ((max_tokens_per_seq + 255) / 256) >= ((int64_t)1 << 24)) return KVD_ERR_UNSUPPORTED;
  if (b == 0 || max_tokens_per_seq == 0 || n_slots == 0) return KVD_OK;
  if (!block_table || !context_lens || !out_start || !slots) return KVD_ERR_INVALID_ARG;
  clear_stale_error();
  KVD_TRY_HIP(kvd::launch_slot_mapping(block_table, max_blocks_per_seq, b, context_lens, first_token, out_start,
                                       max_tokens_per_seq, slots, n_slots, static_cast<hipStream_t>(hip_stream)));
  return KVD_OK;
}

kvd_status kvd_decode_plan(const kvd_pool* pool, const kvd_decode_args* args, int32_t* chunk_tokens,
                           int32_t* n_chunks) {
  if (!pool) return KVD_ERR_INVALID_ARG;
  DecodePlan pl;
  kvd_status st = plan_decode(pool->v, args, &pl);
  if (st != KVD_OK) return st;
  if (chunk_tokens) *chunk_tokens = pl.chunk;
  if (n_chunks) *n_chunks = pl.n_chunks;
  return KVD_OK;
}

kvd_status kvd_decode_workspace_bytes(const kvd_pool* pool, const kvd_decode_args* args, size_t* bytes) {
  if (!pool || !bytes) return KVD_ERR_INVALID_ARG;
  DecodePlan pl;
  kvd_status st = plan_decode(pool->v, args, &pl);
  if (st != KVD_OK) return st;
  *bytes = pl.total;
  return KVD_OK;
}

kvd_status kvd_decode_attn(const kvd_pool* pool, int32_t layer, const kvd_decode_args* args, void* hip_stream) {
  return decode_common(pool, layer, args, hip_stream, false, KVD_BF16, nullptr, nullptr);
}

kvd_status kvd_decode_attn_fp8(const kvd_pool* pool, int32_t layer, const kvd_decode_args* args,
                               void* hip_stream) {
  return decode_common(pool, layer, args, hip_stream, false, KVD_FP8_E4M3, nullptr, nullptr);
}

kvd_status kvd_decode_attn_mixed(const kvd_pool* pool_bf16, const kvd_pool* pool_fp8, int32_t layer,
                                 const kvd_decode_args* args, void* hip_stream) {
  if (!pool_fp8) return KVD_ERR_INVALID_ARG;
  return decode_common(pool_bf16, layer, args, hip_stream, false, KVD_BF16, nullptr, nullptr, pool_fp8);
}

kvd_status kvd_decode_attn_append(const kvd_pool* pool, int32_t layer, const kvd_decode_args* args,
                                  const void* new_k, const void* new_v, void* hip_stream) {
  if (!new_k || !new_v) return KVD_ERR_INVALID_ARG;
  return decode_common(pool, layer, args, hip_stream, true, KVD_BF16, nullptr, nullptr, nullptr, new_k, new_v);
}

kvd_status kvd_decode_attn_no_alloc(const kvd_pool* pool, int32_t layer, const kvd_decode_args* args,
                                    void* hip_stream) {
  if (!pool || !args) return KVD_ERR_INVALID_ARG;
  DecodePlan pl;
  kvd_status st = plan_decode(pool->v, args, &pl);
  if (st != KVD_OK) return st;
  if (pl.total > kStaticScratchBytes) return KVD_ERR_WORKSPACE;   // before any HIP call
  char* ws = nullptr;
  st = static_scratch(&ws);
  if (st != KVD_OK) return st;
  return decode_common(pool, layer, args, hip_stream, true, KVD_BF16, nullptr, nullptr, nullptr, nullptr, nullptr,
                       ws, kStaticScratchBytes);
}

kvd_status kvd_decode_partials(const kvd_pool* pool, int32_t layer, const kvd_decode_args* args,
                               float* part_o, float* part_lse, void* hip_stream) {
  if (!part_o || !part_lse) return KVD_ERR_INVALID_ARG;
  return decode_common(pool, layer, args, hip_stream, true, KVD_BF16, part_o, part_lse);
}

kvd_status kvd_merge_partials(const float* part_o, const float* part_lse, int32_t b, int32_t n_q,
                              int32_t n_chunks, int32_t d_h, void* out_bf16, float* lse_out,
                              void* hip_stream) {
  if (b < 0 || n_q < 1 || n_chunks < 1) return KVD_ERR_INVALID_ARG;
  if (d_h != 64 && d_h != 128) return KVD_ERR_UNSUPPORTED;
  if (b == 0) return KVD_OK;
  if (!part_o || !part_lse || !out_bf16) return KVD_ERR_INVALID_ARG;
  if (((uintptr_t)part_o & 15) != 0 || ((uintptr_t)part_lse & 3) != 0 || ((uintptr_t)out_bf16 & 7) != 0 ||
      ((uintptr_t)lse_out & 3) != 0)
    return KVD_ERR_INVALID_ARG;
  if ((int64_t)b * n_q >= ((int64_t)1 << 24)) return KVD_ERR_UNSUPPORTED;   // a wave per head at most
  clear_stale_error();
  KVD_TRY_HIP(kvd::launch_merge(part_o, part_lse, b, n_q, n_chunks, d_h, static_cast<uint16_t*>(out_bf16),
                                lse_out, nullptr, static_cast<hipStream_t>(hip_stream)));
  return KVD_OK;
}

const char* kvd_last_hip_error(void) {
  thread_local char buf[160];
  snprintf(buf, sizeof buf, "%s: %s", hipGetErrorName(t_last_hip), hipGetErrorString(t_last_hip));
  return buf;
}

const char* kvd_status_string(kvd_status s) {
  switch (s) {
    case KVD_OK: return "KVD_OK";
    case KVD_ERR_INVALID_ARG: return "KVD_ERR_INVALID_ARG";
    case KVD_ERR_UNSUPPORTED: return "KVD_ERR_UNSUPPORTED";
    case KVD_ERR_DTYPE: return "KVD_ERR_DTYPE";
    case KVD_ERR_WORKSPACE: return "KVD_ERR_WORKSPACE";
    case KVD_ERR_HIP: return "KVD_ERR_HIP";
    case KVD_ERR_CAPACITY: return "KVD_ERR_CAPACITY";
  }
  return "KVD_ERR_UNKNOWN";
}

kvd_status kvd_debug_gather_offsets(const kvd_pool* pool, int32_t layer, const int32_t* block_table,
                                    int32_t max_blocks_per_seq, int32_t b, int32_t n_tok,
                                    int64_t* out_k, int64_t* out_v, void* hip_stream) {
  if (!pool || layer < 0 || layer >= pool->v.num_layers) return KVD_ERR_INVALID_ARG;
  if (b < 0 || n_tok < 0 || max_blocks_per_seq < 1) return KVD_ERR_INVALID_ARG;
  if ((int64_t)n_tok > (int64_t)kvd::kBlock * max_blocks_per_seq) return KVD_ERR_INVALID_ARG;
  if ((int64_t)b * n_tok == 0) return KVD_OK;
  if (!block_table || !out_k || !out_v) return KVD_ERR_INVALID_ARG;
  clear_stale_error();
  KVD_TRY_HIP(kvd::launch_debug_offsets(pool->v, layer, block_table, max_blocks_per_seq, b, n_tok, out_k, out_v,
                                static_cast<hipStream_t>(hip_stream)));
  return KVD_OK;
}

kvd_status kvd_debug_unit_map(const kvd_pool* pool, const kvd_decode_args* args, int32_t* units,
                              void* hip_stream) {
  if (!pool || !args) return KVD_ERR_INVALID_ARG;
  DecodePlan pl;
  kvd_status st = plan_decode(pool->v, args, &pl);
  if (st != KVD_OK) return st;
  if (args->b == 0) return KVD_OK;
  if (!args->context_lens || !units) return KVD_ERR_INVALID_ARG;
  kvd::DecodeLaunch L{};
  L.context_lens = args->context_lens;
  L.b = args->b;
  L.n_q = args->n_q;
  L.n_kv = pool->v.n_kv;
  L.g = args->n_q / pool->v.n_kv;
  L.max_blocks = args->max_blocks_per_seq;
  L.num_blocks = pool->v.num_blocks;
  L.ctx_bound = pl.ctx_bound;
  L.chunk = pl.chunk;
  L.n_chunks = pl.n_chunks;
  L.chunk_skew = pl.chunk_skew;
  clear_stale_error();
  KVD_TRY_HIP(kvd::launch_debug_units(L, units, static_cast<hipStream_t>(hip_stream)));
  return KVD_OK;
}

kvd_status kvd_debug_fp8_decode(const uint8_t* codes, int32_t n, float* out, void* hip_stream) {
  if (n < 0) return KVD_ERR_INVALID_ARG;
  if (n == 0) return KVD_OK;
  if (!codes || !out) return KVD_ERR_INVALID_ARG;
  clear_stale_error();
  KVD_TRY_HIP(kvd::launch_debug_fp8_decode(codes, n, out, static_cast<hipStream_t>(hip_stream)));
  return KVD_OK;
}

kvd_status kvd_debug_stream_read(const void* data, uint64_t bytes, uint32_t* sink, int32_t grid,
                                 void* hip_stream) {
  if (!data || !sink || grid < 1 || grid > 65536) return KVD_ERR_INVALID_ARG;
  if (bytes < 16 || bytes % 16 != 0 || ((uintptr_t)data & 15) != 0) return KVD_ERR_INVALID_ARG;
  if (bytes >= ((uint64_t)1 << 32)) return KVD_ERR_UNSUPPORTED;
  clear_stale_error();
  KVD_TRY_HIP(kvd::launch_stream_read(data, (uint32_t)bytes, sink, grid, static_cast<hipStream_t>(hip_stream)));
  return KVD_OK;
}

}  // extern "C"
