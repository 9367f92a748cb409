// Internal declarations shared by the host library and the kernel sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvdecode.h"

namespace kvd {

constexpr int kBlock = 16;  // tokens per block

// Host view of a pool: shape plus base pointers and derived strides.
struct PoolView {
  int32_t num_layers, num_blocks, n_kv, head_dim;
  kvd_dtype dtype;
  char* kv_base;
  float* scale_base;
  int64_t elem_bytes;       // 2 (bf16) or 1 (fp8)
  int64_t tile_pair_bytes;  // 2 * 16 * head_dim * elem_bytes
  int64_t layer_bytes;      // num_blocks * n_kv * tile_pair_bytes (< 4 GiB)
};

// Decode launch plan: how the context is split and where the scratch lives.
struct DecodePlan {
  int32_t chunk;            // tokens per chunk (multiple of 16)
  int32_t n_chunks;         // chunks per sequence at max_context_len
  int32_t ctx_bound;        // clamp for every s_i
  int32_t logit_stride;     // row length of the logit scratch (scores only)
  int32_t chunk_skew;       // tokens that pass from the odd to the even chunk of a pair
  bool final_direct;        // one chunk: no partials, the workgroup writes out/lse itself
  bool scores;
  size_t off_part_o, off_part_lse, off_logits, off_lse2, total;
};

// Arguments handed to the decode kernel.
// Pool kinds of a decode launch, and the table-entry bit that marks an FP8
// block in a mixed-precision decode.
constexpr int kBf16 = 0, kFp8 = 1, kMixed = 2;
constexpr int32_t kPrecisionBit = 1 << 30;

struct DecodeLaunch {
  const char* layer_base;   // start of this layer's tile pairs
  uint32_t layer_bytes;     // bytes addressable from layer_base
  const float* layer_scales;  // FP8: this layer's scales; else null
  const uint16_t* q;
  const int32_t* block_table;
  const int32_t* context_lens;
  int32_t b, n_q, n_kv, g, max_blocks, num_blocks, ctx_bound, chunk, n_chunks;
  int32_t chunk_skew;       // 0, or d of the uneven chunk pairs (chunk_span)
  // outputs: either final (out/lse_out) or partials
  uint16_t* out;
  float* lse_out;
  float* part_o;
  float* part_lse;
  float* logits;            // scores: log2-domain scaled logits [b][n_q][logit_stride]
  float* lse2;              // scores: log2-domain lse [b][n_q]
  int32_t logit_stride;
  // mixed precision: the FP8 pool's layer, its scales and block count
  const char* layer_base8;
  uint32_t layer_bytes8;
  const float* layer_scales8;
  int32_t num_blocks8;
  // fused append (or null): bf16 [b][n_kv][D] K and V of token s_i - 1, stored
  // before attention by the workgroup whose chunk holds that token
  const uint16_t* new_k;
  const uint16_t* new_v;
};

hipError_t launch_decode(const DecodeLaunch& a, int head_dim, int kind, bool final_direct,
                         bool scores, hipStream_t stream);

hipError_t launch_debug_units(const DecodeLaunch& a, int32_t* out, hipStream_t stream);

hipError_t launch_merge(const float* part_o, const float* part_lse, int32_t b, int32_t n_q,
                        int32_t n_chunks, int32_t head_dim, uint16_t* out, float* lse_out,
                        float* lse2, hipStream_t stream);

hipError_t launch_score(const float* logits, const float* lse2, const int32_t* context_lens,
                        int32_t ctx_bound, int32_t b, int32_t n_q, int32_t logit_stride,
                        float* score, int32_t score_stride, float weight, hipStream_t stream);

hipError_t launch_write(const PoolView& p, int32_t layer, const uint16_t* k, const uint16_t* v,
                        const int32_t* slot_mapping, int32_t n_tok, hipStream_t stream);

hipError_t launch_slot_mapping(const int32_t* block_table, int32_t max_blocks, int32_t b,
                               const int32_t* context_lens, const int32_t* first_token,
                               const int64_t* out_start, int32_t max_tokens, int32_t* slots,
                               int64_t n_slots, hipStream_t stream);

hipError_t launch_debug_offsets(const PoolView& p, int32_t layer, const int32_t* block_table,
                                int32_t max_blocks, int32_t b, int32_t n_tok, int64_t* out_k,
                                int64_t* out_v, hipStream_t stream);

hipError_t launch_debug_fp8_decode(const uint8_t* codes, int32_t n, float* out,
                                   hipStream_t stream);

hipError_t launch_stream_read(const void* data, uint32_t bytes, uint32_t* sink, int32_t grid,
                              hipStream_t stream);

}  // namespace kvd
