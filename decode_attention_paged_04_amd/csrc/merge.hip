// Log-sum-exp merge of per-chunk partials, and the cumulative-score update
// that needs the merged lse.
#include "device_common.h"
#include "kvd_internal.h"

#include <math.h>

namespace kvd {

// Log-sum-exp merge of one (sequence, query head)'s per-chunk partials by one
// wave: lse = M + ln(sum_c exp(lse_c - M)) with M = max_c lse_c (lane l takes
// chunks l, l + 64, ...; the lanes' values are combined by butterfly
// shuffles), out = sum_c exp(lse_c - lse) * o_c added in chunk order and
// rounded to bf16.  A chunk whose weight is 0 (lse_c = -inf: nothing
// attended) adds nothing and its o_c is never used, so it may hold anything,
// NaN included; no chunk with weight gives out = 0 and lse = -inf.
constexpr float kMergeLog2e = 1.4426950408889634f;

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// po: o_c rows [nc][D]; pl: lse_c [nc] (natural log).  Writes out[0 .. D)
// (bf16), *lse_out and *lse2 (log2 domain) when given.  Lane l owns channels
// l, l + 64, ...; up to BATCH chunks' outputs are loaded before any is used.
template <int D, int BATCH>
__device__ inline void merge_head(const float* __restrict__ po, const float* __restrict__ pl, int nc,
                                  uint16_t* __restrict__ out, float* lse_out, float* lse2) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  float ov[BATCH][PER];
#pragma unroll
  for (int k = 0; k < BATCH; ++k)
#pragma unroll
    for (int p = 0; p < PER; ++p) ov[k][p] = k < nc ? po[(size_t)k * D + lane + 64 * p] : 0.f;
  const float lv = lane < nc ? pl[lane] : -INFINITY;
  float mx = lv;
  for (int c = lane + 64; c < nc; c += 64) mx = fmaxf(mx, pl[c]);
  const float M = wave_max(mx);
  if (M == -INFINITY) {
#pragma unroll
    for (int p = 0; p < PER; ++p) out[lane + 64 * p] = 0;
    if (lane == 0) {
      if (lse_out) *lse_out = -INFINITY;
      if (lse2) *lse2 = -INFINITY;
    }
    return;
  }
  float sm = lane < nc ? expf(lv - M) : 0.f;
  for (int c = lane + 64; c < nc; c += 64) sm += expf(pl[c] - M);
  const float lse = M + logf(wave_sum(sm));
  const float wl = lane < nc ? expf(lv - lse) : 0.f;   // weight of chunk `lane` (< 64)
  float acc[PER];
#pragma unroll
  for (int p = 0; p < PER; ++p) acc[p] = 0.f;
  for (int c0 = 0; c0 < nc; c0 += BATCH) {               // uniform
    if (c0 > 0) {
#pragma unroll
      for (int k = 0; k < BATCH; ++k)
#pragma unroll
        for (int p = 0; p < PER; ++p)
          ov[k][p] = c0 + k < nc ? po[(size_t)(c0 + k) * D + lane + 64 * p] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
      const int c = c0 + k;
      if (c < nc) {                                      // uniform
        const float w = c < 64 ? __shfl(wl, c) : expf(pl[c] - lse);
        if (w != 0.f) {                                  // uniform: an empty chunk's o_c is never used
#pragma unroll
          for (int p = 0; p < PER; ++p) acc[p] += w * ov[k][p];
        }
      }
    }
  }
#pragma unroll
  for (int p = 0; p < PER; ++p) out[lane + 64 * p] = float_to_bf16_bits(acc[p]);
  if (lane == 0) {
    if (lse_out) *lse_out = lse;
    if (lse2) *lse2 = lse * kMergeLog2e;
  }
}

// One wave per (sequence, query head), four heads per workgroup: with many
// heads and few chunks (a large batch of short contexts) a workgroup per head
// would make the launch mostly workgroup dispatch.  merge_head loads up to
// BATCH chunks' outputs before it uses any, so a split of up to BATCH chunks
// costs about one memory round trip.
constexpr int kMergeThreads = 256;

template <int D, int BATCH>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse, int64_t n_heads,
    int32_t n_chunks, uint16_t* __restrict__ out, float* __restrict__ lse_out, float* __restrict__ lse2) {
  const int64_t ih = (int64_t)blockIdx.x * (kMergeThreads / 64) + (threadIdx.x >> 6);
  if (ih >= n_heads) return;                     // the whole wave
  merge_head<D, BATCH>(part_o + ih * n_chunks * D, part_lse + ih * n_chunks, n_chunks, out + ih * D,
                       lse_out ? lse_out + ih : nullptr, lse2 ? lse2 + ih : nullptr);
}

// Slot of token t in the score scratch.  Within each 32-token pair the decode
// kernel holds tokens 8G .. 8G+7 in lane group G and stores the first four of
// every group, then the last four: token 8G + 4h + e goes to slot 16h + 4G + e.
__device__ inline int score_slot(int t) {
  const int r = t & 31;
  return (t & ~31) + 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3);
}

// alpha of one head and token from its log2-domain score and lse; a head that
// attended nothing (lse2 = -inf, every block dropped) gives 0, not NaN.
__device__ inline float weight_of(float x, float lse2) {
  return lse2 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(x - lse2);
}

// score[i][t] += weight / n_q * sum_h exp2(x[i][h][t] - lse2[i][h]) for t < s_i,
// x being the log2-domain scaled scores the decode kernel stored.  Each thread
// owns one token; the heads' loads are issued eight at a time so that they are
// in flight together, and the sum runs in head order.
__global__ __launch_bounds__(256) void score_kernel(const float* __restrict__ logits,
                                                    const float* __restrict__ lse2,
                                                    const int32_t* __restrict__ context_lens,
                                                    int32_t ctx_bound, int32_t n_q,
                                                    int32_t stride, float* __restrict__ score,
                                                    int32_t score_stride, float w_over_nq) {
  constexpr int U = 8;
  const int i = blockIdx.y;
  const int t = blockIdx.x * 256 + threadIdx.x;
  int s = context_lens[i];
  s = s < 0 ? 0 : (s > ctx_bound ? ctx_bound : s);
  if (t >= s) return;
  const float* x = logits + (size_t)i * n_q * stride + score_slot(t);
  const float* ls = lse2 + (size_t)i * n_q;
  float acc = 0.f;
  int h = 0;
  for (; h + U <= n_q; h += U) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = x[(size_t)(h + u) * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) acc += weight_of(v[u], ls[h + u]);
  }
  for (; h < n_q; ++h) acc += weight_of(x[(size_t)h * stride], ls[h]);
  score[(size_t)i * score_stride + t] += w_over_nq * acc;
}

hipError_t launch_merge(const float* part_o, const float* part_lse, int32_t b, int32_t n_q,
                        int32_t n_chunks, int32_t head_dim, uint16_t* out, float* lse_out,
                        float* lse2, hipStream_t stream) {
  const int64_t heads = (int64_t)b * n_q;
  const dim3 grid((unsigned)((heads + kMergeThreads / 64 - 1) / (kMergeThreads / 64)));
  const dim3 block(kMergeThreads);
  if (head_dim == 128) {
    if (n_chunks <= 16)
      hipLaunchKernelGGL((merge_kernel<128, 16>), grid, block, 0, stream, part_o, part_lse, heads, n_chunks, out,
                         lse_out, lse2);
    else
      hipLaunchKernelGGL((merge_kernel<128, 32>), grid, block, 0, stream, part_o, part_lse, heads, n_chunks, out,
                         lse_out, lse2);
  } else {
    if (n_chunks <= 16)
      hipLaunchKernelGGL((merge_kernel<64, 16>), grid, block, 0, stream, part_o, part_lse, heads, n_chunks, out,
                         lse_out, lse2);
    else
      hipLaunchKernelGGL((merge_kernel<64, 32>), grid, block, 0, stream, part_o, part_lse, heads, n_chunks, out,
                         lse_out, lse2);
  }
  return hipGetLastError();
}

hipError_t launch_score(const float* logits, const float* lse2, const int32_t* context_lens,
                        int32_t ctx_bound, int32_t b, int32_t n_q, int32_t logit_stride,
                        float* score, int32_t score_stride, float weight, hipStream_t stream) {
  if (ctx_bound <= 0) return hipSuccess;
  const dim3 grid((unsigned)((ctx_bound + 255) / 256), (unsigned)b);
  hipLaunchKernelGGL(score_kernel, grid, dim3(256), 0, stream, logits, lse2, context_lens,
                     ctx_bound, n_q, logit_stride, score, score_stride, weight / (float)n_q);
  return hipGetLastError();
}

}  // namespace kvd
