// Log-sum-exp merge of per-chunk partials, and the cumulative-score update
// that needs the merged lse.
#include "device_common.h"
#include "kvd_internal.h"

#include <math.h>

namespace kvd {

constexpr float kLog2eMerge = 1.4426950408889634f;
constexpr int kMergeThreads = 256;

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

// Splits of more than kFewChunks chunks (see merge_few_kernel below): one
// workgroup of four waves per (sequence, query head); wave w owns the channels
// [w*D/4, (w+1)*D/4).  lse = M + ln(sum_c exp(lse_c - M)) with M = max_c
// lse_c over all n_chunks chunks; out = sum_c exp(lse_c - lse) * o_c, rounded
// to bf16.  The o_c of a chunk whose weight is 0 (lse_c = -inf) is
// loaded but never used, so it may hold anything, NaN included.  No chunk, or
// only empty ones: out = 0, lse = -inf.
// Every wave computes M and the sum itself with shuffles (no LDS, no
// barrier), and all loads of a batch of up to kBatch chunks per lane are
// issued before any is used, so a merge of a few dozen chunks costs about one
// memory round trip.  Lane l of a wave takes channel l % (D/4) and the chunks
// c = l / (D/4) (mod NG), NG = 256 / D; the NG partial sums of a channel are
// added with shuffles in a fixed order.
template <int D>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse, int32_t n_chunks,
    uint16_t* __restrict__ out, float* __restrict__ lse_out, float* __restrict__ lse2) {
  constexpr int CH = D / 4;                      // channels per wave
  constexpr int NG = 64 / CH;                    // chunk groups per channel
  constexpr int kBatch = 16;                     // chunks per lane loaded at once
  const size_t ih = blockIdx.x;
  // Chunks past a sequence's end, or with nothing attended, carry lse -inf:
  // they weigh 0, so no context length has to be read before the loads go out.
  const int nc = n_chunks;
  const float* pl = part_lse + ih * n_chunks;
  const float* po = part_o + ih * n_chunks * D;
  const int lane = threadIdx.x & 63;
  const int ch = (threadIdx.x >> 6) * CH + lane % CH;
  const int grp = lane / CH;

  // first batch of this lane's partial outputs, loaded before the reductions
  float ov[kBatch];
#pragma unroll
  for (int k = 0; k < kBatch; ++k) {
    const int c = grp + k * NG;
    ov[k] = c < nc ? po[(size_t)c * D + ch] : 0.f;
  }
  // lane c holds lse_c of the first 64 chunks; more chunks are looped over
  const float lv = lane < nc ? pl[lane] : -INFINITY;
  float mx = lv;
  for (int c = lane + 64; c < nc; c += 64) mx = fmaxf(mx, pl[c]);
  const float M = wave_max(mx);
  if (M == -INFINITY) {
    if (grp == 0) out[ih * D + ch] = 0;
    if (threadIdx.x == 0) {
      if (lse_out) lse_out[ih] = -INFINITY;
      if (lse2) lse2[ih] = -INFINITY;
    }
    return;
  }
  float sm = lane < nc ? expf(lv - M) : 0.f;
  for (int c = lane + 64; c < nc; c += 64) sm += expf(pl[c] - M);
  const float lse = M + logf(wave_sum(sm));
  // each lane's weight exp(lse_c - lse) for c = lane, shared by shuffles below
  const float wl = lane < nc ? expf(lv - lse) : 0.f;

  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < kBatch; ++k) {
    const int c = grp + k * NG;                    // < 64: its weight sits in lane c
    const float w = __shfl(wl, c);
    if (c < nc && w != 0.f) acc += w * ov[k];
  }
  for (int c0 = kBatch * NG; c0 < nc; c0 += kBatch * NG) {   // long splits: further batches
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int c = c0 + grp + k * NG;
      ov[k] = c < nc ? po[(size_t)c * D + ch] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int c = c0 + grp + k * NG;
      if (c < nc) {
        const float w = expf(pl[c] - lse);
        if (w != 0.f) acc += w * ov[k];
      }
    }
  }
#pragma unroll
  for (int off = CH; off < 64; off <<= 1) acc += __shfl_xor(acc, off);
  if (grp == 0) out[ih * D + ch] = float_to_bf16_bits(acc);
  if (threadIdx.x == 0) {
    if (lse_out) lse_out[ih] = lse;
    if (lse2) lse2[ih] = lse * kLog2eMerge;
  }
}

// The same merge for splits of at most kFewChunks chunks, one wave per
// (sequence, query head) and four heads per workgroup: with many heads and few
// chunks (a large batch of short contexts) a workgroup per head would make
// the launch mostly workgroup dispatch.  Lane l takes channels l, l + 64, ...
// and all the chunks; lane c holds lse_c.  All partial outputs are loaded
// before the reductions, and each channel's sum runs in chunk order.
constexpr int kFewChunks = 16;

template <int D>
__global__ __launch_bounds__(kMergeThreads) void merge_few_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse, int64_t n_heads,
    int32_t n_chunks, uint16_t* __restrict__ out, float* __restrict__ lse_out, float* __restrict__ lse2) {
  constexpr int PER = D / 64;                    // channels per lane
  const int lane = threadIdx.x & 63;
  const int64_t ih = (int64_t)blockIdx.x * (kMergeThreads / 64) + (threadIdx.x >> 6);
  if (ih >= n_heads) return;                     // the whole wave
  const int nc = n_chunks;                       // 1 .. kFewChunks
  const float* pl = part_lse + ih * nc;
  const float* po = part_o + ih * nc * D + lane;
  float ov[kFewChunks][PER];
#pragma unroll
  for (int c = 0; c < kFewChunks; ++c)
#pragma unroll
    for (int p = 0; p < PER; ++p) ov[c][p] = c < nc ? po[(size_t)c * D + 64 * p] : 0.f;
  const float lv = lane < nc ? pl[lane] : -INFINITY;
  const float M = wave_max(lv);
  uint16_t* o = out + ih * D + lane;
  if (M == -INFINITY) {
#pragma unroll
    for (int p = 0; p < PER; ++p) o[64 * p] = 0;
    if (lane == 0) {
      if (lse_out) lse_out[ih] = -INFINITY;
      if (lse2) lse2[ih] = -INFINITY;
    }
    return;
  }
  const float lse = M + logf(wave_sum(lane < nc ? expf(lv - M) : 0.f));
  const float wl = lane < nc ? expf(lv - lse) : 0.f;
  float acc[PER];
#pragma unroll
  for (int p = 0; p < PER; ++p) acc[p] = 0.f;
#pragma unroll
  for (int c = 0; c < kFewChunks; ++c) {
    if (c < nc) {                                // uniform
      const float w = __shfl(wl, c);
      if (w != 0.f) {                            // uniform: an empty chunk's o_c is never used
#pragma unroll
        for (int p = 0; p < PER; ++p) acc[p] += w * ov[c][p];
      }
    }
  }
#pragma unroll
  for (int p = 0; p < PER; ++p) o[64 * p] = float_to_bf16_bits(acc[p]);
  if (lane == 0) {
    if (lse_out) lse_out[ih] = lse;
    if (lse2) lse2[ih] = lse * kLog2eMerge;
  }
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
  if (n_chunks <= kFewChunks) {
    const int64_t heads = (int64_t)b * n_q;
    const dim3 grid((unsigned)((heads + kMergeThreads / 64 - 1) / (kMergeThreads / 64)));
    if (head_dim == 128)
      hipLaunchKernelGGL(merge_few_kernel<128>, grid, dim3(kMergeThreads), 0, stream, part_o, part_lse, heads,
                         n_chunks, out, lse_out, lse2);
    else
      hipLaunchKernelGGL(merge_few_kernel<64>, grid, dim3(kMergeThreads), 0, stream, part_o, part_lse, heads,
                         n_chunks, out, lse_out, lse2);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((size_t)b * n_q));
  if (head_dim == 128)
    hipLaunchKernelGGL(merge_kernel<128>, grid, dim3(kMergeThreads), 0, stream, part_o, part_lse,
                       n_chunks, out, lse_out, lse2);
  else
    hipLaunchKernelGGL(merge_kernel<64>, grid, dim3(kMergeThreads), 0, stream, part_o, part_lse,
                       n_chunks, out, lse_out, lse2);
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
