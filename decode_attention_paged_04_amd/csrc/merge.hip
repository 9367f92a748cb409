// Log-sum-exp merge of per-chunk partials, and the cumulative-score update
// that needs the merged lse.
#include "device_common.h"
#include "kvd_internal.h"

#include <math.h>

namespace kvd {

// Log-sum-exp merge of one (sequence, query head)'s per-chunk partials:
// lse = M + ln(sum_c exp(lse_c - M)) with M = max_c lse_c, and
// out = sum_c exp(lse_c - lse) * o_c rounded to bf16.  A chunk whose weight
// is 0 (lse_c = -inf: nothing attended) adds nothing, whatever its o_c holds
// (NaN included); no chunk with weight gives out = 0 and lse = -inf.
constexpr float kMergeLog2e = 1.4426950408889634f;

// Max and sum over the lanes that differ only in the row bits (lanes l and
// l ^ Q, l ^ 2Q, ... hold the same four channels of different rows).
template <int Q>
__device__ inline float row_max(float v) {
#pragma unroll
  for (int off = Q; off < 64; off <<= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

template <int Q>
__device__ inline float row_sum(float v) {
#pragma unroll
  for (int off = Q; off < 64; off <<= 1) v += __shfl_xor(v, off);
  return v;
}

// One wave per (head, slice of 256/R channels).  Lane l takes four channels,
// 4(l % Q) .. 4(l % Q) + 3 of the slice (Q = 64/R lanes across), as one
// 16-byte load per chunk, for the chunk rows l/Q, l/Q + R, l/Q + 2R, ...; the
// lanes of a row also read its lse.  KR rows per lane (R * KR chunks) are
// loaded before any is used, so a merge of that many chunks costs about one
// memory round trip; a row past the last chunk reads as lse = -inf and weighs
// 0.  Each lane adds its rows in order, and the R rows' sums are then added
// by butterfly shuffles over the row bits of the lane index: a fixed order
// for given R and KR.  R and KR are picked per launch from the number of heads
// and chunks (merge_shape).  part_o 16-byte aligned, out 8-byte.
template <int D, int R, int KR>
__global__ __launch_bounds__(256) void merge_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse, int64_t n_waves,
    int32_t n_chunks, uint16_t* __restrict__ out, float* __restrict__ lse_out, float* __restrict__ lse2) {
  constexpr int Q = 64 / R;                      // lanes across a row
  constexpr int DS = 4 * Q;                      // channels per wave
  constexpr int S = D / DS;                      // waves per head
  static_assert(S >= 1 && D % DS == 0, "a slice holds at most one head");
  const int64_t wv = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (wv >= n_waves) return;                     // the whole wave
  const int lane = threadIdx.x & 63;
  const int q = lane % Q, r0 = lane / Q;
  const int64_t ih = wv / S;
  const int sl = (int)(wv % S);
  const int nc = n_chunks;
  const float* pl = part_lse + ih * nc;
  const float* po = part_o + ih * nc * D + DS * sl + 4 * q;

  float lv[KR];
  f32x4 ov[KR];
  auto load_group = [&](int c0) {
#pragma unroll
    for (int k = 0; k < KR; ++k) {
      const int c = c0 + r0 + R * k;
      lv[k] = c < nc ? pl[c] : -INFINITY;
      ov[k] = c < nc ? *reinterpret_cast<const f32x4*>(po + (size_t)c * D) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  load_group(0);
  float mx = lv[0];
#pragma unroll
  for (int k = 1; k < KR; ++k) mx = fmaxf(mx, lv[k]);
  for (int c = R * KR + r0; c < nc; c += R) mx = fmaxf(mx, pl[c]);
  const float M = row_max<Q>(mx);
  uint16_t* dst = out + ih * D + DS * sl + 4 * q;
  if (M == -INFINITY) {
    if (r0 == 0) *reinterpret_cast<u32x2*>(dst) = u32x2{0u, 0u};
    if (lane == 0 && sl == 0) {
      if (lse_out) lse_out[ih] = -INFINITY;
      if (lse2) lse2[ih] = -INFINITY;
    }
    return;
  }
  float sm = 0.f;
#pragma unroll
  for (int k = 0; k < KR; ++k) sm += expf(lv[k] - M);
  for (int c = R * KR + r0; c < nc; c += R) sm += expf(pl[c] - M);
  const float lse = M + logf(row_sum<Q>(sm));
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < nc; c0 += R * KR) {      // uniform
    if (c0 > 0) load_group(c0);
#pragma unroll
    for (int k = 0; k < KR; ++k) {
      const float w = expf(lv[k] - lse);
      if (w != 0.f) acc += w * ov[k];
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) acc[e] = row_sum<Q>(acc[e]);
  if (r0 == 0) {
    const uint32_t lo2 = (uint32_t)float_to_bf16_bits(acc[0]) | ((uint32_t)float_to_bf16_bits(acc[1]) << 16);
    const uint32_t hi2 = (uint32_t)float_to_bf16_bits(acc[2]) | ((uint32_t)float_to_bf16_bits(acc[3]) << 16);
    *reinterpret_cast<u32x2*>(dst) = u32x2{lo2, hi2};
  }
  if (lane == 0 && sl == 0) {
    if (lse_out) lse_out[ih] = lse;
    if (lse2) lse2[ih] = lse * kMergeLog2e;
  }
}

// Rows per wave R: from the fewest (one wave per head for d_h = 128) up,
// doubled while the rows stay fewer than the chunks and the doubled launch
// stays below 2,048 waves -- a launch with few heads spreads each head over
// several CUs, one with many keeps a wave per head.  (Measured per call: the 8B
// layer's 32 heads x 32 chunks at R = 16, 3.5 us faster than a wave per head;
// 1,024 heads x 16 chunks at R = 2, 1.4 us faster than at R = 4.)  Rows per lane KR: enough for
// every chunk (a power of two, at most 8; beyond 8R chunks the lanes loop).
static void merge_shape(int64_t heads, int32_t n_chunks, int32_t head_dim, int* r_out, int* kr_out) {
  int r = 256 / head_dim;
  while (r < 16 && r < n_chunks && heads * (head_dim * 2 * r / 256) < 2048) r *= 2;
  int kr = 1;
  while (kr < 8 && r * kr < n_chunks) kr *= 2;
  *r_out = r;
  *kr_out = kr;
}

template <int D, int R, int KR>
static void launch_merge_r(const float* part_o, const float* part_lse, int64_t heads, int32_t n_chunks,
                           uint16_t* out, float* lse_out, float* lse2, hipStream_t stream) {
  const int64_t waves = heads * (D * R / 256);
  // under 1,024 waves, one wave per workgroup spreads them over more CUs
  const int wpg = waves >= 1024 ? 4 : 1;
  const dim3 grid((unsigned)((waves + wpg - 1) / wpg));
  hipLaunchKernelGGL((merge_kernel<D, R, KR>), grid, dim3(64 * wpg), 0, stream, part_o, part_lse, waves,
                     n_chunks, out, lse_out, lse2);
}

template <int D, int R>
static void launch_merge_kr(int kr, const float* part_o, const float* part_lse, int64_t heads, int32_t n_chunks,
                            uint16_t* out, float* lse_out, float* lse2, hipStream_t stream) {
  switch (kr) {
    case 1: launch_merge_r<D, R, 1>(part_o, part_lse, heads, n_chunks, out, lse_out, lse2, stream); break;
    case 2: launch_merge_r<D, R, 2>(part_o, part_lse, heads, n_chunks, out, lse_out, lse2, stream); break;
    case 4: launch_merge_r<D, R, 4>(part_o, part_lse, heads, n_chunks, out, lse_out, lse2, stream); break;
    default: launch_merge_r<D, R, 8>(part_o, part_lse, heads, n_chunks, out, lse_out, lse2, stream); break;
  }
}

template <int D>
static void launch_merge_d(int r, int kr, const float* part_o, const float* part_lse, int64_t heads,
                           int32_t n_chunks, uint16_t* out, float* lse_out, float* lse2, hipStream_t stream) {
  switch (r) {
    case 2:
      if constexpr (D == 128) launch_merge_kr<D, 2>(kr, part_o, part_lse, heads, n_chunks, out, lse_out, lse2, stream);
      break;
    case 4: launch_merge_kr<D, 4>(kr, part_o, part_lse, heads, n_chunks, out, lse_out, lse2, stream); break;
    case 8: launch_merge_kr<D, 8>(kr, part_o, part_lse, heads, n_chunks, out, lse_out, lse2, stream); break;
    default: launch_merge_kr<D, 16>(kr, part_o, part_lse, heads, n_chunks, out, lse_out, lse2, stream); break;
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
  const int64_t heads = (int64_t)b * n_q;
  int r, kr;
  merge_shape(heads, n_chunks, head_dim, &r, &kr);
  if (head_dim == 128)
    launch_merge_d<128>(r, kr, part_o, part_lse, heads, n_chunks, out, lse_out, lse2, stream);
  else
    launch_merge_d<64>(r, kr, part_o, part_lse, heads, n_chunks, out, lse_out, lse2, stream);
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
