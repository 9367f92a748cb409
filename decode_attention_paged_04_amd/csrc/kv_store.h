// Storing token rows into one (block, KV head) tile of the pool: the bf16
// copy and the FP8 E4M3 quantisation.  Shared by the write kernel and the
// decode kernel's fused append, so that both leave the same bytes.
#pragma once

#include "device_common.h"
#include "kvd_internal.h"

#include <math.h>

namespace kvd {

// Nearest-even E4M3FN code of y, saturating at +-448 (sign kept, -0 -> 0x80).
__device__ inline uint32_t e4m3_encode(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fabsf(y);
  uint32_t code;
  if (!(a < 448.0f)) {
    code = 0x7Eu;
  } else if (a < 0.015625f) {                       // below 2^-6: grid of m * 2^-9
    code = (uint32_t)rintf(a * 512.0f);             // exact scaling; rint ties to even
  } else {
    const uint32_t ab = __float_as_uint(a);
    const uint32_t e = (ab >> 23) - 127u + 7u;      // biased E4M3 exponent, 1..15
    const uint32_t mant = ab & 0x7FFFFFu;
    uint32_t q = (e << 3) | (mant >> 20);
    const uint32_t rem = mant & 0xFFFFFu;
    q += (rem > 0x80000u) || (rem == 0x80000u && (q & 1u));   // carry may bump the exponent
    code = q;
  }
  return sign | code;
}

// Widen one E4M3FN code to fp32 with the conversion the decode kernels use
// (exact: every E4M3FN value is a bf16 value).
__device__ inline float e4m3_to_float(uint32_t code) {
  return (float)__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(code, 1.0f, false)[0];
}

// One wave stores rows r0 .. r0+n-1 (n >= 1, r0 + n <= 16) of the K (which = 0)
// or V (which = 1) tile of an FP8 (block, KV head) from bf16 rows src[r *
// row_stride + ch].  Rows below r0 already hold codes under the tile's current
// scale *scale_at.  The tile keeps one scale: absmax / 448 over the old rows as
// they read back (code value x old scale, fp32) and the new rows.  Old codes
// are re-encoded from their read-back values only if the scale changed; new
// rows are encoded under the new scale.  r0 = 0 is the plain block
// quantisation.  Every load is issued before any is used.  Returns the new
// scale (also stored to *scale_at by lane 0).
template <int D>
__device__ inline float fp8_store_rows(uint8_t* __restrict__ tile, float* __restrict__ scale_at, int which,
                                       int r0, int n, const uint16_t* __restrict__ src, size_t row_stride,
                                       int lane) {
  constexpr int CPL = D / 64;                       // channels per lane: lane, lane + 64
  auto at = [&](int r, int ch) -> uint8_t& { return tile[which ? v_elem(r, ch, D) : k_elem(r, ch, D, 1)]; };
  const float s_old = r0 > 0 ? *scale_at : 0.f;
  uint32_t old[kBlock][CPL];
  float fresh[kBlock][CPL];
#pragma unroll
  for (int r = 0; r < kBlock; ++r) {
#pragma unroll
    for (int q = 0; q < CPL; ++q) {
      const int ch = lane + 64 * q;
      old[r][q] = r < r0 ? (uint32_t)at(r, ch) : 0u;
      fresh[r][q] = r < n ? bf16_bits_to_float(src[r * row_stride + ch]) : 0.f;
    }
  }
  float am = 0.f;
#pragma unroll
  for (int r = 0; r < kBlock; ++r) {
#pragma unroll
    for (int q = 0; q < CPL; ++q) {
      if (r < r0) am = fmaxf(am, fabsf(e4m3_to_float(old[r][q]) * s_old));
      if (r < n) am = fmaxf(am, fabsf(fresh[r][q]));
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) am = fmaxf(am, __shfl_xor(am, off));
  const float scale = am / 448.0f;

  const bool reencode = r0 > 0 && scale != s_old;
#pragma unroll
  for (int r = 0; r < kBlock; ++r) {
#pragma unroll
    for (int q = 0; q < CPL; ++q) {
      const int ch = lane + 64 * q;
      if (reencode && r < r0) {
        const float x = e4m3_to_float(old[r][q]) * s_old;
        at(r, ch) = (uint8_t)(scale == 0.f ? 0u : e4m3_encode(x / scale));
      }
      if (r < n) at(r0 + r, ch) = (uint8_t)(scale == 0.f ? 0u : e4m3_encode(fresh[r][q] / scale));
    }
  }
  if (lane == 0) *scale_at = scale;
  return scale;
}

// One wave stores row `row` of a bf16 (block, KV head) tile pair from the K
// and V rows k_row[ch], v_row[ch].
template <int D>
__device__ inline void bf16_store_row(uint16_t* __restrict__ tile, int row, const uint16_t* __restrict__ k_row,
                                      const uint16_t* __restrict__ v_row, int lane) {
#pragma unroll
  for (int ch = lane; ch < D; ch += 64) {
    tile[k_elem(row, ch, D, 2)] = k_row[ch];
    tile[v_elem(row, ch, D)] = v_row[ch];
  }
}

}  // namespace kvd
