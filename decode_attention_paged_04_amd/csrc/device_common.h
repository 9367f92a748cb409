// Device helpers shared by the kernels: vector types, bounded buffer loads,
// the pool addressing rule and the E4M3 -> bf16 widening.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvd {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

// Buffer resource word 3 for gfx9-family raw buffers (32-bit data format);
// with stride 0 the record count is a byte count and every load outside
// [0, num_records) returns zeros instead of touching memory.
constexpr int kRawBufferWord3 = 0x00020000;
constexpr uint32_t kOutOfRange = 0xFFFFFFFFu;

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kRawBufferWord3);
}

// Cache policy of the K/V stream: "nt" (non-temporal).  Every cached byte is
// read exactly once per decode step, so the lines need not be kept; on gfx950
// a plain streaming read of 2 GB measured 7.1 TB/s with the hint against
// 6.2 TB/s without it.
constexpr int kStreamPolicy = 2;

__device__ inline u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kStreamPolicy));
}

__device__ inline u32x2 load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kStreamPolicy));
}

// Read of memory that no kernel writes while this one runs (block tables,
// scales).  Through the constant address space a wave-uniform address becomes a
// scalar load, whose wait (lgkmcnt) is independent of the vector loads and
// stores in flight; a vector load here would need vmcnt(0) before its
// readfirstlane and so drain every K/V load of the wave.
template <typename T>
__device__ inline T load_invariant(const T* p) {
  return *(const __attribute__((address_space(4))) T*)p;
}

// Byte offset, from the start of a layer, of the tile pair of (block p, KV head
// j); kOutOfRange for a block id outside the pool, so every load through it
// reads zeros.
__host__ __device__ inline uint32_t tile_pair_offset(int32_t p, int32_t j, int32_t num_blocks,
                                                     int32_t n_kv, uint32_t tile_pair_bytes) {
  if ((uint32_t)p >= (uint32_t)num_blocks) return kOutOfRange;
  return ((uint32_t)p * (uint32_t)n_kv + (uint32_t)j) * tile_pair_bytes;
}

// Element offsets inside a tile pair (w = elem_bytes, n = 16 / w elements per
// 16 bytes, P = head_dim / n pieces per row).  The K tile is stored as 16-byte
// pieces in the operand order of the decode kernels' q.K^T MFMA.  Channel c
// belongs to MFMA step c / 32 and lane group (c / 8) % 4; a piece holds the
// 8-channel slices of one lane group for n / 8 consecutive steps (one for
// bf16, two for FP8): piece 4 (step / (n/8)) + group of the row, position
// 8 (step % (n/8)) + c % 8.  Row t's piece q is piece (s * P + q) * 8 + r of
// the tile, s = (t / 4) % 2, r = 4 (t / 8) + t % 4, so the 32 lanes that read
// one block in one load instruction read 512 contiguous bytes, and bf16 and
// FP8 tiles put the same channels in the same lanes.  The V tile is
// channel-major: 16 consecutive rows of each channel.
__host__ __device__ inline uint32_t k_elem(int row, int ch, int head_dim, int elem_bytes) {
  const int n = 16 / elem_bytes;
  const int per = n / 8;
  const int s = (row >> 2) & 1;
  const int r = ((row >> 3) << 2) | (row & 3);
  const int step = ch >> 5, group = (ch >> 3) & 3;
  const int q = 4 * (step / per) + group;
  return (uint32_t)(((s * (head_dim / n) + q) * 8 + r) * n + 8 * (step % per) + (ch & 7));
}
__host__ __device__ inline uint32_t v_elem(int row, int ch, int head_dim) {
  return (uint32_t)(16 * head_dim + ch * 16 + row);
}

// Widen 8 E4M3FN codes (two dwords, code k in byte k % 4 of dword k / 4) to
// bf16 in order.  E4M3FN -> bf16 is exact: 3 mantissa bits fit in 7 and the
// exponent range (2^-9 .. 448) lies inside bf16's normal range.  gfx950's
// scaled conversion is used with scale 1.0, i.e. a plain conversion.
__device__ inline bf16x8 e4m3x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

__device__ inline float bf16_bits_to_float(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// Round to nearest even; NaN stays NaN.
__device__ inline uint16_t float_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

}  // namespace kvd
