// Storing new tokens into the pool (bf16 copy, FP8 E4M3 quantisation) and the
// test hooks that expose the decode kernels' addressing, FP8 widening and
// streaming read.
#include "device_common.h"
#include "kv_store.h"
#include "kvd_internal.h"

#include <math.h>

namespace kvd {

// One thread per (token, KV head, channel): K goes token-major, V channel-major.
template <int D>
__global__ __launch_bounds__(256) void write_bf16_kernel(char* __restrict__ layer_base,
                                                         int32_t num_blocks, int32_t n_kv,
                                                         const uint16_t* __restrict__ k,
                                                         const uint16_t* __restrict__ v,
                                                         const int32_t* __restrict__ slots,
                                                         int32_t n_tok) {
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t total = (size_t)n_tok * n_kv * D;
  if (e >= total) return;
  const int ch = (int)(e % D);
  const int j = (int)((e / D) % n_kv);
  const size_t t = e / ((size_t)D * n_kv);
  const int32_t slot = slots[t];
  if (slot < 0) return;
  const int32_t p = slot / kBlock;
  const int row = slot % kBlock;
  if (p >= num_blocks) return;
  uint16_t* tile = reinterpret_cast<uint16_t*>(layer_base + ((size_t)p * n_kv + j) * (2 * kBlock * D * 2));
  tile[k_elem(row, ch, D, 2)] = k[e];
  tile[v_elem(row, ch, D)] = v[e];
}

// One wave per (run, KV head, K|V).  A run is a maximal stretch of entries of
// the slot mapping that fill consecutive rows r0, r0+1, ... of one block; rows
// below r0 already hold codes under the tile's current scale.  The tile keeps
// one scale: absmax / 448 over the old rows as they read back (code value x old
// scale, fp32) and the run's new rows.  Old codes are re-encoded from their
// read-back values only if the scale changed; new rows are encoded under the
// new scale.  A run starting at row 0 is the plain block quantisation.
// The slots around the entry are read with one vector load; the tile is then
// stored by fp8_store_rows.
template <int D>
__global__ __launch_bounds__(64) void write_fp8_kernel(char* __restrict__ layer_base,
                                                       float* __restrict__ layer_scales,
                                                       int32_t num_blocks, int32_t n_kv,
                                                       const uint16_t* __restrict__ k,
                                                       const uint16_t* __restrict__ v,
                                                       const int32_t* __restrict__ slots,
                                                       int32_t n_tok) {
  const int t = blockIdx.x;
  const int j = blockIdx.y;
  const int which = blockIdx.z;                     // 0: K, 1: V
  const int lane = threadIdx.x;
  const int32_t slot = slots[t];
  const int32_t prev = t > 0 ? slots[t - 1] : -2;
  const int32_t next = lane < kBlock - 1 && t + 1 + lane < n_tok ? slots[t + 1 + lane] : -2;
  if (slot < 0) return;
  const int32_t p = slot / kBlock;
  if (p >= num_blocks) return;
  const int r0 = slot % kBlock;
  // Only the first entry of a run does the work; the run goes on while the
  // following entries take the next rows of the same block.
  if (r0 != 0 && prev == slot - 1) return;
  const uint64_t cont = __ballot(lane < kBlock - 1 - r0 && next == slot + 1 + lane);
  const int n = 1 + __builtin_ctzll(~cont);

  const uint16_t* src = (which ? v : k) + ((size_t)t * n_kv + j) * D;
  uint8_t* tile = reinterpret_cast<uint8_t*>(layer_base + ((size_t)p * n_kv + j) * (2 * kBlock * D));
  float* scale_at = layer_scales + ((size_t)j * num_blocks + p) * 2 + which;   // head-major
  fp8_store_rows<D>(tile, scale_at, which, r0, n, src, (size_t)n_kv * D, lane);
}

hipError_t launch_write(const PoolView& pv, int32_t layer, const uint16_t* k, const uint16_t* v,
                        const int32_t* slots, int32_t n_tok, hipStream_t stream) {
  char* base = pv.kv_base + (size_t)layer * (size_t)pv.layer_bytes;
  const int D = pv.head_dim;
  if (pv.dtype == KVD_BF16) {
    const size_t total = (size_t)n_tok * pv.n_kv * D;
    const dim3 grid((unsigned)((total + 255) / 256));
    if (D == 128)
      hipLaunchKernelGGL(write_bf16_kernel<128>, grid, dim3(256), 0, stream, base, pv.num_blocks,
                         pv.n_kv, k, v, slots, n_tok);
    else
      hipLaunchKernelGGL(write_bf16_kernel<64>, grid, dim3(256), 0, stream, base, pv.num_blocks,
                         pv.n_kv, k, v, slots, n_tok);
  } else {
    float* sc = pv.scale_base + (size_t)layer * pv.num_blocks * pv.n_kv * 2;
    const dim3 grid((unsigned)n_tok, (unsigned)pv.n_kv, 2);
    if (D == 128)
      hipLaunchKernelGGL(write_fp8_kernel<128>, grid, dim3(64), 0, stream, base, sc,
                         pv.num_blocks, pv.n_kv, k, v, slots, n_tok);
    else
      hipLaunchKernelGGL(write_fp8_kernel<64>, grid, dim3(64), 0, stream, base, sc,
                         pv.num_blocks, pv.n_kv, k, v, slots, n_tok);
  }
  return hipGetLastError();
}

// Slots of tokens [first_i, s_i) of every sequence i: token t lives in
// physical block block_table[i][t / 16] at in-block row t % 16, slot
// block * 16 + row.  Workgroup x serves sequence x / groups and its tokens
// first_i + 256 (x % groups) + thread; the slot of token t goes to
// slots[out_start[i] + t - first_i].
__global__ __launch_bounds__(256) void slot_mapping_kernel(const int32_t* __restrict__ bt, int32_t max_blocks,
                                                           const int32_t* __restrict__ lens,
                                                           const int32_t* __restrict__ first,
                                                           const int64_t* __restrict__ out_start,
                                                           int32_t groups, int32_t* __restrict__ slots,
                                                           int64_t n_slots) {
  const int i = blockIdx.x / groups;
  const int cap = max_blocks * kBlock;
  int s = lens[i];
  s = s < 0 ? 0 : (s > cap ? cap : s);
  int f = first ? first[i] : 0;
  f = f < 0 ? 0 : (f > s ? s : f);
  const int t = f + (int)(blockIdx.x % groups) * 256 + (int)threadIdx.x;
  if (t >= s) return;
  const int64_t o = out_start[i] + (t - f);
  if (o < 0 || o >= n_slots) return;
  const int32_t e = bt[(size_t)i * max_blocks + t / kBlock];
  // a slot is an int32: blocks from 2^27 on have none
  slots[o] = (e < 0 || e >= (1 << 27)) ? -1 : e * kBlock + t % kBlock;
}

hipError_t launch_slot_mapping(const int32_t* bt, int32_t max_blocks, int32_t b, const int32_t* lens,
                               const int32_t* first, const int64_t* out_start, int32_t max_tokens,
                               int32_t* slots, int64_t n_slots, hipStream_t stream) {
  const int32_t groups = (max_tokens + 255) / 256;
  if (groups == 0 || b == 0) return hipSuccess;
  hipLaunchKernelGGL(slot_mapping_kernel, dim3((unsigned)((int64_t)b * groups)), dim3(256), 0, stream, bt,
                     max_blocks, lens, first, out_start, groups, slots, n_slots);
  return hipGetLastError();
}

// Element offsets of K[t][0] and V[t][0] through the decode kernels' rule.
__global__ __launch_bounds__(256) void debug_offsets_kernel(int64_t layer_elem0, int32_t num_blocks,
                                                            int32_t n_kv, int32_t head_dim,
                                                            int32_t elem_bytes,
                                                            const int32_t* __restrict__ bt,
                                                            int32_t max_blocks, int32_t b,
                                                            int32_t n_tok, int64_t* out_k,
                                                            int64_t* out_v) {
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t total = (size_t)b * n_kv * n_tok;
  if (e >= total) return;
  const int t = (int)(e % n_tok);
  const int j = (int)((e / n_tok) % n_kv);
  const int i = (int)(e / ((size_t)n_tok * n_kv));
  const int32_t p = bt[(size_t)i * max_blocks + t / kBlock];
  const uint32_t tpb = (uint32_t)(2 * kBlock * head_dim * elem_bytes);
  const uint32_t off = tile_pair_offset(p, j, num_blocks, n_kv, tpb);
  if (off == kOutOfRange) {
    out_k[e] = -1;
    out_v[e] = -1;
    return;
  }
  const int64_t tile_elem = layer_elem0 + (int64_t)(off / (uint32_t)elem_bytes);
  out_k[e] = tile_elem + k_elem(t % kBlock, 0, head_dim, elem_bytes);
  out_v[e] = tile_elem + v_elem(t % kBlock, 0, head_dim);
}

hipError_t launch_debug_offsets(const PoolView& pv, int32_t layer, const int32_t* bt,
                                int32_t max_blocks, int32_t b, int32_t n_tok, int64_t* out_k,
                                int64_t* out_v, hipStream_t stream) {
  const size_t total = (size_t)b * pv.n_kv * n_tok;
  if (total == 0) return hipSuccess;
  const int64_t layer_elem0 = (int64_t)layer * pv.layer_bytes / pv.elem_bytes;
  hipLaunchKernelGGL(debug_offsets_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                     stream, layer_elem0, pv.num_blocks, pv.n_kv, pv.head_dim,
                     (int32_t)pv.elem_bytes, bt, max_blocks, b, n_tok, out_k, out_v);
  return hipGetLastError();
}

// Each thread widens 8 codes with the decode kernels' routine.
__global__ __launch_bounds__(256) void debug_fp8_kernel(const uint8_t* __restrict__ codes,
                                                        int32_t n, float* __restrict__ out) {
  const int q = blockIdx.x * 256 + threadIdx.x;
  const int base = q * 8;
  if (base >= n) return;
  uint32_t w[2] = {0u, 0u};
  for (int e = 0; e < 8 && base + e < n; ++e) w[e >> 2] |= (uint32_t)codes[base + e] << (8 * (e & 3));
  const bf16x8 r = e4m3x8_to_bf16x8(w[0], w[1]);
  for (int e = 0; e < 8 && base + e < n; ++e) out[base + e] = (float)r[e];
}

hipError_t launch_debug_fp8_decode(const uint8_t* codes, int32_t n, float* out,
                                   hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int groups = (n + 7) / 8;
  hipLaunchKernelGGL(debug_fp8_kernel, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0,
                     stream, codes, n, out);
  return hipGetLastError();
}

// A plain streaming read of `bytes` bytes with the decode kernels' 16-byte
// non-temporal buffer loads: workgroup w reads 16-byte units w*256*U + u*256 +
// thread, then steps by grid*256*U units, with U loads in flight per thread;
// each thread XORs every 32-bit word it read into sink[w*256 + thread].
template <int U>
__global__ __launch_bounds__(256) void stream_read_kernel(const void* __restrict__ data, uint32_t bytes,
                                                         uint32_t* __restrict__ sink) {
  const __amdgpu_buffer_rsrc_t r = make_rsrc(data, bytes);
  const uint32_t units = bytes / 16;
  const uint32_t stride = gridDim.x * 256u * U;
  uint32_t acc = 0;
  for (uint32_t base = blockIdx.x * 256u * U; base < units; base += stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t k = base + 256u * u + threadIdx.x;
      v[u] = load16(r, k < units ? k * 16u : kOutOfRange);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  sink[blockIdx.x * 256 + threadIdx.x] = acc;
}

hipError_t launch_stream_read(const void* data, uint32_t bytes, uint32_t* sink, int32_t grid,
                              hipStream_t stream) {
  hipLaunchKernelGGL(stream_read_kernel<8>, dim3((unsigned)grid), dim3(256), 0, stream, data, bytes, sink);
  return hipGetLastError();
}

}  // namespace kvd
