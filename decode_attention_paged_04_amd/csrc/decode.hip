// Split-context paged GQA decode attention for gfx950.
//
// One workgroup = one (sequence i, KV head j, context chunk c); its four waves
// take the chunk's 16-token blocks two at a time ("pairs", 32 tokens) in
// round-robin order.  For every pair a wave:
//   * reads the two physical block ids from the block table and streams the
//     pair's K and V tiles from HBM straight into registers, in the operand
//     layout of the 16x16x32 bf16 MFMA (16-byte loads through a bounded buffer
//     resource, so a bad block id reads zeros instead of faulting).  The loads
//     of the wave's next pair are issued before the current pair is consumed,
//     so two pairs (32 KiB for bf16, d_h = 128) are in flight per wave;
//   * computes S = K q^T for all g query heads of KV head j at once (MFMA rows =
//     tokens, columns = heads, so each K tile is read once and shared by the g
//     heads -- the GQA saving);
//   * folds S into a running max / sum per head (online softmax in the log2
//     domain, fp32), and accumulates O^T += V^T P^T with a second MFMA whose
//     rows are channels and columns heads.  P is split into bf16 hi + lo parts
//     so that the product keeps ~16 bits of P (a single bf16 P would add a
//     relative error of ~1e-3 to the output).
// The four waves' (max, sum, O) are then combined through LDS and written
// either as the final bf16 output (single chunk) or as an fp32 partial
// (o_c normalised, lse_c natural log) for the log-sum-exp merge kernel.
//
// Operand layout of v_mfma_f32_16x16x32_bf16 (lane l, G = l / 16, r = l % 16):
// A[row r][k in group G], B[k in group G][col r], D[row 4G + q][col r], q < 4.
// Which 8 of the 32 k indices a group holds is irrelevant here because A and
// B use the same assignment; the code only relies on rows = r, cols = r and
// the D layout.  Token/channel assignment chosen below:
//   * S-tile t (t = 0, 1) row r  <-> pair token 8*(r/4) + 4t + r%4, so lane
//     (G, r) ends up holding, for head r, the pair tokens 8G .. 8G+7
//     (D row 4G+q of tile t is token 8G + 4t + q);
//   * those 8 tokens are exactly the k group G of the P.V product, and they
//     are 8 consecutive rows of block G/2 -- 16 contiguous bytes of one
//     channel row of the channel-major V tile.
#include "device_common.h"
#include "kv_store.h"
#include "kvd_internal.h"

#include <math.h>

#include <type_traits>

namespace kvd {

constexpr int kWaves = 4;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Registers holding one pair's K/V (and, for FP8, its scales) between the
// loads and their use.
template <int D, bool FP8>
struct PairRegs {
  static constexpr int E = FP8 ? 1 : 2;        // bytes per element
  static constexpr int KU = D * E / 64;        // 16-byte K units per lane per S-tile
  static constexpr int NM = D / 16;            // 16-channel tiles of the output
  u32x4 k[2][KU];
  u32x4 v[FP8 ? 1 : NM];                       // bf16 V: 16 B per lane per channel tile
  u32x2 v8[FP8 ? NM : 1];                      // FP8 V: 8 B per lane per channel tile
  float sK, sV;                                // FP8 scales of this lane's block
  uint32_t drop;                               // bit k: block k of the pair is not attended
};

// k index group G of MFMA step c covers channels 32c + 8G .. +7 of q and K
// (for bf16 and FP8 tiles alike: the K layout puts them in that lane).
__device__ inline int qk_channel0(int c, int G) { return 32 * c + 8 * G; }

// Launch order of the (sequence, chunk) units.  Per KV head the grid holds
// b * n_chunks units, n_chunks covering the longest allowed context, but a
// sequence of s tokens fills only ceil(s / chunk) of its chunks.  Workgroup x
// takes unit k = x / n_kv of this order (and the KV head and span chunk_span
// gives it), in three runs:
// the full chunks chunk-major (chunk 0 of every sequence that has it, in
// sequence order, then chunk 1, ...), then the partly filled last chunks, then
// the empty chunks, sequence by sequence.  The hardware hands out workgroups in grid
// order, so the shorter units run last and the final workgroups drain sooner;
// an empty chunk only marks itself empty for the merge (or writes a zero
// output), and at the end of the grid such workgroups no longer hold compute
// units while chunks with tokens wait.  The runs are counted with even chunks
// of C tokens; with uneven chunk pairs a chunk near a sequence's end may hold a
// few more or fewer tokens than that count says, which moves work between the
// runs but never changes which tokens a unit covers.
// Each wave finds its unit itself, in two rounds of loads whatever b is: lane
// l owns sequences [l per, (l + 1) per), per = ceil(b / 64), and counts their
// chunks of each kind (its loads are independent of one another); a prefix
// sum over the lanes finds the lane that owns unit k, and a second prefix sum
// over that lane's sequences finds the sequence and chunk.
struct Unit {
  int i, c, s;                                  // sequence, chunk, clamped context length
};

__device__ inline int wave_inclusive_sum(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(v, d);
    if (lane >= d) v += t;
  }
  return v;
}

__device__ inline Unit locate_unit(const DecodeLaunch& a, int k) {
  const int lane = threadIdx.x & 63;
  auto length = [&](int q) {
    int s = q < a.b ? a.context_lens[q] : 0;
    return s < 0 ? 0 : (s > a.ctx_bound ? a.ctx_bound : s);
  };
  const int per = (a.b + 63) >> 6;              // sequences per lane
  int nf = 0, np = 0, s1 = 0;                   // this lane's full and partly filled chunks
  int nfs[8];                                   // per <= 8: full chunks of each of its sequences
  if (per <= 8) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      nfs[m] = 0;
      if (m < per) {
        const int sl = length(lane * per + m);
        nfs[m] = sl / a.chunk;
        nf += nfs[m];
        np += sl % a.chunk != 0 ? 1 : 0;
        s1 = sl;
      }
    }
  } else {
#pragma unroll 8
    for (int m = 0; m < per; ++m) {
      const int sl = length(lane * per + m);
      nf += sl / a.chunk;
      np += sl % a.chunk != 0 ? 1 : 0;
      s1 = sl;
    }
  }
  const int owned = max(0, min(a.b, (lane + 1) * per) - lane * per);
  const int nd = owned * a.n_chunks - nf - np;  // its empty chunks
  const int n_full = __builtin_amdgcn_readfirstlane(__shfl(wave_inclusive_sum(nf), 63));
  const int n_part = __builtin_amdgcn_readfirstlane(__shfl(wave_inclusive_sum(np), 63));
  const int run = k < n_full ? 0 : (k < n_full + n_part ? 1 : 2);
  const int kk = run == 0 ? k : (run == 1 ? k - n_full : k - n_full - n_part);
  const int cnt = run == 0 ? nf : (run == 1 ? np : nd);
  const int incl = wave_inclusive_sum(cnt);
  const int li = __popcll(__ballot(incl <= kk));       // incl is non-decreasing over the lanes
  int kq = __builtin_amdgcn_readfirstlane(kk - __shfl(incl - cnt, li));   // index among lane li's units
  auto first_of = [&](int sl) {                        // first chunk of the run in a sequence
    const int full = sl / a.chunk;
    return run == 0 ? 0 : (run == 1 ? full : full + (sl % a.chunk != 0 ? 1 : 0));
  };
  if (run == 0 && a.b > 1) {
    // Full chunks chunk-major: chunk c of every sequence that has it, in
    // sequence order, then chunk c + 1.  Sequences that share prefix blocks
    // then read them together, from one XCD's L2 (the workgroups of one KV
    // head share an XCD).  The order only decides which workgroup computes a
    // unit, never its arithmetic.
    if (per == 1 && a.n_chunks <= 64) {                // lane l owns just sequence l
      int kr = kk, c = 0;
      for (;;) {                                       // uniform; ends since kk < n_full
        const uint64_t m = __ballot(nf > c);
        const int cnt_c = __popcll(m);
        if (kr < cnt_c) {
          const int rank = __popcll(m & ((1ull << lane) - 1ull));
          const int i = __builtin_ctzll(__ballot(((m >> lane) & 1ull) && rank == kr));
          return Unit{i, c, __shfl(s1, i)};
        }
        kr -= cnt_c;
        ++c;
      }
    }
    // Any b and chunk count: F(c), the number of full chunks with index below
    // c, is a wave sum (over the lane's counts kept in nfs when it owns at
    // most eight sequences, else recounted from their lengths); a binary
    // search gives the chunk index c with F(c) <= kk < F(c + 1), then a prefix
    // sum over the lanes and a walk over the owning lane's sequences give the
    // (kk - F(c))-th sequence that has chunk c.
    auto below = [&](int c) {                          // this lane's full chunks with index < c
      int t = 0;
      if (per <= 8) {
#pragma unroll
        for (int m = 0; m < 8; ++m) t += min(nfs[m], c);
      } else {
#pragma unroll 8
        for (int m = 0; m < per; ++m) t += min(length(lane * per + m) / a.chunk, c);
      }
      return t;
    };
    auto F = [&](int c) { return __builtin_amdgcn_readfirstlane(__shfl(wave_inclusive_sum(below(c)), 63)); };
    int lo_c = 0, hi_c = a.n_chunks;                   // F(lo_c) <= kk < F(hi_c) = n_full
    while (hi_c - lo_c > 1) {
      const int mid = (lo_c + hi_c) >> 1;
      if (F(mid) <= kk) lo_c = mid;
      else hi_c = mid;
    }
    const int c = lo_c;
    const int kr = kk - F(c);
    int cl = 0;                                        // this lane's sequences that have chunk c
    if (per <= 8) {
#pragma unroll
      for (int m = 0; m < 8; ++m) cl += nfs[m] > c ? 1 : 0;
    } else {
#pragma unroll 8
      for (int m = 0; m < per; ++m) cl += length(lane * per + m) / a.chunk > c ? 1 : 0;
    }
    const int inc = wave_inclusive_sum(cl);
    const int l2 = __popcll(__ballot(inc <= kr));
    int r = __builtin_amdgcn_readfirstlane(kr - __shfl(inc - cl, l2));
    if (per <= 8) {
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const int v = __builtin_amdgcn_readfirstlane(__shfl(nfs[m], l2));
        if (m < per && v > c) {
          if (r == 0) {
            const int q = l2 * per + m;
            return Unit{q, c, length(q)};
          }
          --r;
        }
      }
    } else {
      for (int m = 0; m < per; ++m) {                  // uniform
        const int q = l2 * per + m;
        if (__builtin_amdgcn_readfirstlane(length(q) / a.chunk) > c) {
          if (r == 0) return Unit{q, c, length(q)};
          --r;
        }
      }
    }
  }
  if (per == 1) {                                      // lane l owns just sequence l
    const int sl = __shfl(s1, li);
    return Unit{li, first_of(sl) + kq, sl};
  }
  for (int m0 = 0; m0 < per; m0 += 64) {
    const int q = li * per + m0 + lane;
    const bool in = m0 + lane < per && q < a.b;
    const int sl = in ? length(q) : 0;
    const int full = sl / a.chunk;
    const int part = sl % a.chunk != 0 ? 1 : 0;
    const int c2 = !in ? 0 : (run == 0 ? full : (run == 1 ? part : a.n_chunks - full - part));
    const int incl2 = wave_inclusive_sum(c2);
    const int total = __builtin_amdgcn_readfirstlane(__shfl(incl2, 63));   // uniform: scalar branch
    if (kq < total) {
      const int mi = __popcll(__ballot(incl2 <= kq));
      return Unit{li * per + m0 + mi, __shfl(first_of(sl), mi) + kq - __shfl(incl2 - c2, mi), __shfl(sl, mi)};
    }
    kq -= total;
  }
  return Unit{-1, 0, 0};
}

// The KV head and token span [lo, hi) of chunk c for workgroup x.  Even
// chunks: head x % n_kv, span [c*C, (c+1)*C).  With chunk_skew = d > 0 (an
// even n_kv) the chunks 2p and 2p + 1 of a pair are C + d and C - d long for
// an even head, C - d and C + d for an odd one, and the odd chunk of a pair
// goes to the workgroup of the partner head (j ^ 1): the workgroup with x
// even -- on an even XCD -- always takes the long chunk.  A last chunk
// without a partner keeps [c*C, (c+1)*C).
struct Span {
  int j, lo, hi;
};

__device__ inline Span chunk_span(const DecodeLaunch& a, int x, int c) {
  int j = x % a.n_kv;
  int lo = c * a.chunk, hi = lo + a.chunk;
  if (a.chunk_skew != 0 && (c | 1) < a.n_chunks) {
    j ^= c & 1;
    const int base = (c & ~1) * a.chunk;
    const int mid = base + a.chunk + ((j & 1) == 0 ? a.chunk_skew : -a.chunk_skew);
    lo = (c & 1) ? mid : base;
    hi = (c & 1) ? base + 2 * a.chunk : mid;
  }
  return Span{j, lo, hi};
}

// KIND: kBf16 or kFp8 (one pool), or kMixed (a bf16 and an FP8 pool; each
// table entry names its block's precision in kPrecisionBit -- the page
// header).  A mixed kernel runs two passes, bf16 then FP8, each over the span
// of pairs that holds blocks of its precision; inside a pass an entry of the
// other precision is skipped like a dropped block, so every pass keeps the
// one-precision pipeline (fixed loads in flight, one register set) and the
// softmax state carries from the first pass into the second.
template <int D, int KIND, bool FINAL, bool SCORES>
__global__ __launch_bounds__(64 * kWaves, KIND == kFp8 ? 3 : 2) void decode_kernel(DecodeLaunch a) {
  constexpr bool MIX = KIND == kMixed;
  constexpr int NM = D / 16;                   // 16-channel tiles of the output
  constexpr int NC = D / 32;                   // MFMA steps along the head dim

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave
  const int G = lane >> 4;
  const int r16 = lane & 15;

  const int x = blockIdx.x;
  const Unit u = locate_unit(a, x / a.n_kv);
  // the unit is the same for every lane: keep it in scalar registers
  const int i = __builtin_amdgcn_readfirstlane(u.i);
  const int c = __builtin_amdgcn_readfirstlane(u.c);
  const int s = __builtin_amdgcn_readfirstlane(u.s);
  if (i < 0) return;                            // outside the grid's units (not reached)
  const Span sp = chunk_span(a, x, c);
  const int j = __builtin_amdgcn_readfirstlane(sp.j);
  const int lo = __builtin_amdgcn_readfirstlane(sp.lo);
  const int ntok = min(s, __builtin_amdgcn_readfirstlane(sp.hi)) - lo;
  const int g = a.g;
  const bool head_ok = r16 < g;
  const size_t ih = (size_t)i * a.n_q + (size_t)j * g + r16;   // this lane's head (when head_ok)
  if (!FINAL && ntok <= 0) {
    // Chunk past the end of the sequence: it contributes nothing to the merge.
    if (wave == 0 && G == 0 && head_ok) a.part_lse[ih * a.n_chunks + c] = -INFINITY;
    return;
  }

  // Fused append: the workgroup whose chunk holds token s - 1 first stores that
  // token's K and V rows of head j into the pool, exactly as the write kernel
  // would, and then reads them back like every other row.  FP8: waves 0 and 1
  // re-quantise the K and the V tile; the new scales are kept in registers for
  // this block, because the scalar cache may hold the old ones.  A context
  // length above the bound has no slot for its new token inside the bound (s
  // is the clamped length): nothing is stored, so no cached row is overwritten.
  int32_t app_pid = -1;
  float app_sK = 0.f, app_sV = 0.f;
  if constexpr (!MIX) {
    if (a.new_k != nullptr && s > 0 && s - 1 >= lo && s - 1 < lo + ntok && load_invariant(a.context_lens + i) == s) {
      const int tl = s - 1;
      const int32_t pid = load_invariant(a.block_table + (size_t)i * a.max_blocks + tl / kBlock);
      if (pid >= 0 && pid < a.num_blocks) {
        const uint16_t* kr = a.new_k + ((size_t)i * a.n_kv + j) * D;
        const uint16_t* vr = a.new_v + ((size_t)i * a.n_kv + j) * D;
        constexpr uint32_t kTPB = 2u * kBlock * D * (KIND == kFp8 ? 1 : 2);
        char* tp = const_cast<char*>(a.layer_base) + tile_pair_offset(pid, j, a.num_blocks, a.n_kv, kTPB);
        if constexpr (KIND == kFp8) {
          __shared__ float sh_app[2];
          if (wave < 2) {
            float* sc = const_cast<float*>(a.layer_scales) + ((size_t)j * a.num_blocks + pid) * 2 + wave;
            const float v = fp8_store_rows<D>(reinterpret_cast<uint8_t*>(tp), sc, wave, tl % kBlock, 1,
                                              wave ? vr : kr, 0, lane);
            if (lane == 0) sh_app[wave] = v;
          }
          __syncthreads();
          // uniform: keep them in scalar registers
          app_sK = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(sh_app[0])));
          app_sV = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(sh_app[1])));
        } else {
          if (wave == 0) bf16_store_row<D>(reinterpret_cast<uint16_t*>(tp), tl % kBlock, kr, vr, lane);
          __syncthreads();
        }
        app_pid = pid;
      }
    }
  }

  // q as the B operand of S = K q^T: column r16 = query head j*g + r16.
  bf16x8 qf[NC];
  {
    const uint16_t* qrow = a.q + ih * D;
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (head_ok) raw = *reinterpret_cast<const u32x4*>(qrow + qk_channel0(cc, G));
      qf[cc] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.layer_base, a.layer_bytes);
  const __amdgpu_buffer_rsrc_t rs8 = make_rsrc(MIX ? a.layer_base8 : a.layer_base, MIX ? a.layer_bytes8 : 0u);
  const int32_t* bt = a.block_table + (size_t)i * a.max_blocks + lo / kBlock;
  const float qk_scale = kLog2e * (1.0f / sqrtf((float)D));

  float m = -INFINITY;                          // running max of head r16 (log2 domain)
  float l = 0.f;                                // this lane's share of the running sum
  f32x4 o[NM];
#pragma unroll
  for (int mm = 0; mm < NM; ++mm) o[mm] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int npairs = (ntok + 31) >> 5;

  // One pass over this wave's pairs in [p0, p1), all of precision F8.
  auto run = [&](auto f8tag, int p0, int p1) {
    constexpr bool F8 = decltype(f8tag)::value;
    using R = PairRegs<D, F8>;
    constexpr int EE = R::E;                           // bytes per element
    constexpr uint32_t TPB = 2u * kBlock * D * EE;     // bytes per (block, head) tile pair
    constexpr bool OTHER = MIX && F8;                  // the mixed kernel's FP8 pool
    const __amdgpu_buffer_rsrc_t rx = OTHER ? rs8 : rs;

    // Issue every load of pair p into f.  A pair past the end (p >= npairs)
    // issues the same loads at out-of-range offsets: they return zeros without
    // touching memory, and the number of loads in flight stays the same on every
    // path, so the waits before each use cover exactly the pair being used.
    auto issue = [&](R& f, int p) {
      const bool live = p < p1;
      const int nvalid = min(32, ntok - (p << 5));
      int32_t pid0 = live ? load_invariant(bt + 2 * p) : -1;
      int32_t pid1 = live && nvalid > kBlock ? load_invariant(bt + 2 * p + 1) : -1;
      if constexpr (MIX) {
        // A block of the other precision waits for the other pass.
        if (pid0 >= 0) pid0 = ((pid0 & kPrecisionBit) != 0) == F8 ? (pid0 & ~kPrecisionBit) : -1;
        if (pid1 >= 0) pid1 = ((pid1 & kPrecisionBit) != 0) == F8 ? (pid1 & ~kPrecisionBit) : -1;
      }
      // A negative entry marks a block that is not attended (its loads read
      // nothing, and consume masks its tokens).
      f.drop = (pid0 < 0 ? 1u : 0u) | (pid1 < 0 ? 2u : 0u);
      const uint32_t t0 = tile_pair_offset(pid0, j, OTHER ? a.num_blocks8 : a.num_blocks, a.n_kv, TPB);
      const uint32_t t1 = tile_pair_offset(pid1, j, OTHER ? a.num_blocks8 : a.num_blocks, a.n_kv, TPB);
      // K: S-tile t, row r16 -> block r16/8, in-block row 8*((r16/4)&1) + 4t + r16%4,
      // whose 16-byte unit u for lane group G (piece 4u + G of the row) is K piece
      // ((t*KU + u)*4 + G)*8 + r16%8 of the block: each load reads 512 contiguous
      // bytes per block.
      const uint32_t tk = r16 < 8 ? t0 : t1;
  #pragma unroll
      for (int t = 0; t < 2; ++t) {
  #pragma unroll
        for (int u = 0; u < R::KU; ++u) {
          const uint32_t off = tk + (uint32_t)((((t * R::KU + u) * 4 + G) * 8 + (r16 & 7)) * 16);
          f.k[t][u] = load16(rx, tk == kOutOfRange ? kOutOfRange : off);
        }
      }
      // V (channel-major): channel tile mm, channel 16mm + r16, rows 8(G&1) .. +7
      // of block G/2.
      const uint32_t tv = G < 2 ? t0 : t1;
  #pragma unroll
      for (int mm = 0; mm < NM; ++mm) {
        const uint32_t off = tv + (uint32_t)((v_elem(8 * (G & 1), 16 * mm + r16, D)) * EE);
        const uint32_t o2 = tv == kOutOfRange ? kOutOfRange : off;
        if constexpr (F8) f.v8[mm] = load8(rx, o2);
        else f.v[mm] = load16(rx, o2);
      }
      if constexpr (F8) {
        // fp32 scales of this lane's block (G/2) for K and V; zero for a bad id.
        // Head-major: this head's scales of all blocks are contiguous.
        const float* sc = (OTHER ? a.layer_scales8 : a.layer_scales) +
                          (size_t)j * (OTHER ? a.num_blocks8 : a.num_blocks) * 2;
        float sk0 = t0 == kOutOfRange ? 0.f : load_invariant(sc + (size_t)pid0 * 2 + 0);
        float sv0 = t0 == kOutOfRange ? 0.f : load_invariant(sc + (size_t)pid0 * 2 + 1);
        float sk1 = t1 == kOutOfRange ? 0.f : load_invariant(sc + (size_t)pid1 * 2 + 0);
        float sv1 = t1 == kOutOfRange ? 0.f : load_invariant(sc + (size_t)pid1 * 2 + 1);
        if constexpr (!MIX) {
          if (pid0 == app_pid) { sk0 = app_sK; sv0 = app_sV; }   // the block this call appended to
          if (pid1 == app_pid) { sk1 = app_sK; sv1 = app_sV; }
        }
        f.sK = G < 2 ? sk0 : sk1;
        f.sV = G < 2 ? sv0 : sv1;
      }
    };

    // Fold pair p (held in f) into the running state.
    auto consume = [&](R& f, int p) {
      const int tok0 = p << 5;
      const int nvalid = min(32, ntok - tok0);
      // A pair with both blocks dropped adds nothing (its scores, when stored,
      // are still written as -inf below).
      if constexpr (!SCORES) {
        if (f.drop == 3u) return;
      }

      f32x4 sacc[2];
  #pragma unroll
      for (int t = 0; t < 2; ++t) {
        sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  #pragma unroll
        for (int cc = 0; cc < NC; ++cc) {
          bf16x8 kf;
          if constexpr (F8) {
            const u32x4 w = f.k[t][cc >> 1];
            kf = (cc & 1) ? e4m3x8_to_bf16x8(w[2], w[3]) : e4m3x8_to_bf16x8(w[0], w[1]);
          } else {
            kf = __builtin_bit_cast(bf16x8, f.k[t][cc]);
          }
          sacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[cc], sacc[t], 0, 0, 0);
        }
      }

      // Scaled scores; lane element e = 4t + q is pair token 8G + e.
      float xs[8];
      const float sc_all = F8 ? qk_scale * f.sK : qk_scale;
  #pragma unroll
      for (int t = 0; t < 2; ++t)
  #pragma unroll
        for (int q = 0; q < 4; ++q) xs[4 * t + q] = sacc[t][q] * sc_all;

      const int my_valid = min(8, max(0, nvalid - 8 * G));   // valid tokens among my 8
      if (nvalid < 32) {
  #pragma unroll
        for (int e = 0; e < 8; ++e)
          if (e >= my_valid) xs[e] = -INFINITY;
      }
      // This lane's tokens lie in block G/2 of the pair.
      if (f.drop && ((f.drop >> (G >> 1)) & 1u)) {
  #pragma unroll
        for (int e = 0; e < 8; ++e) xs[e] = -INFINITY;
      }

      if constexpr (SCORES) {
        // Scaled scores of this head and pair, stored pair-permuted (see
        // score_slot): the lanes' first halves form one contiguous 64-byte run,
        // their second halves the next, so each store instruction writes whole
        // runs.
        if (head_ok) {
          float* dst = a.logits + ih * a.logit_stride + lo + tok0 + 4 * G;
          *reinterpret_cast<f32x4*>(dst) = f32x4{xs[0], xs[1], xs[2], xs[3]};
          *reinterpret_cast<f32x4*>(dst + 16) = f32x4{xs[4], xs[5], xs[6], xs[7]};
        }
      }

      float mx = xs[0];
  #pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, xs[e]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float corr = __builtin_amdgcn_exp2f(m - m_use);
      m = m_new;

      float pv[8];
      float psum = 0.f;
  #pragma unroll
      for (int e = 0; e < 8; ++e) {
        pv[e] = __builtin_amdgcn_exp2f(xs[e] - m_use);
        psum += pv[e];
      }
      l = l * corr + psum;
  #pragma unroll
      for (int mm = 0; mm < NM; ++mm) o[mm] *= corr;

      bf16x8 phi, plo;
  #pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pe = F8 ? pv[e] * f.sV : pv[e];
        const __bf16 h = (__bf16)pe;
        phi[e] = h;
        plo[e] = (__bf16)(pe - (float)h);
      }

      // Zero V of tokens past the end so that stale (even NaN) rows contribute 0.
      if (nvalid < 32) {
        if constexpr (F8) {
          uint32_t keep[2];
  #pragma unroll
          for (int w = 0; w < 2; ++w) {
            uint32_t mk = 0;
  #pragma unroll
            for (int bb = 0; bb < 4; ++bb)
              if (4 * w + bb < my_valid) mk |= 0xFFu << (8 * bb);
            keep[w] = mk;
          }
  #pragma unroll
          for (int mm = 0; mm < NM; ++mm) {
            f.v8[mm][0] &= keep[0];
            f.v8[mm][1] &= keep[1];
          }
        } else {
          uint32_t keep[4];
  #pragma unroll
          for (int w = 0; w < 4; ++w)
            keep[w] = (2 * w < my_valid ? 0x0000FFFFu : 0u) | (2 * w + 1 < my_valid ? 0xFFFF0000u : 0u);
  #pragma unroll
          for (int mm = 0; mm < NM; ++mm)
  #pragma unroll
            for (int w = 0; w < 4; ++w) f.v[mm][w] &= keep[w];
        }
      }

      // O^T[channel][head] += V^T P^T, rows = channels 16mm + 4G + q, cols = heads.
  #pragma unroll
      for (int mm = 0; mm < NM; ++mm) {
        bf16x8 vf;
        if constexpr (F8) vf = e4m3x8_to_bf16x8(f.v8[mm][0], f.v8[mm][1]);
        else vf = __builtin_bit_cast(bf16x8, f.v[mm]);
        o[mm] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, phi, o[mm], 0, 0, 0);
        o[mm] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, plo, o[mm], 0, 0, 0);
      }
    };

    // Two register sets: the next pair's loads are in flight while the current
    // pair is consumed.  This wave owns pairs p0 + wave, p0 + wave + kWaves, ...;
    // they are taken two at a time so that every pass through the loop has the
    // same loads outstanding (a load past the end is an out-of-range no-op).
    const int nmine = p1 - p0 > wave ? (p1 - p0 - wave + kWaves - 1) / kWaves : 0;
    if (nmine > 0) {
      R fa, fb;
      int p = p0 + wave;
      issue(fa, p);
      int k = 0;
      for (; k + 1 < nmine; k += 2) {
        issue(fb, p + kWaves);
        consume(fa, p);
        issue(fa, p + 2 * kWaves);
        consume(fb, p + kWaves);
        p += 2 * kWaves;
      }
      if (k < nmine) consume(fa, p);
    }
  };
  if constexpr (MIX) {
    // Each pass visits only the span of pairs that hold a block of its
    // precision.  A row lists one precision's pages before the other's, so the
    // two spans meet rather than overlap; any other row is still right, the
    // spans then overlap and each pass skips the other precision's blocks.
    // Lane l reads the entries of pair g0 + l; ballots give the first and last
    // pair of each precision.
    int lo16 = npairs, hi16 = 0, lo8 = npairs, hi8 = 0;
    for (int g0 = 0; g0 < npairs; g0 += 64) {
      const int p = g0 + lane;
      bool has16 = false, has8 = false;
      if (p < npairs) {
        const int32_t e0 = bt[2 * p];
        const int32_t e1 = ntok - (p << 5) > kBlock ? bt[2 * p + 1] : -1;
        has16 = (e0 >= 0 && !(e0 & kPrecisionBit)) || (e1 >= 0 && !(e1 & kPrecisionBit));
        has8 = (e0 >= 0 && (e0 & kPrecisionBit)) || (e1 >= 0 && (e1 & kPrecisionBit));
      }
      const uint64_t m16 = __ballot(has16), m8 = __ballot(has8);
      if (m16) {
        lo16 = min(lo16, g0 + (int)__builtin_ctzll(m16));
        hi16 = g0 + 64 - (int)__builtin_clzll(m16);
      }
      if (m8) {
        lo8 = min(lo8, g0 + (int)__builtin_ctzll(m8));
        hi8 = g0 + 64 - (int)__builtin_clzll(m8);
      }
    }
    run(std::false_type{}, __builtin_amdgcn_readfirstlane(lo16), __builtin_amdgcn_readfirstlane(max(lo16, hi16)));
    run(std::true_type{}, __builtin_amdgcn_readfirstlane(lo8), __builtin_amdgcn_readfirstlane(max(lo8, hi8)));
  } else {
    run(std::integral_constant<bool, KIND == kFp8>{}, 0, npairs);
  }

  // Whole-head sum of this wave.
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);

  // Combine the waves after one barrier: each wave leaves its max, sum and
  // unscaled output; the readers take the common max and rescale.
  __shared__ float sh_m[kWaves][16];
  __shared__ float sh_l[kWaves][16];
  __shared__ f32x4 sh_o[kWaves][NM][64];
  if (G == 0) {
    sh_m[wave][r16] = m;
    sh_l[wave][r16] = l;
  }
#pragma unroll
  for (int mm = 0; mm < NM; ++mm) sh_o[wave][mm][lane] = o[mm];
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sh_m[w][r16]);
  float fw[kWaves];
  float L = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    fw[w] = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sh_m[w][r16] - M);
    L += sh_l[w][r16] * fw[w];
  }

  const bool empty = !(L > 0.f);
  const float inv_l = empty ? 0.f : 1.0f / L;
  const float lse2 = empty ? -INFINITY : M + __log2f(L);
  for (int mm = wave; mm < NM; mm += kWaves) {
    f32x4 acc = sh_o[0][mm][lane] * fw[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) acc += sh_o[w][mm][lane] * fw[w];
    acc *= inv_l;
    if (!head_ok) continue;
    const int ch = 16 * mm + 4 * G;
    if constexpr (FINAL) {
      uint32_t lo2 = (uint32_t)float_to_bf16_bits(acc[0]) | ((uint32_t)float_to_bf16_bits(acc[1]) << 16);
      uint32_t hi2 = (uint32_t)float_to_bf16_bits(acc[2]) | ((uint32_t)float_to_bf16_bits(acc[3]) << 16);
      *reinterpret_cast<u32x2*>(a.out + ih * D + ch) = u32x2{lo2, hi2};
    } else {
      *reinterpret_cast<f32x4*>(a.part_o + (ih * a.n_chunks + c) * D + ch) = acc;
    }
  }
  if (wave == 0 && G == 0 && head_ok) {
    if constexpr (FINAL) {
      if (a.lse_out) a.lse_out[ih] = lse2 * kLn2;
      if constexpr (SCORES) a.lse2[ih] = lse2;
    } else {
      a.part_lse[ih * a.n_chunks + c] = lse2 * kLn2;
    }
  }
}

// Test hook: the unit each workgroup of a decode launch with these arguments
// takes -- out[6x .. 6x+5] = (sequence, chunk, clamped context length, KV
// head, first token, end token of the chunk) of workgroup x.  One wave per
// workgroup runs locate_unit and chunk_span exactly as the decode kernels do.
__global__ __launch_bounds__(64) void debug_units_kernel(DecodeLaunch a, int32_t* __restrict__ out) {
  const int x = blockIdx.x;
  const Unit u = locate_unit(a, x / a.n_kv);
  const Span sp = chunk_span(a, x, u.c);
  if (threadIdx.x == 0) {
    int32_t* o = out + 6 * (size_t)x;
    o[0] = u.i;
    o[1] = u.c;
    o[2] = u.s;
    o[3] = sp.j;
    o[4] = sp.lo;
    o[5] = sp.hi;
  }
}

hipError_t launch_debug_units(const DecodeLaunch& a, int32_t* out, hipStream_t stream) {
  const dim3 grid((unsigned)((size_t)a.n_chunks * a.b * a.n_kv));
  hipLaunchKernelGGL(debug_units_kernel, grid, dim3(64), 0, stream, a, out);
  return hipGetLastError();
}

template <int D, int KIND>
static hipError_t launch_d(const DecodeLaunch& a, bool final_direct, bool scores,
                           hipStream_t stream) {
  const dim3 grid((unsigned)((size_t)a.n_chunks * a.b * a.n_kv));
  const dim3 block(64 * kWaves);
  if constexpr (KIND == kMixed) {
    // no fused score in a mixed-precision decode (rejected on the host)
    if (final_direct) hipLaunchKernelGGL((decode_kernel<D, KIND, true, false>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((decode_kernel<D, KIND, false, false>), grid, block, 0, stream, a);
  } else if (final_direct) {
    if (scores) hipLaunchKernelGGL((decode_kernel<D, KIND, true, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((decode_kernel<D, KIND, true, false>), grid, block, 0, stream, a);
  } else {
    if (scores) hipLaunchKernelGGL((decode_kernel<D, KIND, false, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((decode_kernel<D, KIND, false, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

template <int D>
static hipError_t launch_kind(const DecodeLaunch& a, int kind, bool final_direct, bool scores,
                              hipStream_t stream) {
  if (kind == kMixed) return launch_d<D, kMixed>(a, final_direct, scores, stream);
  if (kind == kFp8) return launch_d<D, kFp8>(a, final_direct, scores, stream);
  return launch_d<D, kBf16>(a, final_direct, scores, stream);
}

hipError_t launch_decode(const DecodeLaunch& a, int head_dim, int kind, bool final_direct,
                         bool scores, hipStream_t stream) {
  return head_dim == 128 ? launch_kind<128>(a, kind, final_direct, scores, stream)
                         : launch_kind<64>(a, kind, final_direct, scores, stream);
}

}  // namespace kvd
