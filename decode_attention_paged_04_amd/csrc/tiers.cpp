// Host-side tier planning of a tier-restricted decode (gist.science summary
// of "Not all thinking needs HBM", methodology 1-4): blocks ranked by
// cumulative attention score into T0 (HBM), T1 (host memory, prefetched at
// full precision before attention) and T3 (evicted); attention covers T0 and
// T1, expressed as a block-table row whose evicted entries are negative.
#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <numeric>
#include <vector>

#include "kvblocks.h"

namespace {
constexpr int32_t kBlock = 16;
}

extern "C" {

kvd_status kvd_tier_block_scores(const float* token_scores, int32_t n_tokens, double* block_scores) {
  if (n_tokens < 0 || (n_tokens > 0 && (!token_scores || !block_scores))) return KVD_ERR_INVALID_ARG;
  const int32_t nb = (n_tokens + kBlock - 1) / kBlock;
  for (int32_t b = 0; b < nb; ++b) {
    double acc = 0.0;
    for (int32_t t = b * kBlock; t < std::min(n_tokens, (b + 1) * kBlock); ++t) acc += token_scores[t];
    block_scores[b] = acc;
  }
  return KVD_OK;
}

kvd_status kvd_tier_plan(const double* block_scores, int32_t n_blocks, int32_t protect_first,
                         int32_t protect_last, int32_t t0_blocks, int32_t t1_blocks, int8_t* tiers) {
  if (n_blocks < 0 || protect_first < 0 || protect_last < 0 || t0_blocks < 0 || t1_blocks < 0)
    return KVD_ERR_INVALID_ARG;
  if (n_blocks == 0) return KVD_OK;
  if (!block_scores || !tiers) return KVD_ERR_INVALID_ARG;
  for (int32_t b = 0; b < n_blocks; ++b)
    if (!std::isfinite(block_scores[b])) return KVD_ERR_INVALID_ARG;
  try {
    std::vector<int32_t> rest;
    rest.reserve(n_blocks);
    for (int32_t b = 0; b < n_blocks; ++b) {
      const bool prot = b < protect_first || b >= n_blocks - protect_last;
      tiers[b] = prot ? KVD_TIER_T0 : KVD_TIER_T3;
      if (!prot) rest.push_back(b);
    }
    // highest score first; equal scores by position
    std::sort(rest.begin(), rest.end(), [&](int32_t a, int32_t b) {
      return block_scores[a] != block_scores[b] ? block_scores[a] > block_scores[b] : a < b;
    });
    for (size_t r = 0; r < rest.size(); ++r) {
      if ((int64_t)r < t0_blocks) tiers[rest[r]] = KVD_TIER_T0;
      else if ((int64_t)r < (int64_t)t0_blocks + t1_blocks) tiers[rest[r]] = KVD_TIER_T1;
    }
    return KVD_OK;
  } catch (...) {
    return KVD_ERR_CAPACITY;
  }
}

kvd_status kvd_tier_restrict(const int32_t* table_row, const int8_t* tiers, int32_t n_blocks,
                             int32_t* out_row) {
  if (n_blocks < 0 || (n_blocks > 0 && (!table_row || !tiers || !out_row))) return KVD_ERR_INVALID_ARG;
  for (int32_t b = 0; b < n_blocks; ++b)        // check everything before writing (in place allowed)
    if (tiers[b] != KVD_TIER_T0 && tiers[b] != KVD_TIER_T1 && tiers[b] != KVD_TIER_T3) return KVD_ERR_INVALID_ARG;
  for (int32_t b = 0; b < n_blocks; ++b) out_row[b] = tiers[b] == KVD_TIER_T3 ? -1 : table_row[b];
  return KVD_OK;
}

}  // extern "C"

// Mixed-precision rows (kvd_decode_attn_mixed): tier-homogeneous pages of two
// entries, the precision bit on FP8 entries.
extern "C" kvd_status kvd_mixed_row(const int32_t* ids_bf16, int32_t n_bf16, const int32_t* ids_fp8,
                                    int32_t n_fp8, int32_t fp8_last, int32_t tail_tokens, int32_t* row,
                                    int32_t capacity, int32_t* n_entries, int32_t* context_len) {
  constexpr int32_t kBit = 1 << 30;
  if (n_bf16 < 0 || n_fp8 < 0 || capacity < 0 || !n_entries || !context_len) return KVD_ERR_INVALID_ARG;
  if ((n_bf16 > 0 && !ids_bf16) || (n_fp8 > 0 && !ids_fp8)) return KVD_ERR_INVALID_ARG;
  if (fp8_last != 0 && fp8_last != 1) return KVD_ERR_INVALID_ARG;
  const int32_t* first = fp8_last ? ids_bf16 : ids_fp8;
  const int32_t* second = fp8_last ? ids_fp8 : ids_bf16;
  const int32_t nf = fp8_last ? n_bf16 : n_fp8, ns = fp8_last ? n_fp8 : n_bf16;
  const int32_t tf = fp8_last ? 0 : kBit, ts = fp8_last ? kBit : 0;
  const int32_t pad = (ns > 0 && nf % 2) ? 1 : 0;
  const int64_t n = (int64_t)nf + pad + ns;
  if (n > INT32_MAX - 1) return KVD_ERR_INVALID_ARG;
  *n_entries = (int32_t)n;
  *context_len = 0;
  if (n == 0) return KVD_OK;
  if (tail_tokens < 1 || tail_tokens > 16) return KVD_ERR_INVALID_ARG;
  if (n > capacity || !row) return KVD_ERR_INVALID_ARG;
  int32_t k = 0;
  for (int32_t i = 0; i < nf; ++i) {
    if (first[i] < 0 || first[i] >= kBit) return KVD_ERR_INVALID_ARG;
    row[k++] = first[i] | tf;
  }
  if (pad) row[k++] = -1;
  for (int32_t i = 0; i < ns; ++i) {
    if (second[i] < 0 || second[i] >= kBit) return KVD_ERR_INVALID_ARG;
    row[k++] = second[i] | ts;
  }
  *context_len = 16 * (k - 1) + tail_tokens;
  return KVD_OK;
}
