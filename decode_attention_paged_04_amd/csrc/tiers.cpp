// Host-side tier planning of a tier-restricted decode (gist.science summary
// of "Not all thinking needs HBM", methodology 1-4): blocks ranked by
// cumulative attention score into T0 (HBM), T1 (host memory, prefetched at
// full precision before attention) and T3 (evicted); attention covers T0 and
// T1, expressed as a block-table row whose evicted entries are negative.
#include <algorithm>
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
  for (int32_t b = 0; b < n_blocks; ++b) {
    if (tiers[b] != KVD_TIER_T0 && tiers[b] != KVD_TIER_T1 && tiers[b] != KVD_TIER_T3) return KVD_ERR_INVALID_ARG;
    out_row[b] = tiers[b] == KVD_TIER_T3 ? -1 : table_row[b];
  }
  return KVD_OK;
}

}  // extern "C"
