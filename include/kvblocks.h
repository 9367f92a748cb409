/* libkvdecode -- host-side block bookkeeping of a paged KV cache.
 *
 * The decode kernels read K/V through per-sequence block tables; this part of
 * the library decides which physical blocks a sequence gets.  It follows the
 * PagedAttention and prefix-cache paragraphs of froggydisk, "LLM에서 KV
 * 캐시는 얼마나 생길까", section "KV 캐시를 줄이는 기법":
 *   - a new sequence gets just enough 16-token blocks for its prompt; while
 *     decoding, a new block is taken when the last one holds 16 tokens, so a
 *     sequence wastes at most 15 token slots;
 *   - a finished sequence returns its blocks; a block pointed at by several
 *     tables (a shared prefix) counts its users and is returned when the count
 *     reaches 0;
 *   - with the prefix cache on, every full block is looked up by its 16
 *     tokens together with all tokens before it; a new prompt is matched block
 *     by block from the front up to the first miss and the matched blocks are
 *     shared instead of prefilled; a partial last block is never reused;
 *     finished sequences' blocks stay cached and are evicted, least recently
 *     released first, only when no free block is left -- and only blocks no
 *     sequence uses.
 * Choices the page leaves open: free blocks are handed out lowest number
 * first; a finished sequence releases its blocks last to first (the front of
 * a prefix outlives its tail); a full block whose prefix is cached already
 * stays private; a call that cannot get every block it needs fails with
 * KVD_ERR_CAPACITY and changes nothing.  Lookup keys are a 64-bit hash of the
 * token prefix before the block plus the block's own 16 tokens, compared
 * exactly (two different prefixes collide only if their 64-bit hashes do).
 *
 * Host memory only; no HIP call.  A manager is not thread-safe: one thread at
 * a time.  Sequence ids are never reused.  Token ids are opaque int32 values,
 * used only for prefix matching.
 */
#ifndef KVBLOCKS_H
#define KVBLOCKS_H

#include <stdint.h>

#include "kvdecode.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kvd_block_manager kvd_block_manager;

/* A manager over physical blocks 0 .. num_blocks-1 of a pool (all layers
 * share the block ids).  prefix_cache: 0 off, 1 on.  *out is set on KVD_OK. */
kvd_status kvd_bm_create(int32_t num_blocks, int32_t prefix_cache, kvd_block_manager** out);
kvd_status kvd_bm_destroy(kvd_block_manager* bm);

/* A new sequence whose prompt has n_tokens tokens.  tokens: host int32
 * [n_tokens] of token ids, or NULL (then nothing of this sequence is ever
 * cached or matched).  *seq_id gets the new id; *n_cached (may be NULL) the
 * number of leading prompt tokens whose K/V already sit in shared blocks
 * (a multiple of 16) -- only tokens n_cached .. n_tokens-1 need writing.
 * KVD_ERR_CAPACITY if the blocks cannot all be had (nothing changes). */
kvd_status kvd_bm_add_sequence(kvd_block_manager* bm, const int32_t* tokens, int32_t n_tokens,
                               int64_t* seq_id, int32_t* n_cached);

/* Append n tokens to a sequence (a decode step: n = 1), taking new blocks as
 * needed.  tokens: host int32 [n] or NULL (a sequence appended without ids
 * stops registering full blocks).  slots: host int32 [n] receiving each new
 * token's slot, block * 16 + row -- the slot mapping of kvd_write_kv.
 * KVD_ERR_CAPACITY if the blocks cannot be had (nothing changes). */
kvd_status kvd_bm_append(kvd_block_manager* bm, int64_t seq_id, const int32_t* tokens, int32_t n,
                         int32_t* slots);

/* Slots of tokens first .. first+n-1 of a sequence (within its length). */
kvd_status kvd_bm_slots(const kvd_block_manager* bm, int64_t seq_id, int32_t first, int32_t n,
                        int32_t* slots);

/* Length of a sequence in tokens. */
kvd_status kvd_bm_length(const kvd_block_manager* bm, int64_t seq_id, int32_t* length);

/* A sequence's block table.  table: host int32 [capacity]; *n_blocks gets the
 * number of blocks; KVD_ERR_INVALID_ARG if capacity is smaller. */
kvd_status kvd_bm_block_table(const kvd_block_manager* bm, int64_t seq_id, int32_t* table,
                              int32_t capacity, int32_t* n_blocks);

/* The decode call's block table and context lengths for b sequences:
 * table host int32 [b][max_blocks] (unused entries -1), context_lens host
 * int32 [b].  KVD_ERR_INVALID_ARG if a sequence has more than max_blocks
 * blocks or an id is unknown. */
kvd_status kvd_bm_fill_tables(const kvd_block_manager* bm, const int64_t* seq_ids, int32_t b,
                              int32_t* table, int32_t max_blocks, int32_t* context_lens);

/* Finish a sequence: release its blocks (last to first). */
kvd_status kvd_bm_free_sequence(kvd_block_manager* bm, int64_t seq_id);

/* Counts of free (never cached or evicted), cached-but-unused (evictable) and
 * used blocks; any pointer may be NULL.  They always add up to num_blocks. */
kvd_status kvd_bm_counts(const kvd_block_manager* bm, int32_t* free_blocks, int32_t* cached_blocks,
                         int32_t* used_blocks);

/* Number of sequences whose tables hold a block. */
kvd_status kvd_bm_refcount(const kvd_block_manager* bm, int32_t block, int32_t* refcount);

/* ---- tiers of a tier-restricted decode ---------------------------------
 * gist.science summary of "Not all thinking needs HBM", methodology 1-4:
 * tokens are sorted by cumulative attention score (the score output of
 * kvd_decode_attn) into T0 (kept in HBM, with the protected prompt, sinks
 * and recent window), T1 (host memory at full precision, prefetched before
 * every attention step) and the evicted tail T3, re-sorted every 64 decode
 * steps; attention covers T0 and T1, so its result depends only on what was
 * evicted (Proposition 1).  Here the unit is the 16-token block: a block's
 * score is the sum of its tokens' scores (summed in double); the first
 * protect_first and last protect_last blocks are T0; the others are ranked by
 * score, highest first, equal scores by position, and the first t0_blocks go
 * to T0, the next t1_blocks to T1, the rest to T3 (T2 is not used).  Moving
 * T1 between host and device memory is the caller's business: a T1 block
 * only has to be resident, anywhere in the pool, when the decode runs. */
#define KVD_TIER_T0 0
#define KVD_TIER_T1 1
#define KVD_TIER_T3 3

/* block_scores (host double [ceil(n_tokens / 16)]) from token_scores (host
 * fp32 [n_tokens], e.g. one sequence's row of the cumulative score). */
kvd_status kvd_tier_block_scores(const float* token_scores, int32_t n_tokens, double* block_scores);

/* tiers (host int8 [n_blocks], KVD_TIER_*) of one sequence's blocks.  Scores
 * must be finite. */
kvd_status kvd_tier_plan(const double* block_scores, int32_t n_blocks, int32_t protect_first,
                         int32_t protect_last, int32_t t0_blocks, int32_t t1_blocks, int8_t* tiers);

/* out_row = table_row with every T3 entry replaced by -1: the block-table row
 * of a decode over T0 and T1 (host int32 [n_blocks] both; in place allowed). */
kvd_status kvd_tier_restrict(const int32_t* table_row, const int8_t* tiers, int32_t n_blocks,
                             int32_t* out_row);

/* One sequence's block-table row for kvd_decode_attn_mixed (tier-homogeneous
 * pages): the first run's blocks (bf16 if fp8_last, else FP8), a -1 if that
 * run has an odd length and a second run follows, then the second run's
 * blocks; FP8 entries carry bit 30.  The row's last block holds tail_tokens
 * (1..16) tokens, every other block 16, so *context_len = 16 * (entries - 1)
 * + tail_tokens.  ids: host int32 block ids in [0, 2^30); row: host int32
 * [capacity]; *n_entries is set even when capacity is too small
 * (KVD_ERR_INVALID_ARG). */
kvd_status kvd_mixed_row(const int32_t* ids_bf16, int32_t n_bf16, const int32_t* ids_fp8, int32_t n_fp8,
                         int32_t fp8_last, int32_t tail_tokens, int32_t* row, int32_t capacity,
                         int32_t* n_entries, int32_t* context_len);

#ifdef __cplusplus
}
#endif

#endif /* KVBLOCKS_H */
