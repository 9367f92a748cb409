/*
 * libkvdecode -- one decode step of grouped-query attention over a paged KV
 * cache, for AMD Instinct MI355X (gfx950).
 *
 * What is computed.  For every sequence i of a batch and every query head h,
 * the single new query q[i][h] attends to all s_i cached K/V rows of its
 * sequence: scores q.k / sqrt(d_h), a softmax over them, and the weighted sum
 * of the V rows (froggydisk "LLM에서 KV 캐시는 얼마나 생길까", section
 * "KV 캐시란").  Query heads share KV heads in contiguous groups of
 * g = n_q / n_kv: query head h reads KV head floor(h / g) (same section: 32
 * query heads over 8 KV heads).  s_i counts every cached token including the
 * current one; there is no mask.  The rows are found through a per-sequence
 * block table over fixed 16-token blocks, so the physical placement of the
 * blocks cannot change the result (same page, PagedAttention paragraph).
 *
 * Ownership.  Every device buffer is allocated, owned and freed by the
 * caller.  The library never allocates or frees device memory and keeps no
 * mutable global state, with one exception: the fixed per-device scratch of
 * kvd_decode_attn_no_alloc.  A pool handle holds host metadata only; it is
 * immutable after creation and may be shared by threads and streams.
 * Buffers must stay alive until the stream work that uses them completes.
 *
 * Errors.  Every call returns a kvd_status and nothing aborts.  Shape,
 * dtype and size errors are detected on the host before any launch; launch
 * failures map to KVD_ERR_HIP.  No call synchronises the device.  Values that
 * live in device memory (context lengths, block ids, slot ids) are not
 * validated on the host: context lengths are clamped into [0, bound] (see
 * kvd_decode_args), block ids outside [0, num_blocks) read as zero K/V, and
 * write slots outside the pool are skipped.  No device access can leave the
 * caller's buffers.
 *
 * Streams.  `hip_stream` is a hipStream_t passed as void*; NULL is the null
 * stream.  All work of one call is enqueued on that stream in order.
 */
#ifndef KVDECODE_H
#define KVDECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVD_OK = 0,
  KVD_ERR_INVALID_ARG = 1,  /* null pointer, negative or inconsistent size   */
  KVD_ERR_UNSUPPORTED = 2,  /* valid but not built: d_h, block size, sizes   */
  KVD_ERR_DTYPE = 3,        /* bf16 entry point on an FP8 pool or vice versa */
  KVD_ERR_WORKSPACE = 4,    /* workspace missing or too small                */
  KVD_ERR_HIP = 5,          /* a HIP launch or query failed                  */
  KVD_ERR_CAPACITY = 6      /* not enough free blocks (or host memory)       */
} kvd_status;

/* KV element type of a pool.
 * KVD_FP8_E4M3 is the OCP E4M3FN format (1 sign, 4 exponent, 3 mantissa bits,
 * bias 7, largest finite 448, codes 0x7F/0xFF NaN, no infinities), the format
 * with the 448 maximum in froggydisk's FP8 table. */
typedef enum { KVD_BF16 = 0, KVD_FP8_E4M3 = 1 } kvd_dtype;

/* Shape of a paged KV pool.  block_size must be 16 (the block size of the
 * PagedAttention paragraph); head_dim must be 64 or 128. */
typedef struct {
  int32_t num_layers;
  int32_t num_blocks;   /* physical blocks; block ids are shared by all layers */
  int32_t block_size;   /* = 16                                                */
  int32_t n_kv;         /* KV heads                                            */
  int32_t head_dim;     /* 64 or 128                                           */
  kvd_dtype dtype;
} kvd_pool_desc;

/* Pool layout in device memory (w = 2 bytes for bf16, 1 for FP8).
 *
 *   tile pair of (layer l, physical block p, KV head j) starts at element
 *       T = ((l * num_blocks + p) * n_kv + j) * (2 * 16 * head_dim)
 *   K of in-block row t (0..15), channel c, with n = 16 / w elements per 16
 *   bytes, P = head_dim / n, s = (t / 4) % 2, r = 4 (t / 8) + t % 4,
 *   k = n / 8 (MFMA steps per piece), step = c / 32, grp = (c / 8) % 4,
 *   q = 4 (step / k) + grp:
 *       T + ((s * P + q) * 8 + r) * n + 8 (step % k) + c % 8
 *   (for bf16, k = 1 and q = c / 8: piece q holds channels 8q .. 8q + 7)
 *   V of in-block row t,         channel c:  T + 16 * head_dim + c * 16 + t
 *
 * so one (block, head) is one contiguous 2*16*head_dim*w-byte region: the K
 * tile as 16-byte pieces in the decode kernel's MFMA operand order (each
 * piece n channels of one row), then the V tile channel-major.  Logical token t of a
 * sequence lives in physical block table[t / 16] at in-block row t % 16.
 * FP8 pools add fp32 scales, one per (layer, block, KV head) for K and one
 * for V, head-major within a layer, at
 * scale_base[((l * n_kv + j) * num_blocks + p) * 2 + {0: K, 1: V}], so that
 * the scales one KV head reads are contiguous; a stored element decodes to
 * code_value * scale.
 * Each layer of the pool must be smaller than 4 GiB. */
typedef struct kvd_pool kvd_pool;

/* Bytes the caller must allocate for a pool: kv_bytes for K/V (256-byte
 * alignment recommended) and scale_bytes for FP8 scales (0 for bf16).
 * kv_bytes is num_blocks * 16 tokens times the per-token size of froggydisk's
 * section "토큰 하나의 크기": 2 (K and V) x layers x KV heads x head_dim x
 * bytes per element (128 KiB for the Llama 3.1 8B shape in bf16, 320 KiB for
 * 70B, half of that in FP8 -- section "KV 캐시를 줄이는 기법", FP8 paragraph).
 * Either output pointer may be NULL. */
kvd_status kvd_pool_bytes(const kvd_pool_desc* desc, size_t* kv_bytes, size_t* scale_bytes);

/* Create a host handle over caller-owned device memory laid out as above:
 * the memory cut up front into 16-token blocks that block tables then hand
 * out (froggydisk, PagedAttention paragraph of section "KV 캐시를 줄이는 기법").
 * kv_base: device pointer to kv_bytes bytes, 16-byte aligned.
 * scale_base: device pointer to scale_bytes bytes (FP8), NULL for bf16.
 * Host only: makes no HIP call.  *out is set only on KVD_OK;
 * KVD_ERR_CAPACITY if the host handle cannot be allocated. */
kvd_status kvd_create_pool(const kvd_pool_desc* desc, void* kv_base, float* scale_base,
                           kvd_pool** out);
kvd_status kvd_destroy_pool(kvd_pool* pool);

/* Store n_tok new tokens' K and V of one layer into the pool.
 * k, v: device bf16 [n_tok][n_kv][head_dim], contiguous.
 * slot_mapping: device int32 [n_tok]; token r goes to physical block
 *   slot / 16, in-block row slot % 16.  Negative slots are skipped (padding),
 *   as are slots past the pool.
 * bf16 pools: a plain copy into the layout.
 * FP8 pools: every (block, KV head) keeps one scale for K and one for V, and
 *   each element is stored as the nearest-even E4M3 code of x / scale (fp32
 *   division), saturated to +-448; an all-zero tile has scale 0 and zero
 *   codes.  (Scale per block and head, not per layer as the FP8 paragraph of
 *   froggydisk's page suggests.)  The entries of one call that fill
 *   consecutive rows r0, r0+1, ... of a block (consecutive entries slot,
 *   slot+1, ...) form a run:
 *     - r0 = 0 (a prompt, or the first token of a fresh block): scale =
 *       absmax / 448 over the run's rows (fp32, IEEE division);
 *     - r0 > 0 (appending, e.g. one decode token): rows 0 .. r0-1 must hold
 *       codes written earlier; the scale becomes absmax / 448 over those rows
 *       as they read back (code value x old scale, fp32) and the new rows;
 *       the old codes are re-encoded from their read-back values only if the
 *       scale changed.
 *   Within one call a block may receive at most one run; two runs into one
 *   block in the same call race (undefined result).
 *   Rows of a block past the last one written keep whatever they held and are
 *   never read as long as the context lengths exclude them.
 * bf16 pools: n_tok * n_kv * head_dim must stay below 2^32 (one work-item per
 * element), else KVD_ERR_UNSUPPORTED. */
kvd_status kvd_write_kv(const kvd_pool* pool, int32_t layer, const void* k, const void* v,
                        const int32_t* slot_mapping, int32_t n_tok, void* hip_stream);

/* Slot mapping of kvd_write_kv from block tables: the paging rule of
 * froggydisk's PagedAttention paragraph (section "KV 캐시를 줄이는 기법"):
 * the block table says which physical block holds each 16-token logical
 * block of a request, so token t of sequence i lives in physical block
 * block_table[i][t / 16], in-block row t % 16, i.e. slot
 * block_table[i][t / 16] * 16 + t % 16.
 * block_table:  device int32 [b][max_blocks_per_seq].
 * context_lens: device int32 [b]; s_i, clamped into [0, 16 * max_blocks_per_seq].
 * first_token:  device int32 [b] or NULL (all 0); first_i, clamped into
 *               [0, s_i].  Sequence i contributes its tokens first_i .. s_i - 1
 *               (all of them for a prompt; the last one for a decode step).
 * out_start:    device int64 [b]; token t of sequence i is written to
 *               slots[out_start[i] + t - first_i] (packing is the caller's:
 *               usually the exclusive prefix sum of s_i - first_i).
 * max_tokens_per_seq: a host bound on every s_i - first_i (sizes the launch;
 *               tokens beyond it are not written).
 * slots:        device int32 [n_slots]; positions outside [0, n_slots) are
 *               skipped.  A negative table entry (a block not present) or one
 *               of 2^27 and above (no int32 slot) gives slot -1, which
 *               kvd_write_kv skips.
 * Errors: KVD_ERR_INVALID_ARG for negative sizes or a NULL pointer (other than
 * first_token) when there is work; KVD_ERR_UNSUPPORTED when 16 *
 * max_blocks_per_seq reaches 2^31 or b * ceil(max_tokens_per_seq / 256)
 * reaches 2^24 (one launch of 256-work-item workgroups). */
kvd_status kvd_slot_mapping(const int32_t* block_table, int32_t max_blocks_per_seq, int32_t b,
                            const int32_t* context_lens, const int32_t* first_token, const int64_t* out_start,
                            int32_t max_tokens_per_seq, int32_t* slots, int64_t n_slots, void* hip_stream);

/* Arguments of one decode-attention call on one layer. */
typedef struct {
  int32_t b;                  /* sequences                                            */
  int32_t n_q;                /* query heads, a multiple of the pool's n_kv           */
  int32_t max_blocks_per_seq; /* row length of block_table                            */
  int32_t max_context_len;    /* host-known bound on every s_i (sizes the launch)     */
  const void* q;              /* device bf16 [b][n_q][head_dim], post-RoPE, 16-byte   */
                              /* aligned                                              */
  const int32_t* block_table; /* device int32 [b][max_blocks_per_seq]; entries at or  */
                              /* past ceil(s_i / 16) are never read.  A negative     */
                              /* entry marks a block that is not attended: its tokens */
                              /* take no part and nothing of it is read (attention   */
                              /* over a subset of blocks, e.g. the T0 and T1 tiers   */
                              /* of "Not all thinking needs HBM", methodology 3);    */
                              /* with every block dropped a head's output is 0 and   */
                              /* its lse -inf.  Entries >= num_blocks read as zeros  */
                              /* (the result is then undefined).                     */
  const int32_t* context_lens;/* device int32 [b]; s_i is clamped into               */
                              /* [0, min(max_context_len, 16 * max_blocks_per_seq)]  */
  void* out;                  /* device bf16 [b][n_q][head_dim], 8-byte aligned;      */
                              /* s_i = 0 gives zeros                                  */
  float* lse_out;             /* optional device fp32 [b][n_q]: natural-log           */
                              /* log-sum-exp of the scaled scores (-inf if s_i = 0)   */
  int32_t chunk_tokens;       /* context split: 0 = automatic, else a multiple of 16  */
                              /* (of 32 when a score is requested)                    */
  void* workspace;            /* device scratch of kvd_decode_workspace_bytes bytes,  */
  size_t workspace_bytes;     /* 256-byte aligned; may be NULL when that size is 0.   */
                              /* Calls that overlap in time must not share one.       */
  float* score;               /* optional device fp32 [b][score_stride] cumulative    */
  int32_t score_stride;       /* score; >= max_context_len when score is set          */
  float score_weight;         /* score[i][t] += score_weight * mean_h alpha_h(t)      */
  uint32_t flags;             /* KVD_FLAG_* bits (0: the defaults); an unknown bit    */
                              /* gives KVD_ERR_INVALID_ARG                            */
} kvd_decode_args;

/* flags: keep every chunk of an automatic split the same length (no uneven
 * pairs, kvd_decode_plan).  For a batch whose sequences share most of their
 * blocks (a common prompt stored once): its reads are served mostly by the
 * L2, where the XCDs do not differ, and the uneven pairs only unbalance it
 * (measured: 32 requests behind one 16,384-token prompt, 147.6 against
 * 155.3 us per layer call). */
#define KVD_FLAG_EVEN_CHUNKS 1u

/* How a decode call splits the context: chunk length C in tokens and number
 * of chunks.  Chunk c of a sequence covers tokens [c*C, (c+1)*C), except that
 * an automatic split (chunk_tokens = 0) with an even n_kv, two or more chunks,
 * no score and no KVD_FLAG_EVEN_CHUNKS pairs its chunks unevenly: with d = 32 * floor((45 * C + 16000)
 * / 32000) -- about 4.5 % of C in whole 32-token pairs -- (when C is a
 * multiple of 32, d > 0 and C - d >= 32; else d = 0), chunks 2p
 * and 2p + 1 of KV head j cover [2pC, 2pC + C + d) and [2pC + C + d, 2pC + 2C)
 * when j is even, [2pC, 2pC + C - d) and [2pC + C - d, 2pC + 2C) when j is
 * odd; a last chunk without a partner covers [c*C, (c+1)*C).  The workgroups
 * of the longer chunks run on the device's faster half of its XCDs.  The
 * split never changes what is computed, only how the sum over the context is
 * grouped.  Pure host function of the pool and the arguments.  A launch holds
 * fewer than 2^32 work-items and a workgroup 256, so b * n_kv * n_chunks and
 * b * n_q must stay below 2^24 (KVD_ERR_UNSUPPORTED otherwise, from every
 * decode entry point). */
kvd_status kvd_decode_plan(const kvd_pool* pool, const kvd_decode_args* args,
                           int32_t* chunk_tokens, int32_t* n_chunks);

/* Workspace bytes a decode call with these arguments needs (0 when the whole
 * context fits one chunk and no score is requested): the per-chunk partials
 * and, with a score, the scaled scores and lse of the call.  Pure host
 * function. */
kvd_status kvd_decode_workspace_bytes(const kvd_pool* pool, const kvd_decode_args* args,
                                      size_t* bytes);

/* One decode-attention step of one layer on a bf16 pool.
 * Each (sequence, KV head, context chunk) is processed by one workgroup that
 * streams the chunk's K/V blocks once and serves all g query heads of the KV
 * head from them.  With one chunk that workgroup writes the output; with
 * more, a second kernel merges the per-chunk results by log-sum-exp
 * (kvd_merge_partials' arithmetic, restricted to each sequence's chunks).
 * With score a further kernel adds the weights once every head's lse is
 * known.
 * With score set, adds score_weight * (1/n_q) * sum_h alpha_h(t) to
 * score[i][t] for every t < s_i, alpha_h(t) being the softmax weight of
 * token t for head h -- the per-layer term of the cumulative attention score
 * (gist.science summary of "Not all thinking needs HBM", methodology 2); pass
 * score_weight = 1/L to average over L layers.
 * Returns KVD_ERR_DTYPE on an FP8 pool. */
kvd_status kvd_decode_attn(const kvd_pool* pool, int32_t layer, const kvd_decode_args* args,
                           void* hip_stream);

/* Same on an FP8 pool.  Codes are widened to bf16 in registers (exact) and
 * the per-(block, head) scales are applied to the scores (K) and to the
 * softmax weights (V), so no dense K/V is ever written back to memory (the
 * no-reconstruction rule of the Spherical KV summary, §2.1).  Returns
 * KVD_ERR_DTYPE on a bf16 pool. */
kvd_status kvd_decode_attn_fp8(const kvd_pool* pool, int32_t layer, const kvd_decode_args* args,
                               void* hip_stream);

/* A decode step that first stores the step's own token, in one launch.  The
 * token being decoded is already part of its context (s_i counts it) and its
 * K/V go into the sequence's last block (froggydisk, section "KV 캐시를
 * 줄이는 기법", the PagedAttention paragraph: the decode step writes into
 * the partly filled last block).  new_k, new_v: device bf16 [b][n_kv][d_h],
 * the K and V of token s_i - 1 of each sequence.  The call stores them at that
 * token's slot -- block_table[i][(s_i - 1) / 16], row (s_i - 1) % 16 -- with
 * the bytes kvd_write_kv would store (FP8: the tile re-quantised under
 * kvd_write_kv's append rule), then runs the step of kvd_decode_attn
 * (bf16 pool) or kvd_decode_attn_fp8 (FP8 pool) over the context including
 * that token: outputs, lse, score and pool contents equal those of
 * kvd_write_kv followed by the decode call, bit for bit.  The store is done by
 * the workgroups whose chunk holds token s_i - 1, before they read that block.
 * Nothing is stored for a sequence with s_i = 0, with a context length above
 * min(max_context_len, 16 * max_blocks_per_seq) (its token has no slot inside
 * that bound; the step then attends to the clamped context, as kvd_decode_attn
 * does, and every cached row keeps its value), or whose last table entry is
 * negative or >= num_blocks.  Args, workspace and errors as kvd_decode_attn;
 * KVD_ERR_INVALID_ARG if new_k or new_v is NULL. */
kvd_status kvd_decode_attn_append(const kvd_pool* pool, int32_t layer, const kvd_decode_args* args,
                                  const void* new_k, const void* new_v, void* hip_stream);

/* Decode over a mixed-precision block set: bf16 blocks in pool_bf16 and FP8
 * E4M3 blocks in pool_fp8 (both with the same num_layers, n_kv, head_dim;
 * fewer than 2^30 blocks each), following "The KV Cache Is the New Memory
 * Wall" review §5.5 (one paged layout with a precision per block and a keep
 * mask) and the gist.science summary of "Spherical KV" §2.2 (tier-homogeneous
 * pages read in one header-guided pass).  Each block_table entry names its
 * block's pool in bit 30 (set: pool_fp8, block = entry & ~(1 << 30)) -- the
 * page header; a negative entry is a block that is not attended.  Entries
 * may come in any order, precisions alternating or not; a row that lists one
 * precision's blocks, a -1 if that run is odd, then the other's
 * (kvd_mixed_row) keeps pages of two entries tier-homogeneous, and each
 * precision's pass then visits only its own span of the row.  Only the final
 * entry of a row may be partly filled.  The softmax covers the row's blocks
 * whatever their order, so the output is the step over those tokens.
 * No fused score (KVD_ERR_UNSUPPORTED: the rearranged row has no logical
 * token positions).  Workspace, chunking and outputs as kvd_decode_attn (use
 * pool_bf16 for kvd_decode_workspace_bytes).  KVD_ERR_DTYPE if pool_bf16 is
 * not bf16 or pool_fp8 not FP8. */
kvd_status kvd_decode_attn_mixed(const kvd_pool* pool_bf16, const kvd_pool* pool_fp8, int32_t layer,
                                 const kvd_decode_args* args, void* hip_stream);

/* kvd_decode_attn for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same step, on a bf16 or an FP8 pool alike (the pool's dtype picks the
 * kernels, as in kvd_decode_attn_append), with the split partials and score
 * scratch kept in a fixed array the library holds on each device (32 MiB,
 * the first call on a device looks up its address; it stays allocated until
 * the process ends) instead of args->workspace, which is ignored.  Calls
 * whose kvd_decode_workspace_bytes exceeds 32 MiB return KVD_ERR_WORKSPACE
 * before any launch.  The call itself allocates nothing.  Every call on one
 * device uses that device's one array: calls that overlap in time on the same
 * device (on different streams, or from different threads) race and give
 * undefined results; calls in order on one stream are safe.  The stream must
 * belong to the calling thread's current device.  Nothing in the array has to
 * start at any value.  Outputs, lse and score equal those of kvd_decode_attn /
 * kvd_decode_attn_fp8 with a workspace, bit for bit. */
kvd_status kvd_decode_attn_no_alloc(const kvd_pool* pool, int32_t layer, const kvd_decode_args* args,
                                    void* hip_stream);

/* Per-chunk partial results of one decode step of one layer, for a caller
 * that merges them itself -- for example the partials of context shards held
 * by several GPUs, combined with kvd_merge_partials.  Works on bf16 and FP8
 * pools alike.  The context is split as kvd_decode_plan reports and describes
 * (n_chunks chunks per sequence; with an explicit chunk_tokens, chunk c covers
 * tokens [c*chunk, (c+1)*chunk) of each sequence), always as partials (also
 * when n_chunks is 1).
 * part_o:   device fp32 [b][n_q][n_chunks][d_h], 16-byte aligned: each chunk's
 *           own normalised output;
 * part_lse: device fp32 [b][n_q][n_chunks]: natural-log lse of the chunk's
 *           scaled scores, -inf for a chunk past the end of its sequence (whose
 *           part_o row is left unwritten).
 * args->out, lse_out and workspace are not used; args->score must be NULL. */
kvd_status kvd_decode_partials(const kvd_pool* pool, int32_t layer, const kvd_decode_args* args,
                               float* part_o, float* part_lse, void* hip_stream);

/* Merge per-chunk partial results by log-sum-exp.
 * The attention step of froggydisk's section "KV 캐시란" (scores divided by
 * sqrt(128), a softmax over them, the V rows summed with those weights) is a
 * sum over the context's tokens; split into chunks, each chunk's normalised
 * output o_c and log-sum-exp lse_c determine the whole exactly, which is what
 * lets a long context be split over workgroups or over devices (the
 * capacity-bound sharding of "The KV Cache Is the New Memory Wall" review,
 * Tab. 5) and put together here.
 * part_o:   device fp32 [b][n_q][n_chunks][d_h], 16-byte aligned, each chunk's
 *           normalised output
 * part_lse: device fp32 [b][n_q][n_chunks], natural log; -inf marks an empty
 *           chunk, which contributes nothing (its part_o row may hold anything,
 *           NaN included)
 * out_bf16: device bf16 [b][n_q][d_h], 8-byte aligned; lse_out: optional fp32
 *           [b][n_q].
 * lse = M + ln(sum_c exp(lse_c - M)), M = max_c lse_c, and
 * out = sum_c exp(lse_c - lse) * o_c in fp32, rounded to bf16 (nearest even);
 * the order of the fp32 additions is fixed for given b, n_q, n_chunks and d_h,
 * so equal inputs give equal bits.  d_h must be 64 or 128 (else
 * KVD_ERR_UNSUPPORTED); a misaligned or NULL pointer gives KVD_ERR_INVALID_ARG. */
kvd_status kvd_merge_partials(const float* part_o, const float* part_lse, int32_t b, int32_t n_q,
                              int32_t n_chunks, int32_t d_h, void* out_bf16, float* lse_out,
                              void* hip_stream);

/* Static string naming a status. */
const char* kvd_status_string(kvd_status status);

/* Name and description of the HIP error behind the calling thread's most
 * recent KVD_ERR_HIP (like errno: per thread, kept until the next such error;
 * "hipSuccess: ..." if there was none).  The string is owned by the library
 * and valid until the thread's next call of this function. */
const char* kvd_last_hip_error(void);

/* ---- test hooks: expose device-side pieces of the hot path ------------- */

/* Element offsets (in elements of the pool's dtype, from kv_base) of K[t][c=0]
 * and V[t][c=0] for every sequence i, KV head j and token t < n_tok, as the
 * decode kernels compute them.  out_k, out_v: device int64 [b][n_kv][n_tok].
 * Entries for table entries outside [0, num_blocks) are -1. */
kvd_status kvd_debug_gather_offsets(const kvd_pool* pool, int32_t layer, const int32_t* block_table,
                                    int32_t max_blocks_per_seq, int32_t b, int32_t n_tok,
                                    int64_t* out_k, int64_t* out_v, void* hip_stream);

/* The work decomposition of a decode call with these arguments, as its
 * kernels compute it: the grid holds b * n_kv * n_chunks workgroups
 * (kvd_decode_plan), each serving one KV head and one (sequence, chunk) unit,
 * found on the device from the context lengths.  units: device int32
 * [b * n_kv * n_chunks][6], row x = (sequence, chunk, context length after
 * clamping, KV head, first token, end token of the chunk) of workgroup x --
 * the head is x % n_kv and the span [c*C, (c+1)*C) unless the chunks are
 * paired unevenly (kvd_decode_plan).  Only args->b, n_q, max_blocks_per_seq,
 * max_context_len, context_lens, chunk_tokens and score (which constrains the
 * chunking) are used. */
kvd_status kvd_debug_unit_map(const kvd_pool* pool, const kvd_decode_args* args, int32_t* units,
                              void* hip_stream);

/* Decode n E4M3 codes with the decode kernels' own widening routine.
 * codes: device uint8 [n]; out: device fp32 [n]. */
kvd_status kvd_debug_fp8_decode(const uint8_t* codes, int32_t n, float* out, void* hip_stream);

/* A plain streaming read of `bytes` bytes at `data` with the decode kernels'
 * own 16-byte non-temporal loads and nothing else -- the read rate those loads
 * reach on this device, the practical ceiling of a decode launch of the same
 * size (Spherical KV summary §1: decode time is the time to stream the pages).
 * data: device, 16-byte aligned; bytes: a multiple of 16, at least 16 and
 * below 2^32 (else KVD_ERR_UNSUPPORTED); grid: 1 .. 65536 workgroups of 256
 * work-items; sink: device uint32 [grid * 256], each entry the XOR of the
 * 32-bit words its work-item read (so the XOR of all entries is the XOR of
 * every word of the buffer). */
kvd_status kvd_debug_stream_read(const void* data, uint64_t bytes, uint32_t* sink, int32_t grid,
                                 void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* KVDECODE_H */
