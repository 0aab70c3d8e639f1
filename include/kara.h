/*
 * kara.h - C ABI of the Kara decode-time window-compression step on MI355X (gfx950).
 *
 * Kara ("Kara: Efficient Reasoning LLM Serving via Sliding-Window KV Cache
 * Compression", authors' English abstract and section 方法详解 of its
 * shd-paper.top summary page) compresses, while decoding, only the most recent
 * window of generated tokens: it scores the window's KV pairs with
 * bidirectional attention, selects informative ones, grows a subset of them
 * into chunks (Token2Chunk) and keeps the result in a PagedAttention cache.
 *
 * One "unit" is (sequence n, layer l, KV head g).  For every unit the step
 *   1. kara_score_window  : c[j] = sum_{h in group g} sum_{i<W} softmax_j'(q[h,i].k[j']/sqrt(d))[j]
 *   2. kara_select_chunks : seeds = first `seeds` positions of the order (c desc, position asc);
 *                           chunks = [p-radius, p+radius] clipped to the window, merged;
 *                           fill the rest of `budget` with the best positions outside the chunks;
 *                           kept = ascending list of exactly `budget` window positions
 *   3. kara_compact_paged : slot L+r <- slot L+kept[r] (K and V, in place), then every
 *                           sequence's block table drops the blocks past L+budget.
 * The pages give no formula for the score, the Token2Chunk rule or the in-place
 * layout; the definitions above are the plainest readings of their text.
 *
 * Conventions for every entry point
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    allocates nothing, keeps no state between calls and is reentrant, apart
 *    from kara_compress_fused_noalloc's fixed per-device counter array (see
 *    there).
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls only enqueue
 *    work and return; results are ready when the stream reaches them.
 *  - Arguments are checked on the host before anything is enqueued: a call that
 *    returns an error has enqueued nothing and written nothing.
 *  - Device-side contents (block ids, prior lengths, kept lists) are not
 *    checked by the three step calls.  Kernels never access memory outside the
 *    buffers the configuration describes: a read through an out-of-range
 *    table entry (negative or >= num_blocks) returns the row of physical block
 *    0 (it exists whenever there is a sequence), and compaction neither reads
 *    nor writes a slot whose entry is out of range.  The outputs for such a
 *    sequence are unspecified.  kara_validate_tables reports such sequences;
 *    call it before trusting tables built elsewhere.
 *
 * Layouts (row-major, contiguous, element type = cfg.dtype unless stated):
 *   q            [num_seqs][num_layers][window][num_q_heads][head_dim]  window queries
 *   k_cache,
 *   v_cache      [num_layers][num_blocks][num_kv_heads][block_size][head_dim]
 *   block_tables int32 [num_seqs][max_blocks_per_seq]; logical block b of sequence n
 *                lives in physical block block_tables[n][b]
 *   prior_lens   int32 [num_seqs]: L, tokens before the window; the window is the
 *                logical slots [L, L+window)
 *   scores       float [num_seqs][num_layers][num_kv_heads][window]
 *   kept         int32 [num_seqs][num_layers][num_kv_heads][budget], window-relative
 *   mask         uint8 [num_seqs][num_layers][num_kv_heads][window] (optional)
 *   freed_blocks int32 [num_seqs][kara_max_freed(cfg)], -1 padded
 *   num_freed    int32 [num_seqs];  seq_lens int32 [num_seqs] (out: L + budget)
 * Query head h belongs to KV head h / (num_q_heads / num_kv_heads).
 */
#ifndef KARA_H_
#define KARA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define KARA_OK 0
#define KARA_EINVAL (-1)     /* a configuration value or constraint is violated */
#define KARA_ENULL (-2)      /* a required pointer is NULL */
#define KARA_EWORKSPACE (-3) /* workspace missing or smaller than kara_workspace_bytes */
#define KARA_EHIP (-4)       /* the HIP runtime reported an error while enqueueing */
#define KARA_ENOTIMPL (-5)   /* valid request this library does not support */
#define KARA_ESCRATCH (-6)   /* request larger than the fixed scratch of an allocation-free entry point */

/* most sequences one kara_compress_fused_noalloc call may cover */
#define KARA_NOALLOC_MAX_SEQS 65536

/* element types of q, k_cache and v_cache */
#define KARA_BF16 0
#define KARA_F32 1

typedef struct kara_config {
  int32_t num_seqs;      /* >= 0 (0 = nothing to do) */
  int32_t num_layers;    /* >= 1 */
  int32_t num_q_heads;   /* >= 1, multiple of num_kv_heads, (num_q_heads / num_kv_heads) * window <= 2^24 */
  int32_t num_kv_heads;  /* >= 1 */
  int32_t head_dim;      /* 64 or 128 */
  int32_t window;        /* W, 1..8192 */
  int32_t budget;        /* B, 1..W */
  int32_t seeds;         /* s >= 0 */
  int32_t radius;        /* r >= 0, with s*(2r+1) <= B */
  int32_t block_size;    /* power of two, 1..256 */
  int32_t dtype;         /* KARA_BF16 or KARA_F32 */
  int32_t max_blocks_per_seq; /* >= 1, columns of block_tables; times block_size at most 2^30 */
  int64_t num_blocks;    /* physical blocks per layer in k_cache / v_cache: 0..2^31-1, >= 1 if num_seqs > 0 */
} kara_config;

/* Checks a configuration on the host; returns KARA_OK or KARA_EINVAL. */
int kara_check_config(const kara_config* cfg);

/* Bytes of device workspace kara_score_window needs for cfg (0 if none);
 * returns 0 for an invalid cfg. */
size_t kara_workspace_bytes(const kara_config* cfg);

/* Which scorer kara_score_window runs for cfg: 1 = single pass, either with
 * the window's keys resident in registers (bf16, head_dim 128, W <= 1024) or
 * staged in LDS (any other dtype / head_dim with W <= 256, W <= 128 for fp32
 * rows of head_dim 128); 2 = two passes (row log-sum-exp, then column mass;
 * needs the workspace); 0 for an invalid cfg.  All compute the same scores.
 * kara_workspace_bytes is 0 exactly when this is 1 (or cfg is invalid). */
int kara_score_passes(const kara_config* cfg);

/* Columns of freed_blocks: the most blocks one sequence can free, ceil(W/bs)+1. */
int32_t kara_max_freed(const kara_config* cfg);

/*
 * Step 1 - window scores (bidirectional in-window attention; Kara abstract).
 * For every unit writes scores[n][l][g][j] = c[j] as defined above, in fp32.
 * Reads q and the window rows of k_cache through block_tables; q, k_cache,
 * block_tables and prior_lens are not modified.  `workspace` must hold
 * kara_workspace_bytes(cfg) bytes (256-byte aligned); its contents on entry
 * are ignored.  Errors: KARA_EINVAL, KARA_ENULL, KARA_EWORKSPACE, KARA_EHIP.
 */
int kara_score_window(const kara_config* cfg, const void* q, const void* k_cache,
                      const int32_t* block_tables, const int32_t* prior_lens, float* scores,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Step 2 - Token2Chunk selection (Kara abstract: a subset of the selected KV
 * pairs is expanded into chunks).  For every unit reads scores[n][l][g][:] and
 * writes the `budget` kept window positions, strictly ascending, to kept.  If
 * mask is not NULL it also writes mask[..][j] = 1 for kept j, else 0.  The
 * order compares scores as IEEE floats (-0 equals +0) and breaks ties by the
 * lower position; scores must not be NaN.  Errors: KARA_EINVAL, KARA_ENULL,
 * KARA_EHIP.
 */
int kara_select_chunks(const kara_config* cfg, const float* scores, int32_t* kept, uint8_t* mask,
                       void* stream);

/*
 * Largest number of positions the chunks of the bridging rule below can cover:
 * seeds*(2*radius+1) + max(0, seeds-1) * max(0, gap - 2*radius).  -1 if cfg is
 * NULL or seeds, radius or gap is negative.  Host only.
 */
int64_t kara_chunk_bound(const kara_config* cfg, int32_t gap);

/*
 * Step 2, bridging variant of Token2Chunk (the method's lay explainers,
 * gist.science, section "2. Das Token2Chunk-Modul": a chunk is whatever lies
 * between two important positions and has no fixed size).  Same as
 * kara_select_chunks, except that after the radius spans are formed the seeds
 * are taken in ascending position, and two neighbouring seeds p < p' with
 * p' - p - 1 <= gap also keep every position between them.  gap = 0 gives
 * exactly kara_select_chunks.  Requires 0 <= gap <= window and
 * kara_chunk_bound(cfg, gap) <= budget, else KARA_EINVAL.  Same layouts,
 * ownership and errors as kara_select_chunks.
 */
int kara_select_chunks_bridged(const kara_config* cfg, int32_t gap, const float* scores, int32_t* kept,
                               uint8_t* mask, void* stream);

/*
 * Step 3 - in-place compaction into PagedAttention blocks (Kara abstract: the
 * method is adapted to PagedAttention and lowers KV memory).  For every unit
 * and r < budget, the K and V rows of logical slot L+r become the old rows of
 * slot L+kept[r] (all old rows are read before any is overwritten; kept must
 * be strictly ascending in [0, window)).  Then, per sequence, the entries of
 * logical blocks ceil((L+B)/bs) .. ceil((L+W)/bs)-1 are copied in that order
 * to freed_blocks[n][..] (rest -1), set to -1 in block_tables, num_freed[n]
 * gets their count and seq_lens[n] = L + B.  No other byte of k_cache or
 * v_cache changes.  The caller may reuse freed blocks once the stream has
 * passed this call.  Errors: KARA_EINVAL, KARA_ENULL, KARA_EHIP.
 */
int kara_compact_paged(const kara_config* cfg, void* k_cache, void* v_cache, int32_t* block_tables,
                       const int32_t* prior_lens, int32_t* seq_lens, const int32_t* kept,
                       int32_t* freed_blocks, int32_t* num_freed, void* stream);

/*
 * Step 3 when the window is the oldest part of the context not yet compressed
 * (the gist.science explainer of the method, section "3. Der Periodische
 * Zeitplan": the schedule cleans the back end of the current thought), so that
 * tail_lens[n] = T newer tokens follow the window in slots [L+W, L+W+T).  Same
 * as kara_compact_paged, except that after the kept rows those T rows move in
 * order right behind them (slot L+B+t takes the old row of slot L+W+t), the
 * table keeps the blocks of the first L+B+T slots (entries of logical blocks
 * ceil((L+B+T)/bs) .. ceil((L+W+T)/bs)-1 are freed) and seq_lens[n] = L+B+T.
 * tail_lens is int32 [num_seqs] device memory (required); a negative entry
 * counts as 0, and T is clamped to the slots the table can address after the
 * window.  T = 0 gives exactly kara_compact_paged.  Errors: KARA_EINVAL,
 * KARA_ENULL, KARA_EHIP.
 */
int kara_compact_paged_tail(const kara_config* cfg, void* k_cache, void* v_cache, int32_t* block_tables,
                            const int32_t* prior_lens, const int32_t* tail_lens, int32_t* seq_lens,
                            const int32_t* kept, int32_t* freed_blocks, int32_t* num_freed, void* stream);

/*
 * The whole step in one launch: scores, Token2Chunk selection and in-place
 * compaction of every unit, and every sequence's block-table rewrite, with
 * exactly the results of kara_score_window + kara_select_chunks +
 * kara_compact_paged (same layouts and outputs; mask may be NULL).  One
 * workgroup scores a unit, selects from the scores it produced and compacts
 * the unit's rows; the last workgroup of a sequence to finish rewrites that
 * sequence's table.  `done` is int32 [num_seqs] device memory that must hold
 * zeros before the first call; every call returns it to zeros.  Calls that
 * share a `done` array must not run concurrently.  Available when
 * kara_compress_fused_supported(cfg) is 1, which is exactly when
 * kara_score_passes(cfg) is 1 (the single-pass scorers), else KARA_ENOTIMPL.  Other errors: KARA_EINVAL, KARA_ENULL, KARA_EHIP.
 */
int kara_compress_fused_supported(const kara_config* cfg);

int kara_compress_fused(const kara_config* cfg, const void* q, void* k_cache, void* v_cache,
                        int32_t* block_tables, const int32_t* prior_lens, float* scores, int32_t* kept,
                        uint8_t* mask, int32_t* seq_lens, int32_t* freed_blocks, int32_t* num_freed,
                        int32_t* done, void* stream);

/*
 * kara_compress_fused without caller scratch, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, layouts, results and
 * errors as kara_compress_fused, except that the per-sequence counters live in
 * a fixed array of KARA_NOALLOC_MAX_SEQS int32 that the library holds on every
 * GPU it runs on (256 KiB each, until the process ends).  The call allocates
 * nothing: on its first use on a device (which must be the current device,
 * and the device of `stream`) it looks the array's address up once.  Every
 * call clears the counters it uses on `stream` before the pipeline runs.
 * Calls that overlap on one GPU share the array and race: serialise them
 * (one stream, or events).  num_seqs > KARA_NOALLOC_MAX_SEQS gives
 * KARA_ESCRATCH and enqueues nothing; a stream of another device gives
 * KARA_EINVAL.
 */
int kara_compress_fused_noalloc(const kara_config* cfg, const void* q, void* k_cache, void* v_cache,
                                int32_t* block_tables, const int32_t* prior_lens, float* scores, int32_t* kept,
                                uint8_t* mask, int32_t* seq_lens, int32_t* freed_blocks, int32_t* num_freed,
                                void* stream);

/*
 * Consumer of the compacted cache: one decode step of paged attention (Kara
 * abstract: the compressed window lives in a PagedAttention store whose
 * smaller footprint raises output throughput).  For every sequence n, layer
 * and query head h (KV head h / (num_q_heads / num_kv_heads)):
 *   out[n][l][h] = sum_{j < T} softmax_j(q_dec[n][l][h] . k_j / sqrt(head_dim)) v_j
 * over the logical slots j < T = seq_lens[n] of the sequence, read through its
 * block table (after kara_compact_paged, T = L + budget).  T = 0 gives zeros;
 * T is clamped to max_blocks_per_seq * block_size.
 *   q_dec  [num_seqs][num_layers][num_q_heads][head_dim], cfg.dtype
 *   out    float [num_seqs][num_layers][num_q_heads][head_dim]
 *   k_cache, v_cache, block_tables: as above; seq_lens int32 [num_seqs]
 * Only the fields num_seqs, num_layers, num_q_heads, num_kv_heads, head_dim,
 * block_size, dtype, max_blocks_per_seq and num_blocks matter, but the whole
 * configuration must be valid.  workspace: device memory of at least
 * kara_decode_attention_workspace_bytes(cfg) bytes, 256-byte aligned (may be
 * NULL when that is 0); it holds per-split partial results.  Errors:
 * KARA_EINVAL, KARA_ENULL, KARA_EWORKSPACE, KARA_EHIP.
 */
size_t kara_decode_attention_workspace_bytes(const kara_config* cfg);

/* Number of workgroups that share one (sequence, layer, head group) slot range
 * in kara_decode_attention (1 = no merge pass); 0 for an invalid cfg. */
int kara_decode_attention_splits(const kara_config* cfg);

int kara_decode_attention(const kara_config* cfg, const void* q_dec, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, const int32_t* seq_lens, float* out, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * Debug check of the device-side addressing data: for every sequence, L >= 0,
 * L + W <= max_blocks_per_seq * block_size, and every table entry of the
 * logical blocks that hold slots [L - L % bs, L + W) lies in [0, num_blocks).
 * Writes to *bad_seqs (device int32) the number of sequences that fail.
 * Errors: KARA_EINVAL, KARA_ENULL, KARA_EHIP.
 */
int kara_validate_tables(const kara_config* cfg, const int32_t* block_tables,
                         const int32_t* prior_lens, int32_t* bad_seqs, void* stream);

/* Short text for a status code (static storage). */
const char* kara_status_str(int status);

/* HIP error code behind the last KARA_EHIP returned on this thread (0 if none). */
int kara_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KARA_H_ */
