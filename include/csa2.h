/*
 * csa2.h -- C ABI of libcsa2: the global-attention hot path of Compressed
 * Sparse Attention 2 (CSA2) for AMD Instinct MI355X (gfx950).
 *
 * The operation is the one described in "DeepSeek-V4.1-Flash: Pushing the
 * Limits of KV Cache Compression" (report digest), section 2.3 (CSA2),
 * 2.3.1 (Full / Reindex / Reuse modes), 2.3.2 (Hierarchical Sparse Indexer,
 * Fig. 5) and 2.4.4 (FP4 main KV cache), with the sizes of the mer.dev
 * commentary on that report (section 1 setup: 512-d latent, 64 query heads of
 * dim 512, a 32 x 128 indexer, top-k 512, 2048 blocks of 8 positions, SWA
 * window 128; section 2: 356 bytes per entry).
 *
 * Conventions for every entry point
 *   - All array arguments are DEVICE pointers unless marked (host).  The
 *     caller owns every buffer; the library never allocates or frees device
 *     memory and keeps no state except a thread-local error string (and
 *     the static scratch of csa2_select_topk_noalloc, one per GPU).
 *   - Every call enqueues its kernels on `stream` (a hipStream_t, may be 0
 *     for the null stream) and returns without synchronising.
 *   - bf16 values are passed as uint16_t bit patterns.
 *   - Every array must be aligned to at least its element size (8 bytes for
 *     int64, 4 for int32 and fp32); where an entry point states a stronger
 *     alignment (16 bytes for bf16 / byte arrays the kernels read as
 *     vectors and for fp32 attention outputs, 256 for workspaces that hold
 *     maxima levels) that one applies.  A misaligned pointer returns
 *     CSA2_EINVAL.
 *   - Arguments are validated on the host before anything is launched.  A
 *     bad argument returns CSA2_EINVAL (or CSA2_EUNSUPPORTED for a size the
 *     library does not implement, CSA2_EWORKSPACE for a short workspace)
 *     and sets csa2_last_error().  Launch failures return CSA2_EHIP.
 *   - The contents of device arrays (indices, cache bytes) are not checked;
 *     out-of-range indices are undefined behaviour.  With CSA2_CHECK=1 in
 *     the environment, csa2_index_score (q_seq in [0, batch), or >= 0 when
 *     batch is 0; candidate ids in [0, cap)) and csa2_sparse_attend (q_seq
 *     likewise, idx in [-1, cap)) first
 *     range-check their index arrays on the device, synchronise the stream
 *     and return CSA2_EINVAL naming the array if any value is out of range
 *     (checked calls are synchronous and must not be graph-captured).
 *   - No exception or abort crosses the ABI.  Calls are thread-safe.
 *
 * Cache layout (one KV-producing layer, B sequences, `cap` entries each,
 * structure of arrays, entry (b, j) at flat index b * cap + j):
 *   kv_codes  [B][cap][256] u8  E2M1 main-KV codes, channel 2c in the low nibble
 *   kv_scales [B][cap][32]  u8  E4M3FN scale of channels 16g..16g+15
 *   ik_codes  [B][cap][64]  u8  E2M1 indexer-K codes, dim 2c in the low nibble
 *   ik_scales [B][cap][4]   u8  E8M0 scale of dims 32g..32g+31
 * = 288 B main KV + 68 B indexer K = 356 B per entry (commentary, section 2).
 * The bytes are the cache's whole state: saving and restoring it is a copy.
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CSA2_OK = 0,
  CSA2_EINVAL = 1,        /* bad argument (null pointer, size, alignment)  */
  CSA2_EUNSUPPORTED = 2,  /* a size or mode outside what the library does  */
  CSA2_EWORKSPACE = 3,    /* workspace smaller than csa2_workspace_bytes()  */
  CSA2_EHIP = 4           /* the HIP runtime reported an error              */
} csa2_status;

/* Fixed sizes of the path (commentary, section 1 setup). */
#define CSA2_D_LATENT 512   /* main-KV latent channels                        */
#define CSA2_H_INDEX 32     /* indexer heads                                  */
#define CSA2_D_INDEX 128    /* indexer head dim                               */
#define CSA2_H_ATTN 64      /* attention query heads (head dim = CSA2_D_LATENT) */
#define CSA2_MAX_K 2048     /* largest top-k / block count accepted           */
#define CSA2_MAX_SWA 128    /* largest SWA window per query                   */
#define CSA2_MAX_COLS (1 << 24) /* largest score row the selectors accept     */
#define CSA2_MAX_ROPE 64    /* most RoPE channels of csa2_sparse_attend_rope  */

/* Workspace query selectors. */
#define CSA2_OP_TOPK 1
#define CSA2_OP_POOL 2
#define CSA2_OP_ATTEND 3
#define CSA2_OP_SELECT_ATTEND 4   /* csa2_select_attend, n_blocks == 0 */
#define CSA2_OP_POOL_ATTEND 5     /* csa2_select_attend, n_blocks > 0  */

/* One KV-producing layer's cache for B sequences (host struct holding device
 * pointers).  Every pointer must be 16-byte aligned. */
typedef struct {
  uint8_t* kv_codes;
  uint8_t* kv_scales;
  uint8_t* ik_codes;
  uint8_t* ik_scales;
  int64_t cap;            /* entries per sequence (the batch stride) */
  int64_t batch;          /* sequences the arrays hold; 0 = not stated.  Used
                             only by the CSA2_CHECK range check of q_seq.  */
} csa2_cache;

/* Per-sequence decode state of one KV-producing layer (host struct holding
 * device pointers; every pointer 16-byte aligned).  Start from n_tok = 0. */
typedef struct {
  uint16_t* tail_h;       /* [B][m-1][512] bf16 raw latents of the incomplete group (m > 1) */
  uint16_t* tail_z;       /* [B][m-1][512] bf16 their compression logits (m > 1)            */
  int64_t* n_tok;         /* [B] tokens appended so far                                     */
  uint8_t* swa_codes;     /* [B][W][512] E4M3FN SWA rows, a ring: token t in slot t mod W   */
  float* swa_scale;       /* [B][W] fp32 row scale sigma                                    */
  int64_t W;              /* ring slots (the SWA window), 0 <= W <= CSA2_MAX_SWA            */
  int m;                  /* compression ratio of the layer, 1 <= m <= 16                   */
} csa2_state;

/* Name of a status code (static string). */
const char* csa2_status_string(int status);

/* Detail of the last failed call on this thread ("" if none). */
const char* csa2_last_error(void);

/*
 * (1) Compress, quantise and project: steps a1-a3 of the path.
 *
 * Report section 2.3: CSA2 compresses every m raw entries into one with no
 * overlap between the sources of adjacent entries and no absolute position
 * embedding, and obtains the indexer K by projecting the main-KV entry;
 * section 2.4.4: the main KV is stored as E2M1 with one E4M3 scale per 16
 * channels (no second-level scale), the indexer K as OCP MXFP4.
 *
 * For each sequence b and entry j in [0, T/m):
 *   x[c]  = sum_t softmax_t(z[b][jm+t][c]) * h[b][jm+t][c]     (t < m)
 *           (x = h when m == 1; the softmax form follows the commentary,
 *            section 4.1)
 *   s_g   = E4M3FN(RNE, saturating)(max_{c in g} |x[c]| / 6), 16-channel g
 *   code  = E2M1(RNE, saturating)(x[c] / s_g), all +0 when s_g == 0
 *   k[d]  = sum_c w_ik[d][c] * xhat[c]     (xhat = the dequantised main KV)
 *   MXFP4: X = 2^(floor(log2 max|k_g|) - 2) as E8M0 per 32 dims, E2M1(k / X)
 * and writes entry e0 + j of sequence b of `dst`.
 *
 *   h      [B][T][512] bf16  raw latents
 *   z      [B][T][512] bf16  compression logits; may be NULL iff m == 1
 *   B, T   sequences and raw tokens per sequence; T % m == 0
 *   m      compression ratio, 1 <= m <= 16
 *   w_ik   [128][512] bf16   indexer-K projection (output dim x input channel)
 *   dst    cache written at entries [e0, e0 + T/m); requires e0 + T/m <= cap
 */
csa2_status csa2_compress_quant(const uint16_t* h, const uint16_t* z, int B, int64_t T, int m,
                                const uint16_t* w_ik, const csa2_cache* dst, int64_t e0,
                                void* stream);

/*
 * (2) Lightning-indexer scores: step a4 (full scan) and a7 (Reindex scoring
 * of a candidate pool).
 *
 * Report section 2.3 (indexer Q and K score the main-KV entries), section
 * 2.3.2 (the first Full layer scores every causally visible entry; Reindex
 * layers score only the pool); score form of the commentary, section 4.1:
 *   score(q, j) = sum_{h<32} w[q][h] * max(0, sum_{c<128} q_idx[q][h][c] * khat_j[c])
 * with khat the dequantised MXFP4 indexer K.  Accumulation is fp32.
 *
 *   q_idx  [Q][32][128] bf16   indexer queries
 *   w      [Q][32] fp32        per-head weights
 *   q_seq  [Q] int32           sequence (cache row block) of each query
 *   n_vis  [Q] int64           columns to score for each query (<= n_cols)
 *   cand   NULL: column c scores entry c (c < n_vis[q]).
 *          else [Q][ld_cand] int32 entry ids: column c scores entry
 *          cand[q][c] (c < n_vis[q]); entries must be in [0, cap).  Ids at
 *          columns n_vis[q] .. n_cols-1 may hold anything (e.g. -1 padding):
 *          they may be read but are never used.
 *   ld_cand  row stride of cand (ignored when cand is NULL)
 *   Q      queries
 *   n_cols (host) upper bound of n_vis[q], sets the launch size; < 2^29
 *   src    the cache
 *   scores [Q][ld] fp32; columns >= n_vis[q] are not written
 */
csa2_status csa2_index_score(const uint16_t* q_idx, const float* w, const int32_t* q_seq,
                             const int64_t* n_vis, const int32_t* cand, int64_t ld_cand, int Q,
                             int64_t n_cols, const csa2_cache* src, float* scores, int64_t ld,
                             void* stream);

/*
 * (2b) Lightning-indexer scores with an MXFP4 indexer query.
 *
 * Report section 2.4.4 (V4 already trains the indexer queries and keys for
 * the OCP MXFP4 format so that index scoring runs as an FP4 matrix multiply);
 * commentary section 5.  Same arguments, layouts, ownership and errors as
 * csa2_index_score; the only difference is that each query is first
 * quantised with the OCP MX rule the cache uses for the indexer K, per head
 * and 32-dim block:
 *   X = 2^(floor(log2 max|q_g|) - 2) as E8M0 (exponent clamped to
 *   [-127, 127]; an all-zero block gets 2^-127 and +0 codes),
 *   qhat[c] = X * E2M1(RNE, saturating at 6)(q[c] / X)
 * and the score is
 *   score(q, j) = sum_{h<32} w[q][h] * max(0, sum_{c<128} qhat[q][h][c] * khat_j[c])
 * accumulated in fp32 (the FP4 x FP4 products are exact).  The quantised
 * query is not written out.
 */
csa2_status csa2_index_score_fp4q(const uint16_t* q_idx, const float* w, const int32_t* q_seq,
                                  const int64_t* n_vis, const int32_t* cand, int64_t ld_cand,
                                  int Q, int64_t n_cols, const csa2_cache* src, float* scores,
                                  int64_t ld, void* stream);

/*
 * (3a) Per-query top-k: step a5 (and the selection half of a7).
 *
 * Selects, for each query, the min(k, n_valid[q]) columns with the largest
 * score, ties broken towards the lower column (report section 2.3 and Fig. 5:
 * top-512 per query; the tie rule is this library's reading).  Scores are
 * compared as fp32 values (+0 and -0 equal); NaN is not allowed.
 *
 *   scores   [Q][ld] fp32
 *   n_valid  [Q] int64    columns 0..n_valid[q]-1 are candidates
 *   col_ids  NULL: the id of column c is c.  Else [Q][ld] int32 entry ids,
 *            strictly ascending over each query's valid columns (the pool
 *            that csa2_block_pool writes has this form), so that the lower
 *            column is also the lower entry id.
 *   n_cols   (host) upper bound of n_valid[q], <= CSA2_MAX_COLS
 *   k        1 <= k <= CSA2_MAX_K
 *   out      [Q][k] int32 selected ids, ascending, padded with -1
 *   ws       workspace of csa2_workspace_bytes(CSA2_OP_TOPK, Q, n_cols, k) bytes
 */
csa2_status csa2_select_topk(const float* scores, int64_t ld, int Q, const int64_t* n_valid,
                             const int32_t* col_ids, int64_t n_cols, int k, int32_t* out,
                             void* ws, size_t ws_bytes, void* stream);

/*
 * (3a') Per-query top-k without a workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Same selection, arguments,
 * layouts and errors as csa2_select_topk; the maxima the selection keeps
 * between its kernels go to a static scratch array of
 * CSA2_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held until
 * the process ends.  Calls whose Q x n_cols needs more scratch than that
 * (csa2_workspace_bytes(CSA2_OP_TOPK, Q, n_cols, k) > the limit; e.g. up to
 * 4 x 2^20 or 32 x 2^19 columns fit) return CSA2_EUNSUPPORTED.  The call
 * allocates nothing.  Every call on one GPU shares that GPU's scratch:
 * calls that overlap on one GPU (on different streams, or from several
 * threads) race and must be ordered by the caller.
 */
#define CSA2_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
csa2_status csa2_select_topk_noalloc(const float* scores, int64_t ld, int Q,
                                     const int64_t* n_valid, const int32_t* col_ids,
                                     int64_t n_cols, int k, int32_t* out, void* stream);

/*
 * (3b) Hierarchical candidate pool: step a6.
 *
 * Report section 2.3.2 and Fig. 5: the first Full layer of the decoder gives
 * every block of positions the maximum index score among them, keeps the
 * blocks with the highest scores, and collects their positions into a pool
 * (2048 blocks x 8 positions = 16384 candidates) that later Reindex layers
 * search.  Here: aligned blocks [8b, 8b+8) of the first n_valid[q] columns,
 * a partial last block uses its valid columns; blocks ranked by (max desc,
 * block id asc); the first min(n_blocks, #blocks) are kept.
 *
 * The same section has that Full layer also produce the top-k of its own
 * attention from the full scan.  With k <= n_blocks that top-k lies inside
 * the pool (an entry outside it has n_blocks blocks ranked above its own
 * block, each holding an entry that beats or ties it with a lower id), so
 * the call can return it too, selected among the pool's positions, which
 * equals csa2_select_topk over all n_valid columns.
 *
 *   scores, ld, Q, n_valid, n_cols  as for csa2_select_topk (col_ids = identity)
 *   block     positions per block; must be 8
 *   n_blocks  1 <= n_blocks <= CSA2_MAX_K
 *   pool      [Q][n_blocks * block] int32 pooled positions, ascending, -1 padded
 *   pool_len  [Q] int64 number of valid pool entries
 *   k         0 (no top-k) or 1 <= k <= n_blocks
 *   topk      [Q][k] int32 top-k positions, ascending, -1 padded (NULL iff k == 0)
 *   ws        csa2_workspace_bytes(CSA2_OP_POOL, Q, n_cols, n_blocks) bytes
 */
csa2_status csa2_block_pool(const float* scores, int64_t ld, int Q, const int64_t* n_valid,
                            int64_t n_cols, int block, int n_blocks, int32_t* pool,
                            int64_t* pool_len, int k, int32_t* topk, void* ws, size_t ws_bytes,
                            void* stream);

/*
 * (4 + 5) Gather and sparse attention: steps a8 and a9.
 *
 * Report section 2.3: each query attends to its selected main-KV entries
 * together with the layer-local sliding-window KV; the 512-d latent is
 * shared by all 64 heads and used as both key and value (MLA style);
 * section 2.4.4: main KV dequantised from FP4 before attention, SWA KV FP8.
 * For query q and head h, over the rows
 *   main:  xhat_j for j = idx[q][i] (i < k, idx == -1 skipped),
 *          from sequence q_seq[q] of `src`
 *   SWA:   sigma_r * e_r for the swa_len[q] rows r = (swa_start[q] + i) mod T_swa,
 *          i = 0, 1, ..., of sequence q_seq[q] of the SWA arrays (the SWA
 *          arrays are a ring of T_swa slots, as csa2_decode_append keeps it)
 *   l = q[q][h] . row,  p = softmax(l),  out[q][h] = sum p * row,
 *   lse[q][h] = log sum exp(l).
 * q is used as given (the 1/sqrt(512) softmax scale is folded in by the
 * caller).  Logits accumulate in fp32 from exact bf16 operands; the
 * probability-weighted sum uses fp16 probabilities and fp16 values
 * (exact for FP4 main KV) with fp32 accumulation.
 *
 *   q          [Q][64][512] bf16
 *   q_seq      [Q] int32
 *   Q          queries
 *   src        the cache
 *   idx        [Q][k] int32 selected entries (-1 = none); 0 <= k <= CSA2_MAX_K
 *   swa_codes  [B][T_swa][512] u8 E4M3FN; may be NULL iff every swa_len is 0
 *   swa_scale  [B][T_swa] fp32
 *   T_swa      SWA rows per sequence
 *   swa_start  [Q] int64, swa_len [Q] int32 (0 <= swa_len <= CSA2_MAX_SWA);
 *              a window longer than T_swa is cut to T_swa rows, and a
 *              swa_start outside [0, T_swa) gives no SWA rows
 *   out        [Q][64][512] fp32
 *   lse        [Q][64] fp32, or NULL.  A query with no rows gets out = 0,
 *              lse = -inf.
 *   ws         csa2_workspace_bytes(CSA2_OP_ATTEND, Q, 0, k) bytes (partial
 *              states of the row splits).  With a smaller or NULL workspace the
 *              call uses fewer splits (at worst one workgroup per query and
 *              head group), with the same result.  Calls that share one
 *              workspace must not overlap.
 */
csa2_status csa2_sparse_attend(const uint16_t* q, const int32_t* q_seq, int Q, const csa2_cache* src,
                               const int32_t* idx, int k, const uint8_t* swa_codes,
                               const float* swa_scale, int64_t T_swa, const int64_t* swa_start,
                               const int32_t* swa_len, float* out, float* lse, void* ws,
                               size_t ws_bytes, void* stream);

/*
 * (3 + 4 + 5) Selection fused with the gather and the attention, for decode
 * batches: csa2_select_topk (n_blocks == 0) or csa2_block_pool with its
 * top-k (n_blocks > 0) followed by csa2_sparse_attend over the selected
 * entries, in one call whose kernels keep the selected ids on chip.  The
 * report (section 3.2) fuses each layer's steps into few kernels; here
 * every attention workgroup of a query repeats the query's (deterministic)
 * selection instead of reading the ids back from memory.
 *
 * Outputs are those of the separate calls on the same inputs: idx (and
 * pool, pool_len) exactly as csa2_select_topk / csa2_block_pool write them,
 * out and lse the attention csa2_sparse_attend computes over idx (its rows
 * may be split over workgroups differently, so the fp32 rounding of the
 * merge can differ).
 *
 *   scores, ld, Q, n_valid, n_cols   as for csa2_select_topk; Q < 256
 *   col_ids    as for csa2_select_topk; must be NULL when n_blocks > 0
 *   k          1 <= k <= CSA2_MAX_K (and k <= n_blocks when n_blocks > 0)
 *   idx        [Q][k] int32 selected entry ids, ascending, -1 padded
 *   n_blocks   0 (plain top-k) or the pool's block count (blocks of 8)
 *   pool, pool_len  as for csa2_block_pool (NULL when n_blocks == 0)
 *   q, q_seq, src, swa_codes, swa_scale, T_swa, swa_start, swa_len, out,
 *   lse        as for csa2_sparse_attend (the attended rows are idx)
 *   ws         256-byte aligned, csa2_workspace_bytes(CSA2_OP_SELECT_ATTEND or
 *              CSA2_OP_POOL_ATTEND, Q, n_cols, k) bytes (maxima levels and
 *              the attention's partial states); calls sharing a workspace
 *              must not overlap
 */
csa2_status csa2_select_attend(const float* scores, int64_t ld, int Q, const int64_t* n_valid,
                               const int32_t* col_ids, int64_t n_cols, int k, int32_t* idx,
                               int n_blocks, int32_t* pool, int64_t* pool_len, const uint16_t* q,
                               const int32_t* q_seq, const csa2_cache* src,
                               const uint8_t* swa_codes, const float* swa_scale, int64_t T_swa,
                               const int64_t* swa_start, const int32_t* swa_len, float* out,
                               float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * (4b) Full scan that also lays down the selection's block maxima, and the
 * fused selection + attention that starts from them.
 *
 * The report runs each layer as a few fused kernels (section 3.2); here the
 * first pass of the top-k / block-pool selection (the maximum score of
 * every 8 and every 64 consecutive columns, the lowest levels of its 8-way
 * maxima pyramid) moves into the scan's epilogue, so the selection that
 * follows does not read the scores once more before it starts.
 *
 * csa2_index_score_levels = csa2_index_score (or _fp4q with fp4q != 0) with
 * cand = NULL, plus the maxima levels of those scores written into ws, laid
 * out for a selection of mode n_blocks > 0 (block pool) or n_blocks == 0
 * (top-k) over Q x n_cols (levels the scan epilogue cannot produce are
 * computed by a maxima pass after the scan; the contents are the same).
 *   n_cols   <= CSA2_MAX_COLS (and as for csa2_index_score)
 *   n_blocks 0 or the block count of the csa2_select_attend_levels call that
 *            follows (only its sign matters here)
 *   ws       256-byte aligned, at least csa2_workspace_bytes(CSA2_OP_TOPK or
 *            CSA2_OP_POOL, Q, n_cols, 1) bytes: normally the workspace of the
 *            csa2_select_attend_levels call that follows, whose first part
 *            holds the levels
 *
 * csa2_select_attend_levels = csa2_select_attend (same arguments, outputs,
 * workspace and errors) without its own maxima pass: ws must hold the
 * levels a csa2_index_score_levels call wrote for these scores with
 * n_vis == n_valid, the same Q, n_cols and the same sign of n_blocks, and
 * col_ids must be NULL.  Levels from other scores give a wrong (though
 * in-bounds) selection.
 *
 * csa2_select_topk_levels = csa2_select_topk (same arguments, outputs,
 * workspace and errors) likewise without its maxima pass, after a
 * csa2_index_score_levels call with n_blocks == 0 into the same ws (its
 * csa2_workspace_bytes(CSA2_OP_TOPK, Q, n_cols, k) bytes); col_ids NULL.
 */
csa2_status csa2_index_score_levels(const uint16_t* q_idx, const float* w, const int32_t* q_seq,
                                    const int64_t* n_vis, int Q, int64_t n_cols,
                                    const csa2_cache* src, float* scores, int64_t ld, int fp4q,
                                    int n_blocks, void* ws, size_t ws_bytes, void* stream);
csa2_status csa2_select_attend_levels(const float* scores, int64_t ld, int Q,
                                      const int64_t* n_valid, const int32_t* col_ids,
                                      int64_t n_cols, int k, int32_t* idx, int n_blocks,
                                      int32_t* pool, int64_t* pool_len, const uint16_t* q,
                                      const int32_t* q_seq, const csa2_cache* src,
                                      const uint8_t* swa_codes, const float* swa_scale,
                                      int64_t T_swa, const int64_t* swa_start,
                                      const int32_t* swa_len, float* out, float* lse, void* ws,
                                      size_t ws_bytes, void* stream);
csa2_status csa2_select_topk_levels(const float* scores, int64_t ld, int Q,
                                    const int64_t* n_valid, const int32_t* col_ids,
                                    int64_t n_cols, int k, int32_t* out, void* ws,
                                    size_t ws_bytes, void* stream);

/* Rotary position embedding of csa2_sparse_attend_rope (host struct). */
typedef struct {
  const int64_t* q_pos;   /* [Q] position of each query (device); may be NULL iff dims == 0 */
  int dims;               /* rotated channels: the last `dims` of the 512, even, 0..64      */
  float theta;            /* frequency base, finite and > 1 (e.g. 10000)                    */
} csa2_rope;

/*
 * (5b) Fused RoPE - attention - inverse RoPE - cast.
 *
 * The report (section 3.2) runs attention as one fused kernel with RoPE,
 * the attention, a second RoPE and the output cast (FlashMLA's); section
 * 2.4.4: the cache holds latents quantised after RoPE.  Same rows, masks,
 * workspace and errors as csa2_sparse_attend, with:
 *   - pair i of channels (512 - dims + 2i, 512 - dims + 2i + 1) of every
 *     head of q turned by the angle q_pos[q] * theta^(-2i/dims) before the
 *     products: (a, b) -> (a cos - b sin, a sin + b cos);
 *   - the same channels of each head's output turned back by the opposite
 *     angle after the softmax-weighted sum;
 *   - out written as bf16 (round to nearest even) of the fp32 result.
 * Angles are formed and reduced modulo 2 pi in fp64, then used in fp32;
 * the rotated query enters the fp16 products as two fp16 terms (high and
 * low) on its last 64 channels, so its logits keep fp32 accuracy.
 *
 *   rope   the rotation (host struct)
 *   out    [Q][64][512] bf16
 *   lse    [Q][64] fp32 or NULL (unchanged by the rotations)
 */
csa2_status csa2_sparse_attend_rope(const uint16_t* q, const int32_t* q_seq, int Q,
                                    const csa2_cache* src, const int32_t* idx, int k,
                                    const uint8_t* swa_codes, const float* swa_scale,
                                    int64_t T_swa, const int64_t* swa_start,
                                    const int32_t* swa_len, const csa2_rope* rope,
                                    uint16_t* out, float* lse, void* ws, size_t ws_bytes,
                                    void* stream);

/*
 * (6) Decode-time append of one token per sequence.
 *
 * The V4 KV layout ("DeepSeek-V4" page, Fig. 6) keeps per request a
 * fixed-size state block: the SWA entries of the most recent tokens and the
 * uncompressed tail of tokens not yet ready for compression; the classical
 * cache grows by one compressed entry per m tokens (report section 2.3:
 * non-overlapping m-to-1 compression).  For each sequence b, with
 * t = n_tok[b] before the call:
 *   - if (t + 1) % m == 0, the m - 1 tail tokens followed by the new token
 *     are compressed, quantised and projected exactly as csa2_compress_quant
 *     does for one entry, and written as entry (t + 1) / m - 1 of `cache`
 *     (not written if that entry is at or past cache->cap);
 *     otherwise the new token's h and z go to tail slot t % m;
 *   - the new token's SWA latent x = swa_new[b] is stored in ring slot t % W
 *     as sigma = max|x| / 448 (fp32) and codes E4M3FN(RNE, saturating)(x /
 *     sigma), both quotients rounded to fp32 (an all-zero row: sigma = 0,
 *     +0 codes) -- the FP8 SWA row format csa2_sparse_attend reads;
 *   - n_tok[b] = t + 1, and what the sequence's next query sees is written:
 *     n_vis[b] = (t + 1) / m entries, swa_len[b] = min(W, t + 1) SWA rows
 *     starting at ring slot swa_start[b] = (t + 1 - swa_len[b]) mod W.
 *
 *   h_new    [B][512] bf16 raw latent of the new token
 *   z_new    [B][512] bf16 its compression logits; may be NULL iff m == 1
 *   swa_new  [B][512] bf16 its SWA latent; may be NULL iff state->W == 0
 *   B        sequences, 1 <= B <= 65535
 *   w_ik     [128][512] bf16 indexer-K projection
 *   cache    the layer's cache
 *   state    the layer's state block
 *   n_vis, swa_start, swa_len   [B] int64 / int64 / int32 outputs, each may
 *            be NULL; with q_seq[q] = q they are csa2_index_score's n_vis
 *            and csa2_sparse_attend's swa_start / swa_len (T_swa = W)
 * Calls for one state must be ordered on one stream.
 */
csa2_status csa2_decode_append(const uint16_t* h_new, const uint16_t* z_new,
                               const uint16_t* swa_new, int B, const uint16_t* w_ik,
                               const csa2_cache* cache, const csa2_state* state, int64_t* n_vis,
                               int64_t* swa_start, int32_t* swa_len, void* stream);

/* Workspace bytes an operation needs (0 if it needs none).
 *   op      CSA2_OP_TOPK (n_cols, k), CSA2_OP_POOL (n_cols, k = n_blocks),
 *           CSA2_OP_ATTEND (k = entries per query), CSA2_OP_SELECT_ATTEND and
 *           CSA2_OP_POOL_ATTEND (n_cols, k = the top-k)
 */
size_t csa2_workspace_bytes(int op, int Q, int64_t n_cols, int k);

/*
 * Device self-test of the hardware conversion and matrix instructions the
 * kernels rely on (FP4 -> bf16/fp16 and fp32 -> FP4 scaled conversions,
 * FP8 decoding, MFMA operand layouts, wave scans), against plain
 * integer/bit code on the same device.  Writes
 * `n` int32 failure counters to `counts` (device); all zero means pass.
 * Returns the number of counters it writes when counts is NULL.
 */
int csa2_selftest(int32_t* counts, int n, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CSA2_H */
