/*
 * csa2.h -- C ABI of the CSA2 FP4 sparse-attention decode library (libcsa2.so).
 *
 * The library implements, for one MI355X (gfx950) GPU, the decode-time hot path
 * of CSA2 compressed sparse attention over an FP4 global KV cache as the
 * DeepSeek-V4.1-Flash write-ups describe it:
 *   - "DeepSeek AI Released DeepSeek-V4.1-Flash with 1M Context, FP4 KV Cache,
 *     and Cross-Layer Attention Reuse" (MarkTechPost retelling): paragraph 2
 *     (sliding-window attention in every layer, 128-token window), paragraph 3
 *     (Full / Reindex / Reuse layer roles, candidate pool of up to 16,384
 *     positions), paragraph 4 (main KV cache in E2M1 with one E4M3 scale per 16
 *     channels, NVFP4 without the global scale);
 *   - "DeepSeek-v4.1 Flash: Pushing the Limits of KV Cache Compression"
 *     (hackernews.kjhq.dev summary), key points: local sliding window plus
 *     global sparse retrieval plus cross-layer reuse of the main KV and Top-K
 *     indices; a shallow-layer candidate pool bounds the deeper layers' search.
 *
 * A decode layer is composed by the caller:
 *   Full     csa2_index_full -> csa2_topk [-> pool: csa2_topk over the pool]
 *            -> csa2_sparse_decode -> csa2_swa_merge
 *   Reindex  csa2_index_reindex(pool) -> csa2_topk(index_map = pool)
 *            -> csa2_sparse_decode -> csa2_swa_merge
 *   Reuse    csa2_sparse_decode with the previous layer's indices -> csa2_swa_merge
 *
 * Conventions shared by every call:
 *   - Every tensor argument is a DEVICE pointer allocated and owned by the
 *     caller.  The library never allocates, frees or retains caller memory.
 *     Calls that need scratch memory take a caller-provided `workspace` whose
 *     size comes from the matching *_workspace_size() query (the one
 *     allocation-free call near the end of this file uses a fixed static
 *     array of the library's instead).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on that stream and returns without synchronising.  The
 *     library launches no memset/memcpy nodes, so calls may be captured into a
 *     HIP graph.
 *   - Every call checks its arguments on the host first.  On an argument error
 *     it returns a non-zero status before launching anything and leaves the
 *     outputs untouched.  CSA2_ELAUNCH reports a failed launch; device faults
 *     surface at the caller's next synchronisation.
 *   - Debug validation: with the environment variable CSA2_DEBUG set to
 *     anything but "0" (read at every call), the index, selection and
 *     attention calls first check their device-side row_seq entries against
 *     [0, B) and, strictly, window bounds and attention indices (entries the
 *     kernels would otherwise skip: start < 0, len outside [0, 128],
 *     start + len > S, an index outside [-1, T)); they wait for the check and
 *     return CSA2_EINVAL on a bad entry without launching anything else.
 *     Such calls synchronise their stream (not for graph capture).  Page ids
 *     are not checked (the pool size is not an argument).
 *   - Indices are int32 (positions < 2^31); lse values are natural logarithms.
 *   - bf16 tensors are passed as uint16_t bit patterns, E4M3 as uint8_t.
 *   - Unless stated otherwise, every pointer must be 16-byte aligned and every
 *     row-major tensor is dense.
 *   - Formats: E2M1 = OCP FP4 (1 sign, 2 exponent bits, 1 mantissa bit;
 *     magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6); E4M3 = OCP FP8 E4M3FN (bias 7,
 *     max 448, 0x7F/0xFF NaN).
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t csa2_status;
enum {
  CSA2_OK = 0,
  CSA2_EINVAL = 1,     /* null pointer, non-positive size, bad value            */
  CSA2_ESHAPE = 2,     /* a dimension outside what the kernels support          */
  CSA2_EALIGN = 3,     /* a pointer or stride without the required alignment    */
  CSA2_EWORKSPACE = 4, /* workspace pointer NULL or smaller than required       */
  CSA2_ELAUNCH = 5,    /* hipGetLastError() reported a failure after a launch  */
  CSA2_ESCRATCH = 6    /* the shape needs more than the fixed scratch array     */
};

/* Version of this ABI (incremented on any incompatible change). */
int32_t csa2_abi_version(void);

/* Static, NUL-terminated description of a status code. */
const char* csa2_status_str(csa2_status status);

/* ---------------------------------------------------------------------------
 * FP4 pack: latent KV rows -> E2M1 codes + one E4M3 scale per 16 channels.
 * (MarkTechPost retelling, paragraph 4: NVFP4 layout without the global scale.)
 *
 * For each row and each block of 16 channels [16b, 16b+16):
 *   scale = E4M3 value nearest to amax/6 (amax = largest |x| in the block),
 *           ties to the even code, values above 448 saturate to 448;
 *   code  = E2M1 value nearest to x/scale, ties to the even code, clamped at
 *           +-6, sign bit copied from x; a zero scale gives magnitude 0.
 * Byte j of a packed row holds channel 2j in its low nibble, 2j+1 in its high
 * nibble.  Scale byte b of a row covers channels [16b, 16b+16).
 *
 *   x        bf16 [n_rows][C] with row stride x_row_stride elements
 *            (x_row_stride >= C, multiple of 8)
 *   codes    uint8 [n_rows][C/2], row stride codes_row_stride bytes
 *            (>= C/2, multiple of 16)
 *   scales   uint8 [n_rows][C/16], row stride scales_row_stride bytes
 *            (>= C/16, even)
 *   C        channels, a positive multiple of 32
 * The strided outputs let a decode step write its new rows straight into the
 * cache at position T-1 of every sequence (stride T * C/2 bytes).
 * Errors: EINVAL (null pointer, n_rows < 0, bad stride), ESHAPE (C), EALIGN.
 * n_rows == 0 is a no-op.
 * Non-finite input: a block holding a NaN gets the NaN scale 0x7F and
 * magnitude codes 0 (it unpacks to NaN); an infinity counts as a value above
 * 448 * 6 (scale 448, element code +-6).
 * ------------------------------------------------------------------------- */
csa2_status csa2_fp4_pack(const uint16_t* x, int64_t n_rows, int32_t C, int64_t x_row_stride,
                          uint8_t* codes, int64_t codes_row_stride,
                          uint8_t* scales, int64_t scales_row_stride, void* stream);

/* FP4 unpack: x[r][c] = E2M1(code) * E4M3(scale) as bf16 (always exact; a NaN
 * scale byte 0x7F / 0xFF gives NaN).
 *   codes uint8 [n_rows][C/2], scales uint8 [n_rows][C/16] (dense), x bf16
 *   [n_rows][C] (dense).  Same errors as csa2_fp4_pack. */
csa2_status csa2_fp4_unpack(const uint8_t* codes, const uint8_t* scales, int64_t n_rows, int32_t C,
                            uint16_t* x, void* stream);

/* ---------------------------------------------------------------------------
 * Full-mode indexer scores (MarkTechPost retelling, paragraph 3: a Full layer
 * builds fresh indices over the context).
 *
 *   scores[r][j] = sum_{d<64} q_idx[r][d] * k_idx[seq(r)][j][d]   (fp32)
 * for every position j <= row_limit[r]; later positions get -inf.
 *
 *   q_idx      E4M3 [R][64]
 *   k_idx      E4M3 [B][T][64], shared by all layers
 *   row_seq    int32 [R] sequence of each query row, or NULL for row r -> r
 *              (then R must equal B)
 *   row_limit  int64 [R] last visible position of each row (causal prefill),
 *              or NULL for all T positions
 *   scores     fp32 [R][T]
 * E4M3 products are exact; the matrix cores add them in two steps of 32
 * channels into an fp32 accumulator.  The score is the exact value rounded
 * once to fp32 for unit-normal inputs; over arbitrary finite E4M3 bytes the
 * error measured stays below 2^-21 * sum_d |q_d k_d|.  Every scoring call
 * (csa2_index_full, csa2_index_reindex, csa2_index_full_pool and the paged
 * forms) rounds identically, so their scores agree bit for bit.
 * Errors: EINVAL (null pointer, R/B/T <= 0, R != B without row_seq), ESHAPE
 * (T not a multiple of 4, T >= 2^31), EALIGN.
 * ------------------------------------------------------------------------- */
csa2_status csa2_index_full(const uint8_t* q_idx, const uint8_t* k_idx, int32_t R, int32_t B, int64_t T,
                            const int32_t* row_seq, const int64_t* row_limit, float* scores,
                            void* stream);

/* The same Full-mode scores through the FP8 matrix instruction
 * (v_mfma_f32_16x16x32_fp8_fp8): the E4M3 bytes go in unconverted, for callers
 * that accept approximate scores (MarkTechPost retelling, paragraph 3: a Full
 * layer scores the whole context; the indexer keys are E4M3).  Arguments,
 * layout and errors as csa2_index_full.  The instruction does not
 * form the exact sum of its 32 products: on unit-normal E4M3 data about half
 * the scores differ from the exactly rounded value, by up to about 2^-15 *
 * sum_d |q_d k_d|; over arbitrary finite E4M3 bytes nearly all do, by up to
 * about 2^-12 * sum_d |q_d k_d| (the stated bound is 2^-10 * sum_d |q_d k_d|).  The selections of this library
 * (csa2_index_full_pool, csa2_topk on csa2_index_full scores) take exact scores
 * and do not use it. */
csa2_status csa2_index_full_fp8(const uint8_t* q_idx, const uint8_t* k_idx, int32_t R, int32_t B, int64_t T,
                                const int32_t* row_seq, const int64_t* row_limit, float* scores, void* stream);

/* Reindex-mode scores (MarkTechPost retelling, paragraph 3: a Reindex layer
 * rescores the shared candidate set; HN summary key points: the deeper layers'
 * cost is bounded by the pool, not the context).
 *
 *   scores[r][p] = q_idx[r] . k_idx[seq(r)][pool[r][p]]  (same arithmetic as
 *   csa2_index_full), and -inf where pool[r][p] < 0 or >= T.
 *   pool int32 [R][P]; scores fp32 [R][P].  P must be a multiple of 4.
 * Errors as csa2_index_full. */
csa2_status csa2_index_reindex(const uint8_t* q_idx, const uint8_t* k_idx, int32_t R, int32_t B, int64_t T,
                               const int32_t* row_seq, const int32_t* pool, int32_t P, float* scores,
                               void* stream);

/* ---------------------------------------------------------------------------
 * Top-K selection (HN summary key points: layers share the same Top-K indices;
 * MarkTechPost paragraph 3: the Full layer's candidate pool of up to 16,384).
 *
 * For each row r: the k_eff = min(k, visible) slots with the largest scores,
 * equal scores going to the lower slot, listed in ascending slot order and
 * padded with -1 up to k.  A slot is visible when its score is not -inf/NaN
 * and (with index_map) its index_map entry is >= 0.
 *
 *   scores     fp32 [R][N], row stride row_stride elements (>= N, multiple of 4)
 *   index_map  int32 [R][N] or NULL; with a map the outputs are index_map
 *              values (positions) instead of slots.  With an ascending map,
 *              "lower slot" is "lower position".
 *   idx_out    int32 [R][k]
 *   score_out  fp32 [R][k] or NULL: the selected scores, NaN in padded slots
 *   workspace  >= csa2_topk_workspace_size(R, N, k) bytes, 256-byte aligned
 * Errors: EINVAL (null, R/N/k <= 0), ESHAPE (N % 4, N >= 2^31), EWORKSPACE.
 * ------------------------------------------------------------------------- */
size_t csa2_topk_workspace_size(int32_t R, int64_t N, int32_t k);
csa2_status csa2_topk(const float* scores, int32_t R, int64_t N, int64_t row_stride, int32_t k,
                      const int32_t* index_map, int32_t* idx_out, float* score_out,
                      void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Candidate pool and its Top-K in one selection (MarkTechPost retelling,
 * paragraph 3: a decoder Full layer fills a pool of up to 16,384 positions
 * for the Reindex layers and takes its own Top-K; the HN summary key points:
 * the deeper layers search only that pool).
 *
 * Equivalent to two csa2_topk calls on the same scores:
 *   pool_idx / pool_scores = csa2_topk(scores, k_pool, index_map, score_out)
 *   top_idx                = csa2_topk(scores, k_top,  index_map)
 * (the top k_top entries are the top k_top of the pool, since k_top <= k_pool),
 * but long rows are read and reduced to candidates only once.
 *
 *   pool_idx    int32 [R][k_pool];  pool_scores fp32 [R][k_pool] or NULL
 *   top_idx     int32 [R][k_top]
 *   workspace   >= csa2_topk_pool_workspace_size(R, N, k_pool) bytes
 * Other arguments and the selection rule as for csa2_topk.
 * Errors: as csa2_topk, and EINVAL when k_top > k_pool.
 * ------------------------------------------------------------------------- */
size_t csa2_topk_pool_workspace_size(int32_t R, int64_t N, int32_t k_pool);
csa2_status csa2_topk_pool(const float* scores, int32_t R, int64_t N, int64_t row_stride, int32_t k_pool,
                           int32_t k_top, const int32_t* index_map, int32_t* pool_idx, float* pool_scores,
                           int32_t* top_idx, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Full-mode scoring and the candidate pool with its Top-K in one call
 * (MarkTechPost retelling, paragraph 3: a decoder Full layer scores the whole
 * context, fills the pool of up to 16,384 positions and takes its Top-K).
 *
 * Equivalent to csa2_index_full(q_idx, k_idx, R, B, T, row_seq, row_limit,
 * scores) followed by csa2_topk_pool(scores, R, T, T, k_pool, k_top, NULL,
 * pool_idx, pool_scores, top_idx): same scores, same selections.  Unless the
 * rows are short (T <= 32,768), the selection streams:
 * a strided sample of each row bounds its k_pool-th score from below, the
 * scoring pass keeps only the positions at or above that bound (in position
 * order, block by block) and the selection finishes on them; the result is
 * exact whatever the bound (too few candidates or massive ties take a slower
 * path inside the call).  With row_seq given and R >= 32 (chunked prefill),
 * runs of rows of one sequence share each key tile in the scoring pass.
 *
 *   scores     fp32 [R][T], written (masked positions -inf), or NULL: no
 *              scores are written (the selection does not need them)
 *   workspace  >= csa2_index_full_pool_workspace_size(R, T, k_pool) bytes
 *              (when the selection streams: about T * 8 bytes of candidate
 *              blocks per row for one batch of rows; the call runs as many row
 *              batches as needed, in order, on the stream.  The size query
 *              asks for batches that keep the workspace below 1 GB for any R;
 *              a larger workspace, e.g. from
 *              csa2_index_full_pool_batch_workspace_size(R, T, k_pool) for a
 *              single batch, runs fewer batches (each costs a few launches).
 *              For short rows: the Top-K workspace and room for the scores
 *              when the caller passes none)
 *   scan_start, scan_end  hipEvent_t handles or NULL: when given, recorded on
 *              the stream right before and right after the scoring kernel
 *              (to time it apart from the selection; with several row batches,
 *              before the first batch's scan and after the last one's)
 * Other arguments as for csa2_index_full and csa2_topk_pool.
 * Errors: as those two calls; ELAUNCH also when an event cannot be recorded.
 * ------------------------------------------------------------------------- */
size_t csa2_index_full_pool_workspace_size(int32_t R, int64_t T, int32_t k_pool);
/* Workspace bytes for streaming batches of rows_per_batch rows of T positions
 * (for T <= 32,768 the call does not stream: as
 * csa2_index_full_pool_workspace_size(rows_per_batch, T, k_pool)). */
size_t csa2_index_full_pool_batch_workspace_size(int32_t rows_per_batch, int64_t T, int32_t k_pool);
/* 1 when csa2_index_full_pool at R rows of T positions selects during the
 * scoring pass (T > 32,768: with scores NULL no score array is written or
 * read), 0 when it scores first and then selects; 0 for non-positive sizes.
 * A host-side query, no GPU work. */
int32_t csa2_index_full_pool_streams(int32_t R, int64_t T);
csa2_status csa2_index_full_pool(const uint8_t* q_idx, const uint8_t* k_idx, int32_t R, int32_t B, int64_t T,
                                 const int32_t* row_seq, const int64_t* row_limit, float* scores,
                                 int32_t k_pool, int32_t k_top, int32_t* pool_idx, float* pool_scores,
                                 int32_t* top_idx, void* workspace, size_t workspace_bytes, void* scan_start,
                                 void* scan_end, void* stream);

/* ---------------------------------------------------------------------------
 * Arithmetic of every attention call below: the matrix cores form q . x with
 * exact products (each 128-channel slice of each head's query is scaled by a
 * power of two into the f16 range, and its partial score takes the power back;
 * window rows, bf16 of any range,
 * use bf16 products), add them in fp32, and run the softmax in fp32; P enters
 * the value products as f16 for cache rows (2^-11 relative) and as a bf16 pair
 * (high part + remainder, about 2^-17) for window rows.  Every finite bf16
 * query and window value is supported; the scores softmax_scale * q . x must
 * stay finite in fp32 (|score| < 2e38).
 * ------------------------------------------------------------------------- */

/* ---------------------------------------------------------------------------
 * Sparse attention over the FP4 cache (HN summary key points: global sparse
 * retrieval over the shared main KV).
 *
 * For each row r and head h, over the valid entries j of idx[r] (0 <= j < T):
 *   xhat_j = dequantised FP4 row j of sequence seq(r) (512 channels)
 *   s_j    = softmax_scale * (q_lat[r][h] . xhat_j)
 *   o[r][h]   = sum_j exp(s_j) xhat_j / sum_j exp(s_j)
 *   lse[r][h] = log(sum_j exp(s_j))        (-inf and o = 0 with no valid j)
 * Every head uses the same latent row as key and value (absorbed multi-head
 * latent attention); queries come in absorbed form.
 *
 *   q_lat   bf16 [R][H][512]
 *   codes   uint8 [B][T][256], scales uint8 [B][T][32]   (csa2_fp4_pack layout)
 *   row_seq int32 [R] or NULL (row r -> sequence r, R == B)
 *   idx     int32 [R][K]; entries < 0 or >= T are skipped
 *   o       fp32 [R][H][512];  lse fp32 [R][H]
 *   H       16, 32, 48 or 64
 *   workspace >= csa2_sparse_decode_workspace_size(R, H, K) bytes
 * Errors: EINVAL, ESHAPE (H), EWORKSPACE, EALIGN.
 * ------------------------------------------------------------------------- */
size_t csa2_sparse_decode_workspace_size(int32_t R, int32_t H, int32_t K);
csa2_status csa2_sparse_decode(const uint16_t* q_lat, int32_t R, int32_t H,
                               const uint8_t* codes, const uint8_t* scales, int32_t B, int64_t T,
                               const int32_t* row_seq, const int32_t* idx, int32_t K,
                               float softmax_scale, float* o, float* lse,
                               void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Sliding-window attention and merge (MarkTechPost retelling, paragraph 2:
 * sliding-window attention runs in every layer over the last 128 tokens;
 * fanout.sh lesson, "What you will learn": the window state is layer-local).
 *
 * For each row r: attention (same formula as csa2_sparse_decode) over the
 * layer's own bf16 rows swa[seq(r)][swa_start[r] + i], i < swa_len[r]
 * (swa_len <= 128), then one softmax over the union with the sparse result:
 *   lse = log(exp(lse_sparse) + exp(lse_window))
 *   o   = exp(lse_sparse - lse) o_sparse + exp(lse_window - lse) o_window
 *
 *   swa        bf16 [B][S][512]
 *   swa_start  int32 [R], swa_len int32 [R]  (0 <= start, start + len <= S,
 *              0 <= len <= 128; checked on the device: out-of-range rows are
 *              skipped)
 *   o_sparse   fp32 [R][H][512] and lse_sparse fp32 [R][H]: the
 *              csa2_sparse_decode result, or both NULL for no sparse part
 *   o_out      fp32 [R][H][512] (may be the same buffer as o_sparse)
 *   lse_out    fp32 [R][H] or NULL (may be the same buffer as lse_sparse)
 *   workspace  >= csa2_swa_merge_workspace_size(R, H) bytes
 * Errors: EINVAL, ESHAPE (H, S), EWORKSPACE, EALIGN.
 * ------------------------------------------------------------------------- */
size_t csa2_swa_merge_workspace_size(int32_t R, int32_t H);
csa2_status csa2_swa_merge(const uint16_t* q_lat, int32_t R, int32_t H,
                           const uint16_t* swa, int32_t B, int32_t S, const int32_t* row_seq,
                           const int32_t* swa_start, const int32_t* swa_len, float softmax_scale,
                           const float* o_sparse, const float* lse_sparse,
                           float* o_out, float* lse_out,
                           void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Sparse attention and window merge in one call: the result equals
 * csa2_sparse_decode followed by csa2_swa_merge with that sparse result (one
 * softmax over the union of the selected cache rows and the window rows), but
 * the window rows are processed as more key tiles of the same launch and a
 * single combine step produces o and lse (two launches instead of four).
 *
 * Arguments as in csa2_sparse_decode and csa2_swa_merge; o fp32 [R][H][512],
 * lse fp32 [R][H].
 *   workspace >= csa2_sparse_swa_decode_workspace_size(R, H, K) bytes
 * Errors: EINVAL, ESHAPE (H), EWORKSPACE, EALIGN.
 * ------------------------------------------------------------------------- */
size_t csa2_sparse_swa_decode_workspace_size(int32_t R, int32_t H, int32_t K);
csa2_status csa2_sparse_swa_decode(const uint16_t* q_lat, int32_t R, int32_t H,
                                   const uint8_t* codes, const uint8_t* scales, int32_t B, int64_t T,
                                   const int32_t* row_seq, const int32_t* idx, int32_t K,
                                   const uint16_t* swa, int32_t S, const int32_t* swa_start,
                                   const int32_t* swa_len, float softmax_scale, float* o, float* lse,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Several layers' csa2_sparse_swa_decode in one launch (HN summary key points:
 * the CSA2 layers reuse one main KV and share Top-K indices across layers;
 * MarkTechPost retelling, paragraph 3: Reuse layers take the previous layer's
 * indices unchanged).  Layer l computes exactly what csa2_sparse_swa_decode
 * computes with its own queries, window and outputs and the index slice
 * idx[layer_idx[l]]; layers that share a slice gather the same cache rows.
 *
 *   L          1 .. 8 layers
 *   q_lat      bf16 [L][R][H][512]
 *   idx        int32 [n][R][K], n > max(layer_idx)
 *   layer_idx  int32 [L], HOST memory: the idx slice of each layer (>= 0)
 *   swa        bf16 [L][B][S][512];  swa_start, swa_len int32 [L][R]
 *   o          fp32 [L][R][H][512];  lse fp32 [L][R][H]
 *   workspace  >= csa2_sparse_swa_decode_layers_workspace_size(L, R, H, K) bytes
 * Other arguments as in csa2_sparse_swa_decode.
 * Errors: EINVAL (also a negative layer_idx entry), ESHAPE (H, L > 8),
 * EWORKSPACE, EALIGN.
 * ------------------------------------------------------------------------- */
size_t csa2_sparse_swa_decode_layers_workspace_size(int32_t L, int32_t R, int32_t H, int32_t K);
csa2_status csa2_sparse_swa_decode_layers(int32_t L, const uint16_t* q_lat, int32_t R, int32_t H,
                                          const uint8_t* codes, const uint8_t* scales, int32_t B, int64_t T,
                                          const int32_t* row_seq, const int32_t* idx, const int32_t* layer_idx,
                                          int32_t K, const uint16_t* swa, int32_t S, const int32_t* swa_start,
                                          const int32_t* swa_len, float softmax_scale, float* o, float* lse,
                                          void* workspace, size_t workspace_bytes, void* stream);


/* ===========================================================================
 * Paged global KV (the Hugging Face paper page's abstract: the global KV cache
 * is kept whole in HBM for serving; mixed serving batches hold sequences of
 * different lengths).  The layout is this library's: every per-position
 * tensor of the cache (the index keys, the FP4 codes and scales) lives in a
 * page pool of n_pages pages of `page` positions, and sequence b's logical
 * position p sits in physical row block_table[b][p / page] * page + p % page
 * of each pool.
 *
 *   block_table  int32 [B][max_blocks] (device): the page of each logical
 *                block of each sequence; a negative entry leaves the block
 *                unmapped (its positions count as invisible)
 *   page         positions per page, a positive multiple of 128 (every
 *                32-position scoring tile lies in one page)
 *   T            the logical capacity, T <= max_blocks * page; a sequence's
 *                own length goes in row_limit / swa_len as in the dense calls
 * The paged calls compute exactly what their dense counterparts compute on
 * the logical sequences.  Extra errors: EINVAL (null table, max_blocks <= 0,
 * page <= 0), ESHAPE (page not a multiple of 128, T > max_blocks * page).
 * ------------------------------------------------------------------------- */

/* csa2_fp4_pack with scattered output rows: input row i goes to row
 * out_rows[i] of codes / scales (a negative entry skips the row), e.g. each
 * sequence's new token into its page slot.  out_rows int64 [n_rows] (device,
 * 8-byte aligned).  Other arguments and errors as csa2_fp4_pack. */
csa2_status csa2_fp4_pack_rows(const uint16_t* x, int64_t n_rows, int32_t C, int64_t x_row_stride,
                               const int64_t* out_rows, uint8_t* codes, int64_t codes_row_stride,
                               uint8_t* scales, int64_t scales_row_stride, void* stream);

/* csa2_index_full over paged keys: k_pages uint8 [n_pages * page][64]. */
csa2_status csa2_index_full_paged(const uint8_t* q_idx, const uint8_t* k_pages, int32_t R, int32_t B, int64_t T,
                                  const int32_t* row_seq, const int64_t* row_limit, const int32_t* block_table,
                                  int64_t max_blocks, int32_t page, float* scores, void* stream);

/* csa2_index_reindex over paged keys (pool entries are logical positions). */
csa2_status csa2_index_reindex_paged(const uint8_t* q_idx, const uint8_t* k_pages, int32_t R, int32_t B,
                                     int64_t T, const int32_t* row_seq, const int32_t* block_table,
                                     int64_t max_blocks, int32_t page, const int32_t* pool, int32_t P,
                                     float* scores, void* stream);

/* csa2_index_full_pool over paged keys (scores may be NULL as there; outputs
 * are logical positions).  Workspace as for the dense call. */
size_t csa2_index_full_pool_paged_workspace_size(int32_t R, int64_t T, int32_t k_pool);
csa2_status csa2_index_full_pool_paged(const uint8_t* q_idx, const uint8_t* k_pages, int32_t R, int32_t B,
                                       int64_t T, const int32_t* row_seq, const int64_t* row_limit,
                                       const int32_t* block_table, int64_t max_blocks, int32_t page,
                                       float* scores, int32_t k_pool, int32_t k_top, int32_t* pool_idx,
                                       float* pool_scores, int32_t* top_idx, void* workspace,
                                       size_t workspace_bytes, void* stream);

/* csa2_sparse_swa_decode_layers over paged FP4 rows: code_pages uint8
 * [n_pages * page][256], scale_pages uint8 [n_pages * page][32]; idx holds
 * logical positions.  Workspace: csa2_sparse_swa_decode_layers_workspace_size. */
csa2_status csa2_sparse_swa_decode_layers_paged(int32_t L, const uint16_t* q_lat, int32_t R, int32_t H,
                                                const uint8_t* code_pages, const uint8_t* scale_pages, int32_t B,
                                                int64_t T, const int32_t* row_seq, const int32_t* block_table,
                                                int64_t max_blocks, int32_t page, const int32_t* idx,
                                                const int32_t* layer_idx, int32_t K, const uint16_t* swa, int32_t S,
                                                const int32_t* swa_start, const int32_t* swa_len,
                                                float softmax_scale, float* o, float* lse, void* workspace,
                                                size_t workspace_bytes, void* stream);
/* -------------------------------------------------------------------------
 * Decode-time append (the step before the path: each new token enters the
 * global FP4 cache, its indexer key enters the key cache, and every layer's
 * sliding window gains its row -- the KV-cache paragraph of the MarkTechPost
 * retelling and the HN summary's key points).  One call per decode step:
 *
 *   new_latent  bf16 [B][512]: the token's latent row, packed as csa2_fp4_pack
 *               into row cache_rows[b] of codes ([.][256]) and scales ([.][32])
 *   cache_rows  int64 [B] (device): the cache row of sequence b's new position
 *               (dense [B][T] caches: b T + t_b; a page pool: its page slot);
 *               a negative entry skips the sequence's cache and key writes
 *   new_keys    E4M3 [B][64] or NULL: copied to row cache_rows[b] of k_idx
 *   new_window  bf16 [L][B][512] or NULL: layer l's window row of the token
 *   swa         bf16 [L][B][S][512], S >= 256: each layer's window kept as a
 *               mirrored ring of 2 x 128 rows: position t is written to rows
 *               t mod 128 and t mod 128 + 128, so the last min(128, t + 1)
 *               positions are rows [start, start + len) with
 *               start = (t + 1) mod 128 once t >= 127 (0 before) and
 *               len = min(128, t + 1), the contiguous window every attention
 *               call of this library reads
 *   tok_pos     int64 [B] (device): t, the new token's position in its sequence
 *               (negative: leave that sequence's window alone)
 *   swa_start, swa_len  int32 [L][B] (device), written with those bounds
 * Errors: EINVAL (B or L < 0, null pointer a given input needs, new_window
 * with L = 0), ESHAPE (S < 256), EALIGN (16-byte rows; 8-byte int64 arrays).
 * ------------------------------------------------------------------------- */
csa2_status csa2_decode_append(int32_t B, int32_t L, const uint16_t* new_latent, const int64_t* cache_rows,
                               uint8_t* codes, uint8_t* scales, const uint8_t* new_keys, uint8_t* k_idx,
                               const uint16_t* new_window, uint16_t* swa, int32_t S, const int64_t* tok_pos,
                               int32_t* swa_start, int32_t* swa_len, void* stream);

/* -------------------------------------------------------------------------
 * Query absorption and output unabsorption (helpers around the attention
 * calls, which take absorbed queries and return latent outputs).  Every head
 * attends over the one 512-channel latent row per position (HN summary key
 * points: the layers share one main KV; MarkTechPost retelling, paragraph 3);
 * head h's key of a latent row x is W_UK[h] x and its value W_UV[h] x, with
 * 128-d head queries and outputs, so the attention of q over keys W_UK x
 * equals the attention of q_lat = W_UK[h]^T q over the latent rows, and the
 * head output is W_UV[h] applied to the latent output.
 *
 *   csa2_absorb_q:   q_lat[r][h][c] = sum_d q[r][h][d] * w_uk[h][d][c]
 *     q      bf16 [R][H][D], D = 128
 *     w_uk   bf16 [H][D][512]
 *     q_lat  bf16 [R][H][512]: the fp32 sum of the exact bf16 products,
 *            rounded once to bf16 (nearest, ties to even)
 *   csa2_unabsorb_o: out[r][h][d] = sum_c w_uv[h][d][c] * o_lat[r][h][c]
 *     o_lat  fp32 [R][H][512] (the attention calls' o)
 *     w_uv   bf16 [H][D][512], D = 128
 *     out    fp32 [R][H][D]: o_lat enters as two bf16 parts (nearest bf16 and
 *            the nearest bf16 of the remainder, about 16 significant bits),
 *            products exact, fp32 accumulation
 * All tensors dense.  R == 0 is a no-op.
 * Errors: EINVAL (R < 0, H <= 0, null pointer), ESHAPE (D != 128,
 * H > 65535, R > 4,194,240), EALIGN (16-byte pointers).
 * ------------------------------------------------------------------------- */
csa2_status csa2_absorb_q(const uint16_t* q, int32_t R, int32_t H, int32_t D, const uint16_t* w_uk,
                          uint16_t* q_lat, void* stream);
csa2_status csa2_unabsorb_o(const float* o_lat, int32_t R, int32_t H, int32_t D, const uint16_t* w_uv,
                            float* out, void* stream);
/* -------------------------------------------------------------------------
 * Allocation-free multi-layer attention, for callers that cannot allocate
 * device memory or pass a workspace: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.
 *
 * csa2_sparse_swa_decode_layers_noalloc computes exactly what
 * csa2_sparse_swa_decode_layers computes (same arguments, same kernels), but
 * its chunk partials go to a scratch array of CSA2_NOALLOC_SCRATCH_BYTES
 * (64 MiB) that the library holds as a static device variable, one per GPU,
 * from the first call on that GPU until the process ends.  The call itself
 * allocates nothing.  The array holds the partials of every shape with
 * K <= 2048 on a 256-CU GPU; a shape whose partials need more returns
 * CSA2_ESCRATCH before launching; a shape that runs each (layer, row)
 * as one chunk needs none (csa2_sparse_swa_decode_layers_workspace_size tells
 * the size the partials would take).  Every call on one GPU shares that GPU's
 * array: calls that can overlap on one GPU (different streams, or threads
 * without ordering) race and give wrong results; calls ordered on one stream
 * are safe.  Nothing in the array needs to start cleared.  CSA2_ELAUNCH also
 * reports a failure to resolve the array's device address.
 * ------------------------------------------------------------------------- */
#define CSA2_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
csa2_status csa2_sparse_swa_decode_layers_noalloc(int32_t L, const uint16_t* q_lat, int32_t R, int32_t H,
                                                  const uint8_t* codes, const uint8_t* scales, int32_t B, int64_t T,
                                                  const int32_t* row_seq, const int32_t* idx,
                                                  const int32_t* layer_idx, int32_t K, const uint16_t* swa, int32_t S,
                                                  const int32_t* swa_start, const int32_t* swa_len,
                                                  float softmax_scale, float* o, float* lse, void* stream);
#ifdef __cplusplus
}
#endif
#endif /* CSA2_H */
