/*
 * csa2.h — C ABI of the CSA2 global-attention hot path for MI355X (gfx950).
 *
 * The calls follow the pages' statement of the problem:
 *   csa2_index_scores      Lightning-Indexer scores, dense or over a candidate pool
 *   csa2_block_candidates  block-max candidate pool (hierarchical sparse indexer)
 *   csa2_topk              token-level top-k selection
 *   csa2_topk_and_block_candidates  both selections of a Full layer at once
 *   csa2_sparse_attn       joint-softmax sparse MQA attention with a sink
 *   csa2_cache_write       a Full layer's main-KV entries and index keys
 * Sources are cited as page + section:
 *   [CSA2]   zdszero.github.io/csa2.html (CSA2 deep-dive)
 *   [3MODES] xhh.club, "DeepSeek-V4.1 model structure (2): CSA2's three modes"
 *   [REPORT] 10100.com, "DeepSeek-V4.1-Flash technical report reading"
 *   [DSA]    zdszero.github.io/dsa.html (DeepSeek Sparse Attention)
 *
 * Conventions for every call:
 *   - Every pointer argument is a DEVICE pointer owned by the caller, unless
 *     stated otherwise.  The library allocates no device memory, keeps no
 *     state between calls and never synchronises: work is enqueued on
 *     `stream` (a hipStream_t passed as void*; NULL = the null stream) and
 *     the call returns once it is enqueued.  Calls are thread-safe.
 *   - Return value: CSA2_OK (0) or a negative csa2_status.  Argument checks
 *     run on the host before anything is enqueued; a failed check enqueues
 *     nothing.  csa2_last_error() gives a message for the last failure on
 *     the calling thread.  No C++ exception crosses this interface.
 *   - Device-side contents (positions, indices, candidate ids) cannot be
 *     checked on the host.  Out-of-range contents are clamped or skipped as
 *     each call states; they never make a kernel read outside the buffers
 *     the caller described.
 *   - Integer positions are main-KV entry positions within a sequence
 *     (0-based).  A query at token position p with compression ratio m sees
 *     the entries [0, (p + 1) / m) of its sequence ([CSA2] "the pool does not
 *     reduce storage").
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
    CSA2_ERR_INVALID_ARG = -1,  /* null pointer, negative size, misaligned pointer or stride */
    CSA2_ERR_UNSUPPORTED = -2,  /* a size or dtype combination outside the compiled kernels */
    CSA2_ERR_WORKSPACE = -3,    /* workspace missing or smaller than the size query returns */
    CSA2_ERR_HIP = -4           /* the HIP runtime reported an error while enqueuing */
} csa2_status;

typedef enum {
    CSA2_F32 = 0,       /* IEEE binary32 */
    CSA2_BF16 = 1,      /* bfloat16 */
    CSA2_FP8_E4M3 = 2,  /* OCP FP8 E4M3FN codes, one byte per element, fp32 scales */
    CSA2_FP4_E2M1 = 3,  /* OCP FP4 E2M1 codes, two per byte (element 2i in the low
                           nibble of byte i), one fp32 scale per 32 elements */
    CSA2_FP4_E2M1_E4M3S16 = 4  /* E2M1 codes as above with one OCP E4M3 scale byte
                                  per 16 elements: the pages' FP4 cache format
                                  ([REPORT] section 6: E2M1 elements, an E4M3 scale
                                  per 16 channels, no second-level scale) */
} csa2_dtype;

/*
 * A [rows, dim] matrix, optionally quantized.  Row r's elements start at
 * (const char*)data + r * row_stride; for quantized dtypes its scales start
 * at scale + r * scale_stride (in floats) and element e of the row decodes
 * to code(e) * scale[e / group], with group = 128 for FP8 index rows and SWA
 * rows and group = 32 for FP4 main-KV rows.  For CSA2_FP4_E2M1_E4M3S16 the
 * scales are E4M3 bytes: `scale` points to bytes (cast to const float*),
 * scale_stride counts bytes and group = 16.  A record layout (codes followed
 * by scales in one row) is described by pointing `scale` into the first
 * record.  `scale` is NULL for F32 and BF16.
 * Alignment: data and row_stride multiples of 16 bytes; scale and
 * scale_stride multiples of 4 bytes (1 float, or 4 E4M3 bytes).
 */
typedef struct {
    const void* data;
    const float* scale;
    int64_t row_stride;     /* bytes */
    int64_t scale_stride;   /* floats */
    csa2_dtype dtype;
} csa2_rows;

/*
 * Paged caches ([DSA] top-k section: the KV cache is paged, so position p of
 * a sequence lives in slot table[p / 64] * 64 + p % 64 of a pool of 64-slot
 * pages, and the top-k hands the sparse kernel slots, not positions; [DSA]
 * implementation notes: a page of the index-key cache holds its 64 keys
 * (64 x 128 B) and then their 64 fp32 scales, 8448 B).
 */
typedef struct {
    const int32_t* table;   /* [B, table_stride] int32: the physical page of each
                               64-position page of each sequence; a negative entry,
                               or a page at or past table_stride, is missing */
    int64_t table_stride;   /* entries per sequence (>= 1) */
    int32_t n_pages;        /* csa2_index_scores: pages in the pool; entries at or
                               past it are missing (>= 1) */
    int64_t page_stride;    /* csa2_index_scores: bytes from one page to the next, in
                               k_idx's data and in its scales alike (the 8448-B page:
                               8448, with scale = data + 8192); 0 = flat rows, page P
                               holding rows 64P .. 64P + 63 of both arrays */
    const int32_t* q_seq;   /* csa2_topk: [Q] sequence of each score row */
} csa2_pages;

/*
 * csa2_index_scores — Lightning-Indexer scores
 *   I[t, s] = sum_h w[t, h] * ReLU(q[t, h] . k[s])
 * ([CSA2] "per-layer attention computation", item 4; [DSA] "Lightning
 * Indexer"), with 32 heads x 128 dims.  q and k are the dequantized rows; for
 * FP8 inputs the kernel multiplies codes exactly in fp32 and applies the
 * q scale to the gate and the k scale after the head sum ([DSA] "fp8 and
 * scale absorption"), which equals the dequantized formula because the
 * scales are positive.  No 1/sqrt(d) or 1/sqrt(H) factor is applied: fold any
 * such factor into w.
 *
 *   q_idx     rows = Q * H_I (row t*H_I + h is q[t, h]), dim d_I.
 *             FP8_E4M3 with one scale per row, or F32.
 *   w         [Q, H_I] contiguous gates, w_dtype BF16 or F32.
 *   k_idx     rows = all entries of all sequences, dim d_I.  With FP8 q_idx:
 *             FP8_E4M3 with one scale per row, or FP4_E2M1_E4M3S16 (the
 *             pages' FP4 index K: 64 code bytes per row, row_stride a
 *             multiple of 16, and 8 E4M3 scale bytes per row at
 *             scale + r * scale_stride bytes; those scales enter the dot
 *             products, and the dequantized keys are exact in f16).  With
 *             F32 q_idx: F32.
 *   seq_base  [B] int64: first k_idx row of each sequence.
 *   q_seq     [Q] int32: sequence of each query (0 <= q_seq < B).
 *   q_pos     [Q] int32: token position of each query (>= 0).
 *   ratio     compression ratio m (1 or 2).
 *   cand      NULL: dense mode.  Row t gets n_cols columns: column s < the
 *             visible count holds I[t, s]; the others hold -inf.
 *             Non-NULL: pool mode ([CSA2] "where attention is computed":
 *             the candidate indexer scores only the candidate blocks).
 *             [Q, n_cand_blocks] int32 block ids; column c*block_size + j of
 *             row t holds I[t, cand[t, c]*block_size + j], or -inf when
 *             cand[t, c] < 0 or that position is not visible.  n_cols must
 *             equal n_cand_blocks * block_size.
 *   scores    [Q, score_stride] fp32 output; score_stride >= n_cols,
 *             multiple of 4; 16-byte aligned.  May be NULL in dense mode
 *             when block_max is given: then only the block maxima are
 *             written (csa2_top_blocks_and_block_candidates and a pool-mode
 *             call over the best blocks give the top-k without the scores).
 *   block_max NULL, or (dense mode only) [Q, block_max_stride] fp32 output:
 *             entry b of row t is the largest score of columns
 *             [b*block_size, (b+1)*block_size) (-inf where none is visible),
 *             for b < ceil(n_cols / block_size) — the block maxima of the
 *             candidate pool ([CSA2] "blocks are not compression"), taken in
 *             the same pass so csa2_block_candidates need not re-read the
 *             scores.  Needs block_size <= 32 and block_max_stride >=
 *             ceil(n_cols / block_size).
 *   pages     NULL, or a paged index-key cache (csa2_pages): position p of
 *             sequence q_seq[t] is read from slot (table[p / 64], p % 64) of
 *             k_idx, at page * page_stride + (p % 64) * row_stride (scales
 *             alike); seq_base is not used (may be NULL); a position whose
 *             page is missing scores -inf.
 *   Supported: H_I = 32, d_I = 128 (FP8); H_I <= 64, d_I = 128 (F32);
 *   block_size in {1, 2, 4, 8, 16, 32, 64}.
 */
int csa2_index_scores(const csa2_rows* q_idx, const void* w, csa2_dtype w_dtype,
                      const csa2_rows* k_idx, const int64_t* seq_base,
                      const int32_t* q_seq, const int32_t* q_pos, int32_t ratio,
                      const int32_t* cand, int32_t n_cand_blocks, int32_t block_size,
                      float* scores, int64_t score_stride, int32_t n_cols,
                      float* block_max, int64_t block_max_stride,
                      int32_t Q, int32_t H_I, int32_t d_I, const csa2_pages* pages,
                      void* stream);

/*
 * csa2_block_candidates — the candidate pool of the hierarchical sparse
 * indexer ([CSA2] "hierarchical sparse indexer", "which positions are in the
 * pool"; [REPORT] section 5).  For row t with n = min(visible, n_cols)
 * columns: blocks of block_size positions are scored by their largest score
 * (a partial last block uses its visible members), the block holding the
 * latest visible position (n - 1) / block_size is always kept (it is ranked
 * first), and the remaining places go to the best blocks, ties to the lower
 * block id; blocks whose maximum is -inf are never chosen.
 *   scores    dense scores as written by csa2_index_scores ([Q, score_stride],
 *             16-byte aligned, score_stride a multiple of 4); may be NULL
 *             when block_max is given.
 *   block_max NULL, or the block maxima csa2_index_scores wrote
 *             ([Q, block_max_stride]); when given, only they are read.
 *   cand      [Q, n_blocks] int32 output: chosen block ids ascending, then -1.
 *   workspace device memory of at least
 *             csa2_block_candidates_workspace_size(Q, n_cols, block_size, n_blocks) bytes
 *             (may be NULL when that size is 0).
 *   Supported: n_blocks <= 4096, block_size in {1, 2, 4, 8, 16, 32, 64}.
 */
int csa2_block_candidates(const float* scores, int64_t score_stride, int32_t n_cols,
                          const float* block_max, int64_t block_max_stride,
                          const int32_t* q_pos, int32_t ratio, int32_t block_size,
                          int32_t n_blocks, int32_t* cand, void* workspace,
                          size_t workspace_bytes, int32_t Q, void* stream);

size_t csa2_block_candidates_workspace_size(int32_t Q, int32_t n_cols, int32_t block_size,
                                            int32_t n_blocks);

/*
 * csa2_topk — token-level top-k ([CSA2] "per-layer attention computation",
 * item 4; [DSA] "Top-k: tokens, not blocks").  Chooses the k largest finite
 * scores of each row, ties to the lower position; -inf is never chosen, so a
 * row with fewer than k finite scores yields all of them ([DSA] "design").
 *   Dense mode (cand == NULL): row t has min(n_cols, visible) columns when
 *             q_pos is given, n_cols when q_pos is NULL; column s is position s.
 *   Pool mode (cand != NULL): rows are compact pool scores as written by
 *             csa2_index_scores in pool mode; column c*block_size + j is
 *             position cand[t, c]*block_size + j; columns with cand < 0 are
 *             never chosen; n_cols must equal n_cand_blocks * block_size.
 *             Ties go to the lower position, i.e. the lower column when cand
 *             is ascending, as csa2_block_candidates writes it.
 *   scores    [Q, score_stride] fp32, 16-byte aligned, score_stride a
 *             multiple of 4 (as csa2_index_scores writes them).
 *   idx       [Q, k] int32 output: chosen positions ascending, then -1.
 *   workspace at least csa2_topk_workspace_size(Q, n_cols, k) bytes.
 *   pages     NULL, or a page table (csa2_pages: table, table_stride, q_seq):
 *             each chosen position p of row t is written as the slot
 *             table[q_seq[t]][p / 64] * 64 + p % 64, in the same order, and
 *             as -1 when its page is missing — the translation the sparse
 *             kernel's slot mode (csa2_attn_io.idx_slots) reads.
 *   Supported: 1 <= k <= 2048.
 */
int csa2_topk(const float* scores, int64_t score_stride, int32_t n_cols,
              const int32_t* q_pos, int32_t ratio, const int32_t* cand,
              int32_t n_cand_blocks, int32_t block_size, int32_t k, int32_t* idx,
              void* workspace, size_t workspace_bytes, int32_t Q, const csa2_pages* pages,
              void* stream);

size_t csa2_topk_workspace_size(int32_t Q, int32_t n_cols, int32_t k);

/*
 * csa2_topk_from_block_max — the dense top-k of csa2_topk (the same indices,
 * bit for bit) computed through the block maxima of the same scores
 * ([CSA2] "hierarchical sparse indexer": the maximum of every 8 consecutive
 * scores is taken in the scoring pass; here it narrows the top-k): the k best
 * blocks under (maximum desc, block asc), then the k best of those blocks'
 * k * block_size scores.  Exact: every score above the k-th best lies in one
 * of at most k - 1 blocks whose maximum exceeds it, and a tied score the
 * lower-position rule takes lies in a block of maximum >= it that the same
 * rule on blocks keeps.
 *   scores     [Q, score_stride] dense rows as in csa2_topk (q_pos required).
 *   block_max  [Q, block_max_stride]: entry b = max of the visible scores
 *              [b block_size, (b + 1) block_size) (-inf if none), as
 *              csa2_index_scores writes them; block_max_stride >=
 *              ceil(n_cols / block_size).
 *   block_size a power of two <= 32.
 *   workspace  at least csa2_topk_from_block_max_workspace_size(Q, n_cols,
 *              k, block_size) bytes, 16-byte aligned.
 *   pages      NULL, or a page table for the output as in csa2_topk.
 *   With k * block_size above 32,768 the rows are selected by the plain
 *   dense top-k (same result, its own workspace size, which the size query
 *   returns).
 *   Errors: as csa2_topk; CSA2_ERR_INVALID_ARG for a missing or misaligned
 *   block_max.
 */
int csa2_topk_from_block_max(const float* scores, int64_t score_stride, int32_t n_cols,
                             const float* block_max, int64_t block_max_stride, const int32_t* q_pos,
                             int32_t ratio, int32_t block_size, int32_t k, int32_t* idx,
                             void* workspace, size_t workspace_bytes, int32_t Q,
                             const csa2_pages* pages, void* stream);

size_t csa2_topk_from_block_max_workspace_size(int32_t Q, int32_t n_cols, int32_t k,
                                                int32_t block_size);

/*
 * csa2_topk_and_block_candidates — a Full layer's own top-k and the block
 * candidate pool it hands to the Reindex layers that follow, from the one set
 * of dense scores ([CSA2] "hierarchical sparse indexer", recall step: the
 * first Full layer picks its own top-k and the candidate blocks from one
 * scoring of every visible position).  The result equals
 *   csa2_topk(scores, score_stride, n_cols, q_pos, ratio, NULL, 0, 1, k, idx, ...)
 *   csa2_block_candidates(scores, score_stride, n_cols, block_max,
 *                         block_max_stride, q_pos, ratio, block_size, n_blocks, cand, ...)
 * bit for bit; the two selections run in shared launches, so neither waits
 * for the other to drain the chip.  Arguments mean what they mean in those
 * two calls; scores is required (the top-k reads it) and q_pos is required.
 *   workspace at least csa2_topk_and_block_candidates_workspace_size(Q,
 *             n_cols, k, block_size, n_blocks) bytes, 16-byte aligned.
 *   pages     NULL, or a page table for the top-k output as in csa2_topk
 *             (the candidate blocks stay block ids: pool scoring reads them
 *             through the same table).
 *   Supported: within both calls' limits (1 <= k <= 2048, n_blocks <= 4096,
 *             block_size a power of two <= 64, ratio 1 or 2).
 */
int csa2_topk_and_block_candidates(const float* scores, int64_t score_stride, int32_t n_cols,
                                   const float* block_max, int64_t block_max_stride,
                                   const int32_t* q_pos, int32_t ratio, int32_t k, int32_t* idx,
                                   int32_t block_size, int32_t n_blocks, int32_t* cand,
                                   void* workspace, size_t workspace_bytes, int32_t Q,
                                   const csa2_pages* pages, void* stream);

size_t csa2_topk_and_block_candidates_workspace_size(int32_t Q, int32_t n_cols, int32_t k,
                                                     int32_t block_size, int32_t n_blocks);

/*
 * csa2_top_blocks_and_block_candidates — a Full layer's two rankings of its
 * block maxima, without its scores ([CSA2] "hierarchical sparse indexer";
 * [DSA] "Top-k: tokens, not blocks"), in shared launches:
 *   top_blocks[t]  the k_blocks best blocks of row t by maximum (ties to the
 *                  lower block; no block forced), ascending, -1 padded:
 *                  csa2_block_candidates' selection without its forced
 *                  latest block;
 *   cand[t]        csa2_block_candidates(NULL, 0, n_cols, block_max, ...)
 *                  bit for bit (the latest visible block forced).
 * Every entry of row t among its k best under (score descending, position
 * ascending) lies in one of its k best blocks (a block holding a kept entry
 * has a maximum at least that entry's, and every block ranked above it is
 * kept).  So with k_blocks = k, scoring only those blocks (csa2_index_scores
 * in pool mode with cand = top_blocks) and taking the top-k of that pool
 * (csa2_topk with cand = top_blocks) gives the dense top-k exactly, as long
 * as the pool scores equal the dense ones (the same arithmetic per key,
 * which the quantized scorer has).
 *   block_max [Q, block_max_stride] from csa2_index_scores (scores may then
 *             be NULL); block_max_stride >= ceil(n_cols / block_size).
 *   top_blocks [Q, k_blocks] int32 output; cand [Q, n_blocks] int32 output.
 *   workspace at least csa2_top_blocks_and_block_candidates_workspace_size(
 *             Q, n_cols, block_size, k_blocks, n_blocks) bytes, 16-byte
 *             aligned.
 *   Supported: 1 <= k_blocks, n_blocks <= 4096; block_size a power of two
 *   <= 64; ratio 1 or 2.
 *   Errors: as csa2_block_candidates for either ranking.
 */
int csa2_top_blocks_and_block_candidates(const float* block_max, int64_t block_max_stride, int32_t n_cols,
                                         const int32_t* q_pos, int32_t ratio, int32_t block_size,
                                         int32_t k_blocks, int32_t* top_blocks, int32_t n_blocks,
                                         int32_t* cand, void* workspace, size_t workspace_bytes, int32_t Q,
                                         void* stream);

size_t csa2_top_blocks_and_block_candidates_workspace_size(int32_t Q, int32_t n_cols, int32_t block_size,
                                                           int32_t k_blocks, int32_t n_blocks);

/*
 * csa2_topk_and_block_candidates_noalloc — csa2_topk_and_block_candidates
 * without a workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  The selection lists live in a static device buffer of
 * csa2_noalloc_scratch_bytes() bytes (16 MiB) that the library holds on every
 * device it runs on until the process ends.  Arguments, outputs and limits
 * are those of csa2_topk_and_block_candidates, and so is the result, bit for
 * bit.  The call allocates nothing; its first call on a device looks the
 * buffer's address up (no allocation) and keeps it.
 *   Errors: CSA2_ERR_WORKSPACE when the sizes need more than the buffer
 *   (csa2_topk_and_block_candidates_workspace_size(Q, n_cols, k, block_size,
 *   n_blocks) > csa2_noalloc_scratch_bytes()); nothing is enqueued then.
 *   Every call on one device shares that device's buffer: calls that may
 *   overlap on one device (different streams, different threads without
 *   ordering) race and must not be issued.  The buffer needs no clearing.
 */
int csa2_topk_and_block_candidates_noalloc(const float* scores, int64_t score_stride,
                                           int32_t n_cols, const float* block_max,
                                           int64_t block_max_stride, const int32_t* q_pos,
                                           int32_t ratio, int32_t k, int32_t* idx,
                                           int32_t block_size, int32_t n_blocks, int32_t* cand,
                                           int32_t Q, const csa2_pages* pages, void* stream);

/* Size in bytes of the static buffer behind the _noalloc entry point. */
size_t csa2_noalloc_scratch_bytes(void);

/*
 * Diagnostics (not on the hot path).
 *
 * csa2_diag_index_scores_fp8_mfma — the dense scores of csa2_index_scores for
 * FP8 q_idx and k_idx (flat rows, H_I = 32, d_I = 128, the same score
 * definition: [DSA] Lightning Indexer, FP8 section), with every 128-dim dot
 * product taken on the FP8 matrix cores straight from the E4M3 codes.
 * csa2_index_scores widens the codes to f16 exactly and accumulates in fp32;
 * this form exists so the FP8 instructions' accumulation can be measured
 * against the 1e-3 score bound.  Arguments as in csa2_index_scores (scores
 * [Q, score_stride], n_cols columns, -inf past the visible count).
 *   Errors: CSA2_ERR_INVALID_ARG / CSA2_ERR_UNSUPPORTED on the host as in
 *   csa2_index_scores; CSA2_ERR_HIP if the launch fails.
 */
int csa2_diag_index_scores_fp8_mfma(const csa2_rows* q_idx, const void* w, csa2_dtype w_dtype,
                                    const csa2_rows* k_idx, const int64_t* seq_base,
                                    const int32_t* q_seq, const int32_t* q_pos, int32_t ratio,
                                    float* scores, int64_t score_stride, int32_t n_cols, int32_t Q,
                                    void* stream);

/*
 * csa2_diag_stream_read — reads bytes from src once, as fast as the chip
 * allows (16-byte non-temporal loads in a grid-stride loop), and computes
 * nothing from them: the practical HBM read ceiling against which the
 * hot path's HBM-bound stages are judged.
 *   src          device memory, 16-byte aligned; bytes a multiple of 16.
 *   sink         device memory of sink_floats floats (>= 1); the kernel runs
 *                min(4096, sink_floats) workgroups, and workgroup i may write
 *                sink[i] (it does so only for a sum no real input reaches).
 *   Errors: CSA2_ERR_INVALID_ARG for null or misaligned arguments;
 *   CSA2_ERR_HIP if the launch fails.
 */
int csa2_diag_stream_read(const void* src, size_t bytes, float* sink, size_t sink_floats, void* stream);

/*
 * csa2_diag_stream_write — fills bytes of dst with value (16-byte
 * non-temporal stores, 4096 workgroups in a grid-stride loop): the write
 * counterpart of csa2_diag_stream_read, and a write of known size for
 * calibrating memory-traffic counters.
 *   dst   device memory, 16-byte aligned; bytes a multiple of 16.
 *   Errors: CSA2_ERR_INVALID_ARG for null or misaligned arguments;
 *   CSA2_ERR_HIP if the launch fails.
 */
int csa2_diag_stream_write(void* dst, size_t bytes, float value, void* stream);

/*
 * csa2_diag_mfma_valu — a loop that measures whether matrix-core products
 * and vector ALU work overlap on one SIMD: 256 workgroups of eight waves
 * (two per SIMD) run iters iterations of eight independent
 * v_mfma_f32_32x32x16_f16 products (mode 1), 64 independent fp32 FMAs
 * (mode 2) or both (mode 3).  The caller times the launches; each thread
 * writes one float of its results to sink.
 *   sink   device memory of at least 256 * 512 floats (sink_floats).
 *   Errors: CSA2_ERR_INVALID_ARG for a null sink, a short sink, mode not in
 *   1..3 or iters < 1; CSA2_ERR_HIP if the launch fails.
 */
int csa2_diag_mfma_valu(int32_t mode, int32_t iters, float* sink, size_t sink_floats, void* stream);

/*
 * csa2_sparse_attn — core sparse attention ([CSA2] "per-layer attention
 * computation"; [3MODES] Q&A on Reuse layers).  For query t at position p of
 * sequence b and head i, the keys are the SWA rows of positions
 * [max(lo_b, swa_pos0[b], p - window + 1, 0), p] (oldest first) followed
 * by the main rows
 * idx[t, j] >= 0; K = V (MQA, one 512-dim vector per key).  With
 * z_j = softmax_scale * q[t, i] . K_j:
 *   out[t, i] = sum_j exp(z_j) K_j / (sum_j exp(z_j) + exp(attn_sink[i]))
 *   lse[t, i] = log(sum_j exp(z_j) + exp(attn_sink[i]))
 * The sink is a raw logit and enters only the denominator.  A position in
 * both the window and idx contributes both vectors.  RoPE is already applied
 * to the cached rows; the kernel applies none.
 *
 *   q         [Q, H, D] contiguous, q_dtype BF16 or F32.
 *   main_kv   rows = all main-KV entries: FP4_E2M1 with 16 scales per row
 *             (e.g. 320-byte records: 256 code bytes then 16 fp32 scales),
 *             FP4_E2M1_E4M3S16 with 32 E4M3 scale bytes per row (the pages'
 *             288-byte record: 256 code bytes then the scales; [CSA2] SGLang
 *             section; scale rows 8-byte aligned), or F32.
 *   main_base [B] int64: first main_kv row of each sequence.
 *   idx       [Q, k] int32 main positions; entries < 0 are skipped, and so
 *             are entries at or beyond the query's visible count
 *             (q_pos + 1) / ratio, so no row outside the visible prefix of the
 *             sequence is read.
 *   swa_kv    the layer's SWA rows: FP8_E4M3 with 4 scales per row (e.g.
 *             528-byte records), or F32.  Position p of sequence b is row
 *             swa_base[b] + p - swa_pos0[b]; positions below swa_pos0[b] are
 *             skipped, so the caller stores at least the window of every query.
 *   swa_lo    NULL (lo = 0) or [B] int32 first position of the bounded-replay
 *             segment ([CSA2] "CED": the query at i sees SWA keys in
 *             [max(s, i - W + 1), i]).
 *   window    W >= 0 (128 in the pages' configuration).
 *   attn_sink [H] fp32.
 *   out       [Q, H, D] output, out_dtype BF16 or F32.
 *   lse       NULL or [Q, H] fp32 output.
 *   workspace NULL, or device memory of workspace_bytes bytes the call may
 *             use (contents need not be initialised and are undefined
 *             afterwards).  With at least csa2_sparse_attn_workspace_size(Q,
 *             H, k, window) bytes, small batches split each query's keys
 *             over several workgroups and combine their partial softmax
 *             sums in a second kernel; results are the same up to rounding
 *             order.  With less, each (query, 16 heads) is one workgroup.
 *   io        NULL, or serving-shaped options (csa2_attn_io below).
 *   Supported: D = 512; H a multiple of 16 up to 128; k <= 2048.
 *   Quantized path: q BF16, main FP4_E2M1, swa FP8_E4M3, out BF16 or F32.
 *   Float path: q, main, swa F32, out F32.
 *   Precision of the quantized path: q is converted from bf16 to f16 for the
 *   matrix cores, exactly for |q| in f16's normal range [2^-14, 65504];
 *   smaller magnitudes keep f16's subnormal precision (2^-24 absolute), and
 *   larger ones overflow to infinity, so q entries must stay below 65504 in
 *   magnitude (scale q, not softmax_scale, to meet this).  Dequantized keys
 *   are code x scale rounded once to f16 (exact for the 288-byte records);
 *   probabilities are f16 below 2^8; all sums are fp32.
 */
typedef struct {
    /* NULL, or fp32 [n_rope, 64]: row r holds cos of the 32 RoPE angles of
     * position r, then their sin (the table csa2_cache_write takes).  Dims
     * 448..511 of every head's output are turned back by the query's
     * position before it is written ([CSA2] core formula: the output is
     * inverse-RoPE'd before the grouped output projection): for the pair
     * (x, y) = dims (448 + 2i, 449 + 2i), x' = x cos_i + y sin_i and
     * y' = y cos_i - x sin_i.  A query whose position is outside the table
     * is written unturned.  16-byte aligned. */
    const float* rope_cs;
    int32_t n_rope;
    /* Nonzero: idx holds physical main_kv rows, as csa2_topk writes them
     * through a page table ([DSA] top-k section: the sparse kernel gathers
     * by slot and never needs the positions); entries outside
     * [0, n_main_rows) are skipped, and main_base and the visibility bound
     * are not used (main_base may be NULL). */
    int32_t idx_slots;
    int64_t n_main_rows;
} csa2_attn_io;

int csa2_sparse_attn(const void* q, csa2_dtype q_dtype, const csa2_rows* main_kv,
                     const int64_t* main_base, const int32_t* idx, int32_t k,
                     const csa2_rows* swa_kv, const int64_t* swa_base,
                     const int32_t* swa_pos0, const int32_t* swa_lo, int32_t window,
                     const int32_t* q_seq, const int32_t* q_pos, int32_t ratio,
                     const float* attn_sink, float softmax_scale, void* out,
                     csa2_dtype out_dtype, float* lse, void* workspace,
                     size_t workspace_bytes, int32_t Q, int32_t H, int32_t D,
                     const csa2_attn_io* io, void* stream);

/* Workspace bytes csa2_sparse_attn uses to split keys for Q queries of H
 * heads with k indices and an SWA window of `window` (0 when it would not
 * split). */
size_t csa2_sparse_attn_workspace_size(int32_t Q, int32_t H, int32_t k, int32_t window);

/*
 * csa2_cache_write — a Full layer's write of its main-KV entries and index
 * keys ([CSA2] "per-layer attention computation", item 3; [3MODES]
 * "compression operator simplified" and Q&A "how is indexer K generated";
 * [REPORT] section 6: quantization after RoPE).  A token at position p of
 * sequence s closes entry e = p / ratio when p % ratio == ratio - 1; from the
 * entry's tokens (p - ratio + 1 .. p):
 *   cbar[ch] = sum_j softmax_j(z[j, ch]) c[j, ch]     (ratio 2; c itself for ratio 1)
 *   u        = cbar / sqrt(mean(cbar^2) + eps) * kv_norm_w   (the latent before RoPE)
 *   main     = RoPE(u)                                 dims 448..511 turn
 *   k        = RMSNorm(u W_IK^T) * k_norm_w, then RoPE  dims 64..127 turn
 * and writes main to row main_base[s] + e of main_out and k to row
 * k_base[s] + e of k_out, quantized to their dtypes.  RoPE turns adjacent
 * pairs (2i, 2i+1) of the turned dims by angle i of table row e * ratio (the
 * entry's first token): x' = x cos - y sin, y' = x sin + y cos.  Quantization:
 * per group, scale = amax / 6 (E2M1) or amax / 448 (E4M3) kept in fp32 (1.0
 * for an all-zero group), or for FP4_E2M1_E4M3S16 amax / 6 rounded to E4M3
 * (1.0 for an all-zero group, 2^-9 where the rounding gives zero); each
 * element is the nearest code of x / scale, ties to even, saturating.  With
 * ratio 2 an entry exists only once both of its tokens do ([CSA2] "the pool
 * does not reduce storage": n tokens hold n / 2 entries).
 *
 *   c, z      bf16 token rows, row t at (const char*)c + t * cz_stride (512
 *             values each; cz_stride >= 1024, both 16-byte aligned).  z holds
 *             the compressor's gate logits and is required for ratio 2 (NULL
 *             allowed for ratio 1).
 *   tok_seq   [T] int32 sequence of each token (tokens of sequence ids outside
 *             [0, B) write nothing).
 *   tok_pos   [T] int32 position of each token (negative: nothing written).
 *             A sequence's tokens in one call are consecutive rows at
 *             consecutive positions.
 *   ratio     m, 1 or 2.
 *   pend      NULL, or (ratio 2) bf16 [B, 2, 512]: the c row then the z row of
 *             the token that opened each sequence's incomplete pair, 16-byte
 *             aligned.  A token at an odd position whose partner is not the
 *             previous row of the call takes the partner from pend (without
 *             pend it writes nothing).  After every entry has read it, the
 *             call stores there the token that ends each sequence's run at an
 *             even position.  Calls that share pend must not overlap.
 *   B         number of sequences (length of main_base, k_base and pend).
 *   kv_norm_w [512] fp32, 16-byte aligned.
 *   w_ik      bf16 [128, 512] row-major (a linear layer's weight:
 *             k[n] = sum_c u[c] w_ik[n, c]), 16-byte aligned; required when
 *             k_out is given.
 *   k_norm_w  [128] fp32, 16-byte aligned; required when k_out is given.
 *   eps       RMSNorm epsilon (>= 0), both norms.
 *   rope_cs   fp32 [n_rope, 64], 16-byte aligned: row r holds cos of the 32
 *             angles of position r, then their sin.  An entry whose row
 *             e * ratio is >= n_rope writes nothing.
 *   main_out  NULL, or rows written: F32 (512 floats), FP4_E2M1 (256 code
 *             bytes and 16 fp32 scales, e.g. the 320-byte record) or
 *             FP4_E2M1_E4M3S16 (256 code bytes and 32 E4M3 scale bytes, e.g.
 *             the pages' 288-byte record).
 *   main_base [B] int64 first main_out row of each sequence; rows outside
 *             [0, main_rows) are not written.
 *   k_out     NULL, or rows written: F32 (128 floats), FP8_E4M3 (128 code
 *             bytes and one fp32 scale) or FP4_E2M1_E4M3S16 (64 code bytes
 *             and 8 E4M3 scale bytes).
 *   k_base    [B] int64 first k_out row of each sequence; rows outside
 *             [0, k_rows) are not written.
 *   At least one of main_out and k_out is given.  Rows follow the csa2_rows
 *   alignment rules (F32 rows 16-byte aligned).
 */
int csa2_cache_write(const void* c, const void* z, int64_t cz_stride, const int32_t* tok_seq,
                     const int32_t* tok_pos, int32_t T, int32_t ratio, void* pend, int32_t B,
                     const float* kv_norm_w, const void* w_ik, const float* k_norm_w, float eps,
                     const float* rope_cs, int32_t n_rope, const csa2_rows* main_out,
                     const int64_t* main_base, int64_t main_rows, const csa2_rows* k_out,
                     const int64_t* k_base, int64_t k_rows, void* stream);

/* Name of a status code (static string). */
const char* csa2_status_string(int status);

/* Message describing the last failed call on the calling thread (static
 * thread-local buffer; empty when no call has failed). */
const char* csa2_last_error(void);

/* Library version: major * 10000 + minor * 100 + patch. */
int csa2_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CSA2_H */
