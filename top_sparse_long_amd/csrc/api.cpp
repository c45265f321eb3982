// C ABI of the CSA2 hot path: host-side argument checks, then the launchers.
// Every check runs before anything is enqueued; no call allocates device
// memory or synchronises.
#include "../../include/csa2.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "kernels.h"

namespace {

thread_local char g_err[512];

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return CSA2_OK;
  return fail(CSA2_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int log2_exact(int v) {
  if (v <= 0 || (v & (v - 1))) return -1;
  int s = 0;
  while ((1 << s) < v) ++s;
  return s;
}

#define REQUIRE(cond, status, ...) \
  do {                             \
    if (!(cond)) return fail(status, __VA_ARGS__); \
  } while (0)

}  // namespace

extern "C" {

const char* csa2_status_string(int status) {
  switch (status) {
    case CSA2_OK: return "CSA2_OK";
    case CSA2_ERR_INVALID_ARG: return "CSA2_ERR_INVALID_ARG";
    case CSA2_ERR_UNSUPPORTED: return "CSA2_ERR_UNSUPPORTED";
    case CSA2_ERR_WORKSPACE: return "CSA2_ERR_WORKSPACE";
    case CSA2_ERR_HIP: return "CSA2_ERR_HIP";
    default: return "CSA2_ERR_UNKNOWN";
  }
}

const char* csa2_last_error(void) { return g_err; }

int csa2_version(void) { return 100; }

int csa2_index_scores(const csa2_rows* q_idx, const void* w, csa2_dtype w_dtype,
                      const csa2_rows* k_idx, const int64_t* seq_base, const int32_t* q_seq,
                      const int32_t* q_pos, int32_t ratio, const int32_t* cand,
                      int32_t n_cand_blocks, int32_t block_size, float* scores,
                      int64_t score_stride, int32_t n_cols, float* block_max,
                      int64_t block_max_stride, int32_t Q, int32_t H_I, int32_t d_I,
                      const csa2_pages* pages, void* stream) {
  g_err[0] = 0;
  REQUIRE(q_idx && k_idx && w && (seq_base || pages) && q_seq && q_pos && (scores || block_max),
          CSA2_ERR_INVALID_ARG, "csa2_index_scores: null pointer argument");
  REQUIRE(scores || !cand, CSA2_ERR_INVALID_ARG, "csa2_index_scores: pool mode writes scores (null scores)");
  if (pages)
    REQUIRE(pages->table && pages->table_stride >= 1 && pages->n_pages >= 1 && pages->page_stride >= 0 &&
                pages->page_stride % 16 == 0,
            CSA2_ERR_INVALID_ARG,
            "csa2_index_scores: pages needs a table, table_stride >= 1, n_pages >= 1 and a page_stride "
            ">= 0, multiple of 16");
  REQUIRE(q_idx->data && k_idx->data, CSA2_ERR_INVALID_ARG, "csa2_index_scores: null row data");
  REQUIRE(Q >= 0 && n_cols >= 0, CSA2_ERR_INVALID_ARG, "csa2_index_scores: negative size");
  REQUIRE(ratio == 1 || ratio == 2, CSA2_ERR_UNSUPPORTED, "csa2_index_scores: ratio must be 1 or 2");
  REQUIRE(d_I == 128, CSA2_ERR_UNSUPPORTED, "csa2_index_scores: d_I must be 128 (got %d)", d_I);
  REQUIRE(w_dtype == CSA2_BF16 || w_dtype == CSA2_F32, CSA2_ERR_UNSUPPORTED,
          "csa2_index_scores: gates must be BF16 or F32");
  const bool k_fp4 = k_idx->dtype == CSA2_FP4_E2M1_E4M3S16;
  REQUIRE(q_idx->dtype == k_idx->dtype || (q_idx->dtype == CSA2_FP8_E4M3 && k_fp4),
          CSA2_ERR_UNSUPPORTED,
          "csa2_index_scores: k_idx must share q_idx's dtype (or be FP4_E2M1_E4M3S16 with FP8 q_idx)");
  if (scores) {
    REQUIRE(score_stride >= n_cols && score_stride % 4 == 0, CSA2_ERR_INVALID_ARG,
            "csa2_index_scores: score_stride must be >= n_cols and a multiple of 4");
    REQUIRE(aligned(scores, 16), CSA2_ERR_INVALID_ARG, "csa2_index_scores: scores must be 16-byte aligned");
  }
  REQUIRE(aligned(q_idx->data, 16) && aligned(k_idx->data, 16) && q_idx->row_stride % 16 == 0 &&
              k_idx->row_stride % 16 == 0 && q_idx->row_stride > 0 && k_idx->row_stride > 0,
          CSA2_ERR_INVALID_ARG, "csa2_index_scores: rows must be 16-byte aligned");
  int bshift = 0;
  if (cand || block_max) {
    bshift = log2_exact(block_size);
    REQUIRE(bshift >= 0 && bshift <= 6, CSA2_ERR_UNSUPPORTED,
            "csa2_index_scores: block_size must be a power of two <= 64");
  }
  if (cand) {
    REQUIRE(n_cand_blocks >= 0 && (int64_t)n_cand_blocks * block_size == n_cols,
            CSA2_ERR_INVALID_ARG, "csa2_index_scores: pool mode needs n_cols == n_cand_blocks * block_size");
    REQUIRE(!block_max, CSA2_ERR_INVALID_ARG, "csa2_index_scores: block_max is a dense-mode output");
  }
  if (block_max) {
    REQUIRE(bshift <= 5, CSA2_ERR_UNSUPPORTED, "csa2_index_scores: block_max needs block_size <= 32");
    REQUIRE(block_max_stride >= ((int64_t)n_cols + block_size - 1) / block_size, CSA2_ERR_INVALID_ARG,
            "csa2_index_scores: block_max_stride below ceil(n_cols / block_size)");
    REQUIRE(aligned(block_max, 4), CSA2_ERR_INVALID_ARG, "csa2_index_scores: block_max must be 4-byte aligned");
  }
  csa2::IndexScoreArgs a = {};
  a.q = (const uint8_t*)q_idx->data;
  a.q_scale = q_idx->scale;
  a.q_row_stride = q_idx->row_stride;
  a.q_scale_stride = q_idx->scale_stride;
  a.w = w;
  a.w_bf16 = (w_dtype == CSA2_BF16);
  a.k = (const uint8_t*)k_idx->data;
  a.k_scale = k_idx->scale;
  a.k_row_stride = k_idx->row_stride;
  a.k_scale_stride = k_idx->scale_stride;
  a.k_scale_bytes = k_fp4 ? k_idx->scale_stride : k_idx->scale_stride * (int64_t)sizeof(float);
  a.k_fp4 = k_fp4 ? 1 : 0;
  if (pages) {
    a.page_table = pages->table;
    a.pt_stride = pages->table_stride;
    a.n_pages = pages->n_pages;
    a.k_page_bytes = pages->page_stride ? pages->page_stride : csa2::PAGE_SLOTS * k_idx->row_stride;
    a.s_page_bytes = pages->page_stride ? pages->page_stride : csa2::PAGE_SLOTS * a.k_scale_bytes;
  }
  a.seq_base = seq_base;
  a.q_seq = q_seq;
  a.q_pos = q_pos;
  a.ratio = ratio;
  a.cand = cand;
  a.n_cand_blocks = n_cand_blocks;
  a.block_shift = bshift;
  a.scores = scores;
  a.score_stride = score_stride;
  a.n_cols = n_cols;
  a.block_max = block_max;
  a.block_max_stride = block_max_stride;
  a.Q = Q;
  a.H = H_I;
  if (Q == 0 || n_cols == 0) return CSA2_OK;
  if (q_idx->dtype == CSA2_FP8_E4M3) {
    REQUIRE(H_I == 32, CSA2_ERR_UNSUPPORTED, "csa2_index_scores: FP8 path needs H_I == 32 (got %d)", H_I);
    REQUIRE(q_idx->scale && k_idx->scale, CSA2_ERR_INVALID_ARG, "csa2_index_scores: FP8 rows need scales");
    REQUIRE(q_idx->row_stride >= 128 && k_idx->row_stride >= (k_fp4 ? 64 : 128), CSA2_ERR_INVALID_ARG,
            "csa2_index_scores: row stride below the row's code bytes");
    if (k_fp4)
      REQUIRE(aligned(k_idx->scale, 4) && k_idx->scale_stride >= 8 && k_idx->scale_stride % 4 == 0,
              CSA2_ERR_INVALID_ARG,
              "csa2_index_scores: FP4 key scales need 4-byte alignment and a stride >= 8 bytes, multiple of 4");
    return hip_status(csa2::launch_index_scores_fp8(a, (hipStream_t)stream), "csa2_index_scores");
  }
  if (q_idx->dtype == CSA2_F32) {
    REQUIRE(H_I >= 1 && H_I <= 64, CSA2_ERR_UNSUPPORTED, "csa2_index_scores: F32 path needs 1 <= H_I <= 64");
    REQUIRE(q_idx->row_stride >= 512 && k_idx->row_stride >= 512, CSA2_ERR_INVALID_ARG,
            "csa2_index_scores: F32 row stride below 512 bytes");
    return hip_status(csa2::launch_index_scores_f32(a, (hipStream_t)stream), "csa2_index_scores");
  }
  return fail(CSA2_ERR_UNSUPPORTED, "csa2_index_scores: rows must be FP8_E4M3 or F32");
}

int csa2_diag_index_scores_fp8_mfma(const csa2_rows* q_idx, const void* w, csa2_dtype w_dtype,
                                    const csa2_rows* k_idx, const int64_t* seq_base,
                                    const int32_t* q_seq, const int32_t* q_pos, int32_t ratio,
                                    float* scores, int64_t score_stride, int32_t n_cols, int32_t Q,
                                    void* stream) {
  g_err[0] = 0;
  REQUIRE(q_idx && k_idx && w && seq_base && q_seq && q_pos && scores && q_idx->data && k_idx->data &&
              q_idx->scale && k_idx->scale,
          CSA2_ERR_INVALID_ARG, "csa2_diag_index_scores_fp8_mfma: null pointer argument");
  REQUIRE(q_idx->dtype == CSA2_FP8_E4M3 && k_idx->dtype == CSA2_FP8_E4M3, CSA2_ERR_UNSUPPORTED,
          "csa2_diag_index_scores_fp8_mfma: q_idx and k_idx must be FP8_E4M3");
  REQUIRE(w_dtype == CSA2_BF16 || w_dtype == CSA2_F32, CSA2_ERR_UNSUPPORTED,
          "csa2_diag_index_scores_fp8_mfma: gates must be BF16 or F32");
  REQUIRE(ratio == 1 || ratio == 2, CSA2_ERR_UNSUPPORTED, "csa2_diag_index_scores_fp8_mfma: ratio must be 1 or 2");
  REQUIRE(Q >= 0 && n_cols >= 0 && score_stride >= n_cols, CSA2_ERR_INVALID_ARG,
          "csa2_diag_index_scores_fp8_mfma: bad size or stride");
  REQUIRE(aligned(q_idx->data, 16) && aligned(k_idx->data, 16) && q_idx->row_stride % 16 == 0 &&
              k_idx->row_stride % 16 == 0 && q_idx->row_stride >= 128 && k_idx->row_stride >= 128,
          CSA2_ERR_INVALID_ARG, "csa2_diag_index_scores_fp8_mfma: rows must be 16-byte aligned, >= 128 bytes");
  if (Q == 0 || n_cols == 0) return CSA2_OK;
  csa2::IndexScoreArgs a = {};
  a.q = (const uint8_t*)q_idx->data;
  a.q_scale = q_idx->scale;
  a.q_row_stride = q_idx->row_stride;
  a.q_scale_stride = q_idx->scale_stride;
  a.w = w;
  a.w_bf16 = (w_dtype == CSA2_BF16);
  a.k = (const uint8_t*)k_idx->data;
  a.k_scale = k_idx->scale;
  a.k_row_stride = k_idx->row_stride;
  a.k_scale_stride = k_idx->scale_stride;
  a.k_scale_bytes = k_idx->scale_stride * (int64_t)sizeof(float);
  a.seq_base = seq_base;
  a.q_seq = q_seq;
  a.q_pos = q_pos;
  a.ratio = ratio;
  a.scores = scores;
  a.score_stride = score_stride;
  a.n_cols = n_cols;
  a.Q = Q;
  a.H = 32;
  return hip_status(csa2::launch_index_scores_fp8mma_diag(a, (hipStream_t)stream),
                    "csa2_diag_index_scores_fp8_mfma");
}

int csa2_diag_stream_read(const void* src, size_t bytes, float* sink, size_t sink_floats, void* stream) {
  g_err[0] = 0;
  REQUIRE(src && sink, CSA2_ERR_INVALID_ARG, "csa2_diag_stream_read: null pointer argument");
  REQUIRE(aligned(src, 16) && bytes % 16 == 0, CSA2_ERR_INVALID_ARG,
          "csa2_diag_stream_read: src must be 16-byte aligned and bytes a multiple of 16");
  REQUIRE(sink_floats >= 1, CSA2_ERR_INVALID_ARG, "csa2_diag_stream_read: sink must hold at least one float");
  if (bytes == 0) return CSA2_OK;
  const int n_blocks = (int)std::min<size_t>(4096, sink_floats);
  return hip_status(csa2::launch_stream_read(src, bytes, sink, n_blocks, (hipStream_t)stream),
                    "csa2_diag_stream_read");
}

int csa2_diag_stream_write(void* dst, size_t bytes, float value, void* stream) {
  g_err[0] = 0;
  REQUIRE(dst, CSA2_ERR_INVALID_ARG, "csa2_diag_stream_write: null pointer argument");
  REQUIRE(aligned(dst, 16) && bytes % 16 == 0, CSA2_ERR_INVALID_ARG,
          "csa2_diag_stream_write: dst must be 16-byte aligned and bytes a multiple of 16");
  if (bytes == 0) return CSA2_OK;
  return hip_status(csa2::launch_stream_write(dst, bytes, value, 4096, (hipStream_t)stream),
                    "csa2_diag_stream_write");
}

int csa2_diag_mfma_valu(int32_t mode, int32_t iters, float* sink, size_t sink_floats, void* stream) {
  g_err[0] = 0;
  REQUIRE(sink, CSA2_ERR_INVALID_ARG, "csa2_diag_mfma_valu: null sink");
  REQUIRE(mode >= 1 && mode <= 3, CSA2_ERR_INVALID_ARG, "csa2_diag_mfma_valu: mode must be 1, 2 or 3");
  REQUIRE(iters >= 1, CSA2_ERR_INVALID_ARG, "csa2_diag_mfma_valu: iters must be positive");
  REQUIRE(sink_floats >= (size_t)csa2::MV_BLOCKS * 512, CSA2_ERR_INVALID_ARG,
          "csa2_diag_mfma_valu: sink must hold 256 * 512 floats");
  return hip_status(csa2::launch_mfma_valu(mode, iters, sink, (hipStream_t)stream), "csa2_diag_mfma_valu");
}

size_t csa2_topk_workspace_size(int32_t Q, int32_t n_cols, int32_t k) {
  if (Q <= 0 || n_cols <= 0 || k <= 0) return 0;
  return csa2::select_workspace_bytes(Q, n_cols, k);
}

size_t csa2_block_candidates_workspace_size(int32_t Q, int32_t n_cols, int32_t block_size,
                                            int32_t n_blocks) {
  if (Q <= 0 || n_cols <= 0 || n_blocks <= 0 || block_size <= 0) return 0;
  const int64_t nb = ((int64_t)n_cols + block_size - 1) / block_size;
  return csa2::select_workspace_bytes(Q, nb, n_blocks);
}

static int check_select_common(const char* fn, const float* scores, int64_t score_stride,
                               int32_t n_cols, int32_t k, const void* out, int32_t Q) {
  REQUIRE(scores && out, CSA2_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  REQUIRE(Q >= 0 && n_cols >= 0, CSA2_ERR_INVALID_ARG, "%s: negative size", fn);
  REQUIRE(score_stride >= n_cols && score_stride % 4 == 0, CSA2_ERR_INVALID_ARG,
          "%s: score_stride must be >= n_cols and a multiple of 4", fn);
  REQUIRE(aligned(scores, 16), CSA2_ERR_INVALID_ARG, "%s: scores must be 16-byte aligned", fn);
  REQUIRE(k >= 1, CSA2_ERR_INVALID_ARG, "%s: k must be positive", fn);
  return CSA2_OK;
}

// Checks of csa2_block_candidates; fills the selection arguments and the
// number of blocks per row.
static int prep_block_candidates(const float* scores, int64_t score_stride, int32_t n_cols,
                                 const float* block_max, int64_t block_max_stride,
                                 const int32_t* q_pos, int32_t ratio, int32_t block_size,
                                 int32_t n_blocks, int32_t* cand, void* workspace,
                                 size_t workspace_bytes, int32_t Q, csa2::SelectArgs* out,
                                 int64_t* n_rows) {
  if (block_max) {
    // the maxima replace the scores; the stride and alignment checks of the
    // scores apply to a stand-in that is never read
    REQUIRE(cand, CSA2_ERR_INVALID_ARG, "csa2_block_candidates: null pointer argument");
    REQUIRE(Q >= 0 && n_cols >= 0 && n_blocks >= 1, CSA2_ERR_INVALID_ARG,
            "csa2_block_candidates: bad size");
    REQUIRE(block_size > 0 && block_max_stride >= ((int64_t)n_cols + block_size - 1) / block_size,
            CSA2_ERR_INVALID_ARG, "csa2_block_candidates: block_max_stride below the block count");
    REQUIRE(aligned(block_max, 4), CSA2_ERR_INVALID_ARG, "csa2_block_candidates: block_max must be 4-byte aligned");
  } else {
    int st = check_select_common("csa2_block_candidates", scores, score_stride, n_cols, n_blocks,
                                 cand, Q);
    if (st) return st;
  }
  REQUIRE(q_pos, CSA2_ERR_INVALID_ARG, "csa2_block_candidates: q_pos is required");
  REQUIRE(ratio == 1 || ratio == 2, CSA2_ERR_UNSUPPORTED, "csa2_block_candidates: ratio must be 1 or 2");
  const int bshift = log2_exact(block_size);
  REQUIRE(bshift >= 0 && bshift <= 6, CSA2_ERR_UNSUPPORTED,
          "csa2_block_candidates: block_size must be a power of two <= 64");
  REQUIRE(n_blocks <= 4096, CSA2_ERR_UNSUPPORTED, "csa2_block_candidates: n_blocks above 4096");
  const size_t need = csa2_block_candidates_workspace_size(Q, n_cols, block_size, n_blocks);
  REQUIRE(workspace_bytes >= need && (need == 0 || workspace), CSA2_ERR_WORKSPACE,
          "csa2_block_candidates: workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  REQUIRE(aligned(workspace, 16), CSA2_ERR_INVALID_ARG, "csa2_block_candidates: workspace must be 16-byte aligned");
  csa2::SelectArgs a = {};
  a.scores = scores;
  a.score_stride = score_stride;
  a.n_cols = n_cols;
  a.block_max = block_max;
  a.block_max_stride = block_max_stride;
  a.q_pos = q_pos;
  a.ratio = ratio;
  a.block_shift = bshift;
  a.k = n_blocks;
  a.out_idx = cand;
  a.workspace = workspace;
  a.Q = Q;
  *out = a;
  *n_rows = ((int64_t)n_cols + block_size - 1) / block_size;
  return CSA2_OK;
}

int csa2_block_candidates(const float* scores, int64_t score_stride, int32_t n_cols,
                          const float* block_max, int64_t block_max_stride,
                          const int32_t* q_pos, int32_t ratio, int32_t block_size,
                          int32_t n_blocks, int32_t* cand, void* workspace,
                          size_t workspace_bytes, int32_t Q, void* stream) {
  g_err[0] = 0;
  csa2::SelectArgs a;
  int64_t nb = 0;
  const int st = prep_block_candidates(scores, score_stride, n_cols, block_max, block_max_stride,
                                       q_pos, ratio, block_size, n_blocks, cand, workspace,
                                       workspace_bytes, Q, &a, &nb);
  if (st != CSA2_OK || Q == 0) return st;
  return hip_status(csa2::launch_select(csa2::SEL_BLOCKMAX, a, nb, (hipStream_t)stream),
                    "csa2_block_candidates");
}

static int prep_topk(const float* scores, int64_t score_stride, int32_t n_cols,
                     const int32_t* q_pos, int32_t ratio, const int32_t* cand,
                     int32_t n_cand_blocks, int32_t block_size, int32_t k, int32_t* idx,
                     void* workspace, size_t workspace_bytes, int32_t Q, const csa2_pages* pages,
                     csa2::SelectArgs* out) {
  int st = check_select_common("csa2_topk", scores, score_stride, n_cols, k, idx, Q);
  if (st) return st;
  if (pages)
    REQUIRE(pages->table && pages->q_seq && pages->table_stride >= 1, CSA2_ERR_INVALID_ARG,
            "csa2_topk: pages needs a table, q_seq and table_stride >= 1");
  REQUIRE(k <= 2048, CSA2_ERR_UNSUPPORTED, "csa2_topk: k above 2048");
  if (q_pos) REQUIRE(ratio == 1 || ratio == 2, CSA2_ERR_UNSUPPORTED, "csa2_topk: ratio must be 1 or 2");
  int bshift = 0;
  if (cand) {
    bshift = log2_exact(block_size);
    REQUIRE(bshift >= 0 && bshift <= 6, CSA2_ERR_UNSUPPORTED,
            "csa2_topk: block_size must be a power of two <= 64");
    REQUIRE(n_cand_blocks >= 0 && (int64_t)n_cand_blocks * block_size == n_cols,
            CSA2_ERR_INVALID_ARG, "csa2_topk: pool mode needs n_cols == n_cand_blocks * block_size");
  }
  const size_t need = csa2_topk_workspace_size(Q, n_cols, k);
  REQUIRE(workspace_bytes >= need && (need == 0 || workspace), CSA2_ERR_WORKSPACE,
          "csa2_topk: workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  REQUIRE(aligned(workspace, 16), CSA2_ERR_INVALID_ARG, "csa2_topk: workspace must be 16-byte aligned");
  csa2::SelectArgs a = {};
  a.scores = scores;
  a.score_stride = score_stride;
  a.n_cols = n_cols;
  a.q_pos = cand ? nullptr : q_pos;
  a.ratio = ratio;
  a.cand = cand;
  a.n_cand_blocks = n_cand_blocks;
  a.block_shift = bshift;
  a.k = k;
  a.out_idx = idx;
  a.workspace = workspace;
  a.Q = Q;
  if (pages) {
    a.page_table = pages->table;
    a.pt_stride = pages->table_stride;
    a.pt_seq = pages->q_seq;
  }
  *out = a;
  return CSA2_OK;
}

int csa2_topk(const float* scores, int64_t score_stride, int32_t n_cols, const int32_t* q_pos,
              int32_t ratio, const int32_t* cand, int32_t n_cand_blocks, int32_t block_size,
              int32_t k, int32_t* idx, void* workspace, size_t workspace_bytes, int32_t Q,
              const csa2_pages* pages, void* stream) {
  g_err[0] = 0;
  csa2::SelectArgs a;
  const int st = prep_topk(scores, score_stride, n_cols, q_pos, ratio, cand, n_cand_blocks,
                           block_size, k, idx, workspace, workspace_bytes, Q, pages, &a);
  if (st != CSA2_OK || Q == 0) return st;
  return hip_status(csa2::launch_select(cand ? csa2::SEL_POOL : csa2::SEL_DENSE, a, n_cols,
                                        (hipStream_t)stream),
                    "csa2_topk");
}

static size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }

size_t csa2_topk_from_block_max_workspace_size(int32_t Q, int32_t n_cols, int32_t k,
                                                int32_t block_size) {
  if (Q <= 0 || n_cols <= 0 || k <= 0 || block_size <= 0) return 0;
  const int shift = log2_exact(block_size);
  const int64_t nb = ((int64_t)n_cols + block_size - 1) / block_size;
  if (shift >= 0 && csa2::top_via_blocks_supported(k, shift))
    return csa2::top_via_blocks_workspace_bytes(Q, nb, k);
  return csa2_topk_workspace_size(Q, n_cols, k);
}

int csa2_topk_from_block_max(const float* scores, int64_t score_stride, int32_t n_cols,
                             const float* block_max, int64_t block_max_stride, const int32_t* q_pos,
                             int32_t ratio, int32_t block_size, int32_t k, int32_t* idx,
                             void* workspace, size_t workspace_bytes, int32_t Q,
                             const csa2_pages* pages, void* stream) {
  g_err[0] = 0;
  REQUIRE(q_pos, CSA2_ERR_INVALID_ARG, "csa2_topk_from_block_max: q_pos is required");
  const int shift = log2_exact(block_size);
  REQUIRE(shift >= 0 && shift <= 5, CSA2_ERR_UNSUPPORTED,
          "csa2_topk_from_block_max: block_size must be a power of two <= 32");
  REQUIRE(block_max && block_max_stride >= ((int64_t)n_cols + block_size - 1) / block_size &&
              aligned(block_max, 4),
          CSA2_ERR_INVALID_ARG,
          "csa2_topk_from_block_max: block_max must be 4-byte aligned with a stride >= ceil(n_cols / block_size)");
  const int64_t nb = ((int64_t)n_cols + block_size - 1) / block_size;
  if (!csa2::top_via_blocks_supported(k, shift))
    return csa2_topk(scores, score_stride, n_cols, q_pos, ratio, nullptr, 0, block_size, k, idx,
                     workspace, workspace_bytes, Q, pages, stream);
  const size_t need = Q > 0 && k > 0 && n_cols > 0 ? csa2::top_via_blocks_workspace_bytes(Q, nb, k) : 0;
  REQUIRE(workspace_bytes >= need && (need == 0 || workspace), CSA2_ERR_WORKSPACE,
          "csa2_topk_from_block_max: workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  csa2::SelectArgs a;
  // the plain top-k's argument checks (its own workspace size does not apply here)
  int st = prep_topk(scores, score_stride, n_cols, q_pos, ratio, nullptr, 0, block_size, k, idx,
                     workspace, (size_t)-1, Q, pages, &a);
  if (st != CSA2_OK) return st;
  if (Q == 0 || n_cols == 0) return CSA2_OK;
  a.block_max = block_max;
  a.block_max_stride = block_max_stride;
  a.block_shift = shift;
  a.workspace = workspace;
  return hip_status(csa2::launch_topk_via_blocks(a, nb, (hipStream_t)stream), "csa2_topk_from_block_max");
}



// Workspace of the combined call's top-k: enough for the dense route and,
// when the shapes allow it, for the route through block maxima.
static size_t pair_topk_bytes(int32_t Q, int32_t n_cols, int32_t k, int32_t block_size) {
  size_t b = csa2_topk_workspace_size(Q, n_cols, k);
  const int shift = log2_exact(block_size);
  if (Q > 0 && n_cols > 0 && k > 0 && shift >= 0 && csa2::top_via_blocks_supported(k, shift)) {
    const int64_t nb = ((int64_t)n_cols + block_size - 1) / block_size;
    b = std::max(b, csa2::top_via_blocks_workspace_bytes(Q, nb, k));
  }
  return b;
}

size_t csa2_topk_and_block_candidates_workspace_size(int32_t Q, int32_t n_cols, int32_t k,
                                                     int32_t block_size, int32_t n_blocks) {
  return align16(pair_topk_bytes(Q, n_cols, k, block_size)) +
         csa2_block_candidates_workspace_size(Q, n_cols, block_size, n_blocks);
}

// Both selections of a Full layer.  With from_scratch the lists go to the
// library's static scratch buffer instead of a caller workspace: the checks
// run against a stand-in address (never dereferenced), and the real address
// is looked up only once every check has passed.
static int topk_and_blocks(const float* scores, int64_t score_stride, int32_t n_cols,
                           const float* block_max, int64_t block_max_stride, const int32_t* q_pos,
                           int32_t ratio, int32_t k, int32_t* idx, int32_t block_size,
                           int32_t n_blocks, int32_t* cand, void* workspace,
                           size_t workspace_bytes, int32_t Q, const csa2_pages* pages,
                           void* stream, bool from_scratch) {
  const char* fn = from_scratch ? "csa2_topk_and_block_candidates_noalloc"
                                : "csa2_topk_and_block_candidates";
  REQUIRE(q_pos, CSA2_ERR_INVALID_ARG, "%s: q_pos is required", fn);
  // the top-k's workspace comes first, the pool's follows at a 16-byte boundary
  const size_t ws_t = align16(pair_topk_bytes(Q, n_cols, k, block_size));
  if (from_scratch) {
    const size_t need = csa2_topk_and_block_candidates_workspace_size(Q, n_cols, k, block_size, n_blocks);
    REQUIRE(need <= csa2::SELECT_SCRATCH_BYTES, CSA2_ERR_WORKSPACE,
            "%s: these sizes need %zu bytes of scratch, above the %zu-byte static buffer "
            "(use csa2_topk_and_block_candidates with a workspace)",
            fn, need, csa2::SELECT_SCRATCH_BYTES);
    workspace = (void*)(uintptr_t)256;   // stand-in for the checks only
    workspace_bytes = need;
  }
  const size_t ws_b = workspace_bytes > ws_t ? workspace_bytes - ws_t : 0;
  uint8_t* ws = (uint8_t*)workspace;
  csa2::SelectArgs at, ab;
  int64_t nb = 0;
  int st = prep_topk(scores, score_stride, n_cols, q_pos, ratio, nullptr, 0, block_size, k, idx,
                     workspace, workspace_bytes < ws_t ? workspace_bytes : ws_t, Q, pages, &at);
  if (st != CSA2_OK) return st;
  st = prep_block_candidates(scores, score_stride, n_cols, block_max, block_max_stride, q_pos,
                             ratio, block_size, n_blocks, cand, ws_b ? ws + ws_t : nullptr, ws_b,
                             Q, &ab, &nb);
  if (st != CSA2_OK || Q == 0) return st;
  if (from_scratch) {
    void* base = nullptr;
    if (workspace_bytes > 0) {
      const hipError_t e = csa2::select_scratch(&base);
      if (e != hipSuccess) return hip_status(e, "csa2_topk_and_block_candidates_noalloc: scratch lookup");
    }
    at.workspace = base;
    ab.workspace = ws_b ? (uint8_t*)base + ws_t : nullptr;
  }
  // with block maxima the top-k ranks blocks first (same result)
  const bool via = block_max && csa2::top_via_blocks_supported(k, ab.block_shift);
  int64_t t_len = n_cols;
  if (via) {
    at.block_max = block_max;
    at.block_max_stride = block_max_stride;
    at.block_shift = ab.block_shift;
    t_len = ((int64_t)n_cols + block_size - 1) / block_size;
  }
  return hip_status(csa2::launch_topk_and_blocks(at, t_len, via, ab, nb, (hipStream_t)stream), fn);
}

int csa2_topk_and_block_candidates(const float* scores, int64_t score_stride, int32_t n_cols,
                                   const float* block_max, int64_t block_max_stride,
                                   const int32_t* q_pos, int32_t ratio, int32_t k, int32_t* idx,
                                   int32_t block_size, int32_t n_blocks, int32_t* cand,
                                   void* workspace, size_t workspace_bytes, int32_t Q,
                                   const csa2_pages* pages, void* stream) {
  g_err[0] = 0;
  return topk_and_blocks(scores, score_stride, n_cols, block_max, block_max_stride, q_pos, ratio, k,
                         idx, block_size, n_blocks, cand, workspace, workspace_bytes, Q, pages,
                         stream, false);
}

size_t csa2_top_blocks_and_block_candidates_workspace_size(int32_t Q, int32_t n_cols, int32_t block_size,
                                                           int32_t k_blocks, int32_t n_blocks) {
  return align16(csa2_block_candidates_workspace_size(Q, n_cols, block_size, k_blocks)) +
         csa2_block_candidates_workspace_size(Q, n_cols, block_size, n_blocks);
}

int csa2_top_blocks_and_block_candidates(const float* block_max, int64_t block_max_stride, int32_t n_cols,
                                         const int32_t* q_pos, int32_t ratio, int32_t block_size,
                                         int32_t k_blocks, int32_t* top_blocks, int32_t n_blocks,
                                         int32_t* cand, void* workspace, size_t workspace_bytes, int32_t Q,
                                         void* stream) {
  g_err[0] = 0;
  REQUIRE(block_max && top_blocks && cand, CSA2_ERR_INVALID_ARG,
          "csa2_top_blocks_and_block_candidates: null pointer argument");
  // the best blocks' workspace comes first, the candidates' follows at a
  // 16-byte boundary
  const size_t ws_t = align16(csa2_block_candidates_workspace_size(Q, n_cols, block_size, k_blocks));
  const size_t ws_b = workspace_bytes > ws_t ? workspace_bytes - ws_t : 0;
  csa2::SelectArgs at, ab;
  int64_t n_rows = 0;
  int st = prep_block_candidates(nullptr, 0, n_cols, block_max, block_max_stride, q_pos, ratio, block_size,
                                 k_blocks, top_blocks, workspace, workspace_bytes < ws_t ? workspace_bytes : ws_t,
                                 Q, &at, &n_rows);
  if (st != CSA2_OK) return st;
  st = prep_block_candidates(nullptr, 0, n_cols, block_max, block_max_stride, q_pos, ratio, block_size,
                             n_blocks, cand, ws_b ? (uint8_t*)workspace + ws_t : nullptr, ws_b, Q, &ab, &n_rows);
  if (st != CSA2_OK || Q == 0 || n_rows == 0) return st;
  return hip_status(csa2::launch_top_blocks_and_blocks(at, ab, n_rows, (hipStream_t)stream),
                    "csa2_top_blocks_and_block_candidates");
}

size_t csa2_noalloc_scratch_bytes(void) { return csa2::SELECT_SCRATCH_BYTES; }

int csa2_topk_and_block_candidates_noalloc(const float* scores, int64_t score_stride,
                                           int32_t n_cols, const float* block_max,
                                           int64_t block_max_stride, const int32_t* q_pos,
                                           int32_t ratio, int32_t k, int32_t* idx,
                                           int32_t block_size, int32_t n_blocks, int32_t* cand,
                                           int32_t Q, const csa2_pages* pages, void* stream) {
  g_err[0] = 0;
  return topk_and_blocks(scores, score_stride, n_cols, block_max, block_max_stride, q_pos, ratio, k,
                         idx, block_size, n_blocks, cand, nullptr, 0, Q, pages, stream, true);
}

int csa2_sparse_attn(const void* q, csa2_dtype q_dtype, const csa2_rows* main_kv,
                     const int64_t* main_base, const int32_t* idx, int32_t k,
                     const csa2_rows* swa_kv, const int64_t* swa_base, const int32_t* swa_pos0,
                     const int32_t* swa_lo, int32_t window, const int32_t* q_seq,
                     const int32_t* q_pos, int32_t ratio, const float* attn_sink,
                     float softmax_scale, void* out, csa2_dtype out_dtype, float* lse,
                     void* workspace, size_t workspace_bytes, int32_t Q, int32_t H, int32_t D,
                     const csa2_attn_io* io, void* stream) {
  g_err[0] = 0;
  const bool slots = io && io->idx_slots;
  REQUIRE(q && main_kv && (main_base || slots) && idx && swa_kv && swa_base && swa_pos0 && q_seq &&
              q_pos && attn_sink && out,
          CSA2_ERR_INVALID_ARG, "csa2_sparse_attn: null pointer argument");
  if (io) {
    REQUIRE(io->n_rope >= 0 && (!slots || io->n_main_rows >= 0), CSA2_ERR_INVALID_ARG,
            "csa2_sparse_attn: negative size in io");
    REQUIRE(!io->rope_cs || aligned(io->rope_cs, 16), CSA2_ERR_INVALID_ARG,
            "csa2_sparse_attn: io->rope_cs must be 16-byte aligned");
  }
  REQUIRE(main_kv->data && swa_kv->data, CSA2_ERR_INVALID_ARG, "csa2_sparse_attn: null row data");
  REQUIRE(Q >= 0 && k >= 0 && window >= 0, CSA2_ERR_INVALID_ARG, "csa2_sparse_attn: negative size");
  REQUIRE(D == 512, CSA2_ERR_UNSUPPORTED, "csa2_sparse_attn: D must be 512 (got %d)", D);
  REQUIRE(H >= 16 && H <= 128 && H % 16 == 0, CSA2_ERR_UNSUPPORTED,
          "csa2_sparse_attn: H must be a multiple of 16 in [16, 128] (got %d)", H);
  REQUIRE(k <= 2048, CSA2_ERR_UNSUPPORTED, "csa2_sparse_attn: k above 2048");
  REQUIRE(ratio == 1 || ratio == 2, CSA2_ERR_UNSUPPORTED, "csa2_sparse_attn: ratio must be 1 or 2");
  REQUIRE(aligned(q, 16) && aligned(out, 16), CSA2_ERR_INVALID_ARG,
          "csa2_sparse_attn: q and out must be 16-byte aligned");
  REQUIRE(aligned(main_kv->data, 16) && aligned(swa_kv->data, 16) && main_kv->row_stride % 16 == 0 &&
              swa_kv->row_stride % 16 == 0 && main_kv->row_stride > 0 && swa_kv->row_stride > 0,
          CSA2_ERR_INVALID_ARG, "csa2_sparse_attn: rows must be 16-byte aligned");
  csa2::AttnArgs a = {};
  a.q = q;
  a.main = (const uint8_t*)main_kv->data;
  a.main_scale = main_kv->scale;
  a.main_stride = main_kv->row_stride;
  a.main_scale_stride = main_kv->scale_stride;
  a.main_s16 = main_kv->dtype == CSA2_FP4_E2M1_E4M3S16 ? 1 : 0;
  a.main_base = main_base;
  a.idx = idx;
  a.k = k;
  a.swa = (const uint8_t*)swa_kv->data;
  a.swa_scale = swa_kv->scale;
  a.swa_stride = swa_kv->row_stride;
  a.swa_scale_stride = swa_kv->scale_stride;
  a.swa_base = swa_base;
  a.swa_pos0 = swa_pos0;
  a.swa_lo = swa_lo;
  a.window = window;
  a.q_seq = q_seq;
  a.q_pos = q_pos;
  a.ratio = ratio;
  a.sink = attn_sink;
  a.scale = softmax_scale;
  a.out = out;
  a.out_bf16 = (out_dtype == CSA2_BF16);
  a.lse = lse;
  a.Q = Q;
  a.H = H;
  a.idx_slots = slots ? 1 : 0;
  a.n_main_rows = slots ? io->n_main_rows : 0;
  a.rope = io ? io->rope_cs : nullptr;
  a.n_rope = io ? io->n_rope : 0;
  const bool s16 = main_kv->dtype == CSA2_FP4_E2M1_E4M3S16;
  const bool quant = q_dtype == CSA2_BF16 && (main_kv->dtype == CSA2_FP4_E2M1 || s16) &&
                     swa_kv->dtype == CSA2_FP8_E4M3 &&
                     (out_dtype == CSA2_BF16 || out_dtype == CSA2_F32);
  const bool f32 = q_dtype == CSA2_F32 && main_kv->dtype == CSA2_F32 && swa_kv->dtype == CSA2_F32 &&
                   out_dtype == CSA2_F32;
  REQUIRE(quant || f32, CSA2_ERR_UNSUPPORTED,
          "csa2_sparse_attn: supported dtypes are (q BF16, main FP4_E2M1 or FP4_E2M1_E4M3S16, "
          "swa FP8_E4M3, out BF16|F32) "
          "and (all F32)");
  if (quant) {
    REQUIRE(main_kv->scale && swa_kv->scale, CSA2_ERR_INVALID_ARG, "csa2_sparse_attn: quantized rows need scales");
    REQUIRE(main_kv->row_stride >= 256 && swa_kv->row_stride >= 512, CSA2_ERR_INVALID_ARG,
            "csa2_sparse_attn: row stride below the code bytes of a row");
    if (s16)
      REQUIRE(aligned(main_kv->scale, 8) && main_kv->scale_stride % 8 == 0 && main_kv->scale_stride >= 32,
              CSA2_ERR_INVALID_ARG,
              "csa2_sparse_attn: E4M3 main-KV scales must be 8-byte aligned rows of >= 32 bytes");
    else
      REQUIRE(aligned(main_kv->scale, 16) && main_kv->scale_stride % 4 == 0 && main_kv->scale_stride >= 16,
              CSA2_ERR_INVALID_ARG, "csa2_sparse_attn: FP4 scales must be 16-byte aligned rows of >= 16 floats");
    REQUIRE(aligned(swa_kv->scale, 4) && swa_kv->scale_stride >= 4, CSA2_ERR_INVALID_ARG,
            "csa2_sparse_attn: FP8 SWA rows need 4 scales each");
  } else {
    REQUIRE(main_kv->row_stride >= 2048 && swa_kv->row_stride >= 2048, CSA2_ERR_INVALID_ARG,
            "csa2_sparse_attn: F32 row stride below 2048 bytes");
    REQUIRE((int64_t)window + k <= 8192, CSA2_ERR_UNSUPPORTED, "csa2_sparse_attn: F32 path needs window + k <= 8192");
  }
  if (Q == 0) return CSA2_OK;
  a.n_split = 1;
  a.part = nullptr;
  if (quant && workspace) {
    const size_t need = csa2_sparse_attn_workspace_size(Q, H, k, window);
    if (need > 0 && workspace_bytes >= need) {
      REQUIRE(aligned(workspace, 16), CSA2_ERR_INVALID_ARG, "csa2_sparse_attn: workspace must be 16-byte aligned");
      a.n_split = csa2::attn_splits(Q, H, k, window);
      a.part = (float*)workspace;
    }
  }
  if (quant) return hip_status(csa2::launch_sparse_attn_quant(a, (hipStream_t)stream), "csa2_sparse_attn");
  return hip_status(csa2::launch_sparse_attn_f32(a, (hipStream_t)stream), "csa2_sparse_attn");
}

size_t csa2_sparse_attn_workspace_size(int32_t Q, int32_t H, int32_t k, int32_t window) {
  if (Q <= 0 || H < 16 || k < 0 || window < 0) return 0;
  const int ns = csa2::attn_splits(Q, H, k, window);
  if (ns <= 1) return 0;
  return (size_t)Q * (size_t)(H / 16) * (size_t)ns * csa2::ATTN_PART_FLOATS * sizeof(float);
}

int csa2_cache_write(const void* c, const void* z, int64_t cz_stride, const int32_t* tok_seq,
                     const int32_t* tok_pos, int32_t T, int32_t ratio, void* pend, int32_t B,
                     const float* kv_norm_w, const void* w_ik, const float* k_norm_w, float eps,
                     const float* rope_cs, int32_t n_rope, const csa2_rows* main_out,
                     const int64_t* main_base, int64_t main_rows, const csa2_rows* k_out,
                     const int64_t* k_base, int64_t k_rows, void* stream) {
  g_err[0] = 0;
  REQUIRE(c && kv_norm_w && rope_cs, CSA2_ERR_INVALID_ARG, "csa2_cache_write: null pointer argument");
  REQUIRE(T >= 0 && B >= 0 && n_rope >= 0 && main_rows >= 0 && k_rows >= 0, CSA2_ERR_INVALID_ARG,
          "csa2_cache_write: negative size");
  REQUIRE(T == 0 || (tok_seq && tok_pos), CSA2_ERR_INVALID_ARG, "csa2_cache_write: null token arrays");
  REQUIRE(ratio == 1 || ratio == 2, CSA2_ERR_UNSUPPORTED, "csa2_cache_write: ratio must be 1 or 2");
  REQUIRE(ratio == 1 || z, CSA2_ERR_INVALID_ARG, "csa2_cache_write: ratio 2 needs the gate rows z");
  REQUIRE(main_out || k_out, CSA2_ERR_INVALID_ARG, "csa2_cache_write: no output rows given");
  REQUIRE(eps >= 0.f && eps < INFINITY, CSA2_ERR_INVALID_ARG, "csa2_cache_write: eps must be finite and >= 0");
  REQUIRE(cz_stride >= 1024 && cz_stride % 16 == 0 && aligned(c, 16) && (!z || aligned(z, 16)),
          CSA2_ERR_INVALID_ARG, "csa2_cache_write: c and z rows must be 16-byte aligned with stride >= 1024 bytes");
  REQUIRE(aligned(kv_norm_w, 16) && aligned(rope_cs, 16), CSA2_ERR_INVALID_ARG,
          "csa2_cache_write: kv_norm_w and rope_cs must be 16-byte aligned");
  REQUIRE(!pend || aligned(pend, 16), CSA2_ERR_INVALID_ARG, "csa2_cache_write: pend must be 16-byte aligned");
  csa2::CacheWriteArgs a = {};
  a.c = (const uint16_t*)c;
  a.z = (const uint16_t*)z;
  a.cz_stride = cz_stride;
  a.tok_seq = tok_seq;
  a.tok_pos = tok_pos;
  a.T = T;
  a.ratio = ratio;
  a.pend = ratio == 2 ? (uint16_t*)pend : nullptr;
  a.B = B;
  a.kv_w = kv_norm_w;
  a.eps = eps;
  a.rope = rope_cs;
  a.n_rope = n_rope;
  if (main_out) {
    REQUIRE(main_base && main_out->data, CSA2_ERR_INVALID_ARG, "csa2_cache_write: main_out needs data and main_base");
    REQUIRE(aligned(main_out->data, 16) && main_out->row_stride % 16 == 0, CSA2_ERR_INVALID_ARG,
            "csa2_cache_write: main rows must be 16-byte aligned");
    a.main = (uint8_t*)main_out->data;
    a.main_stride = main_out->row_stride;
    a.main_base = main_base;
    a.main_rows = main_rows;
    switch (main_out->dtype) {
      case CSA2_F32:
        REQUIRE(main_out->row_stride >= 2048, CSA2_ERR_INVALID_ARG, "csa2_cache_write: F32 main rows below 2048 bytes");
        a.main_fmt = csa2::CW_F32;
        break;
      case CSA2_FP4_E2M1:
        REQUIRE(main_out->row_stride >= 256 && main_out->scale && aligned(main_out->scale, 4) &&
                    main_out->scale_stride >= 16,
                CSA2_ERR_INVALID_ARG, "csa2_cache_write: FP4 main rows need 256 code bytes and 16 fp32 scales");
        a.main_fmt = csa2::CW_FP4;
        a.main_scale = (uint8_t*)main_out->scale;
        a.main_scale_stride = main_out->scale_stride * 4;
        break;
      case CSA2_FP4_E2M1_E4M3S16:
        REQUIRE(main_out->row_stride >= 256 && main_out->scale && main_out->scale_stride >= 32, CSA2_ERR_INVALID_ARG,
                "csa2_cache_write: FP4 main rows need 256 code bytes and 32 E4M3 scale bytes");
        a.main_fmt = csa2::CW_S16;
        a.main_scale = (uint8_t*)main_out->scale;
        a.main_scale_stride = main_out->scale_stride;
        break;
      default:
        return fail(CSA2_ERR_UNSUPPORTED, "csa2_cache_write: main rows must be F32, FP4_E2M1 or FP4_E2M1_E4M3S16");
    }
  }
  if (k_out) {
    REQUIRE(k_base && k_out->data && w_ik && k_norm_w, CSA2_ERR_INVALID_ARG,
            "csa2_cache_write: k_out needs data, k_base, w_ik and k_norm_w");
    REQUIRE(aligned(w_ik, 16) && aligned(k_norm_w, 16), CSA2_ERR_INVALID_ARG,
            "csa2_cache_write: w_ik and k_norm_w must be 16-byte aligned");
    REQUIRE(aligned(k_out->data, 16) && k_out->row_stride % 16 == 0, CSA2_ERR_INVALID_ARG,
            "csa2_cache_write: index-key rows must be 16-byte aligned");
    a.w_ik = (const uint16_t*)w_ik;
    a.k_w = k_norm_w;
    a.kd = (uint8_t*)k_out->data;
    a.k_stride = k_out->row_stride;
    a.k_base = k_base;
    a.k_rows = k_rows;
    switch (k_out->dtype) {
      case CSA2_F32:
        REQUIRE(k_out->row_stride >= 512, CSA2_ERR_INVALID_ARG, "csa2_cache_write: F32 key rows below 512 bytes");
        a.k_fmt = csa2::CW_F32;
        break;
      case CSA2_FP8_E4M3:
        REQUIRE(k_out->row_stride >= 128 && k_out->scale && aligned(k_out->scale, 4) && k_out->scale_stride >= 1,
                CSA2_ERR_INVALID_ARG, "csa2_cache_write: FP8 key rows need 128 code bytes and one fp32 scale");
        a.k_fmt = csa2::CW_FP8;
        a.k_scale = (uint8_t*)k_out->scale;
        a.k_scale_stride = k_out->scale_stride * 4;
        break;
      case CSA2_FP4_E2M1_E4M3S16:
        REQUIRE(k_out->row_stride >= 64 && k_out->scale && k_out->scale_stride >= 8, CSA2_ERR_INVALID_ARG,
                "csa2_cache_write: FP4 key rows need 64 code bytes and 8 E4M3 scale bytes");
        a.k_fmt = csa2::CW_S16;
        a.k_scale = (uint8_t*)k_out->scale;
        a.k_scale_stride = k_out->scale_stride;
        break;
      default:
        return fail(CSA2_ERR_UNSUPPORTED, "csa2_cache_write: key rows must be F32, FP8_E4M3 or FP4_E2M1_E4M3S16");
    }
  }
  if (T == 0) return CSA2_OK;
  return hip_status(csa2::launch_cache_write(a, (hipStream_t)stream), "csa2_cache_write");
}

}  // extern "C"
