// Internal launch interface between the C-ABI layer (api.cpp) and the HIP
// kernels.  Every launcher enqueues on the given stream and returns the HIP
// status of the launch; argument validation happens before, in api.cpp.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

struct IndexScoreArgs {
  const uint8_t* q;          // FP8 codes or fp32 values, row (t*H + h)
  const float* q_scale;      // one per row (FP8), else null
  int64_t q_row_stride;      // bytes
  int64_t q_scale_stride;    // floats
  const void* w;             // [Q, H] gates
  int w_bf16;                // 1: bf16 gates, 0: fp32 gates
  const uint8_t* k;          // index-K rows
  const float* k_scale;      // FP8 keys: one fp32 scale per row
  int64_t k_row_stride;
  int64_t k_scale_stride;    // floats (FP8 keys) or bytes (FP4 keys)
  int k_fp4;                 // 1: E2M1 keys (64 B per row), one E4M3 scale byte per 16 dims at
                             //    (const uint8_t*)k_scale + row * k_scale_stride
  const int64_t* seq_base;
  const int32_t* q_seq;
  const int32_t* q_pos;
  int ratio;
  const int32_t* cand;       // null: dense
  int n_cand_blocks;
  int block_shift;
  float* scores;
  int64_t score_stride;
  int n_cols;
  float* block_max;          // optional fused block maxima (dense mode)
  int64_t block_max_stride;
  int sub_per_wg;            // 256-column sub-chunks streamed by one workgroup (sizes the grid at launch)
  int blocks_per_wg;         // query-tiled kernel: 256-key blocks streamed by one workgroup (set at launch)
  int Q;
  int H;
  int64_t k_scale_bytes;     // scale stride of a key row in bytes
  // paged keys: position p of sequence b is slot (page_table[b][p / 64], p % 64);
  // a slot's key and scale sit page * page_bytes + (p % 64) * stride into k and k_scale
  const int32_t* page_table; // null: flat rows from seq_base
  int64_t pt_stride;
  int n_pages;
  int64_t k_page_bytes;
  int64_t s_page_bytes;
};

constexpr int PAGE_SLOTS = 64;

// Physical page of position-page pi of sequence b, or -1 when it is missing
// (negative, past the table row or past the pool).
__device__ __forceinline__ int key_page(const IndexScoreArgs& a, int b, int pi) {
  const int pg = pi < a.pt_stride ? a.page_table[(int64_t)b * a.pt_stride + pi] : -1;
  return (pg >= 0 && pg < a.n_pages) ? pg : -1;
}

// Byte offsets of the key row and of its scale(s) for position pos (>= 0)
// of sequence b: rows from base, or (PAGED) slot pos % 64 of page pg (slot 0
// of page 0 when pg < 0).
template <bool PAGED>
__device__ __forceinline__ void key_offsets(const IndexScoreArgs& a, int64_t base, int pos, int pg,
                                            int64_t& ko, int64_t& so) {
  if (!PAGED) {
    const int64_t row = base + pos;
    ko = row * a.k_row_stride;
    so = row * a.k_scale_bytes;
    return;
  }
  const int o = pg < 0 ? 0 : (pos & (PAGE_SLOTS - 1));
  const int64_t p = pg < 0 ? 0 : pg;
  ko = p * a.k_page_bytes + (int64_t)o * a.k_row_stride;
  so = p * a.s_page_bytes + (int64_t)o * a.k_scale_bytes;
}

// Dense FP8 calls with at least this many queries use the query-tiled
// (prefill) kernel; smaller batches score each query on its own.
constexpr int PF_MIN_Q = 256;

hipError_t launch_index_scores_fp8(const IndexScoreArgs& a, hipStream_t s);
hipError_t launch_index_scores_f32(const IndexScoreArgs& a, hipStream_t s);
// Diagnostic: dense FP8 scores with the contraction on the FP8 matrix cores.
hipError_t launch_index_scores_fp8mma_diag(const IndexScoreArgs& a, hipStream_t s);

// Selection (top-k and block candidates) -------------------------------------
// SEL_BLOCKMAX ranks blocks with the latest visible one forced in (block
// candidates); SEL_BLOCKTOP ranks every block by its maximum; SEL_GATHER
// selects among the scores of the blocks a SEL_BLOCKTOP list names.
enum SelMode { SEL_DENSE = 0, SEL_POOL = 1, SEL_BLOCKMAX = 2, SEL_LIST = 3, SEL_GATHER = 4,
               SEL_BLOCKTOP = 5 };

constexpr int SEL_CAP = 32768;       // entries per chunk read from scores
constexpr int SEL_CAP_LIST = 16384;  // (key, position) pairs per chunk

struct SelectPlan {
  int n_stages;          // launches
  int chunk1;            // entries per chunk of the first stage
  int n_chunks1;
  int64_t list_len[8];   // length of the candidate list written by stage i
  int64_t ws_list_max;   // longest list (entries per row)
};

// rows_len: the longest row (entries; blocks for block candidates)
SelectPlan plan_select(int Q, int64_t rows_len, int k);
size_t select_workspace_bytes(int Q, int64_t rows_len, int k);

struct SelectArgs {
  const float* scores;
  int64_t score_stride;
  int n_cols;
  const float* block_max;    // block candidates: precomputed maxima, or null
  int64_t block_max_stride;
  const int32_t* q_pos;      // may be null (dense top-k: rows of n_cols)
  int ratio;
  const int32_t* cand;       // pool mode
  int n_cand_blocks;
  int block_shift;
  int k;
  int32_t* out_idx;          // [Q, k]
  void* workspace;
  int Q;
  // top-k output through a page table: position p of row t is written as
  // slot page_table[pt_seq[t]][p / 64] * 64 + p % 64 (-1 for a missing page)
  const int32_t* page_table;
  int64_t pt_stride;
  const int32_t* pt_seq;
};

hipError_t launch_select(int mode, const SelectArgs& a, int64_t rows_len, hipStream_t s);
// The allocation-free selection entry point's scratch: a static device array
// of SELECT_SCRATCH_BYTES per device; select_scratch() gives its address on
// the current device (looked up once per device).
constexpr size_t SELECT_SCRATCH_BYTES = (size_t)16 << 20;
hipError_t select_scratch(void** ptr);
// Top-k and block candidates of the same rows: the stages of both run
// paired in shared launches (their workspaces must not overlap).  With
// topk_via_blocks the top-k goes through the block maxima (topk_len is then
// the blocks per row, and topk.block_max the maxima).
hipError_t launch_topk_and_blocks(const SelectArgs& topk, int64_t topk_len, bool topk_via_blocks,
                                  const SelectArgs& blocks, int64_t blocks_len, hipStream_t s);
// Top-k through the block maxima: the k best blocks (ranked in the stages of
// an ordinary selection over the maxima), then the k best of their
// k * block_size scores in one chunk, so k * block_size is at most SEL_CAP;
// workspace: top_via_blocks_workspace_bytes.
bool top_via_blocks_supported(int k, int block_shift);
size_t top_via_blocks_workspace_bytes(int Q, int64_t n_blocks, int k);
hipError_t launch_topk_via_blocks(const SelectArgs& a, int64_t n_blocks, hipStream_t s);
// The k best blocks by maximum (top.k of them, none forced, block indices
// to top.out_idx) and the block candidates of the same n_rows maxima, in
// shared launches; separate workspaces.
hipError_t launch_top_blocks_and_blocks(const SelectArgs& top, const SelectArgs& blocks, int64_t n_rows,
                                        hipStream_t s);

// Sparse attention -----------------------------------------------------------
struct AttnArgs {
  const void* q;             // [Q, H, 512] bf16 or fp32
  const uint8_t* main;       // main-KV rows
  const float* main_scale;   // fp32 per 32 dims, or E4M3 bytes per 16 dims (main_s16)
  int64_t main_stride;       // bytes
  int64_t main_scale_stride; // floats, or bytes (main_s16)
  int main_s16;              // 1: the pages' 288-B record scales (E4M3, one per 16 dims)
  const int64_t* main_base;
  const int32_t* idx;
  int k;
  const uint8_t* swa;
  const float* swa_scale;
  int64_t swa_stride;
  int64_t swa_scale_stride;
  const int64_t* swa_base;
  const int32_t* swa_pos0;
  const int32_t* swa_lo;
  int window;
  const int32_t* q_seq;
  const int32_t* q_pos;
  int ratio;                 // visibility of idx entries
  const float* sink;
  float scale;               // softmax scale (natural-log units)
  void* out;
  int out_bf16;
  float* lse;
  int Q;
  int H;
  int n_split;               // key splits per (query, head group); 1 = no split
  float* part;               // [Q][H/16][n_split] partial records when n_split > 1
  int idx_slots;             // 1: idx holds physical main rows, bounded by n_main_rows
  int64_t n_main_rows;
  const float* rope;         // null, or [n_rope][64] cos / sin: the output's dims 448..511
  int n_rope;                //   are turned back by the query's position
};

// Partial record of one split: m[16] (log2 units), l[16], O[16][512], fp32.
constexpr int ATTN_PART_FLOATS = 16 + 16 + 16 * 512;
int attn_splits(int Q, int H, int k, int window);

hipError_t launch_sparse_attn_quant(const AttnArgs& a, hipStream_t s);
hipError_t launch_sparse_attn_f32(const AttnArgs& a, hipStream_t s);

// Full-layer cache write ------------------------------------------------------
enum CacheFmt { CW_F32 = 0, CW_FP4 = 1, CW_FP8 = 1, CW_S16 = 2 };

struct CacheWriteArgs {
  const uint16_t* c;         // bf16 token rows [T, 512]
  const uint16_t* z;         // bf16 gate rows (ratio 2)
  int64_t cz_stride;         // bytes
  const int32_t* tok_seq;
  const int32_t* tok_pos;
  int T;
  int ratio;
  uint16_t* pend;            // [B][2][512] bf16 (c row, z row), or null
  int B;
  const float* kv_w;         // [512] RMSNorm weight of the latent
  const uint16_t* w_ik;      // [128, 512] bf16
  const float* k_w;          // [128] RMSNorm weight of the index key
  float eps;
  const float* rope;         // [n_rope][64]: cos of the 32 frequencies, then sin
  int n_rope;
  uint8_t* main;             // main-KV rows (null: not written)
  uint8_t* main_scale;
  int64_t main_stride;       // bytes
  int64_t main_scale_stride; // bytes
  int main_fmt;              // CW_F32, CW_FP4 (fp32 scale per 32), CW_S16 (E4M3 per 16)
  const int64_t* main_base;
  int64_t main_rows;
  uint8_t* kd;               // index-key rows (null: not written)
  uint8_t* k_scale;
  int64_t k_stride;
  int64_t k_scale_stride;    // bytes
  int k_fmt;                 // CW_F32, CW_FP8 (fp32 scale per row), CW_S16
  const int64_t* k_base;
  int64_t k_rows;
};

hipError_t launch_cache_write(const CacheWriteArgs& a, hipStream_t s);

// Diagnostics ------------------------------------------------------------------
// Streaming read of bytes (a multiple of 16) from src by n_blocks workgroups.
hipError_t launch_stream_read(const void* src, size_t bytes, float* sink, int n_blocks, hipStream_t s);
// Fill of bytes (a multiple of 16) at dst with value by n_blocks workgroups.
hipError_t launch_stream_write(void* dst, size_t bytes, float value, int n_blocks, hipStream_t s);
// MFMA / VALU overlap loop (mode 1: products, 2: FMAs, 3: both); sink holds
// MV_BLOCKS * 512 floats.
constexpr int MV_BLOCKS = 256;
hipError_t launch_mfma_valu(int mode, int iters, float* sink, hipStream_t s);

}  // namespace csa2
