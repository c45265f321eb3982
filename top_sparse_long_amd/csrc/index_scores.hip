// Lightning-Indexer scoring for the CSA2 hot path on gfx950.
//
//   I[t, s] = sum_h w[t, h] * ReLU(q[t, h] . k[s])      (32 heads x 128 dims)
//
// (CSA2 page, "per-layer attention computation", item 4; DSA page,
// "Lightning Indexer".)  For FP8 rows the kernel follows the dataflow of the
// DSA page's "fp8 and scale absorption" section: the code products are exact,
// the q scale is folded into the gate, the ReLU-weighted head sum is taken,
// and the per-key scale multiplies the sum.
//
// Contraction: every E4M3 code is exactly representable in f16, so the codes
// are widened in registers (v_cvt_scalef32_pk_f16_fp8 with scale 1) and fed to
// v_mfma_f32_32x32x16_f16, whose 22-bit products are exact and whose sums
// carry fp32 precision.  The FP8 MFMA forms of gfx950 were measured to
// accumulate with about 17 significant bits, which on Gaussian data with the
// usual cancellation breaks a 1e-3 relative bound on the scores; the f16 form
// keeps the decode kernel HBM-bound all the same (8 f16 MFMAs of 32 cycles
// per 4 KB key tile per wave).
//
// Layout: A = q of one query (32 heads x 16 k), B = 32 keys (16 k x 32 keys);
// eight MFMAs cover d = 128.  Lane l owns row/column l % 32 and the 64
// contiguous bytes [64 * (l / 32), +64) of that 128-byte row (8 bytes per
// MFMA); both operands use the same assignment, so every product q[d] k[d]
// is summed exactly once.  The accumulator layout is the standard 32x32 one
// (accumulator j of lane l: head 8 (j / 4) + 4 (l / 32) + j % 4, key l % 32),
// so the ReLU-weighted head sum is 16 in-register FMAs plus one exchange with
// the lane 32 away.  Each wave requests the rows of its next sub-chunk
// before contracting the current one (a ring of IS_NBUF register buffers).
//
// Optional fused output: the block maximum of every block_size (<= 32)
// consecutive columns (the first step of the CSA2 page's candidate pool:
// "blocks are not compression"), taken over the scores in registers, or in
// LDS by a storing wave when only the maxima are written.
#include "kernels.h"

#include <algorithm>

namespace csa2 {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

#ifndef CSA2_IS_WAVES
#define CSA2_IS_WAVES 4
#endif
#ifndef CSA2_IS_TILES
#define CSA2_IS_TILES 2
#endif
constexpr int IS_WAVES = CSA2_IS_WAVES;                      // waves per workgroup
constexpr int IS_TILES = CSA2_IS_TILES;                      // 32-key tiles per wave per sub-chunk
// Dense calls of at most this many keys (queries x columns) use one tile per
// wave per sub-chunk: twice the workgroups, each lighter (measured: 128K x 8
// queries 33.4 against 34.4 us; neutral at 2M keys, slower at 16M).  Pool
// calls (candidate blocks, at most a decode batch x the pool) always do
// (64 x 16,384 candidate keys 36.2 -> 35.2 us, 8 x 16,384 9.0 -> 8.9).
#ifndef CSA2_IS_ONE_TILE
#define CSA2_IS_ONE_TILE (3 << 19)
#endif
constexpr int64_t IS_ONE_TILE_MAX_KEYS = CSA2_IS_ONE_TILE;
#ifndef CSA2_IS_RESIDENT
#define CSA2_IS_RESIDENT 768
#endif
constexpr int IS_RESIDENT_WGS = CSA2_IS_RESIDENT;            // about one round on 256 CUs
#ifndef CSA2_IS_RESIDENT_ONE
#define CSA2_IS_RESIDENT_ONE 1024
#endif
// the one-tile form of dense calls (lighter workgroups): measured on 128K x 8
// queries with scores, 768 -> 1024 workgroups 31.6 -> 30.9 us
constexpr int IS_RESIDENT_WGS_ONE = CSA2_IS_RESIDENT_ONE;
#ifndef CSA2_IS_NBUF
#define CSA2_IS_NBUF 2
#endif
// sub-chunk buffers per wave (measured on 64 x 256K keys: 2 buffers 469 us,
// 3 557 us, 4 555 us -- the extra registers cost occupancy)
constexpr int IS_NBUF = CSA2_IS_NBUF;
#ifndef CSA2_IS_UF
#define CSA2_IS_UF 4
#endif
// Calls that write only block maxima: sub-chunks per batch handed to the
// storing wave (measured on 64 x 256K keys: 2, 4 and 8 within 1 %)
constexpr int IS_UF = CSA2_IS_UF;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

__device__ __forceinline__ float load_gate(const IndexScoreArgs& a, int t, int h) {
  if (a.w_bf16) return bf16_to_f32(((const uint16_t*)a.w)[(int64_t)t * a.H + h]);
  return ((const float*)a.w)[(int64_t)t * a.H + h];
}

__device__ __forceinline__ int visible_count(int pos, int ratio) {
  return (int)(((int64_t)pos + 1) / ratio);
}

// Position (within the sequence) scored by column `col` of row t, or -1.
template <bool POOL>
__device__ __forceinline__ int column_position(const IndexScoreArgs& a, int t, int col, int nvis) {
  if (col >= a.n_cols) return -1;
  int p;
  if (POOL) {
    const int c = a.cand[(int64_t)t * a.n_cand_blocks + (col >> a.block_shift)];
    if (c < 0) return -1;
    p = (c << a.block_shift) | (col & ((1 << a.block_shift) - 1));
  } else {
    p = col;
  }
  return (p < nvis) ? p : -1;
}

// 8 E4M3 codes (two dwords) -> 8 f16 values, exactly.
__device__ __forceinline__ v8h fp8x8_to_f16(uint32_t lo, uint32_t hi) {
  const v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
  const v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
  const v2h c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
  const v2h d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
  return (v8h){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// 8 E2M1 codes (one dword, element 2i in the low nibble of byte i) times an
// E4M3 scale already widened to f16 -> 8 f16 values, exactly: a code has at
// most 2 significant bits and an E4M3 scale at most 4, so the product fits
// f16's 11 (and 6 * 448 is far inside its range).
__device__ __forceinline__ v8h fp4x8_to_f16(uint32_t x, _Float16 s) {
  const v2h s2 = {s, s};
  const v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 0) * s2;
  const v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 1) * s2;
  const v2h c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 2) * s2;
  const v2h d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 3) * s2;
  return (v8h){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// The 16-dim groups j = 0..3 of a lane's 64 dims as B operands: FP8 codes in
// raw[j] (16 bytes), or E2M1 codes in raw[j / 2][2 (j % 2)], raw[..][+1] with
// the E4M3 scales of the four groups in one dword.
template <bool K4>
__device__ __forceinline__ void key_operands(const v4u raw[4], uint32_t scales, int j, v8h& b0, v8h& b1) {
  if (K4) {
    const v2h s01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(scales, 1.0f, false);
    const v2h s23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(scales, 1.0f, true);
    const _Float16 sj = (j == 0) ? s01[0] : (j == 1) ? s01[1] : (j == 2) ? s23[0] : s23[1];
    b0 = fp4x8_to_f16(raw[j >> 1][2 * (j & 1)], sj);
    b1 = fp4x8_to_f16(raw[j >> 1][2 * (j & 1) + 1], sj);
  } else {
    b0 = fp8x8_to_f16(raw[j][0], raw[j][1]);
    b1 = fp8x8_to_f16(raw[j][2], raw[j][3]);
  }
}

// ReLU of a float as one integer max: non-negative floats are non-negative
// as int32, negative floats are negative (so they become +0).
__device__ __forceinline__ float relu(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// sum over a lane's 16 heads of gate * ReLU(score), in four independent
// chains: one chain of 16 dependent FMAs left the VALU waiting on every
// result
__device__ __forceinline__ float gated_relu_sum(const float (&gate)[16], const v16f& acc) {
  float p[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 16; ++j) p[j & 3] = fmaf(gate[j], relu(acc[j]), p[j & 3]);
  return (p[0] + p[1]) + (p[2] + p[3]);
}

// v + (the value of the lane 32 away), in every lane (gfx950 permlane swap:
// no LDS round trip).
__device__ __forceinline__ float add_half_swap(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Maximum over aligned groups of bs consecutive lanes (bs a power of two,
// at most 32), valid at the first lane of each group.  DPP moves within
// 16-lane rows; only bs = 32 crosses rows.
__device__ __forceinline__ float group_max(float m, int bs) {
#define CSA2_DPP(x, ctrl) __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), ctrl, 0xF, 0xF, false))
  if (bs > 1) m = fmaxf(m, CSA2_DPP(m, 0xB1));   // quad_perm [1,0,3,2]: lane ^ 1
  if (bs > 2) m = fmaxf(m, CSA2_DPP(m, 0x4E));   // quad_perm [2,3,0,1]: lane ^ 2
  if (bs > 4) m = fmaxf(m, CSA2_DPP(m, 0x12C));  // row_ror 12: lane + 4 (mod 16)
  if (bs > 8) m = fmaxf(m, CSA2_DPP(m, 0x128));  // row_ror 8: lane + 8 (mod 16)
#undef CSA2_DPP
  if (bs > 16) m = fmaxf(m, __shfl_xor(m, 16));
  return m;
}

// SC: the scores are written (otherwise only the block maxima: a call that
// re-scores the best blocks' keys instead of reading the scores back).
//
// Calls without scores (dense, block maxima only) add a fifth, storing
// wave: the four scoring waves hand each batch of IS_UF sub-chunks' scores
// over in LDS (one barrier per batch), and the storing wave writes the
// block maxima of whole sub-chunks, 16-32 consecutive values per store
// instead of 4 per tile and wave.  Measured on 64 x 256K keys: 399 -> 372
// us (stores removed altogether: 355 us).  With scores written (the
// smaller decode calls) the same hand-over measured slower (128K x 8
// queries 31.5 -> 33.7 us), so those waves store their own tiles.
template <bool POOL, bool W_BF16, bool K4, bool PAGED, int TILES, bool SC>
__global__ __launch_bounds__(64 * (SC ? IS_WAVES : IS_WAVES + 1)) void index_scores_fp8_kernel(IndexScoreArgs a) {
  constexpr int SUB = IS_WAVES * 32 * TILES;   // columns per sub-chunk
  constexpr bool SW = !SC;                     // a storing wave
  static_assert(!(POOL && SW), "pool calls always write their scores");
  __shared__ __attribute__((aligned(16))) float s_res[SW ? 2 : 1][SW ? IS_UF * SUB : 1];   // a batch's scores, by column
  const int t = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5;
  const int r = lane & 31;

  const int nvis = visible_count(a.q_pos[t], a.ratio);
  const int bseq = a.q_seq[t];
  const int64_t base = PAGED ? 0 : a.seq_base[bseq];
  // This workgroup's sub-chunks are blockIdx.x, blockIdx.x + gridDim.x, ...
  // of the row, so at any moment the workgroups of a query stream
  // neighbouring sub-chunks (measured about 4 % faster than contiguous runs).
  const int col_begin = blockIdx.x * SUB;
  const int col_end = a.n_cols;
  const int col_step = gridDim.x * SUB;
  float* out = SC ? a.scores + (int64_t)t * a.score_stride : nullptr;
  float* bm_row = (!POOL && a.block_max) ? a.block_max + (int64_t)t * a.block_max_stride : nullptr;
  // Dense mode: columns past the visible prefix only need -inf.
  const int limit = (nvis <= 0) ? 0 : (POOL ? a.n_cols : min(a.n_cols, nvis));

  // q (head r, bytes [64 half, +64)) and the gate of head r are loaded
  // first and used after the first key loads are issued, so one round trip
  // covers all of them.
  v4u qraw[4];
  {
    const v4u* qsrc = (const v4u*)(a.q + (int64_t)(t * 32 + r) * a.q_row_stride + 64 * half);
#pragma unroll
    for (int j = 0; j < 4; ++j) qraw[j] = qsrc[j];
  }
  float g_r;
  if (W_BF16)
    g_r = bf16_to_f32(((const uint16_t*)a.w)[(int64_t)t * 32 + r]);
  else
    g_r = ((const float*)a.w)[(int64_t)t * 32 + r];
  const float qs_r = a.q_scale[(int64_t)(t * 32 + r) * a.q_scale_stride];

  if (limit == 0) {
    // nothing visible: every column of this workgroup is -inf
    for (int c0 = col_begin; c0 < col_end; c0 += col_step)
      for (int c = c0 + threadIdx.x; c < min(col_end, c0 + SUB); c += blockDim.x) {
        if (SC) out[c] = -INFINITY;
        if (bm_row && (c & ((1 << a.block_shift) - 1)) == 0) bm_row[c >> a.block_shift] = -INFINITY;
      }
    return;
  }

  // start column n sub-chunks on, clamped to the row's end (no overflow)
  auto ahead = [&](int c, int n) { return (int)min((int64_t)c + (int64_t)n * col_step, (int64_t)col_end); };
  if (SW && wave == IS_WAVES) {
    // the storing wave: one barrier per batch, then the batch's block
    // maxima from LDS (vector memory operations complete in order per wave,
    // so no scoring wave's wait for key rows includes a store)
    for (int c0 = col_begin, it = 0; c0 < col_end; c0 += IS_UF * col_step, ++it) {
      __syncthreads();
      if (!bm_row) continue;
      const float* res = s_res[it & 1];
      const int sh = a.block_shift;
#pragma unroll
      for (int ph = 0; ph < IS_UF; ++ph) {
        const int sc0 = ahead(c0, ph);
        if (sc0 >= col_end) break;
        for (int j = lane; j < (SUB >> sh); j += 64) {
          const float* v = res + ph * SUB + (j << sh);
          float m = v[0];
          for (int e = 1; e < (1 << sh); ++e) m = fmaxf(m, v[e]);
          if (sc0 + (j << sh) < col_end) bm_row[(sc0 >> sh) + j] = m;
        }
      }
    }
    return;
  }

  // One sub-chunk = SUB columns; this wave's tiles in it are columns
  // sc0 + (i * IS_WAVES + wave) * 32 + [0, 32).  Every load is
  // unconditional: lanes whose column scores nothing read position 0 of the
  // sequence (visible, since limit > 0) and are masked afterwards.
  struct Sub {
    v4u raw[TILES][4];
    float ks[TILES];
    int pos[TILES];
  };
  // Pool calls: the candidate block of each lane's column is requested one
  // sub-chunk ahead of its rows (cq), so a sub-chunk's row addresses never
  // wait for a lookup issued in the same phase; the lookup is unconditional
  // (columns past the row read its last entry and are masked below).
  int cq[TILES];
  auto cand_load = [&](int sc0) {
    if (!POOL) return;
#pragma unroll
    for (int i = 0; i < TILES; ++i) {
      const int col = min(sc0 + (i * IS_WAVES + wave) * 32 + r, a.n_cols - 1);
      cq[i] = a.cand[(int64_t)t * a.n_cand_blocks + (col >> a.block_shift)];
    }
  };
  auto load_sub = [&](int sc0, Sub& S) {
#pragma unroll
    for (int i = 0; i < TILES; ++i) {
      const int tcol = sc0 + (i * IS_WAVES + wave) * 32;
      if (POOL) {
        const int col = tcol + r;
        const int p = (cq[i] << a.block_shift) | (col & ((1 << a.block_shift) - 1));
        S.pos[i] = (tcol < limit && col < a.n_cols && cq[i] >= 0 && p < nvis) ? p : -1;
      } else {
        S.pos[i] = (tcol < limit) ? column_position<POOL>(a, t, tcol + r, nvis) : -1;
      }
      int pg = 0;
      if (PAGED) {
        // dense: a 32-column tile lies in one 64-slot page (one scalar
        // lookup per tile); pool: each lane's position has its own page
        pg = POOL ? key_page(a, bseq, max(S.pos[i], 0) >> 6)
                  : key_page(a, bseq, __builtin_amdgcn_readfirstlane(tcol >> 6));
        if (pg < 0) S.pos[i] = -1;
      }
      int64_t ko, so;
      key_offsets<PAGED>(a, base, max(S.pos[i], 0), pg, ko, so);
      if (K4) {
        // 32 code bytes and the dword of the four E4M3 scales of this half
        const v4u* src = (const v4u*)(a.k + ko + 32 * half);
        S.raw[i][0] = src[0];
        S.raw[i][1] = src[1];
        S.ks[i] = __uint_as_float(*(const uint32_t*)((const uint8_t*)a.k_scale + so + 4 * half));
      } else {
        const v4u* src = (const v4u*)(a.k + ko + 64 * half);
#pragma unroll
        for (int j = 0; j < 4; ++j) S.raw[i][j] = src[j];
        S.ks[i] = *(const float*)((const uint8_t*)a.k_scale + so);
      }
    }
  };

  // The loads are unconditional: sub-chunks past the row's end read row 0
  // (every column there has position -1) and are never used.  A load under
  // a branch would make the wait before each contraction count for the
  // worst path, which is to say for the next sub-chunk's rows as well.
  Sub buf[IS_NBUF];
  cand_load(col_begin);
#pragma unroll
  for (int k = 0; k + 1 < IS_NBUF; ++k) {
    load_sub(ahead(col_begin, k), buf[k]);
    cand_load(ahead(col_begin, k + 1));
  }

  // A operand widened to f16; gate of head r with the q scale folded in,
  // then the 16 heads this lane's accumulators hold.
  v8h qa[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    qa[2 * j] = fp8x8_to_f16(qraw[j][0], qraw[j][1]);
    qa[2 * j + 1] = fp8x8_to_f16(qraw[j][2], qraw[j][3]);
  }
  g_r *= qs_r;
  float gate[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) gate[j] = __shfl(g_r, 8 * (j >> 2) + 4 * half + (j & 3));

  auto compute_sub = [&](int sc0, const Sub& S, float (&scs)[TILES]) {
#pragma unroll
    for (int i = 0; i < TILES; ++i) {
      const int tcol = sc0 + (i * IS_WAVES + wave) * 32;
      if (tcol >= col_end) break;
      const int col = tcol + r;
      float sc = -INFINITY;
      if (tcol < limit) {
        v16f acc = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v8h b0, b1;
          key_operands<K4>(S.raw[i], __float_as_uint(S.ks[i]), j, b0, b1);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(qa[2 * j], b0, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(qa[2 * j + 1], b1, acc, 0, 0, 0);
        }
        const float v = add_half_swap(gated_relu_sum(gate, acc));
        // FP8 keys: the per-key scale multiplies the head sum; FP4 keys
        // carry their scales inside the operands
        sc = (S.pos[i] >= 0) ? (K4 ? v : v * S.ks[i]) : -INFINITY;
      }
      scs[i] = sc;
      if (SW) continue;
      if (SC && half == 0 && col < a.n_cols) out[col] = sc;
      if (bm_row) {
        // maximum over aligned groups of block_size lanes (block_size <= 32)
        const float m = group_max(sc, 1 << a.block_shift);
        if (half == 0 && (r & ((1 << a.block_shift) - 1)) == 0 && col < a.n_cols) bm_row[col >> a.block_shift] = m;
      }
    }
  };

  // Stream over this workgroup's sub-chunks through a ring of IS_NBUF
  // buffers: the next IS_NBUF - 1 sub-chunks' rows are in flight while the
  // current one is contracted, so HBM stays busy for the whole life of the
  // workgroup.
  if (!SW) {
    for (int c0 = col_begin; c0 < col_end; c0 += IS_NBUF * col_step) {
#pragma unroll
      for (int ph = 0; ph < IS_NBUF; ++ph) {
        const int cc = c0 + ph * col_step;
        if (cc >= col_end) break;
        load_sub(ahead(cc, IS_NBUF - 1), buf[(ph + IS_NBUF - 1) % IS_NBUF]);
        cand_load(ahead(cc, IS_NBUF));
        float scs[TILES];
        compute_sub(cc, buf[ph], scs);
      }
    }
    return;
  }
  // with a storing wave: batches of IS_UF sub-chunks, their scores handed
  // over in LDS (the storing wave reads a batch's buffer while the next
  // batch fills the other)
  static_assert(IS_UF % IS_NBUF == 0, "a batch is a whole number of rings");
  for (int c0 = col_begin, it = 0; c0 < col_end; c0 += IS_UF * col_step, ++it) {
    float scb[IS_UF][TILES];
#pragma unroll
    for (int ph = 0; ph < IS_UF; ++ph)
#pragma unroll
      for (int i = 0; i < TILES; ++i) scb[ph][i] = -INFINITY;
#pragma unroll
    for (int ph = 0; ph < IS_UF; ++ph) {
      const int cc = c0 + ph * col_step;
      if (cc >= col_end) break;
      load_sub(ahead(cc, IS_NBUF - 1), buf[(ph + IS_NBUF - 1) % IS_NBUF]);
      compute_sub(cc, buf[ph % IS_NBUF], scb[ph]);
    }
    if (half == 0) {
#pragma unroll
      for (int ph = 0; ph < IS_UF; ++ph)
#pragma unroll
        for (int i = 0; i < TILES; ++i) s_res[it & 1][ph * SUB + (i * IS_WAVES + wave) * 32 + r] = scb[ph][i];
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Many queries over one sequence (a prefill chunk): keys are shared, so the
// contraction is a real matrix product and the kernel is MFMA-bound.
//
// One workgroup = 16 consecutive queries x a run of blocks_per_wg blocks of 256
// keys.  Each key block's E4M3 rows are widened to f16 once and staged in LDS
// (double-buffered: the next block's bytes are in registers while the current
// block is contracted); each of the 8 waves keeps the A operands of 2 queries
// (32 heads x 128 dims each) in registers, reads every B operand once from
// LDS and uses it for both queries.  Operand mapping and epilogue are those of
// the per-query kernel above.  Queries of the tile that belong to different
// sequences are handled in separate passes over the same key range.
constexpr int PF_Q = 16;                 // queries per workgroup
constexpr int PF_KB = 256;               // keys per staged block
constexpr int PF_WAVES = 8;
constexpr int PF_MIN_BLOCKS = 8;         // key blocks per workgroup, at least
constexpr int PF_TARGET_WGS = 256;       // about one long-lived workgroup per CU
constexpr int PF_RS = 272;               // LDS row stride of an f16 key row (bytes)

template <bool W_BF16, bool K4, bool PAGED>
__global__ __launch_bounds__(64 * PF_WAVES) void index_scores_prefill_kernel(IndexScoreArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t s_k[2][PF_KB * PF_RS];
  __shared__ float s_ks[2][PF_KB];
  // Each wave's scores of the current block for its two queries, stored to
  // memory (with their block maxima) at the start of the next block.  Stores
  // in the block loop would otherwise be outstanding when the next block's
  // staged rows are waited for (vector memory counters retire in order),
  // stalling every block on the latency of its last stores.  Wave-private.
  __shared__ __attribute__((aligned(16))) float s_out[PF_WAVES][2][PF_KB];

  const int t0 = blockIdx.y * PF_Q;
  const int blk0 = blockIdx.x * a.blocks_per_wg;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5;
  const int r = lane & 31;
  const int nq = min(PF_Q, a.Q - t0);
  const int n_blk = min(a.blocks_per_wg, (a.n_cols + PF_KB - 1) / PF_KB - blk0);

  // this wave's two queries
  int tq[2], nv[2], sq[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int qi = 2 * wave + i;
    tq[i] = t0 + qi;
    const bool live = qi < nq;
    nv[i] = live ? visible_count(a.q_pos[tq[i]], a.ratio) : 0;
    sq[i] = live ? a.q_seq[tq[i]] : -1;
  }

  // A operands (head r, bytes [64 half, +64) of the row) and gates
  v8h qa[2][8];
  float gate[2][16];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int tt = min(tq[i], a.Q - 1);
    const v4u* qsrc = (const v4u*)(a.q + (int64_t)(tt * 32 + r) * a.q_row_stride + 64 * half);
    v4u qraw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) qraw[j] = qsrc[j];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      qa[i][2 * j] = fp8x8_to_f16(qraw[j][0], qraw[j][1]);
      qa[i][2 * j + 1] = fp8x8_to_f16(qraw[j][2], qraw[j][3]);
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int h = 8 * (j >> 2) + 4 * half + (j & 3);
      const float wv = W_BF16 ? bf16_to_f32(((const uint16_t*)a.w)[(int64_t)tt * 32 + h])
                              : ((const float*)a.w)[(int64_t)tt * 32 + h];
      gate[i][j] = wv * a.q_scale[(int64_t)(tt * 32 + h) * a.q_scale_stride];
    }
  }

  // staging assignment: thread -> (key kk of the block, 64-byte half hh)
  const int kk = threadIdx.x >> 1;
  const int hh = threadIdx.x & 1;

  const int bshift = a.block_shift;
  const bool vec_out = ((uintptr_t)a.scores & 15) == 0 && (a.score_stride & 3) == 0;
  // store the staged block starting at column colb (lane: 4 consecutive
  // columns of each active query's row), then its block maxima, taken here
  // from the staged scores (lane: one block)
  auto flush = [&](int colb, bool act0, bool act1) {
    const int ncols = min(PF_KB, a.n_cols - colb);
    const int c = 4 * lane;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (!(i ? act1 : act0)) continue;
      const v4f v = *(const v4f*)&s_out[wave][i][c];
      if (a.scores) {
        float* dst = a.scores + (int64_t)tq[i] * a.score_stride + colb + c;
        if (vec_out && c + 4 <= ncols) {
          *(v4f*)dst = v;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (c + e < ncols) dst[e] = v[e];
        }
      }
      if (a.block_max) {
        const int bs = 1 << bshift;
        float* bm = a.block_max + (int64_t)tq[i] * a.block_max_stride;
        if (bs >= 4) {
          // the lane's 4 columns, then aligned groups of bs / 4 lanes
          float m = -INFINITY;
#pragma unroll
          for (int e = 0; e < 4; ++e) m = fmaxf(m, (c + e < ncols) ? v[e] : -INFINITY);
          m = group_max(m, bs >> 2);
          if ((lane & ((bs >> 2) - 1)) == 0 && c < ncols) bm[(colb + c) >> bshift] = m;
        } else {
          const int nb = (ncols + bs - 1) >> bshift;
          for (int bi = lane; bi < nb; bi += 64) {
            const int e_end = min(bs, ncols - bi * bs);
            float m = -INFINITY;
            for (int e = 0; e < e_end; ++e) m = fmaxf(m, s_out[wave][i][bi * bs + e]);
            bm[(colb >> bshift) + bi] = m;
          }
        }
      }
    }
  };

  for (int pass = 0; pass < nq; ++pass) {
    // one pass per distinct sequence among the tile's queries (in order of
    // first appearance); every value below is uniform across the workgroup
    const int b = a.q_seq[t0 + pass];
    bool seen = false;
    for (int j = 0; j < pass; ++j) seen |= (a.q_seq[t0 + j] == b);
    if (seen) continue;
    int maxvis = 0;
    for (int j = 0; j < nq; ++j)
      if (a.q_seq[t0 + j] == b) maxvis = max(maxvis, visible_count(a.q_pos[t0 + j], a.ratio));
    const int64_t base = PAGED ? 0 : a.seq_base[b];
    const bool act[2] = {sq[0] == b, sq[1] == b};

    // raw bytes of one block: key kk, bytes [64 hh, +64), and its scale
    v4u kraw[4];
    float kscale = 0.f;
    bool kok = true;   // false: the key's page is missing (its scale is staged as NaN)
    auto load_block = [&](int blk) {
      // rows past the last visible entry repeat it (masked later)
      const int col = min(blk * PF_KB + kk, max(maxvis - 1, 0));
      const int pg = PAGED ? key_page(a, b, col >> 6) : 0;
      kok = pg >= 0;
      int64_t ko, so;
      key_offsets<PAGED>(a, base, col, pg, ko, so);
      if (K4) {
        const v4u* src = (const v4u*)(a.k + ko + 32 * hh);
        kraw[0] = src[0];
        kraw[1] = src[1];
        kscale = __uint_as_float(*(const uint32_t*)((const uint8_t*)a.k_scale + so + 4 * hh));
      } else {
        const v4u* src = (const v4u*)(a.k + ko + 64 * hh);
#pragma unroll
        for (int j = 0; j < 4; ++j) kraw[j] = src[j];
        kscale = *(const float*)((const uint8_t*)a.k_scale + so);
      }
    };
    auto store_block = [&](int buf) {
      uint8_t* dst = s_k[buf] + kk * PF_RS + 128 * hh;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v8h b0, b1;
        key_operands<K4>(kraw, __float_as_uint(kscale), j, b0, b1);
        *(v8h*)(dst + 32 * j) = b0;
        *(v8h*)(dst + 32 * j + 16) = b1;
      }
      if (hh == 0) s_ks[buf][kk] = kok ? (K4 ? 1.0f : kscale) : __uint_as_float(0x7FC00000u);
    };

    if (maxvis > 0) {
      load_block(blk0);
      store_block(0);
    }
    __syncthreads();
    for (int j = 0; j < n_blk; ++j) {
      const int blk = blk0 + j;
      const int buf = j & 1;
      const int colb = blk * PF_KB;
      // the previous block's results go out before this block's loads
      if (j > 0) flush(colb - PF_KB, act[0], act[1]);
      // blocks wholly past the pass's furthest visible column are not staged
      const bool more = (j + 1 < n_blk) && (blk + 1) * PF_KB < maxvis;
      if (more) load_block(blk + 1);
      // B operands of the next tile are read from LDS while the current
      // tile's MFMAs and epilogue run; tiles past maxvis are not contracted
      // (causal skip), their columns are written -inf below
      const int n_col_tiles = min(PF_KB / 32, (a.n_cols - colb + 31) / 32);
      const int n_tiles = min(n_col_tiles, max(0, (maxvis - colb + 31) / 32));
      v8h kb[8];
      auto read_kb = [&](int tile) {
        const uint8_t* krow = s_k[buf] + (tile * 32 + r) * PF_RS + 128 * half;
#pragma unroll
        for (int m = 0; m < 8; ++m) kb[m] = *(const v8h*)(krow + 16 * m);
      };
      if (n_tiles > 0) read_kb(0);
#pragma unroll 1
      for (int tile = 0; tile < n_tiles; ++tile) {
        const int tcol = colb + tile * 32;
        const int col = tcol + r;
        const float ks = s_ks[buf][tile * 32 + r];
        // both queries' chains interleaved; columns a query does not see
        // (within the pass's visible range) are masked
        v16f acc[2] = {{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f},
                       {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(qa[0][m], kb[m], acc[0], 0, 0, 0);
          acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(qa[1][m], kb[m], acc[1], 0, 0, 0);
        }
        if (tile + 1 < n_tiles) read_kb(tile + 1);
        float sc[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const float v = add_half_swap(gated_relu_sum(gate[i], acc[i]));
          sc[i] = (act[i] && col < nv[i] && ks == ks) ? v * ks : -INFINITY;
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          if (!act[i]) continue;
          if (half == 0) s_out[wave][i][tile * 32 + r] = sc[i];
        }
      }
      for (int tile = n_tiles; tile < n_col_tiles; ++tile) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          if (!act[i]) continue;
          if (half == 0) s_out[wave][i][tile * 32 + r] = -INFINITY;
        }
      }
      if (more) store_block(buf ^ 1);
      __syncthreads();
    }
    if (n_blk > 0) flush((blk0 + n_blk - 1) * PF_KB, act[0], act[1]);
  }
}

// ---------------------------------------------------------------------------
// Diagnostic form, not on the hot path: the same dense scores with each
// query-key block of 32 heads x 32 keys contracted on the FP8 matrix cores
// (v_mfma_scale_f32_32x32x64_f8f6f4, unit E8M0 scales) straight from the E4M3
// codes, every other step as in the kernels above.  It exists to measure that
// instruction's accumulation against the score bound; the hot path widens
// the codes to f16 instead (exact) and accumulates in fp32.
typedef int v8i_t __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(64) void index_scores_fp8mma_diag_kernel(IndexScoreArgs a) {
  const int t = blockIdx.y;
  const int col0 = blockIdx.x * 32;
  const int lane = threadIdx.x;
  const int r = lane & 31, g = lane >> 5;
  const int nvis = visible_count(a.q_pos[t], a.ratio);
  const int64_t base = a.seq_base[a.q_seq[t]];
  const int col = col0 + r;
  const int kc = min(col, max(nvis - 1, 0));   // rows past the visible range repeat the last (masked)
  // A: head r, dims [64 s + 32 g, +32); B: key col0 + r, the same dims
  const uint8_t* qrow = a.q + (int64_t)(t * 32 + r) * a.q_row_stride;
  const uint8_t* krow = a.k + (base + kc) * a.k_row_stride;
  v16f acc = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    const v8i_t qa = *(const v8i_t*)(qrow + 64 * st + 32 * g);
    const v8i_t kb = *(const v8i_t*)(krow + 64 * st + 32 * g);
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa, kb, acc, 0, 0, 0, 127, 0, 127);
  }
  // lane (r, g) holds key col0 + r for heads 8 j + 4 g + i
  float v = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 8 * j + 4 * g + i;
      const float gw = load_gate(a, t, h) * a.q_scale[(int64_t)(t * 32 + h) * a.q_scale_stride];
      v = fmaf(gw, relu(acc[4 * j + i]), v);
    }
  v = add_half_swap(v);
  const float ks = *(const float*)((const uint8_t*)a.k_scale + (base + kc) * a.k_scale_bytes);
  if (g == 0 && col < a.n_cols) a.scores[(int64_t)t * a.score_stride + col] = (col < nvis) ? v * ks : -INFINITY;
}

hipError_t launch_index_scores_fp8mma_diag(const IndexScoreArgs& a, hipStream_t s) {
  dim3 grid((a.n_cols + 31) / 32, a.Q);
  hipLaunchKernelGGL(index_scores_fp8mma_diag_kernel, grid, dim3(64), 0, s, a);
  return hipGetLastError();
}

// fp32 rows: one thread per column, heads and dims in a plain loop.  Used for
// float inputs (exact for the small-integer configuration).
template <bool POOL>
__global__ __launch_bounds__(256) void index_scores_f32_kernel(IndexScoreArgs a) {
  __shared__ float sq[64 * 128];
  __shared__ float sw[64];
  const int t = blockIdx.y;
  const int H = a.H;
  for (int i = threadIdx.x; i < H * 128; i += 256) {
    const int h = i >> 7, d = i & 127;
    sq[i] = ((const float*)(a.q + (int64_t)(t * H + h) * a.q_row_stride))[d];
  }
  for (int h = threadIdx.x; h < H; h += 256) sw[h] = load_gate(a, t, h);
  __syncthreads();
  const int nvis = visible_count(a.q_pos[t], a.ratio);
  const int bseq = a.q_seq[t];
  const int64_t base = a.page_table ? 0 : a.seq_base[bseq];
  const int col = blockIdx.x * 256 + threadIdx.x;
  float* out = a.scores + (int64_t)t * a.score_stride;
  int p = column_position<POOL>(a, t, col, nvis);
  float tot = -INFINITY;
  int64_t ko = 0, so = 0;
  if (p >= 0) {
    if (a.page_table) {
      const int pg = key_page(a, bseq, p >> 6);
      if (pg < 0) p = -1;
      else key_offsets<true>(a, base, p, pg, ko, so);
    } else {
      key_offsets<false>(a, base, p, 0, ko, so);
    }
  }
  if (p >= 0) {
    const float* krow = (const float*)(a.k + ko);
    float kv[128];
#pragma unroll
    for (int d = 0; d < 128; d += 4) {
      const float4 x = *(const float4*)(krow + d);
      kv[d] = x.x; kv[d + 1] = x.y; kv[d + 2] = x.z; kv[d + 3] = x.w;
    }
    tot = 0.f;
    for (int h = 0; h < H; ++h) {
      float dot = 0.f;
#pragma unroll
      for (int d = 0; d < 128; ++d) dot = fmaf(sq[h * 128 + d], kv[d], dot);
      tot = fmaf(sw[h], fmaxf(dot, 0.f), tot);
    }
  }
  if (a.scores && col < a.n_cols) out[col] = tot;
  if (!POOL && a.block_max) {
    // 256 consecutive columns per workgroup: wave-level groups of block_size
    float m = tot;
    for (int sh = 1; sh < (1 << a.block_shift); sh <<= 1) m = fmaxf(m, __shfl_xor(m, sh));
    if ((threadIdx.x & ((1 << a.block_shift) - 1)) == 0 && col < a.n_cols)
      a.block_max[(int64_t)t * a.block_max_stride + (col >> a.block_shift)] = m;
  }
}

template <bool W_BF16, bool K4, bool PAGED>
static void launch_prefill(const IndexScoreArgs& a, hipStream_t s) {
  // Long-lived workgroups: the query tiles times the key blocks are dealt out
  // so that about PF_TARGET_WGS workgroups each stream a run of blocks (the
  // per-workgroup prologue -- q operands, gates, the first staged block -- is
  // paid once per run; measured on a 4,096 x 32K chunk: 8 blocks per
  // workgroup 1.15 ms, 32 blocks 1.01 ms, the whole row 0.98 ms).
  IndexScoreArgs b = a;
  const int64_t blocks = (a.n_cols + PF_KB - 1) / PF_KB;
  const int64_t qtiles = (a.Q + PF_Q - 1) / PF_Q;
  b.blocks_per_wg = (int)std::min<int64_t>(
      blocks, std::max<int64_t>(PF_MIN_BLOCKS, blocks * qtiles / PF_TARGET_WGS));
  dim3 grid((unsigned)((blocks + b.blocks_per_wg - 1) / b.blocks_per_wg), (unsigned)qtiles);
  hipLaunchKernelGGL((index_scores_prefill_kernel<W_BF16, K4, PAGED>), grid, dim3(64 * PF_WAVES), 0, s, b);
}

template <bool POOL, bool W_BF16, bool K4, bool PAGED, int TILES, bool SC>
static void launch_decode_t(const IndexScoreArgs& a, hipStream_t s) {
  // sub-chunks per workgroup: enough workgroups for about one resident
  // round, each striding over the sub-chunks of one query's row
  constexpr int SUB = IS_WAVES * 32 * TILES;
  IndexScoreArgs b = a;
  const int64_t subs = (a.n_cols + SUB - 1) / SUB;
  constexpr int64_t RES = (!POOL && TILES == 1) ? IS_RESIDENT_WGS_ONE : IS_RESIDENT_WGS;
  b.sub_per_wg = (int)std::max<int64_t>(1, (subs * a.Q + RES - 1) / RES);
  dim3 grid((unsigned)((subs + b.sub_per_wg - 1) / b.sub_per_wg), a.Q);
  hipLaunchKernelGGL((index_scores_fp8_kernel<POOL, W_BF16, K4, PAGED, TILES, SC>), grid,
                     dim3(64 * (SC ? IS_WAVES : IS_WAVES + 1)), 0, s, b);
}

template <bool POOL, bool W_BF16, bool K4, bool PAGED, bool SC>
static void launch_decode_sc(const IndexScoreArgs& a, hipStream_t s) {
  if (POOL || (int64_t)a.n_cols * a.Q <= IS_ONE_TILE_MAX_KEYS)
    launch_decode_t<POOL, W_BF16, K4, PAGED, 1, SC>(a, s);
  else
    launch_decode_t<POOL, W_BF16, K4, PAGED, IS_TILES, SC>(a, s);
}

template <bool POOL, bool W_BF16, bool K4, bool PAGED>
static void launch_decode(const IndexScoreArgs& a, hipStream_t s) {
  // pool calls always write their scores
  if constexpr (POOL) launch_decode_sc<POOL, W_BF16, K4, PAGED, true>(a, s);
  else if (a.scores) launch_decode_sc<POOL, W_BF16, K4, PAGED, true>(a, s);
  else launch_decode_sc<POOL, W_BF16, K4, PAGED, false>(a, s);
}

template <bool K4, bool PAGED>
static void launch_quant(const IndexScoreArgs& a, hipStream_t s) {
  if (!a.cand && a.Q >= PF_MIN_Q) {
    // many queries: the query-tiled kernel shares every staged key block
    if (a.w_bf16) launch_prefill<true, K4, PAGED>(a, s);
    else launch_prefill<false, K4, PAGED>(a, s);
  } else if (a.cand) {
    if (a.w_bf16) launch_decode<true, true, K4, PAGED>(a, s);
    else launch_decode<true, false, K4, PAGED>(a, s);
  } else {
    if (a.w_bf16) launch_decode<false, true, K4, PAGED>(a, s);
    else launch_decode<false, false, K4, PAGED>(a, s);
  }
}

hipError_t launch_index_scores_fp8(const IndexScoreArgs& a, hipStream_t s) {
  if (a.page_table) {
    if (a.k_fp4) launch_quant<true, true>(a, s);
    else launch_quant<false, true>(a, s);
  } else {
    if (a.k_fp4) launch_quant<true, false>(a, s);
    else launch_quant<false, false>(a, s);
  }
  return hipGetLastError();
}

hipError_t launch_index_scores_f32(const IndexScoreArgs& a, hipStream_t s) {
  dim3 grid((a.n_cols + 255) / 256, a.Q);
  if (a.cand)
    hipLaunchKernelGGL(index_scores_f32_kernel<true>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(index_scores_f32_kernel<false>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace csa2
