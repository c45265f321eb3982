// Top-k selection and block-candidate selection for the CSA2 hot path.
//
// Both calls choose, per row, the k best entries under the strict order
// (value descending, position ascending) among entries whose value is above
// -inf, and emit the chosen positions ascending, padded with -1 (DSA page,
// "Top-k: tokens, not blocks"; CSA2 page, "hierarchical sparse indexer" and
// "where attention is computed" for the block pool with the latest block
// forced).
//
// One workgroup of 1024 threads selects within a chunk of up to 32768
// entries, kept in registers as order-preserving 32-bit keys (entry
// j * 1024 + tid is thread tid's j-th key, so loads are coalesced):
//   1. load the chunk (dense scores, pool scores, block maxima of 8-score
//      blocks, or a (key, position) list from a previous stage);
//   2. if more than k entries are selectable, radix-select the k-th largest
//      key T with 8-bit digit passes over LDS histograms, stopping as soon as
//      the threshold bucket is taken whole;
//   3. move the keys to blocked ownership through LDS (thread tid holds
//      entries [EMAX tid, +EMAX)) and compact in position order with one
//      thread-level scan: every key > T, then the first (k - #greater) keys
//      equal to T, which applies the lower-position tie rule exactly.
// Long rows are cut into chunks; each chunk's k winners (already in position
// order) form a shorter list, and further stages select from the lists until
// one chunk holds the row.  A strict total order makes this exact: an entry
// among the row's k best is among its chunk's k best.
#include "kernels.h"

#include <algorithm>
#include <mutex>

namespace csa2 {

constexpr int SEL_THREADS = 1024;   // threads of a workgroup
// Stages over chunks of at most 4,096 entries with many workgroups run 256
// threads (16 entries each, as a 16,384-entry chunk has with 1,024): four
// waves per barrier instead of sixteen, and several workgroups per CU to hide
// each one's latency chains (the m = 2 chunk's block-route top-k: 118 ->
// 82 us).  Small grids keep 1,024 threads, whose shorter per-thread work
// is what sets their latency (the 8-query decode selections were 1-2 us
// slower with 256).
constexpr int SEL_SMALL_THREADS = 256;
constexpr int SEL_SMALL_MIN_WGS = 1024;   // grids at least this large use them
constexpr int SEL_BATCH = 8;               // loads in flight per thread
constexpr uint32_t KEY_NEG_INF = 0x007FFFFFu;  // key of -inf: selectable keys are larger
constexpr uint32_t KEY_POS_INF = 0xFF800000u;  // key of +inf (the forced latest block)
constexpr uint32_t KEY_PAD = 0u;               // padding in candidate lists

__device__ __forceinline__ uint32_t float_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct StageArgs {
  SelectArgs s;
  const uint32_t* in_key;
  const int32_t* in_pos;
  int64_t in_len;        // list length per row (LIST mode)
  int chunk;             // entries per chunk
  uint32_t* out_key;     // list output, [Q][out_stride]; null for the final stage
  int32_t* out_pos;
  int64_t out_stride;
};

// A selected position as written: itself, or its physical slot through the
// page table (-1 when its page is missing).
__device__ __forceinline__ int32_t out_slot(const SelectArgs& s, int t, int32_t pos) {
  if (!s.page_table || pos < 0) return pos;
  const int64_t pi = pos >> 6;
  const int32_t pg = pi < s.pt_stride ? s.page_table[(int64_t)s.pt_seq[t] * s.pt_stride + pi] : -1;
  return pg >= 0 ? pg * PAGE_SLOTS + (pos & (PAGE_SLOTS - 1)) : -1;
}

__device__ __forceinline__ int sel_visible(const SelectArgs& s, int t) {
  return (int)(((int64_t)s.q_pos[t] + 1) / s.ratio);
}

template <int MODE>
__device__ __forceinline__ int64_t row_length(const StageArgs& a, int t) {
  const SelectArgs& s = a.s;
  if (MODE == SEL_DENSE) return s.q_pos ? min(s.n_cols, sel_visible(s, t)) : s.n_cols;
  if (MODE == SEL_POOL) return s.n_cols;
  if (MODE == SEL_BLOCKMAX || MODE == SEL_BLOCKTOP) {
    const int n = min(s.n_cols, sel_visible(s, t));
    return n <= 0 ? 0 : ((n - 1) >> s.block_shift) + 1;
  }
  if (MODE == SEL_GATHER) return a.in_len << s.block_shift;
  return a.in_len;
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP (no LDS):
// Hillis-Steele within each row of 16 lanes, then row_bcast:15 carries row
// totals into rows 1 and 3 and row_bcast:31 carries the first half's total
// into rows 2 and 3.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x, int lane) {
  (void)lane;
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

__device__ __forceinline__ int lanes_below(uint64_t mask, int lane) {
  return __popcll(mask & ((1ull << lane) - 1ull));
}

// Block-wide exclusive scan of one value per thread (NT threads).
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t x, int lane, int wave,
                                                    uint32_t* s_wsum, uint32_t* total) {
  uint32_t incl = wave_incl_scan(x, lane);
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const uint32_t v = s_wsum[w];
    before += (w < wave) ? v : 0u;
    all += v;
  }
  *total = all;
  return before + incl - x;
}

// LDS bytes of one selection body of capacity CAP: the radix histogram
// shares its bytes with the transpose buffer (the two are never live at the
// same time), then the scan partials and the threshold words.
template <int CAP, int NT>
struct SelSmem {
  static constexpr int HIST = (256 * 16 + 256) * 4;
  static constexpr int TR = (CAP + 4 * NT) * 4;
  static constexpr int WSUM = 16 * 4;
  static constexpr int BODY = HIST > TR ? HIST : TR;
  static constexpr int BYTES = BODY + WSUM + 16;
};

template <int MODE, int CAP, int NT>
__device__ __forceinline__ void select_body(const StageArgs& a, int c, int t, uint8_t* smem) {
  constexpr int EMAX = CAP / NT;   // entries per thread at most
  constexpr int NAUX = (MODE == SEL_POOL || MODE == SEL_LIST || MODE == SEL_GATHER) ? EMAX : 1;
  // first digit: 16 interleaved copies of the 256-bin histogram (bin b,
  // copy c at 16 b + c), so lanes that hit the same bin land on 16 different
  // banks (scores share few top bytes); later digits: one copy after them.
  uint32_t* s_hist = (uint32_t*)smem;
  // transpose buffer: entry p of the chunk at p + 4 (p / EMAX), so that each
  // thread's EMAX consecutive entries start on a different bank group
  uint32_t* s_tr = (uint32_t*)smem;   // same bytes as s_hist
  uint32_t* s_wsum = (uint32_t*)(smem + SelSmem<CAP, NT>::BODY);
  uint32_t& s_bucket = *(uint32_t*)(smem + SelSmem<CAP, NT>::BODY + SelSmem<CAP, NT>::WSUM);
  uint32_t& s_above = (&s_bucket)[1];
  uint32_t& s_bcnt = (&s_bucket)[2];

  const SelectArgs& s = a.s;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  const int64_t L = row_length<MODE>(a, t);
  const int64_t g0 = (int64_t)c * a.chunk;
  const int count = (int)max((int64_t)0, min((int64_t)a.chunk, L - g0));
  const float* row = s.scores + (int64_t)t * s.score_stride;

  // Striped ownership: entry j * NT + tid of the chunk is this
  // thread's j-th key, so every load instruction reads consecutive addresses.
  // Loads are unconditional, from indices clamped into the chunk, and masked
  // afterwards, so they are all in flight together.
  uint32_t key[EMAX];
  int32_t aux[(MODE == SEL_POOL || MODE == SEL_LIST || MODE == SEL_GATHER) ? EMAX : 1];   // block id / position
  if (count > 0) {
    const int last = count - 1;
    if (MODE == SEL_DENSE || MODE == SEL_POOL) {
      float v[EMAX];
#pragma unroll
      for (int j = 0; j < EMAX; ++j) v[j] = row[g0 + min(j * NT + tid, last)];
      if (MODE == SEL_POOL) {
#pragma unroll
        for (int j = 0; j < EMAX; ++j) {
          const int64_t g = g0 + min(j * NT + tid, last);
          aux[j % NAUX] =
              s.cand[(int64_t)t * s.n_cand_blocks + (int)(g >> s.block_shift)];
        }
      }
#pragma unroll
      for (int j = 0; j < EMAX; ++j) {
        const bool in = j * NT + tid < count;
        uint32_t kk = in ? float_key(v[j]) : KEY_PAD;
        if (MODE == SEL_POOL && in && aux[j % NAUX] < 0)
          kk = KEY_NEG_INF;
        key[j] = kk;
      }
    } else if (MODE == SEL_LIST) {
      const uint32_t* ik = a.in_key + (int64_t)t * a.in_len + g0;
      const int32_t* ip = a.in_pos + (int64_t)t * a.in_len + g0;
#pragma unroll
      for (int j = 0; j < EMAX; ++j) {
        key[j] = ik[min(j * NT + tid, last)];
        aux[j % NAUX] = ip[min(j * NT + tid, last)];
      }
#pragma unroll
      for (int j = 0; j < EMAX; ++j)
        if (j * NT + tid >= count) key[j] = KEY_PAD;
    } else if (MODE == SEL_GATHER) {
      // entry e is score (block << shift) + (e % block_size) of list block
      // e / block_size (block -1: nothing); positions past the row or the
      // visible count are not selectable
      const int32_t* ib = a.in_pos + (int64_t)t * a.in_len;
      const int bs = 1 << s.block_shift;
      const int nv = min(s.n_cols, sel_visible(s, t));
      int32_t blk[EMAX];
#pragma unroll
      for (int j = 0; j < EMAX; ++j) blk[j] = ib[(g0 + min(j * NT + tid, last)) >> s.block_shift];
      float v[EMAX];
#pragma unroll
      for (int j = 0; j < EMAX; ++j) {
        const int e = (int)(g0 + min(j * NT + tid, last));
        const int p = blk[j] >= 0 ? (blk[j] << s.block_shift) + (e & (bs - 1)) : -1;
        aux[j] = (p >= 0 && p < nv) ? p : -1;
        v[j] = row[max(aux[j], 0)];
      }
#pragma unroll
      for (int j = 0; j < EMAX; ++j) {
        const bool in = j * NT + tid < count;
        key[j] = !in ? KEY_PAD : (aux[j] >= 0 ? float_key(v[j]) : KEY_NEG_INF);
      }
    } else {   // SEL_BLOCKMAX, SEL_BLOCKTOP
      // blocks before the last visible one are complete; the last one is
      // forced and never read (reads are clamped below it) -- unless every
      // block is ranked by its maximum (SEL_BLOCKTOP), when all are read
      constexpr bool FORCE = MODE == SEL_BLOCKMAX;
      const int64_t lim = FORCE ? ((L >= 2) ? L - 2 : 0) : max(L - 1, (int64_t)0);
      float m[EMAX];
      if (s.block_max) {
#pragma unroll
        for (int j = 0; j < EMAX; ++j)
          m[j] = s.block_max[(int64_t)t * s.block_max_stride + min(g0 + min(j * NT + tid, last), lim)];
      } else if (L >= (FORCE ? 2 : 1)) {
        const int bs = 1 << s.block_shift;
#pragma unroll
        for (int j = 0; j < EMAX; ++j) {
          const float* src = row + (min(g0 + min(j * NT + tid, last), lim) << s.block_shift);
          float mm = -INFINITY;
          if (bs >= 4) {
            for (int p = 0; p < bs; p += 4) {
              const float4 x = *(const float4*)(src + p);
              mm = fmaxf(mm, fmaxf(fmaxf(x.x, x.y), fmaxf(x.z, x.w)));
            }
          } else {
            for (int p = 0; p < bs; ++p) mm = fmaxf(mm, src[p]);
          }
          m[j] = mm;
        }
      } else {
#pragma unroll
        for (int j = 0; j < EMAX; ++j) m[j] = -INFINITY;
      }
#pragma unroll
      for (int j = 0; j < EMAX; ++j) {
        const int i = j * NT + tid;
        uint32_t kk = KEY_PAD;
        // the block of the latest visible position is always kept (unless
        // every block is ranked by its maximum)
        if (i < count) kk = (FORCE && g0 + i == L - 1) ? KEY_POS_INF : float_key(m[j]);
        key[j] = kk;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < EMAX; ++j) key[j] = KEY_PAD;
  }

  // Striped -> blocked ownership through LDS: thread tid now holds entries
  // [EMAX tid, EMAX tid + EMAX) of the chunk in key[0..EMAX), so position
  // order is (thread, j) and compaction needs one thread-level scan.
  {
#pragma unroll
    for (int j = 0; j < EMAX; ++j) {
      const int pe = j * NT + tid;
      s_tr[pe + 4 * (pe / EMAX)] = key[j];
    }
    __syncthreads();
    const uint32_t* src = s_tr + (EMAX + 4) * tid;
#pragma unroll
    for (int i = 0; i < EMAX / 4; ++i) {
      const uint4 v = *(const uint4*)(src + 4 * i);
      key[4 * i] = v.x;
      key[4 * i + 1] = v.y;
      key[4 * i + 2] = v.z;
      key[4 * i + 3] = v.w;
    }
    if (MODE == SEL_POOL || MODE == SEL_LIST || MODE == SEL_GATHER) {
      __syncthreads();
#pragma unroll
      for (int j = 0; j < EMAX; ++j) {
        const int pe = j * NT + tid;
        s_tr[pe + 4 * (pe / EMAX)] = (uint32_t)aux[j % NAUX];
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < EMAX / 4; ++i) {
        const uint4 v = *(const uint4*)(src + 4 * i);
        aux[(4 * i) % NAUX] = (int32_t)v.x;
        aux[(4 * i + 1) % NAUX] = (int32_t)v.y;
        aux[(4 * i + 2) % NAUX] = (int32_t)v.z;
        aux[(4 * i + 3) % NAUX] = (int32_t)v.w;
      }
    }
  }

  const int k = s.k;
  const uint32_t copy = (uint32_t)lane & 15u;

  // radix select of the k-th largest selectable key ---------------------------
  // Histograms count selectable keys only (above the -inf key), so the first
  // pass also yields their number; a chunk with at most k of them takes all.
  uint32_t T = KEY_NEG_INF, keq = 0;
  {
    // The first digit counts every selectable key into 16 interleaved
    // copies; later digits count only the keys inside the current prefix
    // (few, so the atomics are predicated) into one plain 256-bin copy,
    // which wave 0 reads and clears for the next pass.  A pass costs two
    // barriers: one after the counting atomics, one after wave 0 has found
    // the threshold bucket.  Lane l of wave 0 owns buckets 255 - l - 64 q
    // (q = 0..3): consecutive lanes read consecutive buckets, and bucket
    // order (highest first) is q-major, so four wave scans give the suffix
    // counts.
    uint32_t& s_all = (&s_bucket)[3];
    __syncthreads();   // the transposed entries have been read: s_tr becomes the histogram
    uint32_t* s_hist1 = s_hist + 256 * 16;
    for (int i = tid; i < 256 * 16 + 256; i += NT) s_hist[i] = 0;
    __syncthreads();
    uint32_t prefix = 0, mask = 0, krem = (uint32_t)k;
    for (int shift = 24; shift >= 0; shift -= 8) {
      if (shift == 24) {
#pragma unroll
        for (int j = 0; j < EMAX; ++j) {
          const uint32_t inc = (key[j] > KEY_NEG_INF) ? 1u : 0u;
          __hip_atomic_fetch_add(&s_hist[((key[j] >> 24) & 255u) * 16u + copy], inc,
                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
      } else {
#pragma unroll
        for (int j = 0; j < EMAX; ++j) {
          if (key[j] > KEY_NEG_INF && (key[j] & mask) == prefix)
            __hip_atomic_fetch_add(&s_hist1[(key[j] >> shift) & 255u], 1u,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
      }
      __syncthreads();
      if (wave == 0) {
        uint32_t cq[4];
        if (shift == 24) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint4* hb = (const uint4*)(s_hist + (255 - lane - 64 * q) * 16);
            uint32_t c4 = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const uint4 v = hb[i];
              c4 += v.x + v.y + v.z + v.w;
            }
            cq[q] = c4;
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint32_t* hb = s_hist1 + 255 - lane - 64 * q;
            cq[q] = *hb;
            *hb = 0u;
          }
        }
        uint32_t base = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t incl = wave_incl_scan(cq[q], lane);
          const uint32_t run = base + incl - cq[q];   // keys in higher buckets
          if (run < krem && run + cq[q] >= krem) {
            s_bucket = 255u - (uint32_t)(lane + 64 * q);
            s_above = run;
            s_bcnt = cq[q];
          }
          base += (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
        }
        if (lane == 0) s_all = base;
      }
      __syncthreads();
      if (shift == 24 && s_all <= (uint32_t)k) break;   // everything selectable is taken
      krem -= s_above;
      prefix |= s_bucket << shift;
      mask |= 255u << shift;
      if (s_bcnt == krem) {
        // the whole threshold bucket is taken: the k best are the keys >= prefix
        T = prefix - 1u;
        keq = 0;
        break;
      }
      if (shift == 0) {
        T = prefix;
        keq = krem;
      }
    }
  }

  // The output is staged in the (now free) transpose buffer -- positions at
  // [0, k), and for a list output the keys at [0, k) and positions at
  // [k, 2k) -- and written in order after one barrier: coalesced stores
  // instead of one sparsely active store instruction per held entry, and a
  // final top-k through a page table issues all of its lookups together.

  // order-preserving compaction ----------------------------------------------
  // Thread tid holds positions [EMAX tid, +EMAX) in order.  One block scan of
  // the packed per-thread counts (keys > T low half, keys == T high half)
  // gives every thread the number of earlier keys > T and == T; an entry's
  // output slot is (#earlier > T) + min(#earlier == T, keq), and a key == T
  // is taken only among the first keq of them in position order.
  const int my0 = EMAX * tid;   // first entry of this thread within the chunk
  uint32_t cg = 0, ce = 0;
#pragma unroll
  for (int j = 0; j < EMAX; ++j) {
    cg += (key[j] > T) ? 1u : 0u;
    ce += (key[j] == T && my0 + j < count) ? 1u : 0u;
  }
  uint32_t tot_packed;
  const uint32_t ex = block_excl_scan<NT>(cg | (ce << 16), lane, wave, s_wsum, &tot_packed);
  const uint32_t total = (tot_packed & 0xFFFFu) + min(tot_packed >> 16, keq);
  uint32_t rg = ex & 0xFFFFu, re = ex >> 16;
#pragma unroll
  for (int j = 0; j < EMAX; ++j) {
    const bool gt = key[j] > T;
    const bool eq = key[j] == T && my0 + j < count;
    if (gt || (eq && re < keq)) {
      const uint32_t o = rg + min(re, keq);
      const int64_t g = g0 + my0 + j;
      int32_t pos;
      if (MODE == SEL_DENSE || MODE == SEL_BLOCKMAX || MODE == SEL_BLOCKTOP) {
        pos = (int32_t)g;
      } else if (MODE == SEL_POOL) {
        pos = (aux[j % NAUX] << s.block_shift) |
              (int)(g & ((1 << s.block_shift) - 1));
      } else {   // SEL_LIST, SEL_GATHER
        pos = aux[j % NAUX];
      }
      if (a.out_key) {
        s_tr[o] = key[j];
        s_tr[k + o] = (uint32_t)pos;
      } else {
        s_tr[o] = (uint32_t)pos;
      }
    }
    rg += gt ? 1u : 0u;
    re += eq ? 1u : 0u;
  }
  // padding
  for (int q = (int)total + tid; q < k; q += NT) {
    if (a.out_key) {
      s_tr[q] = KEY_PAD;
      s_tr[k + q] = 0xFFFFFFFFu;
    } else {
      s_tr[q] = 0xFFFFFFFFu;
    }
  }
  __syncthreads();
  if (a.out_key) {
    const int64_t off = (int64_t)t * a.out_stride + (int64_t)c * k;
    for (int q = tid; q < k; q += NT) {
      a.out_key[off + q] = s_tr[q];
      a.out_pos[off + q] = (int32_t)s_tr[k + q];
    }
  } else if (s.page_table) {
    for (int q = tid; q < k; q += NT)
      s.out_idx[(int64_t)t * k + q] = out_slot(s, t, (int32_t)s_tr[q]);
  } else {
    for (int q = tid; q < k; q += NT) s.out_idx[(int64_t)t * k + q] = (int32_t)s_tr[q];
  }
}

template <int MODE, int CAP, int NT>
__global__ __launch_bounds__(NT) void select_kernel(StageArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[SelSmem<CAP, NT>::BYTES];
  select_body<MODE, CAP, NT>(a, blockIdx.x, blockIdx.y, smem);
}

// Two independent selections over the same queries in one launch (the
// columns of the grid before n1 run the first, the rest the second), with
// one LDS buffer sized for the larger of the two.
template <int M1, int C1, int M2, int C2>
__global__ __launch_bounds__(SEL_THREADS) void select_pair_kernel(StageArgs a1, StageArgs a2, int n1) {
  constexpr int NT = SEL_THREADS;
  constexpr int B1 = SelSmem<C1, NT>::BYTES, B2 = SelSmem<C2, NT>::BYTES;
  __shared__ __attribute__((aligned(16))) uint8_t smem[B1 > B2 ? B1 : B2];
  if ((int)blockIdx.x < n1)
    select_body<M1, C1, NT>(a1, blockIdx.x, blockIdx.y, smem);
  else
    select_body<M2, C2, NT>(a2, blockIdx.x - n1, blockIdx.y, smem);
}

// ---------------------------------------------------------------------------
// host-side planning

static int pow2_ceil(int64_t x) {
  int p = 1;
  while (p < x && p < (1 << 30)) p <<= 1;
  return p;
}

SelectPlan plan_select(int Q, int64_t rows_len, int k) {
  SelectPlan p = {};
  if (rows_len <= SEL_CAP) {
    p.n_stages = 1;
    p.chunk1 = SEL_CAP;
    p.n_chunks1 = 1;
    p.ws_list_max = 0;
    return p;
  }
  // first stage: enough workgroups to spread the row over the chip, and a
  // reduction of at least 4x per chunk
  int c1 = pow2_ceil((rows_len * (int64_t)Q + 255) / 256);
  c1 = max(c1, pow2_ceil(4 * (int64_t)k));
  c1 = min(c1, SEL_CAP);
  p.chunk1 = c1;
  p.n_chunks1 = (int)((rows_len + c1 - 1) / c1);
  int64_t len = (int64_t)p.n_chunks1 * k;
  int st = 0;
  p.list_len[st++] = len;
  p.ws_list_max = len;
  while (len > SEL_CAP_LIST && st < 7) {
    const int64_t nch = (len + SEL_CAP_LIST - 1) / SEL_CAP_LIST;
    len = nch * k;
    p.list_len[st++] = len;
  }
  p.n_stages = st + 1;
  return p;
}

// Scratch of the allocation-free entry point: the selection lists live in a
// file-scope device array instead of a caller workspace.  Host code never
// passes the array's name to a kernel (on the host it is a stand-in, not a
// device address): the address is looked up once per device with
// hipGetSymbolAddress, with that device current, and kept.  Every call on a
// device shares that device's array; the lists are written before they are
// read, so nothing needs clearing between calls.
static __device__ __align__(256) uint8_t scratch[SELECT_SCRATCH_BYTES];

hipError_t select_scratch(void** ptr) {
  constexpr int MAX_DEVICES = 64;
  static std::mutex mu;
  static void* addr[MAX_DEVICES] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

size_t select_workspace_bytes(int Q, int64_t rows_len, int k) {
  const SelectPlan p = plan_select(Q, rows_len, k);
  if (p.n_stages == 1) return 0;
  // two ping-pong lists of (key, position) pairs
  return (size_t)2 * (size_t)Q * (size_t)p.ws_list_max * 8u;
}

// smallest compiled capacity that holds n entries
static int fit_cap(int64_t n) {
  if (n <= 4096) return 4096;
  if (n <= 16384) return 16384;
  return SEL_CAP;
}

template <int MODE>
static hipError_t launch_stage(const StageArgs& a, int cap, int nchunks, int Q, hipStream_t s) {
  // the staged output (k positions, or k keys and k positions for a list)
  // must fit the transpose buffer of the capacity that runs: at least
  // CAP + 4 * threads entries (the planner keeps a list's chunk >= 4 k)
  const int64_t staged = a.out_key ? 2 * (int64_t)a.s.k : (int64_t)a.s.k;
  if (staged > (int64_t)(cap <= 4096 ? 4096 : cap) + 4 * SEL_SMALL_THREADS) return hipErrorInvalidValue;
  const dim3 grid(nchunks, Q), block(SEL_THREADS);
  if (cap <= 4096 && (int64_t)nchunks * Q >= SEL_SMALL_MIN_WGS)
    hipLaunchKernelGGL((select_kernel<MODE, 4096, SEL_SMALL_THREADS>), grid, dim3(SEL_SMALL_THREADS), 0, s, a);
  else if (cap <= 4096)
    hipLaunchKernelGGL((select_kernel<MODE, 4096, SEL_THREADS>), grid, block, 0, s, a);
  else if (MODE == SEL_LIST || cap <= 16384)   // list stages hold at most SEL_CAP_LIST
    hipLaunchKernelGGL((select_kernel<MODE, 16384, SEL_THREADS>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((select_kernel<MODE, (MODE == SEL_LIST ? 16384 : SEL_CAP), SEL_THREADS>), grid, block, 0,
                       s, a);
  return hipGetLastError();
}

// One launch of a selection: its mode, compiled capacity, chunk count and
// arguments.  The first stage reads the scores (or block maxima); list
// stages read the previous stage's (key, position) lists.
struct Stage {
  int mode;
  int cap;
  int nch;
  StageArgs a;
};
constexpr int SEL_MAX_STAGES = 8;

static int make_stages(int first_mode, const SelectArgs& sa, int64_t rows_len, Stage* st) {
  const SelectPlan p = plan_select(sa.Q, rows_len, sa.k);
  Stage& f = st[0];
  f = Stage{};
  f.mode = first_mode;
  f.a.s = sa;
  if (p.n_stages == 1) {
    f.cap = fit_cap(rows_len);
    f.a.chunk = f.cap;
    f.a.out_key = nullptr;
    f.nch = 1;
    return 1;
  }
  uint8_t* ws = (uint8_t*)sa.workspace;
  const size_t list_bytes = (size_t)sa.Q * (size_t)p.ws_list_max * 4u;
  uint32_t* key_buf[2] = {(uint32_t*)ws, (uint32_t*)(ws + 2 * list_bytes)};
  int32_t* pos_buf[2] = {(int32_t*)(ws + list_bytes), (int32_t*)(ws + 3 * list_bytes)};
  f.a.chunk = p.chunk1;
  f.a.out_key = key_buf[0];
  f.a.out_pos = pos_buf[0];
  f.a.out_stride = p.list_len[0];
  f.cap = fit_cap(p.chunk1);
  f.nch = p.n_chunks1;
  int cur = 0;
  for (int i = 1; i < p.n_stages; ++i) {
    Stage& b = st[i];
    b = Stage{};
    b.mode = SEL_LIST;
    b.a.s = sa;
    b.a.in_key = key_buf[cur];
    b.a.in_pos = pos_buf[cur];
    b.a.in_len = p.list_len[i - 1];
    if (i == p.n_stages - 1) {
      b.cap = min(fit_cap(b.a.in_len), SEL_CAP_LIST);
      b.a.chunk = fit_cap(b.a.in_len);
      b.a.out_key = nullptr;
      b.nch = 1;
    } else {
      b.cap = SEL_CAP_LIST;
      b.a.chunk = SEL_CAP_LIST;
      b.a.out_key = key_buf[cur ^ 1];
      b.a.out_pos = pos_buf[cur ^ 1];
      b.a.out_stride = p.list_len[i];
      b.nch = (int)((b.a.in_len + SEL_CAP_LIST - 1) / SEL_CAP_LIST);
    }
    cur ^= 1;
  }
  return p.n_stages;
}

static hipError_t launch_one(const Stage& st, int Q, hipStream_t s) {
  switch (st.mode) {
    case SEL_GATHER: return launch_stage<SEL_GATHER>(st.a, st.cap, st.nch, Q, s);
    case SEL_DENSE: return launch_stage<SEL_DENSE>(st.a, st.cap, st.nch, Q, s);
    case SEL_POOL: return launch_stage<SEL_POOL>(st.a, st.cap, st.nch, Q, s);
    case SEL_BLOCKMAX: return launch_stage<SEL_BLOCKMAX>(st.a, st.cap, st.nch, Q, s);
    case SEL_BLOCKTOP: return launch_stage<SEL_BLOCKTOP>(st.a, st.cap, st.nch, Q, s);
    default: return launch_stage<SEL_LIST>(st.a, st.cap, st.nch, Q, s);
  }
}

hipError_t launch_select(int mode, const SelectArgs& sa, int64_t rows_len, hipStream_t s) {
  Stage st[SEL_MAX_STAGES];
  const int n = make_stages(mode, sa, rows_len, st);
  for (int i = 0; i < n; ++i) {
    const hipError_t e = launch_one(st[i], sa.Q, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Top-k through the block maxima (exact).  Let T be the k-th best score of
// the row.  Every score above T lies in a block whose maximum is above T, and
// there are at most k - 1 such blocks, so all of them are among the k best
// blocks under (maximum desc, block asc).  The scores equal to T that the
// tie rule takes are the lowest-position ones; a block holding one has
// maximum >= T, and if its maximum equals T, every block of maximum T before
// it also holds a score T at a lower position, so it is among the first
// blocks of maximum T and is kept too.  Hence the k best scores are the k
// best among the k best blocks' scores.  The first stages rank the blocks
// (the latest block is not forced here) into a (key, block) list in block
// order; the last gathers each listed block's scores and selects from them,
// so the positions come out ascending.
bool top_via_blocks_supported(int k, int block_shift) {
  return ((int64_t)k << block_shift) <= SEL_CAP;
}

size_t top_via_blocks_workspace_bytes(int Q, int64_t n_blocks, int k) {
  return std::max(select_workspace_bytes(Q, n_blocks, k), (size_t)Q * (size_t)k * 8u);
}

// The stages of the top-k through block maxima: the ranking's stages, the
// last of them writing its k blocks as a (key, block) list (at the start of
// the workspace when it is the only stage, else into the ping-pong buffer it
// does not read), then the gather.  Returns the number of stages.
static int make_via_blocks_stages(const SelectArgs& sa, int64_t n_blocks, Stage* st) {
  SelectArgs sb = sa;
  sb.page_table = nullptr;   // the ranking lists blocks, not positions
  const int n = make_stages(SEL_BLOCKTOP, sb, n_blocks, st);
  uint8_t* ws = (uint8_t*)sa.workspace;
  uint8_t* list = ws;
  size_t list_bytes = (size_t)sa.Q * (size_t)sa.k * 4u;
  if (n > 1) {
    const SelectPlan p = plan_select(sa.Q, n_blocks, sa.k);
    list_bytes = (size_t)sa.Q * (size_t)p.ws_list_max * 4u;
    if ((const uint8_t*)st[n - 1].a.in_key == ws) list = ws + 2 * list_bytes;
  }
  Stage& last = st[n - 1];
  last.a.out_key = (uint32_t*)list;
  last.a.out_pos = (int32_t*)(list + list_bytes);
  last.a.out_stride = sa.k;
  Stage& g = st[n];
  const int64_t n2 = (int64_t)sa.k << sa.block_shift;
  g = Stage{};
  g.mode = SEL_GATHER;
  g.a.s = sa;
  g.a.in_key = last.a.out_key;
  g.a.in_pos = last.a.out_pos;
  g.a.in_len = sa.k;
  g.a.chunk = fit_cap(n2);
  g.cap = fit_cap(n2);
  g.nch = 1;
  g.a.out_key = nullptr;
  return n + 1;
}

hipError_t launch_topk_via_blocks(const SelectArgs& sa, int64_t n_blocks, hipStream_t s) {
  Stage st[SEL_MAX_STAGES + 1];
  const int n = make_via_blocks_stages(sa, n_blocks, st);
  for (int i = 0; i < n; ++i) {
    const hipError_t e = launch_one(st[i], sa.Q, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Paired launches: the first selection's stage in grid columns [0, n1), the
// second's after it.  The first side is the top-k (DENSE first, then LIST
// stages; or through block maxima: BLOCKTOP, LIST stages, GATHER), the
// second the block candidates (BLOCKMAX, then LIST).
template <int M1, int C1, int M2, int C2>
static void launch_pair_k(const Stage& x, const Stage& y, int Q, hipStream_t s) {
  const dim3 grid(x.nch + y.nch, Q), block(SEL_THREADS);
  hipLaunchKernelGGL((select_pair_kernel<M1, C1, M2, C2>), grid, block, 0, s, x.a, y.a, x.nch);
}

template <int M1, int C1, int M2>
static void pair_c2(const Stage& x, const Stage& y, int Q, hipStream_t s) {
  if (y.cap <= 4096) launch_pair_k<M1, C1, M2, 4096>(x, y, Q, s);
  else if (y.cap <= 16384 || M2 == SEL_LIST) launch_pair_k<M1, C1, M2, 16384>(x, y, Q, s);
  else launch_pair_k<M1, C1, M2, (M2 == SEL_LIST ? 16384 : SEL_CAP)>(x, y, Q, s);
}

template <int M1, int M2>
static void pair_c1(const Stage& x, const Stage& y, int Q, hipStream_t s) {
  if (x.cap <= 4096) pair_c2<M1, 4096, M2>(x, y, Q, s);
  else if (x.cap <= 16384 || M1 == SEL_LIST) pair_c2<M1, 16384, M2>(x, y, Q, s);
  else pair_c2<M1, (M1 == SEL_LIST ? 16384 : SEL_CAP), M2>(x, y, Q, s);
}

template <int M1>
static void pair_m2(const Stage& x, const Stage& y, int Q, hipStream_t s) {
  if (y.mode == SEL_LIST) pair_c1<M1, SEL_LIST>(x, y, Q, s);
  else pair_c1<M1, SEL_BLOCKMAX>(x, y, Q, s);
}

static hipError_t launch_pair(const Stage& x, const Stage& y, int Q, hipStream_t s) {
  switch (x.mode) {
    case SEL_DENSE: pair_m2<SEL_DENSE>(x, y, Q, s); break;
    case SEL_BLOCKTOP: pair_m2<SEL_BLOCKTOP>(x, y, Q, s); break;
    case SEL_GATHER: pair_m2<SEL_GATHER>(x, y, Q, s); break;
    default: pair_m2<SEL_LIST>(x, y, Q, s); break;
  }
  return hipGetLastError();
}

hipError_t launch_topk_and_blocks(const SelectArgs& topk, int64_t topk_len, bool topk_via_blocks,
                                  const SelectArgs& blocks, int64_t blocks_len, hipStream_t s) {
  Stage t[SEL_MAX_STAGES + 1], b[SEL_MAX_STAGES];
  const int nt = topk_via_blocks ? make_via_blocks_stages(topk, topk_len, t)
                                 : make_stages(SEL_DENSE, topk, topk_len, t);
  const int nb = make_stages(SEL_BLOCKMAX, blocks, blocks_len, b);
  // The dense route's stages are aligned at their ends, so the shorter
  // sequence runs beside the longer one's last stages (the final stages are
  // the single-workgroup-per-row ones that leave most of the chip idle).
  // Through block maxima both sequences open with a pass over the same
  // maxima, so they are aligned at their starts and the gather runs last.
  const int n = max(nt, nb);
  for (int j = 0; j < n; ++j) {
    const int it = topk_via_blocks ? j : j - (n - nt);
    const int ib = topk_via_blocks ? j : j - (n - nb);
    hipError_t e;
    const bool ht = it >= 0 && it < nt, hb = ib >= 0 && ib < nb;
    if (ht && hb) e = launch_pair(t[it], b[ib], topk.Q, s);
    else if (ht) e = launch_one(t[it], topk.Q, s);
    else e = launch_one(b[ib], topk.Q, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// The best blocks (SEL_BLOCKTOP, no block forced) and the block candidates
// (SEL_BLOCKMAX) of the same block maxima, in shared launches aligned at
// their starts; both final stages write block indices.
hipError_t launch_top_blocks_and_blocks(const SelectArgs& top, const SelectArgs& blocks, int64_t n_rows,
                                        hipStream_t s) {
  Stage t[SEL_MAX_STAGES], b[SEL_MAX_STAGES];
  const int nt = make_stages(SEL_BLOCKTOP, top, n_rows, t);
  const int nb = make_stages(SEL_BLOCKMAX, blocks, n_rows, b);
  for (int j = 0; j < max(nt, nb); ++j) {
    hipError_t e;
    if (j < nt && j < nb) e = launch_pair(t[j], b[j], top.Q, s);
    else if (j < nt) e = launch_one(t[j], top.Q, s);
    else e = launch_one(b[j], top.Q, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace csa2
