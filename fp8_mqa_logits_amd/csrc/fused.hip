// Fused FP8 MQA logits + per-row top-k without a logits matrix in HBM.
//
// Follows vLLM PR #60618, "What this PR does" (scoring, sampled gate,
// candidate emission, per-row selection, exact rescan, heaviest-first block
// claims) and the API page "fused_mqa_topk" (contract and output convention),
// laid out for gfx950 as ten launches on the caller's stream (eleven in the
// deterministic mode):
//   * prologue: heaviest-first order of the 32-row blocks, counters cleared
//     (one workgroup), and the FP8 score error bounds of every key and row
//     (the other workgroups);
//   * gate (persistent): per block, a strided sample of the keys gives each
//     row an admission threshold with a safe margin over its k-th key's
//     expected sample rank; rows with n <= k get their output here;
//   * refine (persistent, usually empty): rows whose threshold bin was
//     crowded have their sample binned again, finer;
//   * scan (persistent, 8 waves of 4 rows per workgroup): keys stream through
//     LDS in 128-key stages filled by direct global->LDS loads; each wave
//     scores its 4 rows with FP8 MFMAs (the rows' q and weights stay in
//     VGPRs) and appends the keys that reach a row's threshold to that row's
//     candidate slab (a ballot, an mbcnt and two buffer stores per row and
//     chunk, no atomics: a row belongs to one wave); a full slab is merged in
//     place (the best records and their ties stay, the threshold rises);
//   * select (one wave per row): every candidate's exact score lies within a
//     proven bound of its FP8 score (FP8 MFMA scores are approximate on
//     gfx950, see common.h); the keys whose interval can reach the row's k-th
//     score are rescored exactly (bf16 MFMA), the keys wholly above it are
//     taken, and the row is accepted only when no other key's interval, and
//     no key left out by the admission bound, can reach the k-th exact score;
//   * bounded rescan and finish, up to three rounds: a row that could not be
//     certified has every visible key scored exactly, in key slices spread
//     over all waves, against a lower bound of its k-th score, and its top k
//     selected from the keys above the bound (an overfull round raises the
//     bound for the next);
//   * exact (persistent): rows with fewer than k candidates, or whose
//     bounded rescan overfilled the slab in every round, are rescanned with
//     exact scores and a streaming top-k merge;
//   * sort (deterministic mode only): each row's keys in ascending order.
// Each phase is its own kernel so that each gets the registers it needs (the
// scan loop in particular holds no state of the other phases).
#include "common.h"
#include "launch.h"

namespace mqa {

constexpr int kWaves = kFusedWaves;
constexpr int kThreads = kWaves * kWave;
constexpr int kRowsPerWave = 4;
constexpr int kBlockRows = kWaves * kRowsPerWave;  // 32
static_assert(kBlockRows == kFusedBlockRows, "block rows");
constexpr int kGateBins = 512;
constexpr int kGateOff = 64;  // bins above the first-tile maximum
// A row's threshold bin that holds more sample keys than this and than the ks
// the threshold is placed at is binned again, finer (fused_refine_kernel).
constexpr int kGateCrowded = 48;
constexpr int kHistWords = 2048;
constexpr int kSelWaves = 4;        // rows (waves) per select workgroup
// The select's window around the estimated k-th FP8 score, in histogram bins
// beyond the one bin of binning slack on each side.
constexpr int kWinBins = 1;

// Header words (the first 12 mirror struct mqa_stats in mqa_topk.h).
enum : int {
  H_CLAIM = 0, H_SHORT = 1, H_GATED = 2, H_EXACT = 3, H_RESCAN = 4, H_UNDER = 5,
  H_COMPACT = 6, H_UNCERT = 7, H_CAND_LO = 8, H_CAND_HI = 9, H_BAND_LO = 10, H_BAND_HI = 11,
  H_ERRMAX = 12,  // largest |exact - FP8| / bound seen in a band (fp32 bits, >= 0)
  H_XQ = 16,      // blocks queued for the exact rescan
  H_XCLAIM = 17,  // exact-rescan claim counter
  H_GCLAIM = 18,  // gate claim counter
  H_RQ = 19,      // rows queued for the bounded rescan (then 21, 23 for rounds 1, 2)
  H_RCLAIM = 20,  // work-item claim counter of the bounded rescan (then 22, 24)
  H_FQ = 30,      // blocks queued for the gate's fine pass
  H_FCLAIM = 31,  // claim counter of the fine pass
  H_BQ = 32,      // rows queued for the exact block scan (two-level source calls)
  H_BCLAIM = 33,  // its claim counter
  // rows the select could not certify, by the first reason (statistics): too
  // many keys above the window or too few around it, a taken record's
  // interval reaching tau, a dropped record's reaching tau, the admission
  // bound reaching tau
  H_FAIL_COUNT = 26, H_FAIL_ABOVE = 27, H_FAIL_BELOW = 28, H_FAIL_ADMIT = 29
};

enum RowMode : int { M_OFF = 0, M_SHORT = 1, M_ALL = 2, M_GATED = 3, M_EXACT = 4 };

constexpr int kRescanKeys = 2048;  // keys per bounded-rescan work item
constexpr int kRescanRounds = 3;    // bounded-rescan rounds before the exact rescan

// Candidate capacity of a slab row (SMALL_CAP: just above k, to exercise the
// merges in tests).
__device__ __forceinline__ int slab_cap(const FusedParams& p) {
  return (p.flags & 4u) ? p.topk + 2 * kWave : kCap;
}

// Deterministic mode (MQA_FLAG_DETERMINISTIC): ties at a row's k-th exact
// score go to the smallest keys, certificates are strict, and each row's
// output is sorted by key.
__device__ __forceinline__ bool det_mode(const FusedParams& p) { return (p.flags & 64u) != 0u; }

// 64 index heads (p.hm == 2): the real row of virtual row v, whether v is a
// partner (the second 32 heads of its row), and the output row of v.
__device__ __forceinline__ int real_row(const FusedParams& p, int v) { return v >> (p.hm - 1); }
__device__ __forceinline__ bool partner_row(const FusedParams& p, int v) {
  return (v & (p.hm - 1)) != 0;
}
__device__ __forceinline__ int32_t* out_row(const FusedParams& p, int v) {
  return p.out + (int64_t)real_row(p, v) * p.topk;
}

// The FP8 error bound factor of lead row r: its own, or with 64 heads the
// sum of both halves' (each bounds its half's score), widened by 2^-8 for
// the fp32 addition of the two halves' scores.
__device__ __forceinline__ float beta_of(const FusedParams& p, int r) {
  return p.hm == 2 ? (p.beta[r] + p.beta[r + 1]) * (1.f + 0x1p-8f) : p.beta[r];
}

// Exact score of a chunk's keys (lane l: key l) for a row: one 32-head query,
// or the two halves' exact head sums added before the scale (64 heads). Every
// exact score of the path is computed this way, so equal keys score equal.
__device__ __forceinline__ float exact_score(const QueryRow& qr, const QueryRow* qr2,
                                             const KeyTile& kt, float sc) {
  float u = score_chunk_exact(qr, kt);
  if (qr2) u += score_chunk_exact(*qr2, kt);
  return u * sc;
}

__device__ __forceinline__ float exact_score(const QueryRowB& qb, const KeyTile& kt, float sc) {
  return score_chunk_exact(qb, kt) * sc;
}

// exact_score(qr, qr2, ...) from queries converted to bf16 once (the same
// bits: the halves' head sums added, then the scale)
__device__ __forceinline__ float exact_score(const QueryRowB& qb, const QueryRowB* qb2,
                                             const KeyTile& kt, float sc) {
  float u = score_chunk_exact(qb, kt);
  if (qb2) u += score_chunk_exact(*qb2, kt);
  return u * sc;
}

__device__ __forceinline__ void row_range(const FusedParams& p, int r, int& s, int& e) {
  int a = p.starts[real_row(p, r)], b = p.ends[real_row(p, r)];
  a = a < 0 ? 0 : (a > p.keys ? p.keys : a);
  b = b < a ? a : (b > p.keys ? p.keys : b);
  s = a;
  e = b;
}

// ---------------------------------------------------------------------------
// Key sources. The keys' e4m3 codes come from the gathered k array, from the
// paged indexer cache (vLLM PR #60618, "Motivation": 132 B per token, the
// 128-byte e4m3 key and its four-byte UE8M0 scale) through one page table for
// the call's key numbering, or, for decode-shaped calls, from the cache
// through one page-table row per request (the PR's review thread: the decode
// follow-up, many requests of a few query rows each). Every kernel that reads
// key bytes has an instance per source, so the gathered one compiles as if the
// others did not exist.
enum KeySrc : int { SRC_GATHER = 0, SRC_PAGED = 1, SRC_DECODE = 2 };

// 64-key chunks per LDS stage: one per packed request (up to four) in decode,
// else two.
template <int SRC>
constexpr int stage_chunks() {
  return SRC == SRC_DECODE ? 4 : 2;
}
template <int SRC>
constexpr int stage_keys() {
  return stage_chunks<SRC>() * kChunk;
}

__device__ __forceinline__ int clamp_page(const FusedParams& p, int pg) {
  return pg < 0 ? 0 : (pg >= p.num_pages ? p.num_pages - 1 : pg);
}

// The page-table entry of key `key` (in decode: position `key` of request
// `req`, its table row's entries clamped to the row).
template <int SRC>
__device__ __forceinline__ const int32_t* table_entry(const FusedParams& p, int key, int req) {
  if constexpr (SRC == SRC_DECODE) {
    int i = key >> p.page_shift;
    i = i < p.table_stride ? i : p.table_stride - 1;
    return p.table + (int64_t)req * p.table_stride + i;
  } else {
    return p.table + (key >> p.page_shift);
  }
}

// Row of key `key` in cache page `pg` (clamped into the cache).
__device__ __forceinline__ const uint8_t* page_row(const FusedParams& p, int pg, int key) {
  return p.k + (int64_t)clamp_page(p, pg) * p.page_bytes +
         (int64_t)(key & ((1 << p.page_shift) - 1)) * kDim;
}

template <int SRC>
__device__ __forceinline__ const uint8_t* key_row(const FusedParams& p, int key, int req = 0) {
  if constexpr (SRC == SRC_GATHER) {
    return p.k + (int64_t)key * kDim;
  } else {
    return page_row(p, *table_entry<SRC>(p, key, req), key);
  }
}

// UE8M0 decode (API page "fused_mqa_topk", fused_mqa_topk_key_scales): the
// low byte e of a scale word is the fp32 with bit pattern e << 23 (e = 0
// gives +0.0).
__device__ __forceinline__ float ue8m0(uint32_t w) { return __uint_as_float((w & 0xFFu) << 23); }

// The scale word of key `key` of cache page `pg`.
__device__ __forceinline__ const uint32_t* page_scale(const FusedParams& p, int pg, int key) {
  const int P = 1 << p.page_shift;
  return reinterpret_cast<const uint32_t*>(p.k + (int64_t)clamp_page(p, pg) * p.page_bytes +
                                           (int64_t)P * kDim + 4 * (int64_t)(key & (P - 1)));
}

// The decoded scale of key `key` read from its source (the prologue's view;
// the other kernels of the gathered and paged sources read the prologue's
// copy in keyinfo).
template <int SRC>
__device__ __forceinline__ float key_scale(const FusedParams& p, int key, int req = 0) {
  if constexpr (SRC == SRC_GATHER) {
    return p.scales[key];
  } else {
    return ue8m0(*page_scale(p, *table_entry<SRC>(p, key, req), key));
  }
}

// The scale of key `key` as the scan scored it: the prologue's keyinfo copy,
// or in decode (no keyinfo) straight from the cache.
template <int SRC>
__device__ __forceinline__ float scan_scale(const FusedParams& p, int key, int req) {
  if constexpr (SRC == SRC_DECODE) {
    return key_scale<SRC>(p, key, req);
  } else {
    return p.keyinfo[2 * (int64_t)key];
  }
}

// B operands of up to 64 arbitrary keys (lane l: key keyidx[t] of sub-tile t,
// bytes 32 * (l / 16) ..), from any source (decode: of request req).
template <int SRC>
__device__ __forceinline__ void load_keys_rows(KeyTile& kt, const FusedParams& p,
                                               const int* keyidx, int req = 0) {
  if constexpr (SRC == SRC_GATHER) {
    load_keys_gather(kt, p.k, keyidx);
  } else {
    const int g = lane_id() >> 4;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint8_t* r = key_row<SRC>(p, keyidx[t], req) + 32 * g;
      const uint4 x0 = *reinterpret_cast<const uint4*>(r);
      const uint4 x1 = *reinterpret_cast<const uint4*>(r + 16);
      kt.kb[t] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                     (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
    }
  }
}

// Decode blocks. A request's rows are split into parts of up to 8 rows
// (dec_parts = ceil(R / 8) parts of R rows); a block packs kDecPack = 4 parts
// (of one or several requests), each owning 8 row slots, two waves. Slot j of
// block b holds row 8 (part % dec_parts) + j % 8 of request part / dec_parts,
// part = 4 b + j / 8; p.rows marks an empty slot. Otherwise slot j of block b
// is row 32 b + j.
constexpr int kDecPack = 4;
constexpr int kDecSlots = kFusedBlockRows / kDecPack;  // 8

template <int SRC>
__device__ __forceinline__ int slot_row(const FusedParams& p, int b, int slot) {
  if constexpr (SRC == SRC_DECODE) {
    const int part = b * kDecPack + slot / kDecSlots;
    const int q = part / p.dec_parts;
    const int j = (part - q * p.dec_parts) * kDecSlots + slot % kDecSlots;
    return (j < p.dec_rows && q < p.nreq) ? q * p.dec_rows + j : p.rows;
  } else {
    return b * kFusedBlockRows + slot;
  }
}

// The block of row r (either layout).
__device__ __forceinline__ int block_of(const FusedParams& p, int r) {
  if (!p.dec_rows) return r / kFusedBlockRows;
  const int q = r / p.dec_rows;
  return (q * p.dec_parts + (r - q * p.dec_rows) / kDecSlots) / kDecPack;
}

// The part (0 .. 3) of its block whose rows a wave holds in decode.
template <int SRC>
__device__ __forceinline__ int wave_group(int w) {
  if constexpr (SRC == SRC_DECODE) {
    return w / (kFusedWaves / kDecPack);
  } else {
    return 0;
  }
}

// Score of the wave's 4 rows for a 64-key chunk, one row after the other
// (fewer registers than score4's overlap of consecutive rows; for decode,
// whose scan waits on its key copies more than on its MFMAs).
__device__ __forceinline__ void score4_serial(float E[4], const QueryRow* qr, const FoldOp& fo,
                                              const KeyTile& kt, float sc) {
  FoldTerms f;
  RowAcc a;
  fold_terms(f, fo, kt);
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    mfma_row(a, qr[i], kt);
    E[i] = reduce_heads_abs(qr[i], a, f, i) * sc;
  }
}

// ---------------------------------------------------------------------------
// FP8 score error bounds.
//
// The FP8 MFMA (16x16x128; measured on gfx950) splits a 128-term dot product
// into 16 groups of 8 consecutive dimensions. In each group it truncates every
// product toward zero to a multiple of 2^(E - 13), E being the largest
// exponent sum e(a) + e(b) over the group's nonzero products (e: the unbiased
// exponent of an e4m3 code, -6 for subnormals), and it adds the 16 group sums
// one after another in fp32, each addition within one ulp. The product that
// sets E is exact, so a group loses less than
// 7 * 2^(E - 13) <= 7 * 2^-13 * max_d x(a_d) * max_d x(b_d), with x(v) =
// 2^e(v) for v != 0 and x(0) = 0, and the additions lose at most 2^-19 of the
// dot's sum of |products|. Summed over heads (with |w|), groups, and the relu
// fold's terms, the FP8 score of key j in row r is within beta_r * nhat_j of
// its exact score, where
//   nhat_j  = scale_j * sum_g max_{d in g} x(k_jd), rounded up to 12 bits;
//   beta_r  = 2^-13 * (4.5 alpha + 3.5 phi + 2 fmax) * (1 + 2^-10);
//   alpha   = max_g sum_h |w_rh| * max_{d in g} x(q_rhd);
//   fmax    = max_d |f_rd|, f_r = sum_h w_rh q_rh (the fold vector);
//   phi     = the power of two at or below 1.0625 * fmax.
// The head MFMAs' truncation contributes 3.5 alpha (the relu fold halves
// every term) and their fp32 additions 0.25 alpha; the fold-term MFMAs
// 3.5 phi plus 0.4 fmax; the fold's four-term residual and the fp32 rounding
// of f 1.0 fmax + 0.25 alpha; the fp32 epilogue and the record arithmetic
// 0.15 alpha + 0.1 fmax (|q_d| < 2 x(q_d), sum_d |k_d| < 16 sum_g max x).

// x(v) of the largest e4m3 magnitude among the 8 codes of (lo, hi): x is
// nondecreasing in the code's magnitude bits, so it is x of their maximum.
__device__ __forceinline__ float xhat8(uint32_t lo, uint32_t hi) {
  uint32_t m = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const uint32_t c0 = (lo >> (8 * b)) & 0x7Fu, c1 = (hi >> (8 * b)) & 0x7Fu;
    m = c0 > m ? c0 : m;
    m = c1 > m ? c1 : m;
  }
  if (m == 0) return 0.f;
  const uint32_t f = m >> 3;  // exponent field; 0 for subnormals (exponent -6 as field 1)
  return __uint_as_float(((f > 1u ? f : 1u) + 120u) << 23);
}

__device__ __forceinline__ float row_beta(float alpha, float fmax) {
  const float fm = fmax * 1.0625f * (1.f + 0x1p-12f);
  const uint32_t ex = __float_as_uint(fm) & 0x7F800000u;
  const float phi = ex ? __uint_as_float(ex) : fm;  // fm itself when subnormal
  return 0x1p-13f * (4.5f * alpha + 3.5f * phi + 2.f * fmax) * (1.f + 0x1p-10f);
}

// nhat of a key from its unscaled group-maximum sum x (exact: a sum of 16
// powers of two) and its scale: rounded up, and kept to its top 12 bits.
__device__ __forceinline__ float key_nhat(float x, float scale) {
  float v = x * scale;  // a power-of-two scale: exact unless tiny
  if (v == 0.f) return 0.f;
  v = v < 0x1p-100f ? 0x1p-100f : v;
  return __uint_as_float((__float_as_uint(v) + 0xFFFFFu) & ~kKeyMask);
}

// Workgroup 0: heaviest-first block order and the reset of the header and of
// the per-block flags. A block's cost is the union range its non-short rows
// scan (one thread per row, LDS min/max per block); blocks are counting-sorted
// by cost in 1024 buckets of 1024 keys, descending.
// Workgroups 1..: nhat of every key (4 keys per wave) and beta of every row (a
// wave per row).
constexpr int kMaxBlocks = kMaxBatchRows / kBlockRows;
constexpr int kPrologueThreads = 1024;

template <int SRC>
__device__ __forceinline__ void prologue_bounds(const FusedParams& p) {
  const int l = lane_id();
  const int nwaves = (gridDim.x - 1) * (kPrologueThreads / kWave);
  // (decode keeps no keyinfo: its scan bounds each key from the key itself)
  const int kunits = SRC == SRC_DECODE ? 0 : (p.keys + 3) / 4;
  const int units = kunits + p.rows;
  for (int u = (blockIdx.x - 1) * (kPrologueThreads / kWave) + wave_id(); u < units;
       u += nwaves) {
    const int g = l & 15;  // dimension group: dims 8g .. 8g + 7
    if (u < kunits) {
      const int key = 4 * u + (l >> 4);
      float x = 0.f;
      if (key < p.keys) {
        const uint2 v = *reinterpret_cast<const uint2*>(key_row<SRC>(p, key) + 8 * g);
        x = xhat8(v.x, v.y);
        // paged prefill: the keys are also compacted into the workspace,
        // where the later kernels read them as gathered keys
        if constexpr (SRC == SRC_PAGED)
          *reinterpret_cast<uint2*>(p.kc + (int64_t)key * kDim + 8 * g) = v;
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) x += __shfl_xor(x, o, 64);
      if (g == 0 && key < p.keys) {
        const float sc = key_scale<SRC>(p, key);
        *reinterpret_cast<float2*>(p.keyinfo + 2 * (int64_t)key) = float2{sc, key_nhat(x, sc)};
      }
    } else {
      // lane (g, quarter): heads quarter, quarter + 4, ... of dim group g
      const int64_t r = u - kunits;
      const int hq = l >> 4;
      float a = 0.f;
      float f[8];
#pragma unroll
      for (int d = 0; d < 8; ++d) f[d] = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int h = hq + 4 * i;
        const float w = p.weights[r * kHeads + h];
        const uint2 v = *reinterpret_cast<const uint2*>(p.q + (r * kHeads + h) * kDim + 8 * g);
        a = __builtin_fmaf(__builtin_fabsf(w), xhat8(v.x, v.y), a);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          f[b] = __builtin_fmaf(w, e4m3_to_f32((int)v.x, b), f[b]);
          f[4 + b] = __builtin_fmaf(w, e4m3_to_f32((int)v.y, b), f[4 + b]);
        }
      }
      a += __shfl_xor(a, 16, 64);
      a += __shfl_xor(a, 32, 64);
      float fm = 0.f;
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        float t = f[d] + __shfl_xor(f[d], 16, 64);
        t += __shfl_xor(t, 32, 64);
        fm = __builtin_fmaxf(fm, __builtin_fabsf(t));
      }
      const float alpha = wave_max(a);
      const float fmax = wave_max(fm);
      if (l == 0) p.beta[r] = row_beta(alpha, fmax);
    }
  }
}

template <int SRC>
__global__ __launch_bounds__(kPrologueThreads) void fused_prologue_kernel(FusedParams p) {
  __shared__ int cnt[1024];
  __shared__ int off[1024];
  __shared__ int blo[kMaxBlocks], bhi[kMaxBlocks];
  if (blockIdx.x > 0) {
    prologue_bounds<SRC>(p);
    return;
  }
  const int tid = threadIdx.x;
  cnt[tid] = 0;
  if (tid < 64) p.header[tid] = 0;
  for (int b = tid; b < p.nblocks; b += 1024) {
    p.xflag[b] = 0;
    p.fflag[b] = 0;
    blo[b] = p.keys;
    bhi[b] = 0;
  }
  __syncthreads();
#pragma unroll 4
  for (int r = tid; r < p.rows; r += 1024) {
    int s, e;
    row_range(p, r, s, e);
    if (e - s > p.topk) {
      atomicMin(&blo[block_of(p, r)], s);
      atomicMax(&bhi[block_of(p, r)], e);
    }
  }
  __syncthreads();
  for (int b = tid; b < p.nblocks; b += 1024) {
    const int c = (bhi[b] > blo[b] ? bhi[b] - blo[b] : 0) >> 10;
    bhi[b] = c > 1023 ? 1023 : c;  // bucket
    atomicAdd(&cnt[bhi[b]], 1);
  }
  __syncthreads();
  // off[c] = number of blocks in buckets above c: a suffix sum over the 1024
  // buckets (thread t holds bucket 1023 - t; wave scans, then the 16 wave
  // totals)
  {
    const int v = cnt[1023 - tid];
    const int incl = wave_incl_scan(v);
    if (lane_id() == kWave - 1) off[tid >> 6] = incl;  // wave totals (off[0..15] reused below)
    __syncthreads();
    int before = 0;
    for (int i = 0; i < (tid >> 6); ++i) before += off[i];
    __syncthreads();
    off[1023 - tid] = before + incl - v;
  }
  __syncthreads();
  for (int b = tid; b < p.nblocks; b += 1024) p.order[atomicAdd(&off[bhi[b]], 1)] = b;
}

struct RowState {
  int r;        // row id
  int s, e;     // clamped visible range
  int mode;     // RowMode
  float thr;    // admission threshold
  int strict;   // admit score > thr (1) or >= thr (0)
  int cnt;      // records appended to the slab
  float beta;   // the row's FP8 error bound factor (0: not scored)
};

// Rows of block b owned by the calling wave (modes off, thresholds open).
template <int SRC>
__device__ __forceinline__ void wave_rows(const FusedParams& p, int b, RowState* rs) {
  const int w = wave_id();
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    RowState& r = rs[i];
    r.r = slot_row<SRC>(p, b, w * kRowsPerWave + i);
    r.cnt = 0;
    r.strict = 0;
    r.thr = -__builtin_inff();
    r.mode = M_OFF;
    r.beta = 0.f;
    r.s = r.e = 0;
    if (r.r < p.rows) row_range(p, r.r, r.s, r.e);
  }
}

// 64 heads: the partner slots (odd) of the wave carry the second 32 heads of
// the lead rows before them; for every lead row in `mode` (or M_ALL with
// M_GATED), load the partner's query (weights times wscale, as the lead's)
// and take it into the fold (frows, when given).
__device__ __forceinline__ void load_partners(const FusedParams& p, const RowState* rs,
                                              QueryRow* qr, int* frows, int mode,
                                              float wscale) {
  if (p.hm != 2) return;
#pragma unroll
  for (int i = 1; i < kRowsPerWave; i += 2) {
    const int m = rs[i - 1].mode;
    if (m == mode || (mode == M_GATED && m == M_ALL)) {
      load_query(qr[i], p.q, p.weights, rs[i].r, wscale);
      if (frows) frows[i] = rs[i].r;
    }
  }
}

// 64 heads: a lead row's score is its slot's plus its partner's.
__device__ __forceinline__ void combine_halves(const FusedParams& p, float* E) {
  if (p.hm == 2) {
    E[0] += E[1];
    E[2] += E[3];
  }
}

// A row's error bound factor as a wave-uniform (scalar) value: in the scan
// loop it is an SGPR operand of the admission FMA, not one of the VGPRs.
__device__ __forceinline__ float row_beta_of(const FusedParams& p, int r) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(beta_of(p, r))));
}

__device__ __forceinline__ void zero_query(QueryRow& qr) {
  qr.qa[0] = qr.qa[1] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int v = 0; v < 8; ++v) qr.w[v] = 0.f;
}

// The union range of the live rows over the workgroup's waves (wlo/whi: this
// wave's) and the OR of a per-wave flag. All threads call it.
__device__ __forceinline__ void block_union(int* wlo_s, int* whi_s, int* wf_s, int wlo, int whi,
                                            int flag, int keys, int& lo, int& hi, int& any) {
  const int w = wave_id();
  if (lane_id() == 0) {
    wlo_s[w] = wlo;
    whi_s[w] = whi;
    wf_s[w] = flag;
  }
  __syncthreads();
  lo = keys;
  hi = 0;
  any = 0;
  for (int i = 0; i < kWaves; ++i) {
    lo = wlo_s[i] < lo ? wlo_s[i] : lo;
    hi = whi_s[i] > hi ? whi_s[i] : hi;
    any |= wf_s[i];
  }
  __syncthreads();
}

// Keys move through LDS in stages of kStageChunks 64-key chunks, copied by
// direct global->LDS loads into two stage buffers. Each kernel declares the
// buffers as separate __shared__ arrays so that the compiler can tell the one
// being filled from the one being read (and does not wait for the copy in
// flight before reading the other).

// A stage's per-key floats: the scales, then (stage-keys floats further, so
// that one LDS address serves both reads) the error bound factors nhat; in
// decode only the raw scale words. The paged and decode sources also keep the
// page of each stage key (pg), copied one stage ahead so that a stage's key
// copies never wait for a page-table read.
struct Stages {
  uint8_t* k[2];
  float* s[2];
  int32_t* pg[2];
};

#define MQA_DECLARE_STAGES(name, SRC)                                                 \
  __shared__ __align__(16) uint8_t name##_k0[stage_chunks<SRC>() * kChunkBytes];     \
  __shared__ __align__(16) uint8_t name##_k1[stage_chunks<SRC>() * kChunkBytes];     \
  __shared__ __align__(16) float name##_s0[2 * stage_keys<SRC>()];                    \
  __shared__ __align__(16) float name##_s1[2 * stage_keys<SRC>()];                    \
  __shared__ __align__(16) int32_t name##_p0[SRC == SRC_GATHER ? 4 : stage_keys<SRC>()]; \
  __shared__ __align__(16) int32_t name##_p1[SRC == SRC_GATHER ? 4 : stage_keys<SRC>()]; \
  const Stages name = {{name##_k0, name##_k1}, {name##_s0, name##_s1}, {name##_p0, name##_p1}}

// Smallest float above a finite x: "score > x" is "score >= next_up(x)".
__device__ __forceinline__ float next_up(float x) {
  if (x == 0.f) return __int_as_float(1);
  const int b = __float_as_int(x);
  return __int_as_float(b > 0 ? b + 1 : b - 1);
}

// The row's admission test as one ">=" threshold. NaN admits nothing: not
// even a +inf or NaN score, which a key outside every row's range may have
// (the unused slots of a paged cache's last page hold arbitrary bytes).
__device__ __forceinline__ float admit_thr(const RowState& r, bool live) {
  if (!live) return __builtin_nanf("");
  return r.strict ? next_up(r.thr) : r.thr;
}

// The calling wave's 4 slab rows of block b, its merge buffers and its LDS
// histogram. Slab row r (a row id) holds kSlabRow (score, key) records in two
// arrays; the scan appends with buffer stores through one raw buffer that
// spans the wave's score rows through its key rows (the host keeps the
// distance between the two arrays below 2^31 bytes).
struct SlabRefs {
  float* sE0;                  // score slab row of the wave's row 0 (row i at + i * kSlabRow)
  int32_t* sI0;                // key slab row of the wave's row 0
  __amdgpu_buffer_rsrc_t buf;  // 4-byte records from sE0 through the end of the wave's key rows
  int delta;                   // byte distance from the score rows to the key rows
  uint32_t* hist;
  int cap;   // a row merges once it holds more records than this
  int keep;  // records a merge keeps (ties of the last one aside)
  __device__ float* sE(int i) const { return sE0 + i * kSlabRow; }
  __device__ int32_t* sI(int i) const { return sI0 + i * kSlabRow; }
};

// seg >= 0: key segment seg of a split scan (p.nseg > 1), whose records go to
// records [seg * R, (seg + 1) * R) of each slab row, R = kSlabRow / nseg, with
// a capacity of R - 64 (one more chunk fits past it); seg < 0: the whole row.
// Slab row i of the wave is row0 + i: the wave's rows are consecutive row
// ids (in decode, rows of one request; its empty slots never write).
template <int SRC>
__device__ __forceinline__ SlabRefs slab_refs(const FusedParams& p, int b, uint32_t* hist,
                                              int keep, int seg = -1) {
  SlabRefs sr;
  int r0 = slot_row<SRC>(p, b, wave_id() * kRowsPerWave);
  r0 = r0 < p.rows ? r0 : 0;
  const int64_t row0 = r0;
  const int region = kSlabRow / p.nseg;
  const int64_t off = seg > 0 ? (int64_t)seg * region : 0;
  sr.sE0 = p.slabE + row0 * kSlabRow + off;
  sr.sI0 = p.slabI + row0 * kSlabRow + off;
  sr.delta = (int)(reinterpret_cast<const char*>(p.slabI) - reinterpret_cast<const char*>(p.slabE));
  sr.buf = __builtin_amdgcn_make_buffer_rsrc(sr.sE0, 4, sr.delta / 4 + kRowsPerWave * kSlabRow,
                                             kBufferFlags);
  sr.hist = hist;
  sr.cap = slab_cap(p);
  if (seg >= 0 && p.nseg > 1) {
    // SMALL_CAP: a segment's part of the row merges past topk / (2 nseg) + 64
    // records (segments of i.i.d. rows hold about topk / nseg candidates)
    const int c = (p.flags & 4u) ? p.topk / (2 * p.nseg) + kWave : region - kWave;
    sr.cap = c < region - kWave ? c : region - kWave;
  }
  sr.keep = keep < sr.cap - kWave ? keep : sr.cap - kWave;
  return sr;
}

// This wave's merge buffers (persistent workgroup blockIdx.x).
__device__ __forceinline__ float* tmp_e(const FusedParams& p) {
  return p.tmpE + ((int64_t)blockIdx.x * kWaves + wave_id()) * kTmp;
}
__device__ __forceinline__ int32_t* tmp_i(const FusedParams& p) {
  return p.tmpI + ((int64_t)blockIdx.x * kWaves + wave_id()) * kTmp;
}

// Append the passing lanes of one chunk to slab row i of the wave: score and
// key at the same record offset of the score and key rows (buffer stores
// whose lane offset, record (i * kSlabRow + cnt + rank) of the wave's rows,
// comes from one mbcnt). A slab row has room for one more chunk past `cap`;
// a row that went past `cap` is merged down once the whole chunk is scored
// (merge_rows).
__device__ __forceinline__ void emit_rec(RowState& rs, float E, float th, bool valid, int key,
                                         const SlabRefs& sr, int i) {
  const bool pass = valid && E >= th;
  const uint64_t m = __ballot(pass);
  if (pass) {
    const int pos = (int)__builtin_amdgcn_mbcnt_hi(
        (uint32_t)(m >> 32),
        __builtin_amdgcn_mbcnt_lo((uint32_t)m, (uint32_t)(rs.cnt + i * kSlabRow)));
    struct_buffer_store_b32(__float_as_uint(E), sr.buf, pos, 0, 0, 0);
    struct_buffer_store_b32((uint32_t)key, sr.buf, pos, 0, sr.delta, 0);
  }
  rs.cnt += __popcll(m);
}

__device__ __forceinline__ void finish_row(RowState& r, float E, float th, int key, int key0,
                                           const SlabRefs& sr, int i) {
  const bool full = r.s <= key0 && key0 + kChunk <= r.e;
  const bool valid = full || (key >= r.s && key < r.e);
  emit_rec(r, E, th, valid, key, sr, i);
}

// Streaming top-k merge: every row whose slab went past `cap` is cut down to
// its `keep` best records, widened by the records tied with the keep-th best
// while they fit in `room`; the admission threshold rises to a score that
// every dropped record is at most (later records must beat it strictly):
// the best dropped score when every tie stayed, so that rows of heavily tied
// scores keep a gap between the threshold and their k-th score, else the
// keep-th best score. One merge site for the wave's rows, so the select code
// appears once in the scan loop.
// The gated scan records the new threshold in the row's RowInfo at once
// (the row state keeps only the admission bound th).
template <bool EXACT>
__device__ __forceinline__ void merge_rows(const FusedParams& p, RowState* rs, const SlabRefs& sr,
                                           float* th) {
  unsigned todo = 0;
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) todo |= (rs[i].cnt > sr.cap ? 1u : 0u) << i;
  while (todo) {
    const int i = __builtin_ctz(todo);
    todo &= todo - 1;
    float* sE = sr.sE(i);
    int32_t* sI = sr.sI(i);
    float* tE = tmp_e(p);
    int32_t* tI = tmp_i(p);
    int cnt = rs[0].cnt;
#pragma unroll
    for (int j = 1; j < kRowsPerWave; ++j)
      if (i == j) cnt = rs[j].cnt;
    // the ties may fill half the room above `keep` (and the merge buffers)
    const int half = (sr.cap + sr.keep) >> 1;
    float bound;
    const int kept = wave_select_ties(sE, sI, cnt, sr.keep, half < kTmp ? half : kTmp, sr.hist, bound,
                                      [&](int slot, float e, int idx) {
                                        tE[slot] = e;
                                        tI[slot] = idx;
                                      });
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    for (int t = lane_id(); t < kept; t += kWave) {
      sE[t] = tE[t];
      sI[t] = tI[t];
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
#pragma unroll
    for (int j = 0; j < kRowsPerWave; ++j)
      if (i == j) {
        rs[j].cnt = kept;
        rs[j].thr = bound;
        th[j] = next_up(bound);
        if (!EXACT && p.nseg == 1 && lane_id() == 0) {
          p.rowinfo[rs[j].r].thr = bound;
          p.rowinfo[rs[j].r].strict = 1;
        }
      }
    if ((p.flags & 8u) && lane_id() == 0) atomicAdd(&p.header[H_COMPACT], 1u);
  }
  // The counts are wave-uniform; stating it keeps them, and the scan's
  // per-chunk count updates and capacity tests, in scalar registers.
#pragma unroll
  for (int j = 0; j < kRowsPerWave; ++j) rs[j].cnt = __builtin_amdgcn_readfirstlane(rs[j].cnt);
}

// Stage key j (0 .. stage_keys - 1) of a stage that starts at position key0:
// its key (position) and request. Gathered and paged stages hold the keys
// key0 + j * stride; a decode stage holds, in chunk u = j / 64, the
// positions key0 + (j % 64) * stride of part req0 + u. Keys are clamped to
// the last one and requests to the last request.
template <int SRC>
__device__ __forceinline__ void stage_key(const FusedParams& p, int key0, int stride, int j,
                                          int req0, int& key, int& req) {
  if constexpr (SRC == SRC_DECODE) {
    // chunk u of the stage: part req0 + u (its request's table row)
    const int u = j >> 6;
    key = key0 + (j & (kChunk - 1)) * stride;
    req = (req0 + u) / p.dec_parts;
    req = req < p.nreq ? req : p.nreq - 1;
  } else {
    key = key0 + j * stride;
    req = 0;
  }
  key = key < p.keys ? key : p.keys - 1;
}

// Queue the copy of a stage's page numbers into pdst (paged and decode
// sources; thread j copies the page-table entry of stage key j). Issued a
// stage before the stage's key copies, which read them from LDS.
template <int SRC>
__device__ __forceinline__ void dma_pages(const FusedParams& p, int key0, int stride,
                                          int32_t* pdst, int tid, int req0) {
  if constexpr (SRC != SRC_GATHER) {
    if (tid < stage_keys<SRC>()) {
      // decode: entry t holds the page of stage key 64 (t % 4) + t / 4, so
      // that a thread's four tile copies (one per part) read one 16-byte
      // group
      const int j = SRC == SRC_DECODE ? 64 * (tid & 3) + (tid >> 2) : tid;
      int key, req;
      stage_key<SRC>(p, key0, stride, j, req0, key, req);
      const int32_t* src = table_entry<SRC>(p, key, req);
      __builtin_amdgcn_global_load_lds(src, pdst + (tid & ~63), 4, 0, 0);
    }
  }
}

// Queue direct global->LDS copies of a stage's keys (stage_key), their scales
// and their nhat (decode: their raw scale words) into a stage buffer; pgs
// holds the stage's page numbers (paged and decode sources).
// Slot p of the buffer (16 bytes) holds key j = p / 8, column slice (p % 8) ^
// swz(j); each wave fills 64 consecutive slots per copy. The copies are
// waited for by the barrier that ends the stage before the buffer is read.
template <int SRC>
__device__ __forceinline__ void dma_stage(const FusedParams& p, int key0, int stride,
                                          uint8_t* kdst, float* sdst, const int32_t* pgs,
                                          int tid, int req0) {
  constexpr int SK = stage_keys<SRC>();
  // Issued before the key tiles, so that anything the compiler reloads for
  // it is waited for before the tile copies are in flight.
  if constexpr (SRC == SRC_DECODE) {
    if (tid < SK) {
      int key, req;
      stage_key<SRC>(p, key0, stride, tid, req0, key, req);
      const uint32_t* src = page_scale(p, pgs[4 * (tid & 63) + (tid >> 6)], key);
      __builtin_amdgcn_global_load_lds(src, sdst + (tid & ~63), 4, 0, 0);
    }
  } else if (tid < 2 * SK) {
    // threads [0, SK): scales; [SK, 2 SK): nhat (the two halves of each
    // key's keyinfo pair)
    const int t = tid & (SK - 1);
    const int half = tid / SK;
    int key = key0 + t * stride;
    key = key < p.keys ? key : p.keys - 1;
    // a 32-bit byte offset from the uniform base (keys < 2^20): one VGPR
    const uint32_t off = (uint32_t)(2 * key + half) * 4u;
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(p.keyinfo) + off,
                                     sdst + (tid & ~63), 4, 0, 0);
  }
  if constexpr (SRC == SRC_DECODE) {
    // copy i (one per part): stage key 64 i + tid / 8, slice (tid % 8) ^ swz;
    // the four pages in one LDS read
    static_assert(SK * 8 / kThreads == kDecPack, "one tile copy per part");
    const int jj = tid >> 3;
    const int c = (tid & 7) ^ swz(jj);
    int key, req;
    stage_key<SRC>(p, key0, stride, jj, req0, key, req);
    const int4 pg4 = *reinterpret_cast<const int4*>(pgs + 4 * jj);
    const int pg[4] = {pg4.x, pg4.y, pg4.z, pg4.w};
#pragma unroll
    for (int i = 0; i < kDecPack; ++i) {
      const uint8_t* src = page_row(p, pg[i], key) + 16 * c;
      __builtin_amdgcn_global_load_lds(src, kdst + 16 * ((tid + i * kThreads) & ~63), 16, 0, 0);
    }
  } else {
#pragma unroll
    for (int i = 0; i < SK * 8 / kThreads; ++i) {
      const int slot = tid + i * kThreads;
      const int j = slot >> 3;
      const int c = (slot & 7) ^ swz(j);
      int key, req;
      stage_key<SRC>(p, key0, stride, j, req0, key, req);
      const uint8_t* src;
      if constexpr (SRC == SRC_GATHER)
        src = p.k + (int64_t)key * kDim + 16 * c;
      else
        src = page_row(p, pgs[j], key) + 16 * c;
      __builtin_amdgcn_global_load_lds(src, kdst + 16 * (slot & ~63), 16, 0, 0);
    }
  }
}

// In decode the scan bounds a key's FP8 error from the key's own bytes (there
// is no per-key prologue): with S = sum_d k_d^2, each group's largest |k_d|
// is at most the square root of the group's sum of squares, x(v) <= |v| for
// normal codes and x = 2^-6 for subnormal ones, and by Cauchy-Schwarz the 16
// group terms sum to at most 4 sqrt(S), so
//   sum_g max_{d in g} x(k_d) <= 4 sqrt(S) + 16 * 2^-6.
// S is the diagonal of the FP8 MFMA of each 16-key sub-tile with itself: its
// products are exact squares, and truncation lowers a group's sum by at most
// 7 * 2^-13 of it, so S is taken as the MFMA's value times (1 + 2^-9). Lane l
// gets key l's nhat (rounded up like the prologue's).
__device__ __forceinline__ float decode_nhat(const KeyTile& kt, float scale) {
  const int l = lane_id();
  const int j = l & 15;
  float d[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const v4f z = {0.f, 0.f, 0.f, 0.f};
    const v4f c = mfma_fp8(kt.kb[t], kt.kb[t], z);
    // entry (m, n) of the product sits in lane n + 16 (m / 4), element m % 4:
    // the diagonal entry (j, j) in lane j + 16 (j / 4), element j % 4
    const int v = l & 3;
    const float x = v == 0 ? c[0] : (v == 1 ? c[1] : (v == 2 ? c[2] : c[3]));
    d[t] = __shfl(x, j + 16 * (j >> 2), 64);
  }
  const int t = l >> 4;  // key l is key j of sub-tile t
  const float sq = t == 0 ? d[0] : (t == 1 ? d[1] : (t == 2 ? d[2] : d[3]));
  const float x = __builtin_fmaf(4.f * __builtin_sqrtf(sq * (1.f + 0x1p-9f)), 1.f + 0x1p-20f, 0.25f);
  return key_nhat(x, scale);
}

// Scheduling groups of one region of score4: M MFMAs, each followed by V
// VALU instructions (the region's other VALU instructions after them).
template <int M, int V>
__device__ __forceinline__ void interleave_mfma() {
#pragma unroll
  for (int i = 0; i < M; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, V, 0);
  }
}

// Approximate scores of the wave's 4 rows for a 64-key chunk, lane l <->
// key l: (f.k + sum_h w_h |s_h|) / 2 * scale (relu fold, common.h; the rows'
// weights are loaded halved and the fold operand carries f / 2); rows with
// zeroed operands score 0. Five scheduling regions, fenced by sched
// barriers: the fold and row 0 MFMAs; row r + 1's MFMAs spread through row
// r's head epilogue (r = 0, 1, 2), so that every epilogue reads results
// issued a whole region earlier and each MFMA has VALU work beside it; row
// 3's epilogue. Left to itself the scheduler packs each row's epilogue right
// behind its own MFMAs (shorter live ranges) and the wave then waits for
// their results.
__device__ __forceinline__ void score4(float E[4], const QueryRow* qr, const FoldOp& fo,
                                       const KeyTile& kt, float sc) {
  FoldTerms f;
  RowAcc a0, a1;
  __builtin_amdgcn_sched_barrier(0);
  fold_terms(f, fo, kt);
  mfma_row(a0, qr[0], kt);
  __builtin_amdgcn_sched_barrier(0);
  mfma_row(a1, qr[1], kt);
  E[0] = reduce_heads_abs(qr[0], a0, f, 0) * sc;
  interleave_mfma<8, 5>();
  __builtin_amdgcn_sched_barrier(0);
  mfma_row(a0, qr[2], kt);
  E[1] = reduce_heads_abs(qr[1], a1, f, 1) * sc;
  interleave_mfma<8, 5>();
  __builtin_amdgcn_sched_barrier(0);
  mfma_row(a1, qr[3], kt);
  E[2] = reduce_heads_abs(qr[2], a0, f, 2) * sc;
  interleave_mfma<8, 5>();
  __builtin_amdgcn_sched_barrier(0);
  E[3] = reduce_heads_abs(qr[3], a1, f, 3) * sc;
}

// One scan of keys [lo, hi) for the rows of this wave in `mode` (M_ALL and
// M_GATED rows together, or M_EXACT rows): FP8 MFMA scores, or exact scores
// for EXACT. FP8 rows are pipelined: the MFMAs of the next row are issued
// before the epilogue of the current one. Chunks that every live row of the
// wave covers entirely (almost all of them) take a path with no per-row range
// tests: rows that are not live have an admission threshold of NaN there.
// Decode: the block's parts req0 .. req0 + 3 share the stages (chunk u of a
// stage is part req0 + u's) and this wave's rows are part req0 + grp's.
template <bool EXACT, int SRC>
__device__ __forceinline__ void scan_rows(const FusedParams& p, const Stages& stg, const QueryRow* qr,
                                          const FoldOp& fo, RowState* rs, int mode, int lo,
                                          int hi, const SlabRefs& sr, int req0, int grp) {
  const int tid = threadIdx.x;
  const int l = lane_id();
  constexpr int SC = stage_chunks<SRC>();
  constexpr int SK = stage_keys<SRC>();
  constexpr int G = SRC == SRC_DECODE ? kDecPack : 1;
  const int cps = SC / G;  // 64-position chunks per stage
  const int nch = (hi - lo + kChunk - 1) / kChunk;
  bool live[kRowsPerWave];
  float th[kRowsPerWave];
  int cf = 0, ch = nch, nlive = 0;  // chunks [cf, ch) lie inside every live row
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    live[i] = EXACT ? rs[i].mode == M_EXACT : (rs[i].mode == M_ALL || rs[i].mode == M_GATED);
    th[i] = admit_thr(rs[i], live[i]);
    if (live[i]) {
      ++nlive;
      const int a = (rs[i].s - lo + kChunk - 1) / kChunk;
      const int z = (rs[i].e - lo) / kChunk;
      cf = a > cf ? a : cf;
      ch = z < ch ? z : ch;
    }
  }
  if (nlive == 0) cf = ch = 0;
  const int nst = (nch + cps - 1) / cps;
  // The records of a stage's last chunk (FP8 scan of gathered and paged keys)
  // are appended after the stage barrier: the barrier's fence waits for every
  // store the wave has in flight, and these would be the youngest.
  constexpr bool kDefer = !EXACT && SRC != SRC_DECODE;
  float dE[kRowsPerWave], dth[kRowsPerWave];
  float dnh = 0.f;
  int dkw = 0;
  bool dpend = false;
  auto check_merge = [&]() {
    bool over = false;
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) over |= rs[i].cnt > sr.cap;
    if (over) merge_rows<EXACT>(p, rs, sr, th);
  };
  // One chunk of the stage in LDS (keys kc, scales scl, error bound factors
  // nrm): score the wave's rows and append their candidates (held for after
  // the barrier when `defer`).
  auto chunk = [&](int c, const uint8_t* kc, const float* scl, bool defer) {
    const int key0 = lo + c * kChunk;
    const int key = key0 + l;
    if constexpr (!EXACT) {
      // Each row's admission test as one per-lane threshold: the row's own on
      // interior chunks, NaN for keys outside the row's range on the others,
      // so that scoring and emission are the same code for both (no range
      // tests behind the scores).
      float thl[kRowsPerWave];
      if (c >= cf && c < ch) {
#pragma unroll
        for (int i = 0; i < kRowsPerWave; ++i) thl[i] = th[i];
      } else {
        bool any = false;
#pragma unroll
        for (int i = 0; i < kRowsPerWave; ++i) {
          const bool act = live[i] && rs[i].s < key0 + kChunk && rs[i].e > key0;
          any |= act;
          thl[i] = act && key >= rs[i].s && key < rs[i].e ? th[i] : __builtin_nanf("");
        }
        if (!any) return;
      }
      KeyTile kt;
      float sc, nh;
      int kw;
      float E[4];
      if constexpr (SRC == SRC_DECODE) {
        // (the key's bound after its scores: fewer registers live at once)
        load_keys_lds(kt, kc);
        sc = ue8m0(__float_as_uint(scl[l]));
        score4_serial(E, qr, fo, kt, sc);
        nh = decode_nhat(kt, sc);
        kw = key | __float_as_int(nh);
      } else {
        sc = scl[l];
        nh = scl[SK + l];
        // the record's key word: the key and its nhat bits
        kw = key | __float_as_int(nh);
        load_keys_lds(kt, kc);
        // rows that are not live have zeroed operands and a NaN threshold
        // (64 heads: partner slots are not live; their scores join the lead's)
        score4(E, qr, fo, kt, sc);
        combine_halves(p, E);
      }
      // admission and records by U = E + beta * nhat, an upper bound of the
      // key's exact score
      if (kDefer && defer) {
#pragma unroll
        for (int i = 0; i < kRowsPerWave; ++i) {
          dE[i] = E[i];
          dth[i] = thl[i];
        }
        dnh = nh;
        dkw = kw;
        dpend = true;
        return;  // the capacity check follows the held records
      }
#pragma unroll
      for (int i = 0; i < kRowsPerWave; ++i)
        emit_rec(rs[i], __builtin_fmaf(rs[i].beta, nh, E[i]), thl[i], true, kw, sr, i);
    } else {
      bool act[kRowsPerWave];
      bool any = false;
#pragma unroll
      for (int i = 0; i < kRowsPerWave; ++i) {
        act[i] = live[i] && rs[i].s < key0 + kChunk && rs[i].e > key0;
        any |= act[i];
      }
      if (!any) return;
      const float sc = SRC == SRC_DECODE ? ue8m0(__float_as_uint(scl[l])) : scl[l];
      KeyTile kt;
      load_keys_lds(kt, kc);
      float E[4];
      if (SRC != SRC_DECODE && p.hm == 2) {
        // 64 heads: lead slot i scores with its partner i + 1 (exact_score's
        // order: the halves' head sums added, then the scale)
#pragma unroll
        for (int i = 0; i < kRowsPerWave; i += 2) {
          E[i] = act[i] ? (score_chunk_exact(qr[i], kt) + score_chunk_exact(qr[i + 1], kt)) * sc
                        : 0.f;
          E[i + 1] = 0.f;
        }
      } else {
#pragma unroll
        for (int i = 0; i < kRowsPerWave; ++i)
          E[i] = act[i] ? score_chunk_exact(qr[i], kt) * sc : 0.f;
      }
#pragma unroll
      for (int i = 0; i < kRowsPerWave; ++i)
        if (act[i]) finish_row(rs[i], E[i], th[i], key, key0, sr, i);
    }
    check_merge();
  };
  // One stage: queue the copy of the next stage into the other buffer (its
  // last readers passed the previous barrier), then score this one.
  // (paged and decode sources: the pages of stage st + 2 are copied during
  // stage st, into the page buffer stage st's copies were issued from)
  auto stage = [&](int st, const uint8_t* kcur, const float* scur, uint8_t* knext,
                   float* snext, const int32_t* pnext, int32_t* pafter) {
    if (st + 1 < nst)
      dma_stage<SRC>(p, lo + (st + 1) * cps * kChunk, 1, knext, snext, pnext, tid, req0);
    if (SRC != SRC_GATHER && st + 2 < nst)
      dma_pages<SRC>(p, lo + (st + 2) * cps * kChunk, 1, pafter, tid, req0);
    if constexpr (SRC == SRC_DECODE) {
      // this wave's request's chunks of the stage: u = grp, grp + G, ...
      // (one copy of the chunk code for any G)
#pragma unroll 1
      for (int v = 0; v < cps; ++v) {
        const int u = grp + v * G;
        const int c = st * cps + v;
        if (c < nch) chunk(c, kcur + u * kChunkBytes, scur + u * kChunk, false);
      }
    } else {
#pragma unroll
      for (int u = 0; u < SC; ++u) {
        const int c = st * SC + u;
        if (c < nch) chunk(c, kcur + u * kChunkBytes, scur + u * kChunk, u == SC - 1 || c + 1 == nch);
      }
    }
    __syncthreads();
    if (kDefer && dpend) {
#pragma unroll
      for (int i = 0; i < kRowsPerWave; ++i)
        emit_rec(rs[i], __builtin_fmaf(rs[i].beta, dnh, dE[i]), dth[i], true, dkw, sr, i);
      dpend = false;
      check_merge();
    }
  };
  if constexpr (SRC != SRC_GATHER) {
    dma_pages<SRC>(p, lo, 1, stg.pg[0], tid, req0);
    __syncthreads();
  }
  dma_stage<SRC>(p, lo, 1, stg.k[0], stg.s[0], stg.pg[0], tid, req0);
  if (SRC != SRC_GATHER && nst > 1) dma_pages<SRC>(p, lo + cps * kChunk, 1, stg.pg[1], tid, req0);
  __syncthreads();
  for (int st = 0; st < nst; st += 2) {
    stage(st, stg.k[0], stg.s[0], stg.k[1], stg.s[1], stg.pg[1], stg.pg[0]);
    if (st + 1 < nst) stage(st + 1, stg.k[1], stg.s[1], stg.k[0], stg.s[0], stg.pg[0], stg.pg[1]);
  }
}

// ---------------------------------------------------------------------------
// Gate. A strided sample of the block's keys (512..16384 keys, about span /
// 24, at a fixed integer stride from the start of the block's range) is
// scored like the scan scores; each gated row bins (first-tile maximum -
// score) in kGateBins bins of 1/256 of the first sample tile's score range and
// takes as threshold the lower score edge of the bin where the count of sample keys
// above reaches a safe margin over the k-th key's expected sample rank. Rows with n <= k are answered here (keys 0..n-1, -1 padding).
// The gate's sample of a block whose union range spans `span` keys: S keys
// (about span / 24, a multiple of spp, the positions a stage holds per
// request, 512..16384) at an integer stride from the start of the range.
// Returns the number of stages.
__device__ __forceinline__ int gate_sample(int span, int spp, int& stride) {
  int S = (span / 24) & ~(spp - 1);
  S = S < 512 ? 512 : (S > 16384 ? 16384 : S);
  stride = span / S > 1 ? span / S : 1;
  return S / spp;
}

// The strided sample loop of the gate and of its fine pass: nst stages of the
// keys lo + j * stride (decode: of each packed request), double-buffered,
// each chunk handed to f(position chunk, keys, scales) (decode: only the
// chunks of the calling wave's request grp); the paged and decode sources
// copy the pages a stage ahead, as the scan does.
template <int SRC, class F>
__device__ __forceinline__ void sample_stages(const FusedParams& p, const Stages& stg, int lo,
                                              int stride, int nst, int req0, int grp, int tid,
                                              F f) {
  constexpr int SC = stage_chunks<SRC>();
  constexpr int G = SRC == SRC_DECODE ? kDecPack : 1;
  const int step = SC / G * kChunk * stride;  // positions per stage
  auto stage = [&](int st, const uint8_t* kcur, const float* scur, uint8_t* knext,
                   float* snext, const int32_t* pnext, int32_t* pafter) {
    if (st + 1 < nst)
      dma_stage<SRC>(p, lo + (st + 1) * step, stride, knext, snext, pnext, tid, req0);
    if (SRC != SRC_GATHER && st + 2 < nst)
      dma_pages<SRC>(p, lo + (st + 2) * step, stride, pafter, tid, req0);
    if constexpr (SRC == SRC_DECODE) {
      // this wave's request's chunks: u = grp, grp + G, ... (position chunk
      // st * (SC / G) + v)
#pragma unroll 1
      for (int v = 0; v < SC / G; ++v) {
        const int u = grp + v * G;
        f(st * (SC / G) + v, kcur + u * kChunkBytes, scur + u * kChunk);
      }
    } else {
#pragma unroll
      for (int u = 0; u < SC; ++u) f(st * SC + u, kcur + u * kChunkBytes, scur + u * kChunk);
    }
    __syncthreads();
  };
  if constexpr (SRC != SRC_GATHER) {
    dma_pages<SRC>(p, lo, stride, stg.pg[0], tid, req0);
    __syncthreads();
  }
  dma_stage<SRC>(p, lo, stride, stg.k[0], stg.s[0], stg.pg[0], tid, req0);
  if (SRC != SRC_GATHER && nst > 1) dma_pages<SRC>(p, lo + step, stride, stg.pg[1], tid, req0);
  __syncthreads();
  for (int st = 0; st < nst; st += 2) {
    stage(st, stg.k[0], stg.s[0], stg.k[1], stg.s[1], stg.pg[1], stg.pg[0]);
    if (st + 1 < nst) stage(st + 1, stg.k[1], stg.s[1], stg.k[0], stg.s[0], stg.pg[0], stg.pg[1]);
  }
}

struct __align__(16) GateSmem {
  uint32_t hist[kWaves][kRowsPerWave * kGateBins];
  int block;
  int wlo[kWaves], whi[kWaves], wf[kWaves];
};

template <int SRC>
__global__ __launch_bounds__(kThreads) void fused_gate_kernel(FusedParams p) {
  __shared__ GateSmem sm;
  MQA_DECLARE_STAGES(stg, SRC);
  const int tid = threadIdx.x;
  const int w = wave_id();
  const int l = lane_id();
  const int k = p.topk;
  const int cap = slab_cap(p);
  const bool stats = p.flags & 8u;
  // Work items (block, part): with key segments (p.nseg > 1, few blocks) a
  // block's rows are shared by p.nseg workgroups, part t serving the rows of
  // waves [t * 8 / nseg, (t + 1) * 8 / nseg); every part samples the whole
  // block's union range, so the thresholds do not depend on the split.
  const int parts = p.nseg;
  const int items = p.nblocks * parts;
  for (;;) {
    if (tid == 0) sm.block = (int)atomicAdd(&p.header[H_GCLAIM], 1u);
    __syncthreads();
    const int bi = sm.block;
    if (bi >= items) break;
    const int b = p.order[bi / parts];
    const bool mine = w * parts / kWaves == bi % parts;
    RowState rs[kRowsPerWave];
    QueryRow qr[kRowsPerWave];
    wave_rows<SRC>(p, b, rs);
    int wlo = p.keys, whi = 0, wg = 0;
    int frows[kRowsPerWave];
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      RowState& r = rs[i];
      zero_query(qr[i]);
      frows[i] = -1;
      if (r.r >= p.rows || partner_row(p, r.r)) continue;
      const int n = r.e - r.s;
      if (n <= k) {
        r.mode = M_SHORT;
        if (mine) {
          int32_t* o = out_row(p, r.r);
          for (int j = l; j < k; j += kWave) o[j] = j < n ? j : -1;
          if (stats && l == 0) atomicAdd(&p.header[H_SHORT], 1u);
        }
      } else if (p.flags & 1u) {
        r.mode = M_EXACT;  // forced: straight to the exact rescan
      } else if (n <= 4 * k && n <= cap) {
        r.mode = M_ALL;  // every visible key is a candidate
      } else {
        // rows of other parts count for the union range only
        r.mode = mine ? M_GATED : M_OFF;
        if (mine) {
          load_query(qr[i], p.q, p.weights, r.r, 0.5f);
          frows[i] = r.r;
          r.beta = row_beta_of(p, r.r);
        }
        wlo = r.s < wlo ? r.s : wlo;
        whi = r.e > whi ? r.e : whi;
        wg |= mine ? 1 : 0;  // the part samples only when it serves a gated row
      }
    }
    load_partners(p, rs, qr, frows, M_GATED, 0.5f);
    int lo, hi, any_g;
    block_union(sm.wlo, sm.whi, sm.wf, wlo, whi, wg, p.keys, lo, hi, any_g);
    // the fine pass's hand-over (rbin -1: none)
    int rbin[kRowsPerWave], rneed[kRowsPerWave], rnext[kRowsPerWave];
    float rm0[kRowsPerWave], rinv[kRowsPerWave];
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      rbin[i] = -1;
      rneed[i] = rnext[i] = 0;
      rm0[i] = 0.f;
      rinv[i] = 1.f;
    }
    if (any_g && hi > lo) {
      FoldOp fo;
      build_fold(fo, p.q, p.weights, frows);
      // the sample keys lo + j * stride, j < nst * cps * 64 (in decode, of
      // each packed request)
      constexpr int SC = stage_chunks<SRC>();
      constexpr int SK = stage_keys<SRC>();
      constexpr int G = SRC == SRC_DECODE ? kDecPack : 1;
      const int cps = SC / G;
      const int req0 = b * G;  // decode: the block's first part
      const int grp = wave_group<SRC>(w);
      int stride;
      const int nst = gate_sample(hi - lo, cps * kChunk, stride);
      uint32_t* hist = sm.hist[w];
      for (int i = l; i < kRowsPerWave * kGateBins; i += kWave) hist[i] = 0;
      float m0[kRowsPerWave], inv[kRowsPerWave];
      int have_m0[kRowsPerWave], nsamp[kRowsPerWave];
#pragma unroll
      for (int i = 0; i < kRowsPerWave; ++i) {
        m0[i] = 0.f;
        inv[i] = 1.f;
        have_m0[i] = 0;
        nsamp[i] = 0;
      }
      // The sample is scored as the scan will admit it: by U = E + beta * nhat
      // (E the FP8 score), so that its counts predict the scan's candidates.
      auto chunk = [&](int c, const uint8_t* kc, const float* scl) {
        if (!mine) return;
        const int key = lo + (c * kChunk + l) * stride;
        KeyTile kt;
        float sc, nh;
        float E[4];
        if constexpr (SRC == SRC_DECODE) {
          load_keys_lds(kt, kc);
          sc = ue8m0(__float_as_uint(scl[l]));
          score4(E, qr, fo, kt, sc);
          nh = decode_nhat(kt, sc);
        } else {
          nh = scl[SK + l];
          sc = scl[l];
          load_keys_lds(kt, kc);
          score4(E, qr, fo, kt, sc);
          combine_halves(p, E);
        }
#pragma unroll
        for (int i = 0; i < kRowsPerWave; ++i) E[i] = __builtin_fmaf(rs[i].beta, nh, E[i]);
#pragma unroll
        for (int i = 0; i < kRowsPerWave; ++i) {
          const RowState& r = rs[i];
          if (r.mode != M_GATED) continue;
          const bool valid = key >= r.s && key < r.e;
          const uint64_t vm = __ballot(valid);
          if (vm == 0) continue;
          if (!have_m0[i]) {
            const float mx = wave_max(valid ? E[i] : -__builtin_inff());
            const float mn = wave_min(valid ? E[i] : __builtin_inff());
            float width = (mx - mn) / 256.f;
            if (!(width > 0.f) || !__builtin_isfinite(width))
              width = __builtin_fmaxf(__builtin_fabsf(mx), 1e-30f) * (1.f / 512.f);
            m0[i] = mx;
            inv[i] = 1.f / width;
            have_m0[i] = 1;
          }
          nsamp[i] += __popcll(vm);
          if (valid) {
            const float fb = (m0[i] - E[i]) * inv[i];
            int bin = fb < -1e6f ? 0
                                 : (fb > 1e6f ? kGateBins - 1 : (int)__builtin_floorf(fb) + kGateOff);
            bin = bin < 0 ? 0 : (bin > kGateBins - 1 ? kGateBins - 1 : bin);
            atomicAdd(&hist[i * kGateBins + bin], 1u);
          }
        }
      };
      sample_stages<SRC>(p, stg, lo, stride, nst, req0, grp, tid,
                         [&](int c, const uint8_t* kc, const float* scl) { chunk(c, kc, scl); });
#pragma unroll
      for (int i = 0; i < kRowsPerWave; ++i) {
        RowState& r = rs[i];
        rbin[i] = -1;
        if (r.mode != M_GATED) continue;
        // The sample keys above the row's true k-th score are about
        // Poisson(lam), lam = k * nsamp / n. The threshold is put at the
        // ks-th best sample, ks = lam + 5 sqrt(lam) + 5, so that fewer than k
        // keys pass it with probability below ~1e-6 (about 1.5k candidates
        // at lam ~ 150, more when the sample is thin).
        const int n = r.e - r.s;
        const float lam = (float)p.kgate * (float)nsamp[i] / (float)n;
        const int ks = (int)__builtin_ceilf(lam + 5.f * __builtin_sqrtf(lam) + 5.f);
        float thr = -__builtin_inff();
        if (have_m0[i] && ks >= 1 && ks <= nsamp[i]) {
          // bins kPer*l .. kPer*l + kPer-1 per lane, cumulative from bin 0 (the top)
          constexpr int kPer = kGateBins / kWave;
          int hv[kPer], hsum = 0;
#pragma unroll
          for (int j = 0; j < kPer; ++j) {
            hv[j] = (int)hist[i * kGateBins + kPer * l + j];
            hsum += hv[j];
          }
          const int incl = wave_incl_scan(hsum);
          const uint64_t hit = __ballot(incl >= ks);
          int c = incl - hsum, bstar = kPer * l + kPer - 1;
          // first bin of this lane where the running count reaches ks
          bool found = false;
#pragma unroll
          for (int j = 0; j < kPer; ++j) {
            const bool here = !found && c + hv[j] >= ks;
            bstar = here ? kPer * l + j : bstar;
            found = found || here;
            c += hv[j];
          }
          bstar = __shfl(bstar, hit ? __builtin_ctzll(hit) : 0, 64);
          // The threshold goes down the run of empty bins below bstar to the
          // next sampled score, not to bstar's lower edge: when the scores are
          // heavily tied the k-th key's score sits at the top of a wide gap,
          // and the select's certificate needs that gap as margin (every key
          // left out must score below the k-th exact score, about one error
          // bound under its U).
          int b2 = kGateBins;
#pragma unroll
          for (int j = kPer - 1; j >= 0; --j)
            b2 = (kPer * l + j > bstar && hv[j] > 0) ? kPer * l + j : b2;
          b2 = -wave_max_i(-b2);
          if (hit && bstar < kGateBins - 1) {
            const float lower = (float)(bstar - kGateOff + 1);  // bstar's lower score edge
            const float next = (float)(b2 - kGateOff);           // upper edge of the next sample
            // (a quarter bin above the next sampled bin, so that its scores
            // stay out under rounding; never above bstar's lower edge)
            thr = m0[i] - (b2 < kGateBins ? __builtin_fmaxf(lower, next - 0.25f) : lower) / inv[i];
            // A crowded bin (the first tile's range can be far wider than the
            // spread of scores around the k-th, e.g. with a large common score
            // offset) would admit every key of it: the fine pass bins its
            // samples again.
            int hb = 0, before = 0, cc = incl - hsum;
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
              if (kPer * l + j == bstar) {
                hb = hv[j];
                before = cc;
              }
              cc += hv[j];
            }
            hb = __shfl(hb, bstar / kPer, 64);
            before = __shfl(before, bstar / kPer, 64);
            if (bstar >= 1 && hb > kGateCrowded && hb > ks && !(p.flags & 2u)) {
              rbin[i] = bstar;
              rneed[i] = ks - before;
              rnext[i] = b2;
            }
          }
        }
        if (p.flags & 2u) thr = __builtin_inff();  // forced gate miss
        r.thr = thr;
        rm0[i] = m0[i];
        rinv[i] = inv[i];
      }
    }
    if (mine && l == 0) {
      bool fine = false;
#pragma unroll
      for (int i = 0; i < kRowsPerWave; ++i) {
        const RowState& r = rs[i];
        if (r.r >= p.rows) continue;
        p.rowinfo[r.r] = RowInfo{r.thr, 0, r.mode, 0, 0, 0};
        p.xrow[r.r] = 0;
        if (r.mode == M_GATED) p.rinfo[r.r] = RefineInfo{rm0[i], rinv[i], rbin[i], rneed[i], rnext[i]};
        fine = fine || rbin[i] >= 0;
      }
      // queue the block for the fine pass, once
      if (fine && atomicExch(&p.fflag[b], 1u) == 0u)
        p.fqueue[atomicAdd(&p.header[H_FQ], 1u)] = b;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Scan: every visible key of every live row of a block, candidates to the
// rows' slabs.
// The gate's fine pass, for the blocks the gate queued (a row whose threshold
// bin was crowded). The block's sample is drawn again as the gate drew it
// (the union range of its gated rows, gate_sample), the queued rows score it
// again (the same arithmetic as the gate, so the same scores) and bin the
// samples of their crowded coarse bin in kGateBins fine bins across it; the
// threshold goes into the first fine bin that completes the row's count, with
// the gate's gap rule (down to the next sampled score). Returns at
// once when nothing is queued.
template <int SRC>
__global__ __launch_bounds__(kThreads) void fused_refine_kernel(FusedParams p) {
  __shared__ GateSmem sm;
  MQA_DECLARE_STAGES(stg, SRC);
  const int tid = threadIdx.x;
  const int w = wave_id();
  const int l = lane_id();
  const int nq = (int)p.header[H_FQ];
  if (nq == 0) return;
  for (;;) {
    if (tid == 0) sm.block = (int)atomicAdd(&p.header[H_FCLAIM], 1u);
    __syncthreads();
    const int qi = sm.block;
    if (qi >= nq) break;
    const int b = p.fqueue[qi];
    RowState rs[kRowsPerWave];
    QueryRow qr[kRowsPerWave];
    wave_rows<SRC>(p, b, rs);
    int wlo = p.keys, whi = 0, wfine = 0;
    int frows[kRowsPerWave], rbin[kRowsPerWave], rneed[kRowsPerWave], rnext[kRowsPerWave];
    float m0[kRowsPerWave], inv[kRowsPerWave];
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      RowState& r = rs[i];
      zero_query(qr[i]);
      frows[i] = rbin[i] = -1;
      rneed[i] = rnext[i] = 0;
      m0[i] = 0.f;
      inv[i] = 1.f;
      if (r.r >= p.rows || p.rowinfo[r.r].mode != M_GATED) continue;
      wlo = r.s < wlo ? r.s : wlo;  // the gate's union: every gated row
      whi = r.e > whi ? r.e : whi;
      const RefineInfo f = p.rinfo[r.r];
      if (f.bin < 0) continue;
      rbin[i] = f.bin;
      rneed[i] = f.need;
      rnext[i] = f.next;
      m0[i] = f.m0;
      inv[i] = f.inv;
      load_query(qr[i], p.q, p.weights, r.r, 0.5f);
      frows[i] = r.r;
      r.beta = row_beta_of(p, r.r);
      wfine = 1;
    }
    if (p.hm == 2) {
      // partners of the refined rows (rows with a fine pass have frows set)
#pragma unroll
      for (int i = 1; i < kRowsPerWave; i += 2)
        if (frows[i - 1] >= 0) {
          load_query(qr[i], p.q, p.weights, rs[i].r, 0.5f);
          frows[i] = rs[i].r;
        }
    }
    int lo, hi, unused;
    block_union(sm.wlo, sm.whi, sm.wf, wlo, whi, 0, p.keys, lo, hi, unused);
    if (hi > lo) {
      constexpr int SC = stage_chunks<SRC>();
      constexpr int SK = stage_keys<SRC>();
      constexpr int G = SRC == SRC_DECODE ? kDecPack : 1;
      const int cps = SC / G;
      const int req0 = b * G;  // decode: the block's first part
      const int grp = wave_group<SRC>(w);
      int stride;
      const int nst = gate_sample(hi - lo, cps * kChunk, stride);
      FoldOp fo;
      build_fold(fo, p.q, p.weights, frows);
      uint32_t* hist = sm.hist[w];
      for (int j = l; j < kRowsPerWave * kGateBins; j += kWave) hist[j] = 0;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      auto chunk = [&](int c, const uint8_t* kc, const float* scl) {
        if (!wfine) return;
        const int key = lo + (c * kChunk + l) * stride;
        KeyTile kt;
        float sc, nh;
        float E[4];
        if constexpr (SRC == SRC_DECODE) {
          load_keys_lds(kt, kc);
          sc = ue8m0(__float_as_uint(scl[l]));
          score4(E, qr, fo, kt, sc);
          nh = decode_nhat(kt, sc);
        } else {
          nh = scl[SK + l];
          sc = scl[l];
          load_keys_lds(kt, kc);
          score4(E, qr, fo, kt, sc);
          combine_halves(p, E);
        }
#pragma unroll
        for (int i = 0; i < kRowsPerWave; ++i) E[i] = __builtin_fmaf(rs[i].beta, nh, E[i]);
#pragma unroll
        for (int i = 0; i < kRowsPerWave; ++i) {
          const RowState& r = rs[i];
          if (rbin[i] < 0 || key < r.s || key >= r.e) continue;
          // the gate's coarse bin, by the gate's expression
          const float fb = (m0[i] - E[i]) * inv[i];
          if (fb < -1e6f || fb > 1e6f) continue;
          const float fl = __builtin_floorf(fb);
          if ((int)fl + kGateOff != rbin[i]) continue;
          int f = (int)((fb - fl) * (float)kGateBins);
          f = f < 0 ? 0 : (f > kGateBins - 1 ? kGateBins - 1 : f);
          atomicAdd(&hist[i * kGateBins + f], 1u);
        }
      };
      sample_stages<SRC>(p, stg, lo, stride, nst, req0, grp, tid,
                         [&](int c, const uint8_t* kc, const float* scl) { chunk(c, kc, scl); });
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int i = 0; i < kRowsPerWave; ++i) {
        if (rbin[i] < 0) continue;
        constexpr int kPer = kGateBins / kWave;
        int hv[kPer], hsum = 0;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
          hv[j] = (int)hist[i * kGateBins + kPer * l + j];
          hsum += hv[j];
        }
        const int incl = wave_incl_scan(hsum);
        const uint64_t hit = __ballot(incl >= rneed[i]);
        if (!hit) continue;  // keep the gate's threshold
        int c = incl - hsum, fstar = kPer * l + kPer - 1;
        bool found = false;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
          const bool here = !found && c + hv[j] >= rneed[i];
          fstar = here ? kPer * l + j : fstar;
          found = found || here;
          c += hv[j];
        }
        fstar = __shfl(fstar, __builtin_ctzll(hit), 64);
        int f2 = kGateBins;
#pragma unroll
        for (int j = kPer - 1; j >= 0; --j)
          f2 = (kPer * l + j > fstar && hv[j] > 0) ? kPer * l + j : f2;
        f2 = -wave_max_i(-f2);
        const float base = (float)(rbin[i] - kGateOff);
        const float lower = base + (float)(fstar + 1) / (float)kGateBins;
        float pos = lower;
        if (f2 < kGateBins)
          pos = __builtin_fmaxf(lower, base + ((float)f2 - 0.25f) / (float)kGateBins);
        else if (rnext[i] < kGateBins)
          pos = __builtin_fmaxf(lower, (float)(rnext[i] - kGateOff) - 0.25f);
        if (l == 0) p.rowinfo[rs[i].r].thr = m0[i] - pos / inv[i];
      }
    }
    __syncthreads();
  }
}

struct __align__(16) ScanSmem {
  uint32_t hist[kWaves][kHistWords];
  int block;
  int wlo[kWaves], whi[kWaves], wf[kWaves];
};

// SPLIT: the launch uses key segments (p.nseg > 1); the instance without
// them keeps no segment state.
template <bool SPLIT, int SRC>
__global__ __launch_bounds__(kThreads) void fused_topk_kernel(FusedParams p) {
  __shared__ ScanSmem sm;
  MQA_DECLARE_STAGES(stg, SRC);
  const int tid = threadIdx.x;
  const int w = wave_id();
  const int l = lane_id();
  // work items: (block, key segment), the block order major
  const int nseg = SPLIT ? p.nseg : 1;
  const int items = p.nblocks * nseg;
  for (;;) {
    if (tid == 0) sm.block = (int)atomicAdd(&p.header[H_CLAIM], 1u);
    __syncthreads();
    const int bi = sm.block;
    if (bi >= items) break;
    const int b = p.order[SPLIT ? bi / nseg : bi];
    const int seg = SPLIT ? bi % nseg : 0;
    RowState rs[kRowsPerWave];
    QueryRow qr[kRowsPerWave];
    wave_rows<SRC>(p, b, rs);
    int wlo = p.keys, whi = 0;
    int frows[kRowsPerWave];
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      RowState& r = rs[i];
      zero_query(qr[i]);
      frows[i] = -1;
      if (r.r >= p.rows) continue;
      const RowInfo ri = p.rowinfo[r.r];
      r.mode = ri.mode;
      r.thr = ri.thr;
      if (r.mode == M_ALL || r.mode == M_GATED) {
        load_query(qr[i], p.q, p.weights, r.r, 0.5f);
        frows[i] = r.r;
        r.beta = row_beta_of(p, r.r);
        wlo = r.s < wlo ? r.s : wlo;
        whi = r.e > whi ? r.e : whi;
      }
    }
    load_partners(p, rs, qr, frows, M_GATED, 0.5f);
    int lo, hi, unused;
    block_union(sm.wlo, sm.whi, sm.wf, wlo, whi, 0, p.keys, lo, hi, unused);
    if (SPLIT && hi > lo) {
      // segment seg of the block's key range, in whole chunks
      const int len = ((hi - lo + nseg - 1) / nseg + kChunk - 1) / kChunk * kChunk;
      const int a = lo + seg * len;
      hi = a + len < hi ? a + len : hi;
      lo = a;
    }
    if (hi > lo) {
      FoldOp fo;
      build_fold(fo, p.q, p.weights, frows);
      const SlabRefs sr = slab_refs<SRC>(p, b, sm.hist[w], 2 * p.kgate, SPLIT ? seg : -1);
      scan_rows<false, SRC>(p, stg, qr, fo, rs, M_GATED, lo, hi, sr,
                            b * (SRC == SRC_DECODE ? kDecPack : 1), wave_group<SRC>(w));
    }
    if (l == 0) {
#pragma unroll
      for (int i = 0; i < kRowsPerWave; ++i) {
        const RowState& r = rs[i];
        if (r.mode != M_ALL && r.mode != M_GATED) continue;
        if (!SPLIT)
          p.rowinfo[r.r].cnt = r.cnt;
        else
          p.seg[(int64_t)r.r * kMaxSeg + seg] = SegInfo{r.thr, r.cnt};
      }
    }
    __syncthreads();
  }
}

// Top-k of a row from its FP8-scored candidates (sE, sI)[0..n), n >= k. A
// record holds U = E + B, E the key's FP8 score and B = beta * nhat its error
// bound, and the key word (key | nhat bits), so that the key's exact score
// lies in [U - 2B, U]. Every key without a record scores at most Thi exactly
// (strictly less when thi_lt: the admission bound of a row whose threshold
// never rose; a row scanned in key segments has one per segment, Thi their
// maximum).
//   1. one pass for the range of the FP8 scores E (and the mean bound) and
//      one histogram pass over 2048 equal-width bins of it find the bin of
//      the k-th best E; the window [t_lo, t_hi] is that bin widened by
//      1 + kWinBins bins and a sixteenth of the mean bound on each side;
//   2. records whose whole interval lies above t_hi are taken; records whose
//      interval meets the window form the band, compacted to the front of the
//      slab; the others lie wholly below t_lo;
//   3. the band is rescored exactly (bf16 MFMA) and its best need = k - taken
//      records complete the row; tau is the need-th best exact band score;
//   4. the result is exact when every taken record's interval lies above tau,
//      every other record's below it and Thi does not exceed it (strictly, in
//      the deterministic mode, so that every key scoring tau is in the band).
// Returns false when step 4 fails; `low` then receives a lower bound of the
// row's k-th exact score (the k records found score at least min(tau, the
// lowest taken interval); more than k taken records bound it by t_hi), or
// -inf.
template <int SRC, class Emit>
__device__ bool select_interval(const FusedParams& p, float* sE, int32_t* sI, int n, int k,
                                float beta, float Thi, bool thi_lt, float hint_lo, float hint_hi,
                                const QueryRow& qr, const QueryRow* qr2, int req,
                                uint32_t* hist, float& low, Emit emit) {
  const int l = lane_id();
  constexpr int kBins = kHistWords;
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  // slab rows start on 1 KiB boundaries: 16-byte groups of 4 records
  const float4* e4 = reinterpret_cast<const float4*>(sE);
  const int4* i4 = reinterpret_cast<const int4*>(sI);
  const int n4 = n >> 2;
  auto bnd = [&](int kw) { return beta * __uint_as_float((uint32_t)kw & ~kKeyMask); };
  // The histogram's range: the gate's hint (from its threshold up to twice
  // its first-tile maximum's distance above it; scores outside fall into the
  // end bins) when the row has one, else the records' own range (one pass);
  // also when the k-th best lands in an end bin of the hinted range.
  float mx = hint_hi, mn = hint_lo;
  bool hinted = hint_hi > hint_lo && __builtin_isfinite(hint_hi - hint_lo);
  float bs = 0.f;
  int bk = 0;
  for (int attempt = 0; attempt < 2; ++attempt) {
    if (!hinted) {
      float m = __builtin_inff(), x = -__builtin_inff();
#pragma unroll 2
      for (int i = l; i < n4; i += kWave) {
        const float4 u = e4[i];
        const int4 w4 = i4[i];
        const float a0 = u.x - bnd(w4.x), a1 = u.y - bnd(w4.y), a2 = u.z - bnd(w4.z),
                    a3 = u.w - bnd(w4.w);
        m = __builtin_fminf(m, __builtin_fminf(__builtin_fminf(a0, a1), __builtin_fminf(a2, a3)));
        x = __builtin_fmaxf(x, __builtin_fmaxf(__builtin_fmaxf(a0, a1), __builtin_fmaxf(a2, a3)));
      }
      for (int i = 4 * n4 + l; i < n; i += kWave) {
        const float a0 = sE[i] - bnd(sI[i]);
        m = __builtin_fminf(m, a0);
        x = __builtin_fmaxf(x, a0);
      }
      mx = wave_max(x);
      mn = wave_min(m);
    }
    const float span = mx - mn;
    const float inv = span > 0.f ? (float)(kBins - 1) / span : 0.f;
    auto bin_of = [&](float e) {
      const float f = (mx - e) * inv;
      int b = f < (float)(kBins - 1) ? (int)f : kBins - 1;
      return b < 0 ? 0 : b;
    };
    for (int b = l; b < kBins; b += kWave) hist[b] = 0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    bs = 0.f;
#pragma unroll 2
    for (int i = l; i < n4; i += kWave) {
      const float4 u = e4[i];
      const int4 w4 = i4[i];
      const float b0 = bnd(w4.x), b1 = bnd(w4.y), b2 = bnd(w4.z), b3 = bnd(w4.w);
      atomicAdd(&hist[bin_of(u.x - b0)], 1u);
      atomicAdd(&hist[bin_of(u.y - b1)], 1u);
      atomicAdd(&hist[bin_of(u.z - b2)], 1u);
      atomicAdd(&hist[bin_of(u.w - b3)], 1u);
      bs += (b0 + b1) + (b2 + b3);
    }
    for (int i = 4 * n4 + l; i < n; i += kWave) {
      const float b0 = bnd(sI[i]);
      atomicAdd(&hist[bin_of(sE[i] - b0)], 1u);
      bs += b0;
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    int before;
    bk = first_bin_reaching(hist, kBins, k, before);
    __builtin_amdgcn_wave_barrier();
    if (!(hinted && (bk == 0 || bk == kBins - 1))) break;
    hinted = false;  // the k-th best lies outside the hinted range
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) bs += __shfl_xor(bs, o, 64);
  const float margin = bs / (16.f * (float)n);  // a sixteenth of the mean bound
  const float wbin = mx > mn ? (mx - mn) / (float)(kBins - 1) : 0.f;
  // the k-th best E lies in bin bk, up to one bin of rounding in bin_of
  const float t_lo = mx - (float)(bk + 2 + kWinBins) * wbin - margin;
  const float t_hi = mx - (float)(bk - 1 - kWinBins) * wbin + margin;
  int na = 0, nb = 0;
  // the lowest interval end among the taken records and the highest among
  // the dropped ones
  float a_lo = __builtin_inff(), z_hi = -__builtin_inff();
  // One record: taken (wholly above t_hi), compacted into the band (meets the
  // window), or dropped (wholly below t_lo).
  auto visit = [&](bool in, float u, int32_t kw) {
    const float lo = u - 2.f * bnd(kw);
    const bool up = in && lo > t_hi;
    const bool band = in && !up && u >= t_lo;
    const uint64_t mu = __ballot(up);
    const uint64_t mb = __ballot(band);
    const int key = kw & (int)kKeyMask;
    if (up) {
      const int slot = na + rank_in_mask(mu);
      if (slot < k) emit(slot, key);
      a_lo = __builtin_fminf(a_lo, lo);
    }
    if (in && !up && !band) z_hi = __builtin_fmaxf(z_hi, u);
    // in-place compaction: the targets lie in records already loaded
    if (band) {
      const int pos = nb + rank_in_mask(mb);
      sE[pos] = u;
      sI[pos] = kw;
    }
    na += __popcll(mu);
    nb += __popcll(mb);
  };
  // groups of 4 consecutive records per lane (256 per wave step), the next
  // group's loads issued before the current group is visited
  float4 ev = l < n4 ? e4[l] : float4{0.f, 0.f, 0.f, 0.f};
  int4 iv = l < n4 ? i4[l] : int4{0, 0, 0, 0};
  for (int g0 = 0; g0 < n4; g0 += kWave) {
    const bool in = g0 + l < n4;
    const int gn = g0 + kWave + l;
    const float4 en = gn < n4 ? e4[gn] : float4{0.f, 0.f, 0.f, 0.f};
    const int4 inx = gn < n4 ? i4[gn] : int4{0, 0, 0, 0};
    visit(in, ev.x, iv.x);
    visit(in, ev.y, iv.y);
    visit(in, ev.z, iv.z);
    visit(in, ev.w, iv.w);
    ev = en;
    iv = inx;
  }
  {
    const int i = 4 * n4 + l;
    const bool in = i < n;
    visit(in, in ? sE[i] : 0.f, in ? sI[i] : 0);
  }
  a_lo = wave_min(a_lo);
  z_hi = wave_max(z_hi);
  const int need = k - na;
  const bool stats = p.flags & 8u;
  low = -__builtin_inff();
  if (need < 1 || nb < need) {
    if (need < 1) low = t_hi;  // k or more keys score above t_hi
    if (stats && l == 0) atomicAdd(&p.header[H_FAIL_COUNT], 1u);
    return false;
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  // exact scores of the band, 64 records at a time; the next group's key
  // indices and scales are loaded one group ahead. With MQA_FLAG_STATS the
  // largest |exact - FP8| / bound of the band goes to the header (a check of
  // the bound on the hardware that runs it).
  float ratio = 0.f;
  int keyidx[4];
  float sc = 0.f;
  auto group_refs = [&](int b0, int* ki, float& s_) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int j = b0 + 16 * t + (l & 15);
      ki[t] = sI[j < nb ? j : nb - 1] & (int)kKeyMask;
    }
    const int j = b0 + l;
    s_ = scan_scale<SRC>(p, sI[j < nb ? j : nb - 1] & (int)kKeyMask, req);
  };
  group_refs(0, keyidx, sc);
  for (int b0 = 0; b0 < nb; b0 += kWave) {
    KeyTile kt;
    load_keys_rows<SRC>(kt, p, keyidx, req);
    int kn[4] = {0, 0, 0, 0};
    float scn = 0.f;
    if (b0 + kWave < nb) group_refs(b0 + kWave, kn, scn);
    const int j = b0 + l;
    const float E = exact_score(qr, qr2, kt, sc);
    if (j < nb) {
      const int kw = sI[j];
      if (stats) {
        const float bb = bnd(kw);
        const float dev = __builtin_fabsf(E - (sE[j] - bb));
        ratio = __builtin_fmaxf(ratio, bb > 0.f ? dev / bb : (dev > 0.f ? 1e30f : 0.f));
      }
      sE[j] = E;
      sI[j] = kw & (int)kKeyMask;
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) keyidx[t] = kn[t];
    sc = scn;
  }
  if (stats) {
    ratio = wave_max(ratio);
    if (l == 0) atomicMax(&p.header[H_ERRMAX], __float_as_uint(ratio));
  }
  if (l == 0 && stats)
    atomicAdd(reinterpret_cast<unsigned long long*>(&p.header[H_BAND_LO]), (unsigned long long)nb);
  auto take = [&](int slot, float, int idx) { emit(na + slot, idx); };
  const bool det = det_mode(p);
  const float tau = det ? wave_select_lowkey(sE, sI, nb, need, hist, take)
      : nb <= 256 ? small_select(sE, sI, nb, need, take)
                  : wave_select(sE, sI, nb, need, hist, take);
  low = __builtin_fminf(tau, a_lo);
  // taken records above tau, dropped ones and non-candidates below it
  // (ties at tau are allowed outside the band unless the mode is
  // deterministic)
  const bool ok_a = det ? a_lo > tau : a_lo >= tau;
  const bool ok_z = det ? z_hi < tau : z_hi <= tau;
  const bool ok_nc = (thi_lt || !det) ? Thi <= tau : Thi < tau;
  if (stats && l == 0 && !(ok_a && ok_z && ok_nc))
    atomicAdd(&p.header[!ok_a ? H_FAIL_ABOVE : (!ok_z ? H_FAIL_BELOW : H_FAIL_ADMIT)], 1u);
  return ok_a && ok_z && ok_nc;
}

// Queue row r (of block r / 32) for the exact rescan; each block is queued
// once.
__device__ __forceinline__ void queue_exact(const FusedParams& p, int r) {
  if (lane_id() != 0) return;
  p.xrow[r] = 1;
  const int b = block_of(p, r);
  if (atomicExch(&p.xflag[b], 1u) == 0u) p.xqueue[atomicAdd(&p.header[H_XQ], 1u)] = b;
}

// Queue row r for the bounded rescan: every visible key is scored exactly and
// the keys scoring >= low (a lower bound of the row's k-th exact score) are
// appended to the row's slab.
__device__ __forceinline__ void queue_rescan(const FusedParams& p, int r, float low) {
  if (lane_id() != 0) return;
  p.rowinfo[r].thr = low;
  p.rowinfo[r].cnt = 0;
  p.rowinfo[r].strict = 0;
  p.rowinfo[r].above = 0;
  p.rowinfo[r].filled = 0;
  p.rqueue[atomicAdd(&p.header[H_RQ], 1u)] = r;
}

// Select: one wave per row.
// H2: 64 index heads (rows of two 32-head halves); a separate instance, so
// that the 32-head select keeps its registers.
template <int SRC, bool H2>
__global__ __launch_bounds__(kSelWaves * kWave) __attribute__((amdgpu_waves_per_eu(H2 ? 2 : 4))) void fused_select_kernel(FusedParams p) {
  __shared__ uint32_t hist[kSelWaves][kHistWords];
  const int w = wave_id();
  const int l = lane_id();
  const int k = p.topk;
  const int r = blockIdx.x * kSelWaves + w;
  if (r >= p.rows) return;
  const bool stats = p.flags & 8u;
  const RowInfo ri = p.rowinfo[r];
  if (ri.mode == M_SHORT || ri.mode == M_OFF) return;
  bool ok = false;
  float low = -__builtin_inff();
  const bool forced = ri.mode != M_EXACT && (p.flags & 32u);  // rescan from an open bound
  float* sE = p.slabE + (int64_t)r * kSlabRow;
  int32_t* sI = p.slabI + (int64_t)r * kSlabRow;
  // candidates and admission bound: the row's, or the union of its key
  // segments' (moved down to one run at the start of the slab row; thi bounds
  // every other key's exact score from above)
  int cnt = ri.cnt;
  float thi = ri.thr;
  if (p.nseg > 1 && ri.mode != M_EXACT) {
    const int region = kSlabRow / p.nseg;
    cnt = 0;
    thi = -__builtin_inff();
    for (int sg = 0; sg < p.nseg; ++sg) {
      const SegInfo si = p.seg[(int64_t)r * kMaxSeg + sg];
      thi = __builtin_fmaxf(thi, si.thr);
      const int src = sg * region;
      // forward copy to a lower offset: no lane reads a record already written
      if (sg > 0 && src != cnt) {
        for (int i = l; i < si.cnt; i += kWave) {
          const float e = sE[src + i];
          const int32_t x = sI[src + i];
          sE[cnt + i] = e;
          sI[cnt + i] = x;
        }
      }
      cnt += si.cnt;
    }
  }
  if (ri.mode != M_EXACT && !forced) {
    if (cnt >= k) {
      int s, e;
      row_range(p, r, s, e);
      QueryRow qr, qr2;
      load_query(qr, p.q, p.weights, r);
      if constexpr (H2) load_query(qr2, p.q, p.weights, r + 1);
      int32_t* o = out_row(p, r);
      // non-candidates score below the bound unless a merge raised it (then
      // at most it); split rows are taken as raised
      const bool thi_lt = p.nseg == 1 && ri.strict == 0;
      // the histogram's range from the gate: [thr, m0 + (m0 - thr)], m0 the
      // maximum U of the gate's first sample tile
      float hlo = 0.f, hhi = 0.f;
      if (ri.mode == M_GATED && p.nseg == 1 && ri.strict == 0) {
        const float m0 = p.rinfo[r].m0;
        hlo = ri.thr;
        hhi = m0 + (m0 - ri.thr);
      }
      const int req = p.dec_rows ? r / p.dec_rows : 0;
      ok = select_interval<SRC>(p, sE, sI, cnt, k, beta_of(p, r), thi, thi_lt, hlo, hhi, qr,
                                H2 ? &qr2 : nullptr, req, hist[w], low,
                                [&](int sl, int idx) { o[sl] = idx - s; });
      if (stats && l == 0) {
        atomicAdd(&p.header[ok ? H_GATED : H_UNCERT], 1u);
        atomicAdd(reinterpret_cast<unsigned long long*>(&p.header[H_CAND_LO]),
                  (unsigned long long)cnt);
      }
    } else if (stats && l == 0) {
      atomicAdd(&p.header[H_UNDER], 1u);
    }
  }
  if (!ok) {
    if (forced || low > -__builtin_inff())
      queue_rescan(p, r, low);
    else
      queue_exact(p, r);
  }
}

// ---------------------------------------------------------------------------
// Bounded rescan of the queued rows, in up to three rounds. Work item i of a
// round covers keys [kRescanKeys * (i / ng), kRescanKeys * (i / ng + 1)) of
// the queued rows of group i % ng (groups of R consecutive queue entries;
// slice-major, so that the waves working at one time share their keys in L2);
// one wave per item, claimed from the round's counter. The group's rows share
// each 64-key tile: exact scores (the band rescoring's bf16 MFMA) of 64 keys
// at a time for each row whose range meets them; keys scoring >= the row's
// bound (> in a strict round) get slab slots from the row's counter (slots
// past the slab are counted, not written), and the keys strictly above it are
// counted apart. (64 heads and decode calls take one row per item: a 64-head
// row already holds two query halves, and decode rows of different requests
// read different keys.)
constexpr int kRescanGroup = 3;
template <int SRC, bool H2>
__global__ __launch_bounds__(kThreads) void fused_rescan_kernel(FusedParams p, int round) {
  constexpr int R = (H2 || SRC == SRC_DECODE) ? 1 : kRescanGroup;
  const int l = lane_id();
  const int nq = (int)p.header[H_RQ + 2 * round];
  const int32_t* queue = p.rqueue + (int64_t)round * p.nblocks * kBlockRows;
  const int nsl = (p.keys + kRescanKeys - 1) / kRescanKeys;
  const int ng = (nq + R - 1) / R;
  const int items = ng * nsl;
  if (items == 0) return;  // no claims (one contended counter) when nothing is queued
  for (;;) {
    int it = 0;
    if (l == 0) it = (int)atomicAdd(&p.header[H_RCLAIM + 2 * round], 1u);
    it = __shfl(it, 0, 64);
    if (it >= items) break;
    const int grp = it % ng;
    const int slice = it / ng;
    int rr[R], ka[R], kb[R];
    int lo = p.keys, hi = 0;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int qi = grp * R + i;
      rr[i] = qi < nq ? queue[qi] : -1;
      ka[i] = kb[i] = 0;
      if (rr[i] >= 0) {
        int s, e;
        row_range(p, rr[i], s, e);
        ka[i] = s > slice * kRescanKeys ? s : slice * kRescanKeys;
        kb[i] = e < (slice + 1) * kRescanKeys ? e : (slice + 1) * kRescanKeys;
        if (ka[i] < kb[i]) {
          lo = ka[i] < lo ? ka[i] : lo;
          hi = kb[i] > hi ? kb[i] : hi;
        }
      }
    }
    if (lo >= hi) continue;
    const int req = p.dec_rows ? rr[0] / p.dec_rows : 0;
    QueryRowB qb[R], qb2;
    float low[R];
    bool strict[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int r = rr[i] >= 0 ? rr[i] : rr[0];
      QueryRow qr;
      load_query(qr, p.q, p.weights, r);
      to_bf16(qb[i], qr);
      if constexpr (H2) {
        load_query(qr, p.q, p.weights, r + 1);
        to_bf16(qb2, qr);
      }
      low[i] = p.rowinfo[r].thr;
      strict[i] = p.rowinfo[r].strict != 0;
    }
    for (int k0 = lo; k0 < hi; k0 += kWave) {
      int keyidx[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int j = k0 + 16 * t + (l & 15);
        keyidx[t] = j < hi ? j : hi - 1;
      }
      KeyTile kt;
      load_keys_rows<SRC>(kt, p, keyidx, req);
      const int key = k0 + l;
      const float sc = scan_scale<SRC>(p, key < hi ? key : hi - 1, req);
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const bool valid = key >= ka[i] && key < kb[i];
        if (__ballot(valid) == 0) continue;
        const int r = rr[i];
        const float E = exact_score(qb[i], H2 ? &qb2 : nullptr, kt, sc);
        const bool pass = valid && (strict[i] ? E > low[i] : E >= low[i]);
        const uint64_t m = __ballot(pass);
        if (m == 0) continue;
        const uint64_t ma = __ballot(valid && E > low[i]);
        int base = 0;
        if (l == 0) {
          base = atomicAdd(&p.rowinfo[r].cnt, __popcll(m));
          if (!strict[i] && ma) atomicAdd(&p.rowinfo[r].above, __popcll(ma));
        }
        base = __shfl(base, 0, 64);
        const int pos = base + rank_in_mask(m);
        if (pass && pos < kSlabRow) {
          p.slabE[(int64_t)r * kSlabRow + pos] = E;
          p.slabI[(int64_t)r * kSlabRow + pos] = key;
        }
      }
    }
  }
}

// Top-k of each row of a bounded-rescan round from its slab (one wave per
// row). A row whose keys at or above its bound overfilled the slab gets, in
// the first two rounds, another round: over the keys at or above the k-th best
// exact score among the slab's records when that is a higher bound, else over
// the keys strictly above the bound when k of them are; a row with fewer than
// k such keys, or still too many, goes on to the exact streaming rescan.
__global__ __launch_bounds__(kSelWaves * kWave) void fused_finish_kernel(FusedParams p,
                                                                         int round) {
  __shared__ uint32_t hist[kSelWaves][kHistWords];
  const int w = wave_id();
  const int l = lane_id();
  const int k = p.topk;
  const int nq = (int)p.header[H_RQ + 2 * round];
  const int64_t qrows = (int64_t)p.nblocks * kBlockRows;
  for (int qi = blockIdx.x * kSelWaves + w; qi < nq; qi += gridDim.x * kSelWaves) {
    const int r = p.rqueue[round * qrows + qi];
    const int cnt = p.rowinfo[r].cnt;
    const int filled = p.rowinfo[r].filled;
    const int need = k - filled;  // slots [need, k) were filled by round 0
    float* sE = p.slabE + (int64_t)r * kSlabRow;
    int32_t* sI = p.slabI + (int64_t)r * kSlabRow;
    int s, e;
    row_range(p, r, s, e);
    int32_t* o = out_row(p, r);
    if (cnt >= need && cnt <= kSlabRow) {
      auto put = [&](int sl, float, int idx) { o[sl] = idx - s; };
      if (det_mode(p))
        wave_select_lowkey(sE, sI, cnt, need, hist[w], put);
      else
        wave_select(sE, sI, cnt, need, hist[w], put);
      if ((p.flags & 8u) && l == 0) atomicAdd(&p.header[H_RESCAN], 1u);
      continue;
    }
    if (round + 1 < kRescanRounds && cnt > kSlabRow) {
      // Too many keys at or above the bound. The k-th best stored score is a
      // higher bound when it exceeds it (the second round then takes the keys
      // at or above it); else, when k keys score strictly above the bound
      // (the rest tie with it, e.g. relu's exact zeros), the second round
      // takes those; else the k-th score is the bound itself: stored ties of
      // it fill the last k - above slots and the second round takes the
      // `above` keys strictly above it (not in the deterministic mode, whose
      // ties go to the smallest keys, not to the stored ones).
      const int above = p.rowinfo[r].above;
      const float thr = p.rowinfo[r].thr;
      const float low = wave_kth_value(sE, kSlabRow, k, hist[w]);
      int fill = 0;
      if (!(low > thr) && above < k && !det_mode(p)) {
        fill = k - above;
        int got = 0;
        for (int i0 = 0; i0 < kSlabRow && got < fill; i0 += kWave) {
          const int i = i0 + l;
          const bool tie = i < kSlabRow && sE[i] == thr;
          const uint64_t m = __ballot(tie);
          const int slot = got + rank_in_mask(m);
          if (tie && slot < fill) o[above + slot] = sI[i] - s;
          got += __popcll(m);
        }
        if (got < fill) fill = -1;  // cannot happen: the slab holds >= k - above ties
      }
      if (low > thr || above >= k || fill > 0) {
        if (fill > 0 && above == 0) {
          if ((p.flags & 8u) && l == 0) atomicAdd(&p.header[H_RESCAN], 1u);
          continue;  // every slot holds a tie of the k-th score
        }
        if (l == 0) {
          p.rowinfo[r].thr = low > thr ? low : thr;
          p.rowinfo[r].cnt = 0;
          p.rowinfo[r].above = 0;
          p.rowinfo[r].strict = low > thr ? 0 : 1;
          p.rowinfo[r].filled = low > thr || above >= k ? 0 : fill;
          p.rqueue[(round + 1) * qrows + atomicAdd(&p.header[H_RQ + 2 * (round + 1)], 1u)] = r;
        }
        continue;
      }
    }
    queue_exact(p, r);
  }
}

// ---------------------------------------------------------------------------
// Exact rescan of the queued blocks: exact (bf16 MFMA) scores of every key of
// the flagged rows with a streaming top-k merge, then an exact select.
template <int SRC>
__global__ __launch_bounds__(kThreads) void fused_exact_kernel(FusedParams p) {
  __shared__ ScanSmem sm;
  MQA_DECLARE_STAGES(stg, SRC);
  const int tid = threadIdx.x;
  const int w = wave_id();
  const int l = lane_id();
  const int k = p.topk;
  const int nq = (int)p.header[H_XQ];
  for (;;) {
    if (tid == 0) sm.block = (int)atomicAdd(&p.header[H_XCLAIM], 1u);
    __syncthreads();
    const int qi = sm.block;
    if (qi >= nq) break;
    const int b = p.xqueue[qi];
    RowState rs[kRowsPerWave];
    QueryRow qr[kRowsPerWave];
    wave_rows<SRC>(p, b, rs);
    int wlo = p.keys, whi = 0;
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      RowState& r = rs[i];
      zero_query(qr[i]);
      if (r.r >= p.rows || r.e - r.s <= k || !p.xrow[r.r]) continue;
      r.mode = M_EXACT;
      load_query(qr[i], p.q, p.weights, r.r);
      wlo = r.s < wlo ? r.s : wlo;
      whi = r.e > whi ? r.e : whi;
    }
    load_partners(p, rs, qr, nullptr, M_EXACT, 1.f);
    int lo, hi, unused;
    block_union(sm.wlo, sm.whi, sm.wf, wlo, whi, 0, p.keys, lo, hi, unused);
    if (hi > lo) {
      SlabRefs sr = slab_refs<SRC>(p, b, sm.hist[w], k);
      FoldOp none;
      scan_rows<true, SRC>(p, stg, qr, none, rs, M_EXACT, lo, hi, sr,
                           b * (SRC == SRC_DECODE ? kDecPack : 1), wave_group<SRC>(w));
#pragma unroll
      for (int i = 0; i < kRowsPerWave; ++i) {
        RowState& r = rs[i];
        if (r.mode != M_EXACT) continue;
        int32_t* o = out_row(p, r.r);
        const int base = r.s;
        const int have = r.cnt;
        auto put = [&](int sl, float, int idx) { o[sl] = idx - base; };
        if (det_mode(p))
          wave_select_lowkey(sr.sE(i), sr.sI(i), have, k, sr.hist, put);
        else
          wave_select(sr.sE(i), sr.sI(i), have, k, sr.hist, put);
        for (int j = have + l; j < k; j += kWave) o[j] = -1;
        if ((p.flags & 8u) && l == 0) atomicAdd(&p.header[H_EXACT], 1u);
      }
    }
    __syncthreads();
  }
}

}  // namespace mqa

namespace mqa {

// Ascending bitonic sort of the 64 * E ints at o (16-byte aligned), one wave,
// in registers: lane l holds elements l * E .. l * E + E - 1; stages whose
// stride is below E compare within a lane, the others with lane l ^ (stride /
// E) through a lane-xor shuffle.
template <int E>
__device__ __forceinline__ void wave_sort_asc(int32_t* o) {
  const int l = lane_id();
  int v[E];
  int4* o4 = reinterpret_cast<int4*>(o + l * E);
#pragma unroll
  for (int j = 0; j < E / 4; ++j) {
    const int4 x = o4[j];
    v[4 * j] = x.x;
    v[4 * j + 1] = x.y;
    v[4 * j + 2] = x.z;
    v[4 * j + 3] = x.w;
  }
  for (int size = 2; size <= kWave * E; size <<= 1) {
    // cross-lane stages (stride >= E)
    for (int stride = size >> 1; stride >= E; stride >>= 1) {
      const int lm = stride / E;
      const bool lower = (l & lm) == 0;
#pragma unroll
      for (int j = 0; j < E; ++j) {
        const int p = __shfl_xor(v[j], lm, 64);
        const bool up = ((l * E + j) & size) == 0;
        v[j] = lower == up ? (v[j] < p ? v[j] : p) : (v[j] > p ? v[j] : p);
      }
    }
    // in-lane stages (stride < E, compile-time strides: constant register
    // indices)
#pragma unroll
    for (int stride = E / 2; stride > 0; stride >>= 1) {
      if (stride >= size) continue;
#pragma unroll
      for (int j = 0; j < E; ++j) {
        if (j & stride) continue;  // the pair (j, j + stride)
        const bool up = ((l * E + j) & size) == 0;
        const int a = v[j], b = v[j + stride];
        const int mn = a < b ? a : b, mx = a < b ? b : a;
        v[j] = up ? mn : mx;
        v[j + stride] = up ? mx : mn;
      }
    }
  }
#pragma unroll
  for (int j = 0; j < E / 4; ++j) o4[j] = int4{v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]};
}

// Deterministic mode, last launch: each row with more than k visible keys has
// its k output keys sorted ascending (one wave per row, wave_sort_asc; k is
// 512, 1024 or 2048). Rows with n <= k already hold 0..n-1 and their -1
// padding.
__global__ __launch_bounds__(kSelWaves * kWave) void fused_sort_kernel(FusedParams p) {
  const int r = blockIdx.x * kSelWaves + wave_id();
  if (r >= p.rows || partner_row(p, r)) return;
  const int k = p.topk;
  int s, e;
  row_range(p, r, s, e);
  if (e - s <= k) return;
  int32_t* o = out_row(p, r);
  if (k == 2048)
    wave_sort_asc<32>(o);
  else if (k == 1024)
    wave_sort_asc<16>(o);
  else
    wave_sort_asc<8>(o);
}

}  // namespace mqa

namespace mqa {

// ---------------------------------------------------------------------------
// Consumer rows of DeepSeek-V4.1's two-level candidate selection (vLLM PR
// #60618, "Limitations of this PR -- TODOs": the consumer layers mask their
// scores to the source layer's blocks before their top-k). Row r keeps only
// the keys of its listed blocks of 8 (entry j names keys 8 (j + s / 8) ..
// + 7, inside [s, e); entries < 0 are padding), scores them exactly (the
// band rescoring's bf16 MFMA, so no FP8 bound is involved) into its slab (at
// most 8 nb <= 16384 keys) and selects their top-k there. One wave per row;
// in the deterministic mode the ties of the k-th score go to the smallest
// keys and the row is sorted by key.
// Blocks of 8 keys per row in the two-level selection's block lists.
constexpr int kNbo = 2048;

__global__ __launch_bounds__(kSelWaves * kWave) void masked_topk_kernel(FusedParams p,
                                                                        const int32_t* blocks,
                                                                        int nb) {
  // (the wave's histogram words hold its row's block list until the select)
  static_assert(kHistWords >= kNbo, "block list in the histogram words");
  __shared__ uint32_t hist[kSelWaves][kHistWords];
  int32_t* blw = reinterpret_cast<int32_t*>(hist[wave_id()]);
  const int w = wave_id();
  const int l = lane_id();
  const int k = p.topk;
  const int r = blockIdx.x * kSelWaves + w;
  if (r >= p.rows) return;
  int s, e;
  row_range(p, r, s, e);
  int32_t* o = p.out + (int64_t)r * k;
  float* sE = p.slabE + (int64_t)r * kSlabRow;
  int32_t* sI = p.slabI + (int64_t)r * kSlabRow;
  const int32_t* bl = blocks + (int64_t)r * nb;
  const int64_t b0 = s >> 3;
  QueryRowB qb;
  {
    QueryRow qr;
    load_query(qr, p.q, p.weights, r);
    to_bf16(qb, qr);
  }
  // the row's block list, in LDS (each group of 64 keys reads 8 entries)
  for (int j = l; j < nb; j += kWave) blw[j] = bl[j];
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  int cnt = 0;
  // key of chunk position c (block c0 + c / 8, offset c % 8), or -1
  auto key_at = [&](int c0, int c) -> int {
    const int j = c0 + (c >> 3);
    const int bid = j < nb ? blw[j] : -1;
    if (bid < 0) return -1;
    const int64_t key = (bid + b0) * 8 + (c & 7);
    return (key >= s && key < e) ? (int)key : -1;
  };
  // two groups of 64 keys per step: both groups' key gathers are in flight
  // before either is scored
  for (int c00 = 0; c00 < nb && e > s; c00 += 16) {
    KeyTile kt[2];
    float sc[2];
    int key[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c0 = c00 + 8 * u;
      int keyidx[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int kk = key_at(c0, 16 * t + (l & 15));
        keyidx[t] = kk >= 0 ? kk : s;
      }
      load_keys_rows<SRC_GATHER>(kt[u], p, keyidx);
      key[u] = key_at(c0, l);
      sc[u] = p.scales[key[u] >= 0 ? key[u] : s];
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const bool valid = key[u] >= 0;
      const float E = exact_score(qb, kt[u], sc[u]);
      const uint64_t m = __ballot(valid);
      if (valid) {
        const int pos = cnt + rank_in_mask(m);
        sE[pos] = E;
        sI[pos] = key[u];
      }
      cnt += __popcll(m);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  const bool det = det_mode(p);
  const int m = cnt < k ? cnt : k;
  auto put = [&](int slot, float, int key) { o[slot] = key - s; };
  if (cnt <= k) {
    for (int i = l; i < cnt; i += kWave) o[i] = sI[i] - s;
  } else if (det) {
    wave_select_lowkey(sE, sI, cnt, k, hist[w], put);
  } else {
    wave_select(sE, sI, cnt, k, hist[w], put);
  }
  // padding (the deterministic mode sorts with it at the top of the range)
  for (int i = m + l; i < k; i += kWave) o[i] = det ? 0x7FFFFFFF : -1;
  if (det) {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    if (k == 2048)
      wave_sort_asc<32>(o);
    else if (k == 1024)
      wave_sort_asc<16>(o);
    else
      wave_sort_asc<8>(o);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    for (int i = m + l; i < k; i += kWave) o[i] = -1;
  }
}

// ---------------------------------------------------------------------------
// Source layers of DeepSeek-V4.1's two-level candidate selection (vLLM PR
// #60618, "Limitations of this PR -- TODOs": the source layer also writes,
// per row, the 2048 blocks of 8 keys of largest maximum score). A block is 8
// consecutive keys of the key numbering (block B: keys 8B .. 8B + 7); a row
// names block B as B - s / 8 and scores it by the maximum exact score of its
// visible keys in it.
//
// The block output comes from the key candidates: the gate and the scan of a
// source call run with a key target of at least 2048 (FusedParams.kgate), so
// that a row's candidates (every key whose exact score exceeds the admission
// bound Thi) cover well over 2048 blocks. Then, per row,
//   1. the candidates (in key order, as the scan appends them) are scored
//      exactly and reduced to one record per block: the maximum over the
//      block's candidates, which is the block's true maximum whenever it
//      exceeds Thi (its other keys score at most Thi);
//   2. the 2048 best block records are taken; the result is exact when the
//      2048th best maximum exceeds Thi (every block without a record, and
//      every record at or below Thi, then ranks below it).
// Rows where this does not hold (too few candidate blocks, candidates out of
// key order after a merge, more block records than a wave's merge buffer,
// rows of the exact rescan) go to the exact block scan: every key scored
// exactly, block maxima streamed through a bounded top-2048.

// Rows with at most 2048 visible blocks list them all: 0 .. nb - 1, -1 padded.
__device__ __forceinline__ bool all_blocks(const FusedParams& p, int s, int e, int32_t* ob) {
  const int nb = e > s ? (e - 1) / 8 - s / 8 + 1 : 0;
  if (nb > kNbo) return false;
  for (int i = lane_id(); i < kNbo; i += kWave) ob[i] = i < nb ? i : -1;
  return true;
}

// Queue row r for the exact block scan.
__device__ __forceinline__ void queue_block_scan(const FusedParams& p, int r) {
  if (lane_id() == 0) p.bqueue[atomicAdd(&p.header[H_BQ], 1u)] = r;
}

// The top-2048 of n block records (tE, tI) into ob as block - b0, -1 padded;
// deterministic mode: the smallest blocks at a tie, sorted. Returns the
// smallest selected maximum.
__device__ __forceinline__ float take_blocks(const FusedParams& p, float* tE, int32_t* tI, int n,
                                             int b0, int32_t* ob, uint32_t* hist) {
  const int l = lane_id();
  const bool det = det_mode(p);
  auto put = [&](int slot, float, int blk) { ob[slot] = blk - b0; };
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  const float tau = det ? wave_select_lowkey(tE, tI, n, kNbo, hist, put)
                        : wave_select(tE, tI, n, kNbo, hist, put);
  const int m = n < kNbo ? n : kNbo;
  for (int i = m + l; i < kNbo; i += kWave) ob[i] = det ? 0x7FFFFFFF : -1;
  if (det) {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    wave_sort_asc<32>(ob);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    for (int i = m + l; i < kNbo; i += kWave) ob[i] = -1;
  }
  return tau;
}

// Steps 1-2 above, one wave per row (persistent: the waves' merge buffers
// hold the block records).
__global__ __launch_bounds__(kThreads) void block_select_kernel(FusedParams p) {
  __shared__ uint32_t hist[kWaves][kHistWords];
  const int w = wave_id();
  const int l = lane_id();
  float* tE = tmp_e(p);
  int32_t* tI = tmp_i(p);
  for (int r = blockIdx.x * kWaves + w; r < p.rows; r += gridDim.x * kWaves) {
    int s, e;
    row_range(p, r, s, e);
    int32_t* ob = p.blocks_out + (int64_t)r * kNbo;
    if (all_blocks(p, s, e, ob)) continue;
    const RowInfo ri = p.rowinfo[r];
    if (ri.mode != M_GATED && ri.mode != M_ALL) {
      queue_block_scan(p, r);
      continue;
    }
    QueryRowB qb;
    {
      QueryRow qr;
      load_query(qr, p.q, p.weights, r);
      to_bf16(qb, qr);
    }
    const int32_t* sI = p.slabI + (int64_t)r * kSlabRow;
    const int nseg = p.nseg;
    const int region = kSlabRow / nseg;
    float thi = -__builtin_inff();
    int nbk = 0;          // block records written
    int cur = -1;         // the block carried over from the previous group
    float curm = -__builtin_inff();
    int last = -1;        // the last candidate key seen
    bool ok = true;
    for (int sg = 0; sg < nseg && ok; ++sg) {
      int cnt;
      if (nseg > 1) {
        const SegInfo si = p.seg[(int64_t)r * kMaxSeg + sg];
        thi = __builtin_fmaxf(thi, si.thr);
        cnt = si.cnt;
      } else {
        thi = ri.thr;
        cnt = ri.cnt;
      }
      const int32_t* I = sI + (nseg > 1 ? sg * region : 0);
      // two groups of 64 records per step: both groups' key gathers are in
      // flight before either is scored
      for (int i00 = 0; i00 < cnt && ok; i00 += 2 * kWave) {
        int key[2];
        KeyTile kt[2];
        float sc[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int i = i00 + u * kWave + l;
          key[u] = i < cnt ? (I[i] & (int)kKeyMask) : 0x7FFFFFFF;
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int i0 = i00 + u * kWave;
          const int nv = cnt - i0 < kWave ? (cnt - i0 > 0 ? cnt - i0 : 1) : kWave;
          const int lastk = __shfl(key[u], nv - 1, 64);
          int keyidx[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int j = 16 * t + (l & 15);
            const int kk = __shfl(key[u], j, 64);
            keyidx[t] = j < nv && i0 < cnt ? kk : (i0 < cnt ? lastk : 0);
          }
          load_keys_rows<SRC_GATHER>(kt[u], p, keyidx);
          const int ks = __shfl(keyidx[0], 0, 64);
          sc[u] = p.keyinfo[2 * (int64_t)(i0 + l < cnt ? key[u] : ks)];
        }
        float Es[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) Es[u] = exact_score(qb, kt[u], sc[u]);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int i0 = i00 + u * kWave;
          if (i0 >= cnt || !ok) break;
          const bool valid = i0 + l < cnt;
          const int k1 = key[u];
          // key order (the scan appends ascending keys; a merge may not keep it)
          int prev = __shfl_up(k1, 1, 64);
          prev = l == 0 ? last : prev;
          if (__ballot(valid && k1 <= prev)) {
            ok = false;
            break;
          }
          const int blk = valid ? k1 >> 3 : 0x7FFFFFFF;
          // the maximum over each run of one block's records (at most 8 long)
          float m = valid ? Es[u] : -__builtin_inff();
#pragma unroll
          for (int d = 1; d < 8; d <<= 1) {
            const float om = __shfl_up(m, d, 64);
            const int ob2 = __shfl_up(blk, d, 64);
            if (l >= d && ob2 == blk) m = __builtin_fmaxf(m, om);
          }
          // (wave-uniform) the carried block ended with the previous group:
          // its record; else it continues in this group's first run
          if (cur >= 0 && __shfl(blk, 0, 64) != cur) {
            if (l == 0 && nbk < kTmp) {
              tE[nbk] = curm;
              tI[nbk] = cur;
            }
            ++nbk;
            cur = -1;
          }
          if (blk == cur) m = __builtin_fmaxf(m, curm);
          // a run ends where the next record's block differs; the group's last
          // run is carried into the next group
          const int nxt = __shfl_down(blk, 1, 64);
          const int nv = cnt - i0 < kWave ? cnt - i0 : kWave;  // valid records in this group
          const bool lastv = l == nv - 1;
          const bool end = valid && !lastv && nxt != blk;
          const uint64_t em = __ballot(end);
          if (end) {
            const int pos = nbk + rank_in_mask(em);
            if (pos < kTmp) {
              tE[pos] = m;
              tI[pos] = blk;
            }
          }
          nbk += __popcll(em);
          cur = __shfl(blk, nv - 1, 64);
          curm = __shfl(m, nv - 1, 64);
          last = __shfl(k1, nv - 1, 64);
        }
      }
    }
    if (ok && cur >= 0) {
      if (l == 0 && nbk < kTmp) {
        tE[nbk] = curm;
        tI[nbk] = cur;
      }
      ++nbk;
    }
    // certified when the 2048th best block maximum exceeds the admission bound
    if (!ok || nbk > kTmp || nbk < kNbo ||
        !(take_blocks(p, tE, tI, nbk, s >> 3, ob, hist[w]) > thi))
      queue_block_scan(p, r);
  }
}

// Exact maxima of the 8 blocks of 64 keys from key0 (key0 % 8 == 0) over a
// row's visible range [s, e): lane 8i holds block (key0 >> 3) + i's maximum,
// -inf for a block with no visible key (every lane of a block holds it).
__device__ __forceinline__ void block_max_load(const FusedParams& p, int key0, int s, int e,
                                               KeyTile& kt, float& sc) {
  const int l = lane_id();
  int keyidx[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int j = key0 + 16 * t + (l & 15);
    keyidx[t] = j < s ? s : (j >= e ? e - 1 : j);
  }
  load_keys_rows<SRC_GATHER>(kt, p, keyidx);
  const int key = key0 + l;
  sc = p.keyinfo[2 * (int64_t)(key >= s && key < e ? key : s)];
}
__device__ __forceinline__ float block_max_score(const QueryRowB& qb, const KeyTile& kt, float sc,
                                                 int key0, int s, int e) {
  const int key = key0 + lane_id();
  float m = exact_score(qb, kt, sc);
  m = key >= s && key < e ? m : -__builtin_inff();
  m = __builtin_fmaxf(m, __shfl_xor(m, 1, 64));
  m = __builtin_fmaxf(m, __shfl_xor(m, 2, 64));
  return __builtin_fmaxf(m, __shfl_xor(m, 4, 64));
}

// The exact block scan of the queued rows. When every queued row's block
// maxima fit the merge buffers (the usual case: a few rows), the rows' key
// ranges are split into pieces of kBlockPiece keys that the whole grid's
// waves take one at a time; each piece writes its blocks' maxima to the
// row's array of block records in the merge buffers (row q at q * stride),
// and block_take_kernel selects each row's 2048 from them. Otherwise each
// wave takes whole rows: 64 keys at a time from the row's first 8-aligned
// key, block records at or above the current bound appended to the first half
// of the wave's merge buffer; when it fills, its best 2048 (and the ties of
// the 2048th, in the room left) move to the other half, become the first
// half's contents, and later records must beat the new bound. Block records
// arrive in block order, and the moves keep the ties in that order, so the
// deterministic mode's smallest-block rule holds either way.
constexpr int kBlockPiece = 8192;

__device__ __forceinline__ int64_t block_stride(const FusedParams& p) {
  return (((int64_t)p.keys + 7) / 8 + 1 + 63) & ~(int64_t)63;
}
__device__ __forceinline__ bool block_split(const FusedParams& p, int nq) {
  return (int64_t)nq * block_stride(p) <= (int64_t)gridDim.x * kWaves * kTmp;
}

__global__ __launch_bounds__(kThreads) void block_scan_kernel(FusedParams p) {
  __shared__ uint32_t hist[kWaves][kHistWords];
  const int w = wave_id();
  const int l = lane_id();
  const int nq = (int)p.header[H_BQ];
  if (nq == 0) return;
  if (block_split(p, nq)) {
    // pieces: (queued row q, piece g), g < pieces per row
    const int64_t stride = block_stride(p);
    const int per_row = (p.keys + 7) / kBlockPiece + 1;
    float* bE = p.tmpE;
    int32_t* bI = p.tmpI;
    for (;;) {
      int it = 0;
      if (l == 0) it = (int)atomicAdd(&p.header[H_BCLAIM], 1u);
      it = __shfl(it, 0, 64);
      if (it >= nq * per_row) break;
      const int q = it / per_row, g = it % per_row;
      const int r = p.bqueue[q];
      int s, e;
      row_range(p, r, s, e);
      const int a = (s & ~7) + g * kBlockPiece;
      if (a >= e) continue;
      const int b = a + kBlockPiece < e ? a + kBlockPiece : e;
      QueryRowB qb;
      {
        QueryRow qr;
        load_query(qr, p.q, p.weights, r);
        to_bf16(qb, qr);
      }
      const int b0 = s >> 3;
      float* oE = bE + q * stride;
      int32_t* oI = bI + q * stride;
      for (int key0 = a; key0 < b; key0 += 2 * kWave) {
        KeyTile kt[2];
        float sc[2];
        block_max_load(p, key0, s, e, kt[0], sc[0]);
        const bool two = key0 + kWave < b;
        if (two) block_max_load(p, key0 + kWave, s, e, kt[1], sc[1]);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          if (u == 1 && !two) break;
          const int k0 = key0 + u * kWave;
          const float m = block_max_score(qb, kt[u], sc[u], k0, s, e);
          const int blk = (k0 + l) >> 3;
          if ((l & 7) == 0 && k0 + l < e) {
            oE[blk - b0] = m;
            oI[blk - b0] = blk;
          }
        }
      }
    }
    return;
  }
  constexpr int kHalf = kTmp / 2;
  float* aE = tmp_e(p);
  int32_t* aI = tmp_i(p);
  float* bE = aE + kHalf;
  int32_t* bI = aI + kHalf;
  for (;;) {
    int qi = 0;
    if (l == 0) qi = (int)atomicAdd(&p.header[H_BCLAIM], 1u);
    qi = __shfl(qi, 0, 64);
    if (qi >= nq) break;
    const int r = p.bqueue[qi];
    int s, e;
    row_range(p, r, s, e);
    QueryRowB qb;
    {
      QueryRow qr;
      load_query(qr, p.q, p.weights, r);
      to_bf16(qb, qr);
    }
    float bound = -__builtin_inff();
    bool strict = false;
    int n = 0;
    for (int key0 = s & ~7; key0 < e; key0 += kWave) {
      KeyTile kt;
      float sc;
      block_max_load(p, key0, s, e, kt, sc);
      const float m = block_max_score(qb, kt, sc, key0, s, e);
      const int key = key0 + l;
      const bool lead = (l & 7) == 0 && m > -__builtin_inff() && (strict ? m > bound : m >= bound);
      const uint64_t lm = __ballot(lead);
      if (lead) {
        const int pos = n + rank_in_mask(lm);
        aE[pos] = m;
        aI[pos] = key >> 3;
      }
      n += __popcll(lm);
      if (n > kHalf - 8) {
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
        float nb;
        const int kept = wave_select_ties(aE, aI, n, kNbo, kHalf - 64, hist[w], nb,
                                          [&](int slot, float v, int idx) {
                                            bE[slot] = v;
                                            bI[slot] = idx;
                                          });
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
        for (int t = l; t < kept; t += kWave) {
          aE[t] = bE[t];
          aI[t] = bI[t];
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
        n = kept;
        bound = nb;
        strict = true;
      }
    }
    take_blocks(p, aE, aI, n, s >> 3, p.blocks_out + (int64_t)r * kNbo, hist[w]);
  }
}

// Split block scan, second step: each queued row's 2048 best blocks from its
// array of block records (one wave per row).
__global__ __launch_bounds__(kThreads) void block_take_kernel(FusedParams p) {
  __shared__ uint32_t hist[kWaves][kHistWords];
  const int nq = (int)p.header[H_BQ];
  if (nq == 0 || !block_split(p, nq)) return;
  const int64_t stride = block_stride(p);
  for (int q = blockIdx.x * kWaves + wave_id(); q < nq; q += gridDim.x * kWaves) {
    const int r = p.bqueue[q];
    int s, e;
    row_range(p, r, s, e);
    const int nb = (e - 1) / 8 - s / 8 + 1;  // > 2048: shorter rows list all blocks
    take_blocks(p, p.tmpE + q * stride, p.tmpI + q * stride, nb, s >> 3,
                p.blocks_out + (int64_t)r * kNbo, hist[wave_id()]);
  }
}

// The launch sequence of one row batch, over one key source.
template <int SRC>
int fused_launch_scan(const FusedParams* p, int grid, hipStream_t stream, hipEvent_t scan_begin,
                      hipEvent_t scan_end);

template <int SRC>
int fused_launch_all(const FusedParams* p, int grid, hipStream_t stream, hipEvent_t scan_begin,
                     hipEvent_t scan_end) {
  hipError_t e;
  // workgroup 0 plans; the others (about one per CU, at most the units of
  // bound work) compute the error bounds
  const int units = (SRC == SRC_DECODE ? 0 : (p->keys + 3) / 4) + p->rows;
  const int waves_per_wg = kPrologueThreads / kWave;
  int bwg = (units + waves_per_wg - 1) / waves_per_wg;
  bwg = bwg < grid ? bwg : grid;
  bwg = bwg < 1 ? 1 : bwg;
  hipLaunchKernelGGL(fused_prologue_kernel<SRC>, dim3(1 + bwg), dim3(kPrologueThreads), 0,
                     stream, *p);
  if ((e = hipGetLastError()) != hipSuccess) return (int)e;
  // paged prefill: the prologue compacted the keys into p->kc; every later
  // kernel reads them there as gathered keys
  if constexpr (SRC == SRC_PAGED) {
    FusedParams g = *p;
    g.k = p->kc;
    g.table = nullptr;
    return fused_launch_scan<SRC_GATHER>(&g, grid, stream, scan_begin, scan_end);
  } else {
    return fused_launch_scan<SRC>(p, grid, stream, scan_begin, scan_end);
  }
}

// Everything after the prologue.
template <int SRC>
int fused_launch_scan(const FusedParams* p, int grid, hipStream_t stream, hipEvent_t scan_begin,
                      hipEvent_t scan_end) {
  hipError_t e;
  hipLaunchKernelGGL(fused_gate_kernel<SRC>, dim3(p->scan_grid), dim3(kThreads), 0, stream, *p);
  if ((e = hipGetLastError()) != hipSuccess) return (int)e;
  hipLaunchKernelGGL(fused_refine_kernel<SRC>, dim3(grid), dim3(kThreads), 0, stream, *p);
  if ((e = hipGetLastError()) != hipSuccess) return (int)e;
  if (scan_begin && (e = hipEventRecord(scan_begin, stream)) != hipSuccess) return (int)e;
  if (p->nseg > 1)
    hipLaunchKernelGGL((fused_topk_kernel<true, SRC>), dim3(p->scan_grid), dim3(kThreads), 0,
                       stream, *p);
  else
    hipLaunchKernelGGL((fused_topk_kernel<false, SRC>), dim3(p->scan_grid), dim3(kThreads), 0,
                       stream, *p);
  if ((e = hipGetLastError()) != hipSuccess) return (int)e;
  if (scan_end && (e = hipEventRecord(scan_end, stream)) != hipSuccess) return (int)e;
  if (SRC == SRC_GATHER && p->blocks_out) {
    // two-level source call: the block output, before the select reorders
    // the slabs
    hipLaunchKernelGGL(block_select_kernel, dim3(grid), dim3(kThreads), 0, stream, *p);
    if ((e = hipGetLastError()) != hipSuccess) return (int)e;
    hipLaunchKernelGGL(block_scan_kernel, dim3(grid), dim3(kThreads), 0, stream, *p);
    if ((e = hipGetLastError()) != hipSuccess) return (int)e;
    hipLaunchKernelGGL(block_take_kernel, dim3(grid), dim3(kThreads), 0, stream, *p);
    if ((e = hipGetLastError()) != hipSuccess) return (int)e;
  }
  const int sel = (p->rows + kSelWaves - 1) / kSelWaves;
  // (64 heads: gathered calls only)
  constexpr bool kH2 = SRC != SRC_DECODE;
  if (kH2 && p->hm == 2)
    hipLaunchKernelGGL((fused_select_kernel<SRC, kH2>), dim3(sel), dim3(kSelWaves * kWave), 0,
                       stream, *p);
  else
    hipLaunchKernelGGL((fused_select_kernel<SRC, false>), dim3(sel), dim3(kSelWaves * kWave), 0,
                       stream, *p);
  if ((e = hipGetLastError()) != hipSuccess) return (int)e;
  const int fin = sel < 256 ? sel : 256;
  for (int round = 0; round < kRescanRounds; ++round) {
    if (kH2 && p->hm == 2)
      hipLaunchKernelGGL((fused_rescan_kernel<SRC, kH2>), dim3(2 * grid), dim3(kThreads), 0,
                         stream, *p, round);
    else
      hipLaunchKernelGGL((fused_rescan_kernel<SRC, false>), dim3(2 * grid), dim3(kThreads), 0,
                         stream, *p, round);
    if ((e = hipGetLastError()) != hipSuccess) return (int)e;
    hipLaunchKernelGGL(fused_finish_kernel, dim3(fin), dim3(kSelWaves * kWave), 0, stream, *p,
                       round);
    if ((e = hipGetLastError()) != hipSuccess) return (int)e;
  }
  hipLaunchKernelGGL(fused_exact_kernel<SRC>, dim3(grid), dim3(kThreads), 0, stream, *p);
  if (p->flags & 64u) {
    if ((e = hipGetLastError()) != hipSuccess) return (int)e;
    hipLaunchKernelGGL(fused_sort_kernel, dim3(sel), dim3(kSelWaves * kWave), 0, stream, *p);
  }
  return (int)hipGetLastError();
}

}  // namespace mqa

extern "C" int mqa_fused_launch(const mqa::FusedParams* p, int grid, hipStream_t stream,
                                hipEvent_t scan_begin, hipEvent_t scan_end) {
  if (p->dec_rows)
    return mqa::fused_launch_all<mqa::SRC_DECODE>(p, grid, stream, scan_begin, scan_end);
  return p->table ? mqa::fused_launch_all<mqa::SRC_PAGED>(p, grid, stream, scan_begin, scan_end)
                  : mqa::fused_launch_all<mqa::SRC_GATHER>(p, grid, stream, scan_begin, scan_end);
}

extern "C" int mqa_masked_launch(const mqa::FusedParams* p, const int32_t* blocks, int nb,
                                 hipStream_t stream) {
  const int g = (p->rows + mqa::kSelWaves - 1) / mqa::kSelWaves;
  hipLaunchKernelGGL(mqa::masked_topk_kernel, dim3(g), dim3(mqa::kSelWaves * mqa::kWave), 0,
                     stream, *p, blocks, nb);
  return (int)hipGetLastError();
}

extern "C" int mqa_fused_occupancy(int* wg_per_cu) {
  // the persistent kernels' workgroups per CU, over the gathered and decode
  // sources (paged prefill runs the gathered kernels)
  const void* kernels[] = {
      reinterpret_cast<const void*>(mqa::fused_topk_kernel<false, mqa::SRC_GATHER>),
      reinterpret_cast<const void*>(mqa::fused_topk_kernel<false, mqa::SRC_DECODE>),
      reinterpret_cast<const void*>(mqa::fused_topk_kernel<true, mqa::SRC_DECODE>),
      reinterpret_cast<const void*>(mqa::fused_exact_kernel<mqa::SRC_GATHER>),
      reinterpret_cast<const void*>(mqa::fused_exact_kernel<mqa::SRC_DECODE>),
      reinterpret_cast<const void*>(mqa::fused_gate_kernel<mqa::SRC_GATHER>),
      reinterpret_cast<const void*>(mqa::fused_gate_kernel<mqa::SRC_DECODE>)};
  int best = 1 << 30;
  for (const void* f : kernels) {
    int n = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, f, mqa::kThreads, 0);
    if (e != hipSuccess) return (int)e;
    best = n < best ? n : best;
  }
  *wg_per_cu = best;
  return 0;
}
