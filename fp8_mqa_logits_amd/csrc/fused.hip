// Fused FP8 MQA logits + per-row top-k, one persistent launch per call.
//
// Follows vLLM PR #60618, "What this PR does" (scoring, sampled gate,
// candidate emission, per-row selection, exact rescan, heaviest-first block
// claims) and the API page "fused_mqa_topk" (contract and output convention),
// laid out for gfx950:
//   * a workgroup is 8 waves (512 threads); a block is 32 consecutive query
//     rows, 4 per wave, whose q and weights stay in VGPRs for the whole scan;
//   * keys stream through a double-buffered 8 KiB LDS stage (64 keys) loaded
//     with coalesced 16-byte global loads; every wave reads the stage as FP8
//     MFMA B operands and scores its 4 rows (common.h);
//   * each wave owns its rows, so the gate threshold, the candidate count and
//     the slab cursor of a row are wave-uniform values: emission is a ballot,
//     a popcount and one 8-byte store per passing lane, with no atomics;
//   * the scan ranks with FP8 MFMA scores, which are approximate on gfx950
//     (common.h); the select finds each row's k-th approximate score,
//     recomputes the scores of a band of keys around it exactly (bf16 MFMA)
//     and accepts the row only when the band's largest measured error, times
//     a safety factor, cannot move any key across the cut;
//   * rows whose gate misses, whose slab overflows or whose band cannot be
//     certified are rescanned with exact scores and a streaming top-k merge;
//   * the select, the fallback rescan and its compactions run in the same
//     workgroup right after the block's scan, so no workgroup ever waits for
//     another one.
#include "common.h"
#include "launch.h"

namespace mqa {

constexpr int kWaves = kFusedWaves;
constexpr int kThreads = kWaves * kWave;
constexpr int kRowsPerWave = 4;
constexpr int kBlockRows = kWaves * kRowsPerWave;  // 32
static_assert(kBlockRows == kFusedBlockRows, "block rows");
constexpr int kGateBins = 128;
constexpr int kGateOff = 16;  // bins above the first-tile maximum
constexpr int kHistWords = 2048;

// Header words (mirror of struct mqa_stats in mqa_topk.h).
enum : int {
  H_CLAIM = 0, H_SHORT = 1, H_GATED = 2, H_EXACT = 3, H_OVERFLOW = 4, H_UNDER = 5,
  H_COMPACT = 6, H_UNCERT = 7, H_CAND_LO = 8, H_CAND_HI = 9, H_BAND_LO = 10, H_BAND_HI = 11
};
constexpr int kBand = 32;           // keys on each side of rank k that are rescored exactly
constexpr float kBandSafety = 8.f;  // certificate margin, in units of the band's largest error

enum RowMode : int { M_OFF = 0, M_SHORT = 1, M_ALL = 2, M_GATED = 3, M_EXACT = 4 };



__device__ __forceinline__ void row_range(const FusedParams& p, int r, int& s, int& e) {
  int a = p.starts[r], b = p.ends[r];
  a = a < 0 ? 0 : (a > p.keys ? p.keys : a);
  b = b < a ? a : (b > p.keys ? p.keys : b);
  s = a;
  e = b;
}

// Cost of a block: the union range its non-short rows scan.
__device__ __forceinline__ int block_cost(const FusedParams& p, int b) {
  int lo = p.keys, hi = 0;
  for (int i = 0; i < kBlockRows; ++i) {
    const int r = b * kBlockRows + i;
    if (r >= p.rows) break;
    int s, e;
    row_range(p, r, s, e);
    if (e - s > p.topk) {
      lo = s < lo ? s : lo;
      hi = e > hi ? e : hi;
    }
  }
  return hi > lo ? hi - lo : 0;
}

// Heaviest-first block order (counting sort by cost, 1024 buckets of 1024
// keys, descending) and the reset of the header. One workgroup.
__global__ __launch_bounds__(1024) void fused_plan_kernel(FusedParams p) {
  __shared__ int cnt[1024];
  __shared__ int off[1024];
  const int tid = threadIdx.x;
  cnt[tid] = 0;
  if (tid < 64) p.header[tid] = 0;
  __syncthreads();
  for (int b = tid; b < p.nblocks; b += 1024) {
    const int c = block_cost(p, b) >> 10;
    atomicAdd(&cnt[c > 1023 ? 1023 : c], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int c = 1023; c >= 0; --c) {
      off[c] = acc;
      acc += cnt[c];
    }
  }
  __syncthreads();
  for (int b = tid; b < p.nblocks; b += 1024) {
    int c = block_cost(p, b) >> 10;
    c = c > 1023 ? 1023 : c;
    const int pos = atomicAdd(&off[c], 1);
    p.order[pos] = b;
  }
}

struct RowState {
  int r;        // global row id
  int s, e;     // clamped visible range
  int mode;     // RowMode
  float thr;    // admission threshold
  int strict;   // admit score > thr (1) or >= thr (0)
  int cnt;      // records appended to the slab
  float m0, inv;  // gate: first-tile maximum and inverse bin width
  int have_m0;
  int nsamp;    // gate: sample keys inside the row's range
};

struct __align__(16) FusedSmem {
  uint8_t kbuf[2][kChunkBytes];
  uint32_t hist[kWaves][kHistWords];
  int64_t gath[kChunk];
  int lo, hi, any_gated, any_exact, block;
  int wlo[kWaves], whi[kWaves], wg[kWaves], wx[kWaves];
};

// Append the passing lanes of one chunk to a row's slab; a full slab in
// streaming mode is first compacted to the row's k best records.
__device__ __forceinline__ void emit_chunk(const FusedParams& p, RowState& rs, float E, bool valid,
                                           int64_t key, int cap, float* sE, int32_t* sI,
                                           float* tE, int32_t* tI, uint32_t* hist) {
  bool pass = valid && (rs.strict ? (E > rs.thr) : (E >= rs.thr));
  uint64_t m = __ballot(pass);
  if (m == 0) return;
  int c = __popcll(m);
  if (rs.mode == M_EXACT && rs.cnt + c > cap) {
    // streaming top-k merge: keep the k best so far, raise the threshold
    const int k = p.topk;
    const float kth = wave_select(sE, sI, rs.cnt, k, hist, [&](int slot, float e, int idx) {
      tE[slot] = e;
      tI[slot] = idx;
    });
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    for (int i = lane_id(); i < k; i += kWave) {
      sE[i] = tE[i];
      sI[i] = tI[i];
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    rs.cnt = k;
    rs.thr = kth;
    rs.strict = 1;
    if (p.flags & 8u) {
      if (lane_id() == 0) atomicAdd(&p.header[H_COMPACT], 1u);
    }
    pass = valid && E > rs.thr;
    m = __ballot(pass);
    if (m == 0) return;
    c = __popcll(m);
  }
  if (pass) {
    const int pos = rs.cnt + rank_in_mask(m);
    if (pos < cap) {
      sE[pos] = E;
      sI[pos] = (int32_t)key;
    }
  }
  rs.cnt += c;
}

// One sweep over the keys [lo, hi) for the rows of this wave whose mode is in
// `mode_bits`, with FP8 MFMA scores (EXACT = false) or exact scores.
template <bool EXACT>
__device__ __forceinline__ void scan_block(const FusedParams& p, FusedSmem& sm, const QueryRow* qr, RowState* rs,
                           int mode_bits, int lo, int hi, int cap, float* slabE, int32_t* slabI,
                           float* tE, int32_t* tI) {
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int l = lane_id();
  const int nch = (hi - lo + kChunk - 1) / kChunk;
  uint4 regs[1];
  stage_chunk_regs(regs, p.k, lo, p.keys, tid, kThreads);
  store_chunk_regs(regs, sm.kbuf[0], tid, kThreads);
  __syncthreads();
  for (int c = 0; c < nch; ++c) {
    const int64_t key0 = (int64_t)lo + (int64_t)c * kChunk;
    const bool more = c + 1 < nch;
    if (more) stage_chunk_regs(regs, p.k, key0 + kChunk, p.keys, tid, kThreads);
    const int64_t key = key0 + l;
    const float sc = p.scales[key < p.keys ? key : p.keys - 1];
    bool any = false;
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i)
      any |= ((mode_bits >> rs[i].mode) & 1) && rs[i].s < key0 + kChunk && rs[i].e > key0;
    if (any) {
      KeyTile kt;
      load_keys_lds(kt, sm.kbuf[c & 1]);
#pragma unroll
      for (int i = 0; i < kRowsPerWave; ++i) {
        RowState& r = rs[i];
        if (!((mode_bits >> r.mode) & 1) || r.s >= key0 + kChunk || r.e <= key0) continue;
        const float E = (EXACT ? score_chunk_exact(qr[i], kt) : score_chunk(qr[i], kt)) * sc;
        const bool valid = key >= r.s && key < r.e;
        const int slot = w * kRowsPerWave + i;
        emit_chunk(p, r, E, valid, key, cap, slabE + (int64_t)slot * kCap,
                   slabI + (int64_t)slot * kCap, tE, tI, sm.hist[w]);
      }
    }
    if (more) store_chunk_regs(regs, sm.kbuf[(c + 1) & 1], tid, kThreads);
    __syncthreads();
  }
}

// Top-k of a row from its FP8-scored candidates (sE, sI)[0..n), n >= k, all
// with approximate score >= T (non-candidates score below T):
//   1. the (k-kBand)-th and (k+kBand)-th largest approximate scores vhi, vlo;
//   2. records above vhi are taken; records in [vlo, vhi] (the band) are
//      compacted to the front of the slab; the largest approximate score
//      below the band (or T) and the smallest one above it are kept;
//   3. the band's scores are recomputed exactly and its best k - |above|
//      records are taken by exact score;
//   4. certificate: with D = kBandSafety * (largest |exact - approximate| in
//      the band, floored at 2^-18 of the row's largest score magnitude), the
//      result is exact when every record above the band scores >= tau + D and
//      every record below it <= tau - D (tau = the k-th exact score).
// Returns false when the certificate fails (the caller rescans the row).
template <class Emit>
__device__ bool select_banded(const FusedParams& p, float* sE, int32_t* sI, int n, int k, float T,
                              const QueryRow& qr, uint32_t* hist, unsigned* band_count,
                              Emit emit) {
  const int l = lane_id();
  const float vhi = (k - kBand >= 1) ? wave_kth_value(sE, n, k - kBand, hist) : __builtin_inff();
  const float vlo = (k + kBand <= n) ? wave_kth_value(sE, n, k + kBand, hist) : -__builtin_inff();
  int na = 0, nb = 0;
  float min_above = __builtin_inff(), max_below = -__builtin_inff(), maxabs = 0.f;
  for (int i0 = 0; i0 < n; i0 += kWave) {
    const int i = i0 + l;
    const bool in = i < n;
    const float e = in ? sE[i] : 0.f;
    const int32_t idx = in ? sI[i] : 0;
    const bool up = in && e > vhi;
    const bool band = in && e >= vlo && e <= vhi;
    const uint64_t mu = __ballot(up);
    const uint64_t mb = __ballot(band);
    if (up) {
      const int slot = na + rank_in_mask(mu);
      if (slot < k) emit(slot, idx);
      min_above = __builtin_fminf(min_above, e);
    }
    if (in && e < vlo) max_below = __builtin_fmaxf(max_below, e);
    if (in) maxabs = __builtin_fmaxf(maxabs, __builtin_fabsf(e));
    // in-place compaction: targets lie at or before this chunk, already read
    if (band) {
      const int pos = nb + rank_in_mask(mb);
      sE[pos] = e;
      sI[pos] = idx;
    }
    na += __popcll(mu);
    nb += __popcll(mb);
  }
  min_above = wave_min(min_above);
  max_below = wave_max(max_below);
  maxabs = wave_max(maxabs);
  const int need = k - na;
  if (na >= k || nb < need) return false;
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  // exact scores of the band, 64 records at a time
  float err = 0.f;
  for (int b0 = 0; b0 < nb; b0 += kWave) {
    int keyidx[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int j = b0 + 16 * t + (l & 15);
      keyidx[t] = sI[j < nb ? j : nb - 1];
    }
    KeyTile kt;
    load_keys_gather(kt, p.k, keyidx);
    const int j = b0 + l;
    const int jj = j < nb ? j : nb - 1;
    const float E = score_chunk_exact(qr, kt) * p.scales[sI[jj]];
    if (j < nb) {
      err = __builtin_fmaxf(err, __builtin_fabsf(E - sE[j]));
      sE[j] = E;
    }
  }
  err = wave_max(err);
  if (l == 0 && band_count) atomicAdd(band_count, (unsigned)nb);
  const float tau = wave_select(sE, sI, nb, need, hist,
                                [&](int slot, float, int idx) { emit(na + slot, idx); });
  const float d = kBandSafety * __builtin_fmaxf(err, maxabs * 0x1p-18f);
  const float below = __builtin_fmaxf(max_below, T);
  const bool ok_above = na == 0 || min_above - d >= tau;
  const bool ok_below = below + d <= tau;
  return ok_above && ok_below;
}

// Sampled gate: a strided sample of the block's keys gives each gated row a
// threshold that should keep about 2k candidates. The sample histogram is
// binned relative to the row's maximum over the first sample tile.
__device__ __forceinline__ void gate_block(const FusedParams& p, FusedSmem& sm, const QueryRow* qr, RowState* rs,
                           int lo, int hi) {
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int l = lane_id();
  const int64_t span = hi - lo;
  int S = (int)(span / 16) & ~(kChunk - 1);
  S = S < 1024 ? 1024 : (S > 4096 ? 4096 : S);
  const int nch = S / kChunk;
  uint32_t* hist = sm.hist[w];
  for (int i = l; i < kRowsPerWave * kGateBins; i += kWave) hist[i] = 0;
  uint4 regs[1];
  for (int c = 0; c < nch; ++c) {
    if (tid < kChunk) sm.gath[tid] = lo + ((int64_t)(c * kChunk + tid) * span) / S;
    __syncthreads();
    stage_chunk_regs(regs, p.k, 0, p.keys, tid, kThreads, sm.gath);
    store_chunk_regs(regs, sm.kbuf[0], tid, kThreads);
    __syncthreads();
    const int64_t key = sm.gath[l];
    const float sc = p.scales[key];
    KeyTile kt;
    load_keys_lds(kt, sm.kbuf[0]);
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      RowState& r = rs[i];
      if (r.mode != M_GATED) continue;
      const float E = score_chunk(qr[i], kt) * sc;
      const bool valid = key >= r.s && key < r.e;
      const uint64_t vm = __ballot(valid);
      if (vm == 0) continue;
      if (!r.have_m0) {
        const float mx = wave_max(valid ? E : -__builtin_inff());
        const float mn = wave_min(valid ? E : __builtin_inff());
        float width = (mx - mn) / 64.f;
        if (!(width > 0.f) || !__builtin_isfinite(width))
          width = __builtin_fmaxf(__builtin_fabsf(mx), 1e-30f) * (1.f / 128.f);
        r.m0 = mx;
        r.inv = 1.f / width;
        r.have_m0 = 1;
      }
      r.nsamp += __popcll(vm);
      if (valid) {
        float fb = (r.m0 - E) * r.inv;
        int bin = fb < -1e6f ? 0 : (fb > 1e6f ? kGateBins - 1 : (int)__builtin_floorf(fb) + kGateOff);
        bin = bin < 0 ? 0 : (bin > kGateBins - 1 ? kGateBins - 1 : bin);
        atomicAdd(&hist[i * kGateBins + bin], 1u);
      }
    }
    __syncthreads();
  }
  // thresholds
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    RowState& r = rs[i];
    if (r.mode != M_GATED) continue;
    const int n = r.e - r.s;
    const int64_t target = 2 * (int64_t)p.topk;
    const int ks = (int)((target * r.nsamp + n - 1) / n);
    float thr = -__builtin_inff();
    if (r.have_m0 && ks >= 1 && ks <= r.nsamp) {
      // bins 2l, 2l+1 per lane, cumulative from bin 0 (the top)
      const int h0 = (int)hist[i * kGateBins + 2 * l];
      const int h1 = (int)hist[i * kGateBins + 2 * l + 1];
      const int incl = wave_incl_scan(h0 + h1);
      const uint64_t hit = __ballot(incl >= ks);
      const int src = hit ? __builtin_ctzll(hit) : 63;
      int bstar = 2 * l + ((incl - h1) >= ks ? 0 : 1);
      bstar = __shfl(bstar, src, 64);
      if (bstar < kGateBins - 1) thr = r.m0 - (float)(bstar - kGateOff + 1) / r.inv;
    }
    if (p.flags & 2u) thr = __builtin_inff();  // forced gate miss
    r.thr = thr;
  }
}

__global__ __launch_bounds__(kThreads) void fused_topk_kernel(FusedParams p) {
  __shared__ FusedSmem sm;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int l = lane_id();
  const int k = p.topk;
  const int cap = (p.flags & 4u) ? k + 64 : kCap;
  const bool stats = p.flags & 8u;
  float* slabE = p.slabE + (int64_t)blockIdx.x * kBlockRows * kCap;
  int32_t* slabI = p.slabI + (int64_t)blockIdx.x * kBlockRows * kCap;
  float* tE = p.tmpE + ((int64_t)blockIdx.x * kWaves + w) * kMaxTopk;
  int32_t* tI = p.tmpI + ((int64_t)blockIdx.x * kWaves + w) * kMaxTopk;

  for (;;) {
    if (tid == 0) sm.block = (int)atomicAdd(&p.header[H_CLAIM], 1u);
    __syncthreads();
    const int bi = sm.block;
    if (bi >= p.nblocks) break;
    const int b = p.order[bi];

    // ---- per-row setup (each wave: its 4 rows)
    RowState rs[kRowsPerWave];
    QueryRow qr[kRowsPerWave];
    int wlo = p.keys, whi = 0, wgated = 0, wexact = 0;
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      RowState& r = rs[i];
      r.r = b * kBlockRows + w * kRowsPerWave + i;
      r.cnt = 0;
      r.strict = 0;
      r.thr = -__builtin_inff();
      r.have_m0 = 0;
      r.nsamp = 0;
      r.m0 = 0.f;
      r.inv = 1.f;
      if (r.r >= p.rows) {
        r.mode = M_OFF;
        r.s = r.e = 0;
        continue;
      }
      row_range(p, r.r, r.s, r.e);
      const int n = r.e - r.s;
      if (n <= k) {
        r.mode = M_SHORT;
        int32_t* o = p.out + (int64_t)r.r * k;
        for (int j = l; j < k; j += kWave) o[j] = j < n ? j : -1;
        if (stats && l == 0) atomicAdd(&p.header[H_SHORT], 1u);
        continue;
      }
      load_query(qr[i], p.q, p.weights, r.r);
      wlo = r.s < wlo ? r.s : wlo;
      whi = r.e > whi ? r.e : whi;
      if (p.flags & 1u) {
        r.mode = M_EXACT;
        wexact = 1;
      } else if (n <= 4 * k && n <= cap) {
        r.mode = M_ALL;  // every visible key is a candidate
      } else {
        r.mode = M_GATED;
        wgated = 1;
      }
    }
    if (l == 0) {
      sm.wlo[w] = wlo;
      sm.whi[w] = whi;
      sm.wg[w] = wgated;
      sm.wx[w] = wexact;
    }
    __syncthreads();
    int lo = p.keys, hi = 0, any_g = 0, any_x = 0;
    for (int i = 0; i < kWaves; ++i) {
      lo = sm.wlo[i] < lo ? sm.wlo[i] : lo;
      hi = sm.whi[i] > hi ? sm.whi[i] : hi;
      any_g |= sm.wg[i];
      any_x |= sm.wx[i];
    }
    __syncthreads();
    if (hi > lo) {
      if (any_g) gate_block(p, sm, qr, rs, lo, hi);
      // ---- normal scan (all-candidate and gated rows)
      if (!(p.flags & 1u)) {
        scan_block<false>(p, sm, qr, rs, (1 << M_ALL) | (1 << M_GATED), lo, hi, cap, slabE, slabI,
                          tE, tI);
        // validity check + certified select, per row
        int wx = 0;
#pragma unroll
        for (int i = 0; i < kRowsPerWave; ++i) {
          RowState& r = rs[i];
          if (r.mode != M_ALL && r.mode != M_GATED) continue;
          const int slot = w * kRowsPerWave + i;
          bool ok = false;
          if (r.cnt >= k && r.cnt <= cap) {
            int32_t* o = p.out + (int64_t)r.r * k;
            const int base = r.s;
            ok = select_banded(p, slabE + (int64_t)slot * kCap, slabI + (int64_t)slot * kCap,
                               r.cnt, k, r.thr, qr[i], sm.hist[w],
                               stats ? &p.header[H_BAND_LO] : nullptr,
                               [&](int sl, int idx) { o[sl] = idx - base; });
            if (stats && l == 0) {
              atomicAdd(&p.header[ok ? H_GATED : H_UNCERT], 1u);
              const unsigned long long c = (unsigned long long)r.cnt;
              atomicAdd(reinterpret_cast<unsigned long long*>(&p.header[H_CAND_LO]), c);
            }
          } else if (stats && l == 0) {
            atomicAdd(&p.header[r.cnt > cap ? H_OVERFLOW : H_UNDER], 1u);
          }
          if (!ok) {
            r.mode = M_EXACT;
            r.cnt = 0;
            r.thr = -__builtin_inff();
            r.strict = 0;
            wx = 1;
          }
        }
        if (l == 0) sm.wx[w] = wx;
        __syncthreads();
        any_x = 0;
        for (int i = 0; i < kWaves; ++i) any_x |= sm.wx[i];
        __syncthreads();
      }
      // ---- exact streaming rescan for the rows that need it
      if (any_x) {
        scan_block<true>(p, sm, qr, rs, 1 << M_EXACT, lo, hi, cap, slabE, slabI, tE, tI);
#pragma unroll
        for (int i = 0; i < kRowsPerWave; ++i) {
          RowState& r = rs[i];
          if (r.mode != M_EXACT) continue;
          const int slot = w * kRowsPerWave + i;
          int32_t* o = p.out + (int64_t)r.r * k;
          const int base = r.s;
          const int have = r.cnt < cap ? r.cnt : cap;
          wave_select(slabE + (int64_t)slot * kCap, slabI + (int64_t)slot * kCap, have, k,
                      sm.hist[w], [&](int sl, float, int idx) { o[sl] = idx - base; });
          for (int j = have + l; j < k; j += kWave) o[j] = -1;
          if (stats && l == 0) atomicAdd(&p.header[H_EXACT], 1u);
        }
      }
    }
    __syncthreads();
  }
}

}  // namespace mqa

extern "C" int mqa_fused_launch(const mqa::FusedParams* p, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(mqa::fused_plan_kernel, dim3(1), dim3(1024), 0, stream, *p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return (int)e;
  hipLaunchKernelGGL(mqa::fused_topk_kernel, dim3(grid), dim3(mqa::kThreads), 0, stream, *p);
  return (int)hipGetLastError();
}

extern "C" int mqa_fused_occupancy(int* wg_per_cu) {
  return (int)hipOccupancyMaxActiveBlocksPerMultiprocessor(wg_per_cu, mqa::fused_topk_kernel,
                                                           mqa::kThreads, 0);
}
