// The dense path the fused kernel replaces (vLLM PR #60618, "Motivation": a
// logits pass that writes the fp32 [rows, keys] scores to HBM, then a per-row
// top-k pass that reads them back), plus the UE8M0 key-scale decode (API page
// "fused_mqa_topk", fused_mqa_topk_key_scales).
#include "common.h"
#include "launch.h"

namespace mqa {

typedef float v16f __attribute__((ext_vector_type(16)));

__device__ __forceinline__ v16f mfma32_bf16(v8bf a, v8bf b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Dense logits. The scores must match the exact ones within 1e-5 of the row's
// largest, so the products run on the bf16 MFMA over the exactly converted
// e4m3 values (fp32 accumulation), never on the FP8 MFMA.
//
// A workgroup owns 16 rows (2 per wave) and 2048 columns of the window. Each
// wave keeps its rows' queries in registers as bf16 for the whole kernel; the
// keys pass through LDS 64 at a time, converted to bf16 once per workgroup
// while the next 64 are loaded. Per 32 keys and row a wave issues 8
// v_mfma_f32_32x32x16_bf16 (A: the 32 heads x 16 dims, B: 16 dims x the 32
// keys), which leave each lane with 16 of the 32 heads of one key; the
// weighted relu sum over them, one lane swap with the other 16 heads (both
// rows in one swap) and the key's scale give the logit. The epilogue of one
// 32-key tile (2 x 16 relu + fma per lane and row: as much VALU time as the
// tile's MFMA time) runs while the next tile's MFMAs execute: the two are
// independent, and scheduling groups interleave them. Waves of a SIMD start
// each stage together (one barrier per stage), so without this overlap the
// MFMA unit idles through every epilogue.
//
// K order: in k-step s (0..7) the lanes of half h = lane / 32 supply the 8
// k-indices 8h .. 8h + 7, which stand for dims 64h + 8s .. 64h + 8s + 7 of
// both operands, so every dot product covers all 128 dims once.
constexpr int kLWaves = 8;
constexpr int kLThreads = kLWaves * kWave;
constexpr int kLRows = 2;                      // rows per wave
constexpr int kLBlockRows = kLWaves * kLRows;  // 16
constexpr int kLStage = 64;                    // keys per LDS stage (two tiles)
constexpr int kLCols = 2048;                   // window columns per workgroup
// Buffer-store cache policy bits on gfx950: bit 1 is the non-temporal hint.
constexpr int kStoreNonTemporal = 2;

// LDS index (16-byte slots) of key j's bf16 dims [8s, 8s + 8) in a stage: the
// slot index is XOR-swizzled with j & 15, so 16 consecutive keys read at one
// slot index touch 16 distinct bank groups.
__device__ __forceinline__ int lslot(int j, int s) { return j * 16 + (s ^ (j & 15)); }

__device__ __forceinline__ uint4 as_u4(v8bf v) { return __builtin_bit_cast(uint4, v); }
__device__ __forceinline__ v8bf as_v8bf(uint4 v) { return __builtin_bit_cast(v8bf, v); }

struct TileAcc {
  v16f c[kLRows];
  float sc;  // the scale of the lane's key
};

__global__ __launch_bounds__(kLThreads) void dense_logits_kernel(DenseParams p) {
  __shared__ float ks[2][kLStage];  // the stage keys' scales
  __shared__ __align__(16) uint4 kb[2][kLStage * 16];  // 2 x 16 KiB of bf16 keys
  const int tid = threadIdx.x;
  const int w = wave_id();
  const int l = lane_id();
  const int h = l >> 5;
  const int c32 = l & 31;
  const int c_begin = blockIdx.x * kLCols;
  const int c_end = c_begin + kLCols < p.ncols ? c_begin + kLCols : p.ncols;
  const int win_end = p.col0 + p.ncols;  // first key past the window
  const int r0 = blockIdx.y * kLBlockRows + w * kLRows;
  // queries: lane l holds head l % 32, dims [64h, 64h + 64) of each row;
  // weights: lane l's 16 heads 8g + 4h + e (accumulator element 4g + e)
  v8bf qa[kLRows][8];
  float wt[kLRows][16];
  int rs[kLRows], re[kLRows];
#pragma unroll
  for (int i = 0; i < kLRows; ++i) {
    const int r = r0 + i;
    rs[i] = re[i] = 0;
    if (r < p.rows) {
      int a = p.starts[r], b = p.ends[r];
      a = a < 0 ? 0 : (a > p.keys ? p.keys : a);
      b = b < a ? a : (b > p.keys ? p.keys : b);
      rs[i] = a;
      re[i] = b;
      const uint4* src =
          reinterpret_cast<const uint4*>(p.q + ((int64_t)r * kHeads + c32) * kDim + 64 * h);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint4 x = src[v];
        qa[i][2 * v] = fp8x8_to_bf16((int)x.x, (int)x.y);
        qa[i][2 * v + 1] = fp8x8_to_bf16((int)x.z, (int)x.w);
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 w4 =
            *reinterpret_cast<const float4*>(p.weights + (int64_t)r * kHeads + 8 * g + 4 * h);
        wt[i][4 * g] = w4.x;
        wt[i][4 * g + 1] = w4.y;
        wt[i][4 * g + 2] = w4.z;
        wt[i][4 * g + 3] = w4.w;
      }
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s) qa[i][s] = as_v8bf(uint4{0u, 0u, 0u, 0u});
#pragma unroll
      for (int e = 0; e < 16; ++e) wt[i][e] = 0.f;
    }
  }
  // stage copies: slice v = t + kLThreads * u (u < kLCopies) of a stage is
  // e4m3 bytes [16c, 16c + 16) of stage key v / 8 (c = v % 8), written to
  // bf16 slots 2c and 2c + 1
  constexpr int kLCopies = kLStage * 8 / kLThreads;
  auto gload = [&](int st, uint4* x) {
#pragma unroll
    for (int u = 0; u < kLCopies; ++u) {
      const int v = tid + kLThreads * u;
      int key = p.col0 + c_begin + st * kLStage + (v >> 3);
      key = key < win_end ? key : win_end - 1;
      x[u] = *reinterpret_cast<const uint4*>(p.k + (int64_t)key * kDim + 16 * (v & 7));
    }
  };
  auto lstore = [&](const uint4* x, int buf) {
#pragma unroll
    for (int u = 0; u < kLCopies; ++u) {
      const int v = tid + kLThreads * u;
      kb[buf][lslot(v >> 3, 2 * (v & 7))] = as_u4(fp8x8_to_bf16((int)x[u].x, (int)x[u].y));
      kb[buf][lslot(v >> 3, 2 * (v & 7) + 1)] = as_u4(fp8x8_to_bf16((int)x[u].z, (int)x[u].w));
    }
  };
  // the stage keys' scales: every wave loads and stores all 64 (the same
  // values), which keeps the loop free of branches
  auto sload = [&](int st) {
    int key = p.col0 + c_begin + st * kLStage + (tid & (kLStage - 1));
    key = key < win_end ? key : win_end - 1;
    return p.scales[key];
  };
  // the output rows r0 and r0 + 1 as one buffer resource
  const __amdgpu_buffer_rsrc_t orow = __builtin_amdgcn_make_buffer_rsrc(
      p.logits + (int64_t)r0 * p.ld, 0, (int)(2 * p.ld * 4), kBufferFlags);
  // the MFMAs of one tile (window columns cb .. cb + 31) for both rows
  auto mfmas = [&](int buf, int t, TileAcc& a) {
    v8bf kf[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) kf[s] = as_v8bf(kb[buf][lslot(32 * t + c32, 8 * h + s)]);
    a.sc = ks[buf][32 * t + c32];
#pragma unroll
    for (int i = 0; i < kLRows; ++i)
      a.c[i] = v16f{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f,
                    0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
#pragma unroll
      for (int i = 0; i < kLRows; ++i) a.c[i] = mfma32_bf16(qa[i][s], kf[s], a.c[i]);
    }
  };
  // the epilogue of the tile at window column cb (stores past c_end dropped)
  auto epilogue = [&](const TileAcc& a, int cb) {
    const int key = p.col0 + cb + c32;  // this lane's key
    const float sc = a.sc;
    float part[kLRows];
#pragma unroll
    for (int i = 0; i < kLRows; ++i) {
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc = __builtin_fmaf(wt[i][e], relu(a.c[i][e]), acc);
      part[i] = acc;
    }
    // lanes 0-31 end with row 0's sums over all 32 heads, lanes 32-63 with row 1's
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]),
                                                     __float_as_uint(part[1]), false, false);
    const float tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    const int rsi = h ? rs[1] : rs[0];
    const int rei = h ? re[1] : re[0];
    const bool vis = key >= rsi && key < rei;
    // a buffer store (no branch): lanes of a row past the last or of a
    // column past the tile range get an offset past the resource, and the
    // hardware drops them. Cache policy: non-temporal (the logits are read
    // once, by the top-k pass; with the hint that pass ran 5% faster, the
    // logits pass the same)
    const bool ok = r0 + h < p.rows && cb + c32 < c_end;
    const int off = ok ? (h * (int)p.ld + cb + c32) * 4 : 0x7FFFFFF0;
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(vis ? tot * sc : -__builtin_inff()),
                                          orow, off, 0, kStoreNonTemporal);
  };
  // interleave: one MFMA, then four VALU/LDS instructions of the epilogue
  auto interleave = [&]() {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // VALU
    }
  };
  // Stages always hold two tiles: keys past the window repeat its last key
  // and their stores are dropped, so the loop body has no branch and each
  // tile's MFMAs share one scheduling region with the previous tile's
  // epilogue. The copies for stage st + 1 are issued (and stored to the other
  // buffer) also on the last stage, where they go unused.
  const int nst = (c_end - c_begin + kLStage - 1) / kLStage;
  uint4 x[kLCopies];
  float xs = sload(0);
  gload(0, x);
  lstore(x, 0);
  ks[0][tid & (kLStage - 1)] = xs;
  __syncthreads();
  TileAcc a0, a1;
  gload(1, x);
  xs = sload(1);
  mfmas(0, 0, a0);
  mfmas(0, 1, a1);
  epilogue(a0, c_begin);
  interleave();
  lstore(x, 1);
  ks[1][tid & (kLStage - 1)] = xs;
  __syncthreads();
  for (int st = 1; st < nst; ++st) {
    const int cb0 = c_begin + st * kLStage;
    gload(st + 1, x);
    xs = sload(st + 1);
    mfmas(st & 1, 0, a0);
    epilogue(a1, cb0 - 32);
    interleave();
    mfmas(st & 1, 1, a1);
    epilogue(a0, cb0);
    interleave();
    lstore(x, (st + 1) & 1);
    ks[(st + 1) & 1][tid & (kLStage - 1)] = xs;
    __syncthreads();
  }
  epilogue(a1, c_begin + nst * kLStage - 32);
}

// ---------------------------------------------------------------------------
// Dense per-row top-k: exact, over the row's visible columns of the logits
// window, on the order-preserving uint32 key of each fp32 logit. One
// 1024-thread workgroup per row.
//   - Rows of at most kTLds logits: read once into LDS, radix-selected there.
//   - Longer rows: a stratified sample (runs of 256 logits spread over the
//     row) is binned below its largest key in bins of 2^16 keys (1/128 of a
//     binade); the bins holding the sample ranks expected for the k-th
//     largest, minus and plus a margin of 3 standard deviations plus 6, give
//     two keys hi and lo (the margin also bounds the band: at 2^20 logits and
//     k = 2048 the band holds about 4400). One pass over the row writes every logit above hi
//     to the output and collects those in [lo, hi] in LDS, where the rest of
//     the top-k is selected. When the pass finds more than k above hi, fewer
//     than k at or above lo, or more than kTLds in between, the row falls back
//     to a radix select over the row in global memory (three digit passes
//     and an output pass).
// Radix digits are taken from the top of the keys' actual span (key - base
// over span bits), so that keys packed into a narrow range spread over a
// digit's bins instead of piling into one (LDS atomics on one address
// serialise).
constexpr int kTThreads = 1024;
constexpr int kTLds = 8192;   // logits held in LDS: short rows, the sample, the band
constexpr int kTRun = 256;    // sample run length
constexpr int kTBinShift = 16;

struct TopkShared {
  uint32_t v[kTLds];
  int32_t idx[kTLds];
  uint32_t hist[2048];
  uint32_t red[kTThreads / kWave];
  int digit, above, cnt, up, tie;
};

// Wave-aggregated append: the calling lanes with take set get consecutive
// slots from the LDS counter *ctr (one atomic per wave instead of one per
// lane: same-address LDS atomics serialise); -1 for the others.
__device__ __forceinline__ int wave_append(bool take, int* ctr) {
  const uint64_t m = __ballot(take);
  if (m == 0) return -1;
  const int leader = __builtin_ctzll(m);
  int base = 0;
  if (lane_id() == leader) base = atomicAdd(ctr, __popcll(m));
  base = __shfl(base, leader, 64);
  return take ? base + rank_in_mask(m) : -1;
}

// The largest of n keys get(i) (block-wide).
template <class Get>
__device__ uint32_t block_max_key(TopkShared& sh, Get get, int n) {
  uint32_t m = 0;
  for (int i = threadIdx.x; i < n; i += kTThreads) m = get(i) > m ? get(i) : m;
  m = (uint32_t)wave_max_i((int)(m ^ 0x80000000u)) ^ 0x80000000u;
  if (lane_id() == 0) sh.red[threadIdx.x / kWave] = m;
  __syncthreads();
  uint32_t r = 0;
  for (int w = 0; w < kTThreads / kWave; ++w) r = sh.red[w] > r ? sh.red[w] : r;
  __syncthreads();
  return r;
}

// One wave over hist[0 .. nb) (nb a multiple of 64), bins taken from the
// last down (descending) or from the first up: the bin at which the running
// count reaches need, the count before it (above) and in it (cnt), through
// sh; digit -1 when the bins hold fewer than need.
__device__ void hist_find(TopkShared& sh, int nb, int need, bool descending) {
  const int l = lane_id();
  const int per = nb / kWave;
  auto bin_of = [&](int j) { return descending ? nb - 1 - j : j; };
  int mine = 0;
  // (each lane starts at its own offset in its run of bins: lanes reading
  // bins 32 apart would all hit one LDS bank)
  for (int b = 0; b < per; ++b) mine += (int)sh.hist[bin_of(l * per + ((b + l) & (per - 1)))];
  const int incl = wave_incl_scan(mine);
  const int excl = incl - mine;
  const uint64_t hit = __ballot(incl >= need);
  const int src = hit ? __builtin_ctzll(hit) : -1;
  if (src < 0) {  // fewer than need in all bins
    if (l == 0) {
      sh.digit = -1;
      sh.above = 0;
      sh.cnt = 0;
    }
    return;
  }
  if (l == src) {
    int c = excl;
    for (int b = 0; b < per; ++b) {
      const int bin = bin_of(l * per + b);
      const int h = (int)sh.hist[bin];
      if (c + h >= need) {
        sh.digit = bin;
        sh.above = c;
        sh.cnt = h;
        break;
      }
      c += h;
    }
  }
}

// Radix select over n keys get(i) - base, all in [0, span]: on return the
// keys with ((key - base) & pmask) > prefix are the ones strictly above the
// need-th largest (k - need of them, need updated), and those equal to
// prefix its ties. Digits of up to 11 bits from the top bit of span down;
// stops early once the ties are exactly the ones needed.
template <class Get>
__device__ void block_radix(TopkShared& sh, Get get, int n, int& need, uint32_t base,
                            uint32_t span, uint32_t& prefix, uint32_t& pmask) {
  const int tid = threadIdx.x;
  prefix = 0;
  pmask = 0;
  int top = 32 - __builtin_clz(span | 1u);  // bits to resolve
  while (top > 0) {
    const int width = top < 11 ? top : 11;
    const int shv = top - width;
    const uint32_t dmask = (1u << width) - 1u;
    const int nb = 1 << width;
    const int nbh = nb < kWave ? kWave : nb;
    for (int b = tid; b < nbh; b += kTThreads) sh.hist[b] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kTThreads) {
      const uint32_t key = get(i) - base;
      if ((key & pmask) == prefix) atomicAdd(&sh.hist[(key >> shv) & dmask], 1u);
    }
    __syncthreads();
    if (tid < kWave) hist_find(sh, nbh, need, true);
    __syncthreads();
    need -= sh.above;
    prefix |= (uint32_t)sh.digit << shv;
    pmask |= dmask << shv;
    const bool done = sh.cnt == need;
    __syncthreads();
    if (done) break;
    top = shv;
  }
}

// Writes the selection block_radix found into o[slot0 ..]: the first k - need
// slots take the keys strictly above, the next `need` the first ties;
// out_idx(i) is element i's output value.
template <class Get, class Out>
__device__ void block_emit(TopkShared& sh, Get get, Out out_idx, int n, int k, int need,
                           uint32_t base, uint32_t prefix, uint32_t pmask, int32_t* o, int slot0) {
  const int tid = threadIdx.x;
  if (tid == 0) {
    sh.up = 0;
    sh.tie = 0;
  }
  __syncthreads();
  const int n_above = k - need;
  for (int i = tid; i < n; i += kTThreads) {
    const uint32_t key = (get(i) - base) & pmask;
    const int s = wave_append(key > prefix, &sh.up);
    const int t = wave_append(key == prefix, &sh.tie);
    if (s >= 0 && s < n_above) o[slot0 + s] = out_idx(i);
    if (t >= 0 && t < need) o[slot0 + n_above + t] = out_idx(i);
  }
}

__global__ __launch_bounds__(kTThreads) void dense_topk_kernel(DenseTopkParams p) {
  __shared__ TopkShared sh;
  __shared__ int n_up, n_band;
  __shared__ uint32_t key_hi, key_lo;
  const int tid = threadIdx.x;
  const int r = blockIdx.x;
  const int k = p.topk;
  int s = p.starts[r], e = p.ends[r];
  s = s < 0 ? 0 : (s > p.keys ? p.keys : s);
  e = e < s ? s : (e > p.keys ? p.keys : e);
  const int c_lo = (s > p.col0 ? s : p.col0) - p.col0;
  const int c_hi = (e < p.col0 + p.ncols ? e : p.col0 + p.ncols) - p.col0;
  const int n = c_hi > c_lo ? c_hi - c_lo : 0;
  int32_t* o = p.out + (int64_t)r * k;
  const int shift_out = p.col0 - s + c_lo;  // element i is key - s = i + shift_out
  if (n <= k) {
    for (int j = tid; j < k; j += kTThreads) o[j] = j < n ? j + shift_out : -1;
    return;
  }
  const float* row = p.logits + (int64_t)r * p.ld + c_lo;
  auto plain = [&](int i) { return i + shift_out; };
  auto lkey = [&](int i) { return sh.v[i]; };
  uint32_t prefix, pmask;
  int need = k;
  if (n <= kTLds) {
    for (int i = tid; i < n; i += kTThreads) sh.v[i] = fkey(row[i]);
    __syncthreads();
    block_radix(sh, lkey, n, need, 0u, 0xFFFFFFFFu, prefix, pmask);
    block_emit(sh, lkey, plain, n, k, need, 0u, prefix, pmask, o, 0);
    return;
  }
  // the sample: m logits in runs of 256 spread evenly over the row
  int m = n / 16;
  m = m < 4096 ? 4096 : (m > kTLds ? kTLds : m);
  m = m / kTRun * kTRun;
  const int runs = m / kTRun;
  for (int i = tid; i < m; i += kTThreads) {
    const int run = i / kTRun;
    const int off = (int)((int64_t)run * (n - kTRun) / (runs - 1));
    sh.v[i] = fkey(row[off + i % kTRun]);
  }
  __syncthreads();
  {
    const uint32_t kmax = block_max_key(sh, lkey, m);
    // bins below the sample's largest key: bin b holds keys in
    // (kmax - (b + 1) 2^16, kmax - b 2^16]; lower keys are not counted
    for (int b = tid; b < 2048; b += kTThreads) sh.hist[b] = 0;
    __syncthreads();
    for (int i = tid; i < m; i += kTThreads) {
      const uint32_t d = (kmax - sh.v[i]) >> kTBinShift;
      if (d < 2048u) atomicAdd(&sh.hist[d], 1u);
    }
    __syncthreads();
    const float t = (float)k * (float)m / (float)n;  // expected sample rank of the k-th
    const float dv = 3.f * __builtin_sqrtf(t) + 6.f;
    const int rank_hi = (int)__builtin_floorf(t - dv);
    const int rank_lo = (int)__builtin_ceilf(t + dv);
    uint32_t hi = 0xFFFFFFFFu, lo = 0u;
    if (rank_hi >= 1) {
      if (tid < kWave) hist_find(sh, 2048, rank_hi, false);
      __syncthreads();
      // fewer than rank_hi sample keys lie above bin b's top
      if (sh.digit >= 0) hi = kmax - ((uint32_t)sh.digit << kTBinShift);
      __syncthreads();
    }
    if (rank_lo <= m) {
      if (tid < kWave) hist_find(sh, 2048, rank_lo, false);
      __syncthreads();
      // at least rank_lo sample keys lie at or above bin b's bottom
      if (sh.digit >= 0) {
        const uint32_t drop = ((uint32_t)sh.digit + 1u) << kTBinShift;
        lo = kmax >= drop ? kmax - drop + 1u : 0u;
      }
      __syncthreads();
    }
    if (tid == 0) {
      key_hi = hi;
      key_lo = lo;
      n_up = 0;
      n_band = 0;
    }
    __syncthreads();
  }
  const uint32_t hi = key_hi, lo = key_lo;
  // one pass: above hi to the output, [lo, hi] to LDS. Elements are read
  // four at a time from the first 16-byte aligned one.
  auto take = [&](int i, float f) {
    const uint32_t key = fkey(f);
    if (key > hi) {
      const int u = atomicAdd(&n_up, 1);
      if (u < k) o[u] = i + shift_out;
    } else if (key >= lo) {
      const int b = atomicAdd(&n_band, 1);
      if (b < kTLds) {
        sh.v[b] = key;
        sh.idx[b] = i;
      }
    }
  };
  const int head = (4 - (c_lo & 3)) & 3;  // elements before the first aligned one
  const int h0 = head < n ? head : n;
  if (tid < h0) take(tid, row[tid]);
  const int nv = (n - h0) >> 2;
  const float4* row4 = reinterpret_cast<const float4*>(row + h0);
  // Most logits lie below lo: a float compare clears them first (a float
  // strictly below lo's float has a key below lo; -0/+0 pairs, NaNs and a NaN
  // lo compare false and go through take), and a lane then visits only its
  // remaining elements, so a wave issues take's instructions about once per
  // group of four instead of four times.
  const float lo_f = kfloat(lo);
  auto take4 = [&](int v, float4 f) {
    const int i = h0 + 4 * v;
    uint32_t m = (f.x < lo_f ? 0u : 1u) | (f.y < lo_f ? 0u : 2u) | (f.z < lo_f ? 0u : 4u) |
                 (f.w < lo_f ? 0u : 8u);
    while (m) {
      const int b = __builtin_ctz(m);
      m &= m - 1u;
      take(i + b, b == 0 ? f.x : (b == 1 ? f.y : (b == 2 ? f.z : f.w)));
    }
  };
  int v = tid;
  for (; v + 7 * kTThreads < nv; v += 8 * kTThreads) {  // eight loads in flight
    float4 f[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) f[u] = row4[v + u * kTThreads];
#pragma unroll
    for (int u = 0; u < 8; ++u) take4(v + u * kTThreads, f[u]);
  }
  for (; v < nv; v += kTThreads) take4(v, row4[v]);
  for (int i = h0 + 4 * nv + tid; i < n; i += kTThreads) take(i, row[i]);
  __syncthreads();
  const int up = n_up, band = n_band;
  if (up <= k && up + band >= k && band <= kTLds) {
    const int need0 = k - up;  // the band's share of the top-k
    if (need0 == 0) return;
    need = need0;
    auto bidx = [&](int i) { return sh.idx[i] + shift_out; };
    block_radix(sh, lkey, band, need, lo, hi - lo, prefix, pmask);
    block_emit(sh, lkey, bidx, band, need0, need, lo, prefix, pmask, o, up);
    return;
  }
  // fallback: radix select over the row in global memory
  need = k;
  auto gkey = [&](int i) { return fkey(row[i]); };
  block_radix(sh, gkey, n, need, 0u, 0xFFFFFFFFu, prefix, pmask);
  block_emit(sh, gkey, plain, n, k, need, 0u, prefix, pmask, o, 0);
}

__global__ void key_scales_kernel(const uint32_t* b, float* s, int keys) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j < keys) s[j] = __uint_as_float((b[j] & 0xFFu) << 23);
}

}  // namespace mqa

extern "C" int mqa_dense_logits_launch(const mqa::DenseParams* p, hipStream_t stream) {
  dim3 grid((p->ncols + mqa::kLCols - 1) / mqa::kLCols,
            (p->rows + mqa::kLBlockRows - 1) / mqa::kLBlockRows);
  hipLaunchKernelGGL(mqa::dense_logits_kernel, grid, dim3(mqa::kLThreads), 0, stream, *p);
  return (int)hipGetLastError();
}

extern "C" int mqa_dense_topk_launch(const mqa::DenseTopkParams* p, hipStream_t stream) {
  hipLaunchKernelGGL(mqa::dense_topk_kernel, dim3(p->rows), dim3(mqa::kTThreads), 0, stream, *p);
  return (int)hipGetLastError();
}

extern "C" int mqa_key_scales_launch(const uint8_t* b, float* s, int keys, hipStream_t stream) {
  hipLaunchKernelGGL(mqa::key_scales_kernel, dim3((keys + 255) / 256), dim3(256), 0, stream,
                     reinterpret_cast<const uint32_t*>(b), s, keys);
  return (int)hipGetLastError();
}
