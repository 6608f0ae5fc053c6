// The dense path the fused kernel replaces (vLLM PR #60618, "Motivation": a
// logits pass that writes the fp32 [rows, keys] scores to HBM, then a per-row
// top-k pass that reads them back), plus the UE8M0 key-scale decode (API page
// "fused_mqa_topk", fused_mqa_topk_key_scales).
#include "common.h"
#include "launch.h"

namespace mqa {

constexpr int kDWaves = 8;
constexpr int kDThreads = kDWaves * kWave;
constexpr int kDRowsPerWave = 4;
constexpr int kDBlockRows = kDWaves * kDRowsPerWave;  // 32
constexpr int kDCols = 4 * kChunk;                    // 256 columns per workgroup

// logits[r, c] for a 32-row x 256-column tile; keys staged through LDS as in
// the fused scan, scored with the fp32-accurate bf16 MFMA tile (the written
// logits must match the exact scores within 1e-5 of the row's largest).
__global__ __launch_bounds__(kDThreads) void dense_logits_kernel(DenseParams p) {
  __shared__ __align__(16) uint8_t kbuf[2][kChunkBytes];
  const int tid = threadIdx.x;
  const int w = wave_id();
  const int l = lane_id();
  const int c_begin = blockIdx.x * kDCols;
  const int c_end = c_begin + kDCols < p.ncols ? c_begin + kDCols : p.ncols;
  QueryRow qr[kDRowsPerWave];
  int rr[kDRowsPerWave], rs_[kDRowsPerWave], re_[kDRowsPerWave];
#pragma unroll
  for (int i = 0; i < kDRowsPerWave; ++i) {
    const int r = blockIdx.y * kDBlockRows + w * kDRowsPerWave + i;
    rr[i] = r;
    rs_[i] = re_[i] = 0;
    if (r < p.rows) {
      int a = p.starts[r], b = p.ends[r];
      a = a < 0 ? 0 : (a > p.keys ? p.keys : a);
      b = b < a ? a : (b > p.keys ? p.keys : b);
      rs_[i] = a;
      re_[i] = b;
      load_query(qr[i], p.q, p.weights, r);
    }
  }
  const int nch = (c_end - c_begin + kChunk - 1) / kChunk;
  uint4 regs[1];
  stage_chunk_regs(regs, p.k, p.col0 + c_begin, p.keys, tid, kDThreads);
  store_chunk_regs(regs, kbuf[0], tid, kDThreads);
  __syncthreads();
  for (int c = 0; c < nch; ++c) {
    const int cc0 = c_begin + c * kChunk;
    const bool more = c + 1 < nch;
    if (more) stage_chunk_regs(regs, p.k, p.col0 + cc0 + kChunk, p.keys, tid, kDThreads);
    const int cc = cc0 + l;
    const int64_t key = (int64_t)p.col0 + cc;
    const float sc = p.scales[key < p.keys ? key : p.keys - 1];
    KeyTile kt;
    load_keys_lds(kt, kbuf[c & 1]);
#pragma unroll
    for (int i = 0; i < kDRowsPerWave; ++i) {
      if (rr[i] >= p.rows) continue;
      float E = -__builtin_inff();
      if (rs_[i] < p.col0 + cc0 + kChunk && re_[i] > p.col0 + cc0)
        E = score_chunk_exact(qr[i], kt) * sc;
      const bool valid = key >= rs_[i] && key < re_[i];
      if (cc < c_end) p.logits[(int64_t)rr[i] * p.ld + cc] = valid ? E : -__builtin_inff();
    }
    if (more) store_chunk_regs(regs, kbuf[(c + 1) & 1], tid, kDThreads);
    __syncthreads();
  }
}

// Per-row exact top-k over the row's visible columns of the logits window:
// radix select on the order-preserving uint32 of the fp32 logit (digits of
// 11, 11 and 10 bits, histogram in LDS), then one output pass. One 1024-thread
// workgroup per row.
__global__ __launch_bounds__(1024) void dense_topk_kernel(DenseTopkParams p) {
  __shared__ uint32_t hist[2048];
  __shared__ int sh_digit, sh_above, sh_cnt, cur_up, cur_tie;
  const int tid = threadIdx.x;
  const int r = blockIdx.x;
  const int k = p.topk;
  int s = p.starts[r], e = p.ends[r];
  s = s < 0 ? 0 : (s > p.keys ? p.keys : s);
  e = e < s ? s : (e > p.keys ? p.keys : e);
  int c_lo = (s > p.col0 ? s : p.col0) - p.col0;
  int c_hi = (e < p.col0 + p.ncols ? e : p.col0 + p.ncols) - p.col0;
  const int n = c_hi > c_lo ? c_hi - c_lo : 0;
  int32_t* o = p.out + (int64_t)r * k;
  const int shift_out = p.col0 - s;  // key - s = c + col0 - s
  if (n <= k) {
    for (int j = tid; j < k; j += 1024) o[j] = j < n ? c_lo + j + shift_out : -1;
    return;
  }
  const float* row = p.logits + (int64_t)r * p.ld + c_lo;
  uint32_t prefix = 0, pmask = 0;
  int need = k;
  bool done = false;
  const int shifts[3] = {21, 10, 0};
  const int widths[3] = {11, 11, 10};
  for (int lev = 0; lev < 3 && !done; ++lev) {
    const int sh = shifts[lev];
    const uint32_t dmask = (1u << widths[lev]) - 1u;
    const int nb = 1 << widths[lev];
    for (int b = tid; b < nb; b += 1024) hist[b] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += 1024) {
      const uint32_t key = fkey(row[i]);
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> sh) & dmask], 1u);
    }
    __syncthreads();
    if (tid < kWave) {
      const int l = tid;
      const int per = nb / kWave;
      int mine = 0;
      for (int b = 0; b < per; ++b) mine += (int)hist[nb - 1 - (l * per + b)];
      const int incl = wave_incl_scan(mine);
      const int excl = incl - mine;
      const uint64_t hit = __ballot(incl >= need);
      const int src = hit ? __builtin_ctzll(hit) : 63;
      if (l == src) {
        int c = excl;
        int digit = 0, above = 0, cnt = 0;
        for (int b = 0; b < per; ++b) {
          const int bin = nb - 1 - (l * per + b);
          const int h = (int)hist[bin];
          if (c + h >= need) {
            digit = bin;
            above = c;
            cnt = h;
            break;
          }
          c += h;
        }
        sh_digit = digit;
        sh_above = above;
        sh_cnt = cnt;
      }
    }
    __syncthreads();
    need -= sh_above;
    prefix |= (uint32_t)sh_digit << sh;
    pmask |= dmask << sh;
    if (sh_cnt == need) done = true;
    __syncthreads();
  }
  if (tid == 0) {
    cur_up = 0;
    cur_tie = 0;
  }
  __syncthreads();
  const int n_above = k - need;
  for (int i = tid; i < n; i += 1024) {
    const uint32_t key = fkey(row[i]);
    if ((key & pmask) > prefix) {
      const int slot = atomicAdd(&cur_up, 1);
      if (slot < n_above) o[slot] = c_lo + i + shift_out;
    } else if ((key & pmask) == prefix) {
      const int t = atomicAdd(&cur_tie, 1);
      if (t < need) o[n_above + t] = c_lo + i + shift_out;
    }
  }
}

__global__ void key_scales_kernel(const uint32_t* b, float* s, int keys) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j < keys) s[j] = __uint_as_float((b[j] & 0xFFu) << 23);
}

}  // namespace mqa

extern "C" int mqa_dense_logits_launch(const mqa::DenseParams* p, hipStream_t stream) {
  dim3 grid((p->ncols + mqa::kDCols - 1) / mqa::kDCols, (p->rows + mqa::kDBlockRows - 1) / mqa::kDBlockRows);
  hipLaunchKernelGGL(mqa::dense_logits_kernel, grid, dim3(mqa::kDThreads), 0, stream, *p);
  return (int)hipGetLastError();
}

extern "C" int mqa_dense_topk_launch(const mqa::DenseTopkParams* p, hipStream_t stream) {
  hipLaunchKernelGGL(mqa::dense_topk_kernel, dim3(p->rows), dim3(1024), 0, stream, *p);
  return (int)hipGetLastError();
}

extern "C" int mqa_key_scales_launch(const uint8_t* b, float* s, int keys, hipStream_t stream) {
  hipLaunchKernelGGL(mqa::key_scales_kernel, dim3((keys + 255) / 256), dim3(256), 0, stream,
                     reinterpret_cast<const uint32_t*>(b), s, keys);
  return (int)hipGetLastError();
}
