// Plain CPU oracle for FP8 MQA logits and per-row top-k selection.
//
// TEST INFRASTRUCTURE ONLY. Nothing in the product path (the HIP library and
// its Python binding) may include, link or call this file; only the tests, the
// smoke check and the benchmark's CPU-baseline leg use it. It shares no code,
// header, table or constant with the GPU path.
//
// What it computes (all citations are to the source pages):
//   * vLLM API page "fused_mqa_topk", function fused_mqa_topk_prefill:
//     q [rows,32,128] e4m3, k [keys,128] e4m3, scales [keys] fp32,
//     weights [rows,32] fp32, starts/ends [rows] int32 giving the visible key
//     range [start, end) of each row; output [rows,k] int32 holding each
//     selected key minus the row's start, in no particular order, with -1 in
//     the slots left over when the row sees fewer than k keys.
//   * same page, function fused_mqa_topk_key_scales: a UE8M0 scale byte e
//     decodes to the fp32 whose bit pattern is e << 23.
//   * vLLM PR #60618, "What this PR does" (Scoring): 32 index heads, each
//     head's dot product passes through relu and is weighted by its per-row
//     head weight, and the weighted heads are summed. The same PR's
//     "Limitations of this PR -- TODOs" names DeepSeek-V3.2's 64 index heads:
//     the oracle takes heads = 32 or 64 (q [rows,heads,128], weights
//     [rows,heads]), the same sum over all heads.
//   Reading taken for the full formula (the pages never print it in one
//   piece): logit[r,j] = scale_j * sum_h w[r,h] * relu(q[r,h,:] . k[j,:]).
//
// Precision:
//   * Every e4m3 value is an integer multiple of 2^-9 with magnitude <= 448,
//     so a product of two is a multiple of 2^-18 and a 128-term dot product
//     stays below 2^25 in magnitude: it needs at most 43 significant bits and
//     is therefore EXACT in double in any summation order.
//   * The head sum runs in double, in head order 0..heads-1, is multiplied by the
//     scale in double (a power of two: exact barring underflow) and rounded
//     once to fp32.
//   * Top-k: a full sort of the row by (logit descending, key ascending); the
//     first k keys are the answer. Ties at the k-th score make several answers
//     correct (the API page's use_fused_mqa_topk: the fused op keeps whichever
//     tied keys its atomic updates reach first); this order is one of them.
//
// Pins (tests/test_oracle_pins.py): all 256 e4m3 codes against their closed
// form and a library decoder, UE8M0 spot values, a hand-worked 4-key example,
// the relu identity, the scale bit-pattern rule, closed-form extreme dots, and
// brute-force subset enumeration for the selection.

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <thread>
#include <vector>

namespace {

// 32 index heads (GLM-5.x, DeepSeek-V4.1) or 64 (DeepSeek-V3.2: PR #60618,
// "Limitations of this PR -- TODOs"); the formula is the same sum over heads.
constexpr int kMaxHeads = 64;
constexpr int kDim = 128;

// OCP FP8 E4M3FN (torch.float8_e4m3fn): 1 sign bit, 4 exponent bits with
// bias 7, 3 mantissa bits; exponent field 0 is subnormal (m * 2^-9); the
// codes 0x7F and 0xFF are NaN; there are no infinities; the largest finite
// magnitude is 448.
double e4m3_value(uint8_t code) {
  const int sign = code >> 7;
  const int e = (code >> 3) & 0xF;
  const int m = code & 0x7;
  if (e == 15 && m == 7) return std::numeric_limits<double>::quiet_NaN();
  double mag;
  if (e == 0)
    mag = std::ldexp(static_cast<double>(m), -9);
  else
    mag = std::ldexp(1.0 + m / 8.0, e - 7);
  return sign ? -mag : mag;
}

// Decoded value of every code, filled once when the library loads.
alignas(64) double g_e4m3[256];
struct TableInit {
  TableInit() {
    for (int c = 0; c < 256; ++c) g_e4m3[c] = e4m3_value(static_cast<uint8_t>(c));
  }
} g_table_init;

// fused_mqa_topk_key_scales: view the four bytes as a little-endian int32,
// keep the low byte e, and shift it into the fp32 exponent field.
float ue8m0_scale(const uint8_t* four_bytes) {
  uint32_t word;
  std::memcpy(&word, four_bytes, 4);
  const uint32_t bits = (word & 0xFFu) << 23;
  float f;
  std::memcpy(&f, &bits, 4);
  return f;
}

struct Problem {
  const uint8_t* q;
  const uint8_t* k;
  const float* scales;
  const float* weights;
  const int32_t* starts;
  const int32_t* ends;
  int64_t rows;
  int64_t keys;
  int heads;
};

// Visible range of row r. The pages require [start, end) inside [0, keys);
// values outside are clamped (the same reading the GPU library documents).
void row_range(const Problem& p, int64_t r, int64_t* s, int64_t* e) {
  int64_t a = p.starts[r], b = p.ends[r];
  a = std::min<int64_t>(std::max<int64_t>(a, 0), p.keys);
  b = std::min<int64_t>(std::max<int64_t>(b, a), p.keys);
  *s = a;
  *e = b;
}

// Decoded query of one row, stored dimension-major: qd[d*heads + h].
void decode_query(const Problem& p, int64_t r, double* qd) {
  const uint8_t* qr = p.q + r * p.heads * kDim;
  for (int h = 0; h < p.heads; ++h)
    for (int d = 0; d < kDim; ++d) qd[d * p.heads + h] = g_e4m3[qr[h * kDim + d]];
}

// The per-head dot products s[h] = sum_d q[h,d] * k[j,d] of one key.
// Each s[h] is accumulated over d = 0..127 in order; the loop runs over the
// heads innermost only so that the independent sums advance together.
__attribute__((target_clones("avx512f", "avx2", "default")))
void head_dots(const double* __restrict__ qd, const uint8_t* __restrict__ kj,
               double* __restrict__ s, int heads) {
  double kd[kDim];
  for (int d = 0; d < kDim; ++d) kd[d] = g_e4m3[kj[d]];
  double acc[kMaxHeads];
  for (int h = 0; h < heads; ++h) acc[h] = 0.0;
  for (int d = 0; d < kDim; ++d) {
    const double* qrow = qd + d * heads;
    for (int h = 0; h < heads; ++h) acc[h] += qrow[h] * kd[d];
  }
  for (int h = 0; h < heads; ++h) s[h] = acc[h];
}

// logit[r,j] = scale_j * sum_h w[r,h] * relu(s[h]), head sum in double in
// head order, one rounding to fp32 at the end.
float logit_of(const Problem& p, int64_t r, const double* qd, int64_t j) {
  double s[kMaxHeads];
  head_dots(qd, p.k + j * kDim, s, p.heads);
  const float* w = p.weights + r * p.heads;
  double sum = 0.0;
  for (int h = 0; h < p.heads; ++h) {
    const double relu = s[h] > 0.0 ? s[h] : 0.0;
    sum += static_cast<double>(w[h]) * relu;
  }
  return static_cast<float>(static_cast<double>(p.scales[j]) * sum);
}

bool inputs_in_contract(const Problem& p) {
  if (p.heads != 32 && p.heads != 64) return false;
  for (int64_t i = 0; i < p.rows * p.heads * kDim; ++i)
    if ((p.q[i] & 0x7F) == 0x7F) return false;
  for (int64_t i = 0; i < p.keys * kDim; ++i)
    if ((p.k[i] & 0x7F) == 0x7F) return false;
  for (int64_t i = 0; i < p.keys; ++i)
    if (!std::isfinite(p.scales[i]) || p.scales[i] < 0.0f) return false;
  for (int64_t i = 0; i < p.rows * p.heads; ++i)
    if (!std::isfinite(p.weights[i])) return false;
  return true;
}

// The kk best positions of v[0..n) by (value descending, position ascending):
// a full sort, then the first kk.
void sort_select(const float* v, int64_t n, int64_t kk, int32_t* out) {
  std::vector<int32_t> order(n);
  for (int64_t c = 0; c < n; ++c) order[c] = static_cast<int32_t>(c);
  std::sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
    if (v[a] != v[b]) return v[a] > v[b];
    return a < b;
  });
  for (int64_t c = 0; c < kk && c < n; ++c) out[c] = order[c];
}

template <class F>
void parallel_rows(int64_t n, int nthreads, F&& f) {
  if (nthreads <= 0) nthreads = static_cast<int>(std::thread::hardware_concurrency());
  if (nthreads <= 0) nthreads = 1;
  nthreads = static_cast<int>(std::min<int64_t>(nthreads, std::max<int64_t>(n, 1)));
  std::atomic<int64_t> next{0};
  auto worker = [&]() {
    for (;;) {
      const int64_t i = next.fetch_add(1);
      if (i >= n) break;
      f(i);
    }
  };
  std::vector<std::thread> pool;
  for (int t = 1; t < nthreads; ++t) pool.emplace_back(worker);
  worker();
  for (auto& th : pool) th.join();
}

}  // namespace

extern "C" {

// Returns the decoded value of every e4m3 code (NaN for 0x7F and 0xFF).
void oracle_e4m3_table(double* out256) {
  for (int c = 0; c < 256; ++c) out256[c] = g_e4m3[c];
}

// UE8M0 [keys,4] bytes -> fp32 [keys].
void oracle_key_scales(const uint8_t* bytes, int64_t keys, float* out) {
  for (int64_t j = 0; j < keys; ++j) out[j] = ue8m0_scale(bytes + 4 * j);
}

// Exact per-head dot products of a query row (heads x 128 codes) against one
// key (for the pins).
int oracle_head_dots(const uint8_t* q_row, const uint8_t* k_row, double* out, int heads) {
  if (heads != 32 && heads != 64) return -1;
  double qd[kDim * kMaxHeads];
  for (int h = 0; h < heads; ++h)
    for (int d = 0; d < kDim; ++d) qd[d * heads + h] = g_e4m3[q_row[h * kDim + d]];
  head_dots(qd, k_row, out, heads);
  return 0;
}

// Logits of the selected rows over columns [col0, col0 + ncols) (a column c is
// key col0 + c). Keys outside a row's visible range, and columns past the last
// key, get -inf. out: [nsel, ncols] fp32.
// Returns 0, or -1 if an input is outside the contract (NaN codes, non-finite
// or negative scales, non-finite weights, a bad row id).
int oracle_logits(const uint8_t* q, const uint8_t* k, const float* scales,
                  const float* weights, const int32_t* starts, const int32_t* ends,
                  int64_t rows, int64_t keys, int heads, const int32_t* sel, int64_t nsel,
                  int64_t col0, int64_t ncols, float* out, int nthreads) {
  Problem p{q, k, scales, weights, starts, ends, rows, keys, heads};
  if (!inputs_in_contract(p)) return -1;
  for (int64_t i = 0; i < nsel; ++i)
    if (sel[i] < 0 || sel[i] >= rows) return -1;
  const float ninf = -std::numeric_limits<float>::infinity();
  parallel_rows(nsel, nthreads, [&](int64_t i) {
    const int64_t r = sel[i];
    std::vector<double> qd(kDim * p.heads);
    decode_query(p, r, qd.data());
    int64_t s, e;
    row_range(p, r, &s, &e);
    float* o = out + i * ncols;
    for (int64_t c = 0; c < ncols; ++c) {
      const int64_t j = col0 + c;
      o[c] = (j >= s && j < e) ? logit_of(p, r, qd.data(), j) : ninf;
    }
  });
  return 0;
}

// Top-k of the selected rows. out_idx: [nsel, topk] int32, key - start of the
// k best keys (oracle order: logit descending, key ascending), -1 padded when
// the row sees n <= topk keys (then slots [0, n) hold 0..n-1).
// kth[i]: the k-th largest logit (-inf when n <= topk).
// maxabs[i]: max |logit| over the row's visible keys (0 when n == 0).
// Returns 0, or -1 on inputs outside the contract or topk < 1.
int oracle_topk(const uint8_t* q, const uint8_t* k, const float* scales,
                const float* weights, const int32_t* starts, const int32_t* ends,
                int64_t rows, int64_t keys, int heads, const int32_t* sel, int64_t nsel,
                int64_t topk, int32_t* out_idx, float* kth, float* maxabs,
                int nthreads) {
  Problem p{q, k, scales, weights, starts, ends, rows, keys, heads};
  if (topk < 1 || !inputs_in_contract(p)) return -1;
  for (int64_t i = 0; i < nsel; ++i)
    if (sel[i] < 0 || sel[i] >= rows) return -1;
  parallel_rows(nsel, nthreads, [&](int64_t i) {
    const int64_t r = sel[i];
    std::vector<double> qd(kDim * p.heads);
    decode_query(p, r, qd.data());
    int64_t s, e;
    row_range(p, r, &s, &e);
    const int64_t n = e - s;
    std::vector<float> lg(n);
    float mx = 0.0f;
    for (int64_t c = 0; c < n; ++c) {
      lg[c] = logit_of(p, r, qd.data(), s + c);
      mx = std::max(mx, std::fabs(lg[c]));
    }
    maxabs[i] = mx;
    int32_t* o = out_idx + i * topk;
    if (n <= topk) {
      for (int64_t c = 0; c < topk; ++c) o[c] = c < n ? static_cast<int32_t>(c) : -1;
      kth[i] = -std::numeric_limits<float>::infinity();
      return;
    }
    sort_select(lg.data(), n, topk, o);
    kth[i] = lg[o[topk - 1]];
  });
  return 0;
}

// The selection step of oracle_topk on its own, exposed so that tests can pin
// it against brute-force subset enumeration.
void oracle_select(const float* v, int64_t n, int64_t kk, int32_t* out) {
  sort_select(v, n, kk, out);
}

}  // extern "C"
