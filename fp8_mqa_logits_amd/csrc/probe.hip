// FP8 MFMA throughput probe: the achievable rate of the instruction the scan's
// head tiles use (v_mfma_f32_16x16x128_f8f6f4), measured on the machine that
// runs the scan, so that the scan's MFMA fraction can be read against both the
// published peak and the clock the part actually sustains.
#include "common.h"

namespace mqa {

constexpr int kProbeThreads = 512;  // 8 waves, 2 per SIMD (the scan's occupancy)
constexpr int kProbeChains = 8;     // independent accumulators per wave

// Each wave issues `iters` rounds of kProbeChains independent MFMAs on
// register operands (e4m3 codes 0x30..0x37: 0.5 .. 0.9375, so the sums stay
// finite) and writes one value per thread.
__global__ __launch_bounds__(kProbeThreads) void mfma_peak_kernel(float* out, int iters) {
  const int l = lane_id();
  const int code = 0x30 + (l & 7);
  const int word = code | (code << 8) | (code << 16) | (code << 24);
  const v8i a = {word, word, word, word, word, word, word, word};
  const v8i b = a;
  v4f acc[kProbeChains];
#pragma unroll
  for (int j = 0; j < kProbeChains; ++j) acc[j] = v4f{0.f, 0.f, 0.f, (float)j};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < kProbeChains; ++j) acc[j] = mfma_fp8(a, b, acc[j]);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kProbeChains; ++j) s += (acc[j][0] + acc[j][1]) + (acc[j][2] + acc[j][3]);
  out[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = s;
}

// The scan's FP8 MFMA forms on caller operands (a test aid that pins the
// instruction's accumulation rule): case c = blockIdx.x * 4 + wave. Lane l
// holds row l % 16 of A and of B (bytes 32 * (l / 16) ..), as the scan's
// operands; with scales, lane l supplies A row l % 16's E8M0 scale of K block
// l / 16 and B's scale is 1 (the fold-term form).
template <bool SCALED>
__global__ __launch_bounds__(256) void fp8_mfma_probe_kernel(const uint8_t* __restrict__ a,
                                                             const uint8_t* __restrict__ b,
                                                             const uint8_t* __restrict__ sa,
                                                             float* __restrict__ out, int ncases) {
  const int c = blockIdx.x * 4 + wave_id();
  if (c >= ncases) return;
  const int l = lane_id();
  const int m = l & 15, g = l >> 4;
  const int64_t off = (int64_t)c * 2048 + m * 128 + 32 * g;
  const uint4 a0 = *reinterpret_cast<const uint4*>(a + off);
  const uint4 a1 = *reinterpret_cast<const uint4*>(a + off + 16);
  const uint4 b0 = *reinterpret_cast<const uint4*>(b + off);
  const uint4 b1 = *reinterpret_cast<const uint4*>(b + off + 16);
  const v8i av = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                  (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
  const v8i bv = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w,
                  (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
  const v4f z = {0.f, 0.f, 0.f, 0.f};
  v4f r;
  if constexpr (SCALED) {
    const int s = sa[(int64_t)c * 64 + m * 4 + g];
    r = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, z, 0, 0, 0, s, 0, 127);
  } else {
    r = mfma_fp8(av, bv, z);
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) out[(int64_t)c * 256 + (4 * g + v) * 16 + m] = r[v];
}

}  // namespace mqa

extern "C" int mqa_fp8_mfma_probe_launch(const uint8_t* a, const uint8_t* b, const uint8_t* sa,
                                         float* out, int ncases, hipStream_t stream) {
  const int blocks = (ncases + 3) / 4;
  if (sa)
    hipLaunchKernelGGL(mqa::fp8_mfma_probe_kernel<true>, dim3(blocks), dim3(256), 0, stream, a, b,
                       sa, out, ncases);
  else
    hipLaunchKernelGGL(mqa::fp8_mfma_probe_kernel<false>, dim3(blocks), dim3(256), 0, stream, a,
                       b, sa, out, ncases);
  return (int)hipGetLastError();
}

extern "C" int mqa_mfma_peak_launch(float* out, int workgroups, int iters, hipStream_t stream) {
  hipLaunchKernelGGL(mqa::mfma_peak_kernel, dim3(workgroups), dim3(mqa::kProbeThreads), 0, stream,
                     out, iters);
  return (int)hipGetLastError();
}
