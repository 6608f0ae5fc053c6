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

}  // namespace mqa

extern "C" int mqa_mfma_peak_launch(float* out, int workgroups, int iters, hipStream_t stream) {
  hipLaunchKernelGGL(mqa::mfma_peak_kernel, dim3(workgroups), dim3(mqa::kProbeThreads), 0, stream,
                     out, iters);
  return (int)hipGetLastError();
}
