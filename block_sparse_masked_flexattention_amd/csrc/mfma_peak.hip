// mfma_peak.hip -- measured matrix-unit peak of the part: every wave issues
// nothing but independent chains of v_mfma_f32_32x32x16_bf16 (the product
// instruction of the bf16 forward), so the launch time gives the dense bf16
// rate the hardware sustains, and each wave's shader-clock and real-time
// counters give the clock it ran at.
#include "internal.hpp"

namespace flexattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kPeakThreads = 256;  // 4 waves per work-group
constexpr int kPeakChains = 4;     // independent accumulator chains per wave

__global__ __launch_bounds__(kPeakThreads) void mfma_peak_kernel(int iters, float* sink,
                                                                 uint64_t* clocks) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)(lane + i));
    b[i] = (__bf16)(0.002f * (float)(lane - i));
  }
  f32x16 c[kPeakChains];
#pragma unroll
  for (int j = 0; j < kPeakChains; ++j) c[j] = f32x16{};
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kPeakChains; ++j)
      c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
  }
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < kPeakChains; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc += c[j][r];
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  sink[(size_t)blockIdx.x * kPeakThreads + tid] = acc;
  if (lane == 0) {
    const size_t w = (size_t)blockIdx.x * (kPeakThreads / 64) + wave;
    clocks[2 * w] = t1 - t0;
    clocks[2 * w + 1] = r1 - r0;
  }
}

}  // namespace
}  // namespace flexattn

extern "C" int32_t flex_attn_mfma_peak_probe(int32_t n_workgroups, int32_t iters, float* sink,
                                             uint64_t* clocks, void* stream) {
  if (n_workgroups <= 0 || iters <= 0 || !sink || !clocks) return FLEX_E_INVALID_ARG;
  if (((uintptr_t)sink & 3u) || ((uintptr_t)clocks & 7u)) return FLEX_E_INVALID_ARG;
  hipLaunchKernelGGL(flexattn::mfma_peak_kernel, dim3((unsigned)n_workgroups),
                     dim3(flexattn::kPeakThreads), 0, static_cast<hipStream_t>(stream), iters,
                     sink, clocks);
  return hipGetLastError() == hipSuccess ? FLEX_OK : FLEX_E_HIP;
}
