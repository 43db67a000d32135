// Matrix-core throughput of this GPU for the instruction the chunked-prefill
// kernel is built on (v_mfma_f32_32x32x16_bf16), measured with register
// operands only: no memory traffic, no LDS, eight independent accumulators
// per wavefront.  The bench reports it beside the published dense bf16 peak
// as the rate the matrix cores sustain at the clock they hold under this
// load.  This library is a measuring instrument, not part of the attention
// path, and is built and loaded separately from libmsa.so.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/msa_peaks.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;  // four wavefronts, one per SIMD of a CU
constexpr int kChains = 8;     // independent accumulators per wavefront

__global__ void __launch_bounds__(kThreads) mfma_rate_kernel(int32_t iters, float* sink) {
  const int lane = threadIdx.x % 64;
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = __bf16(float((lane + i) % 17) * (1.0f / 64.0f));
    b[i] = __bf16(float((lane * 3 + i) % 13) * (1.0f / 64.0f));
  }
  f32x16_t c[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) c[j][i] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kChains; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kChains; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += c[j][i];
  sink[size_t(blockIdx.x) * kThreads + threadIdx.x] = s;
}

}  // namespace

// Launches `workgroups` workgroups of 256 threads on `stream` (a hipStream_t,
// NULL for the default stream); every wavefront issues iters x 8 MFMAs, so
// one call performs workgroups * 4 * iters * 8 * 32768 flops.  `sink` is a
// device buffer of workgroups * 256 floats that receives one sum per thread
// (it keeps the results live).  Returns 0 when the launch was accepted, -1
// for arguments outside workgroups in [1, 2^20] and iters in [1, 2^20] or a
// null sink, otherwise the HIP error code of the launch.
extern "C" int msa_peaks_mfma_bf16(int32_t workgroups, int32_t iters, float* sink, void* stream) {
  if (workgroups < 1 || workgroups > (1 << 20) || iters < 1 || iters > (1 << 20) || sink == nullptr)
    return -1;
  hipLaunchKernelGGL(mfma_rate_kernel, dim3(workgroups), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), iters, sink);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? 0 : int(e);
}
