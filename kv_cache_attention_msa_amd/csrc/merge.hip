// a5: log-sum-exp merge of attention partials.
//
// The MSA pseudocode (P1, "Core method 1: MSA") adds up per-segment
// attention results, each scaled by a per-segment normaliser that the pages
// do not define.  It is read here as the log-sum-exp weight, which makes the
// stitched result equal to attention over the union of the keys:
//   M = max_i m_i,  w_i = exp(m_i - M) (0 for an empty partial),
//   L = sum_i w_i l_i,  out = sum_i w_i o_i / L,  lse = M + ln L.
// Partials are visited in their stored (logical) order, so the result is
// deterministic run to run.
//
// One workgroup covers 128 consecutive (head, d) elements of one (sequence,
// row); every thread folds the sequence's partials for its element in one
// pass with a running maximum, eight partials' loads in flight at a time.
#include "msa_internal.h"

namespace msa {
namespace {

constexpr int kThreads = 128;
constexpr int kUnroll = 8;  // partials whose loads are issued together
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ void store_o(void* out, size_t idx, float v, msa_dtype dt) {
  if (dt == MSA_BF16)
    static_cast<uint16_t*>(out)[idx] = f32_to_bf16(v);
  else
    static_cast<float*>(out)[idx] = v;
}

// mode 0: partials [indptr[b], indptr[b+1]); mode 1: derived from the plan
struct MergeArgs {
  const float* o_part;
  const float* m_part;
  const float* l_part;
  const int32_t* part_indptr;
  const msa_segment* segs;
  const int32_t* seg_indptr;
  int32_t S, split_blocks;
  int32_t B, R, H, D;
  msa_dtype out_dtype;
  void* out;
  float* lse;
};

template <int MODE>
__global__ void __launch_bounds__(kThreads) merge_kernel(MergeArgs a) {
  const int b = blockIdx.z, r = blockIdx.y;
  const int e = blockIdx.x * kThreads + threadIdx.x;
  const int HD = a.H * a.D;
  int lo, n;
  if (MODE == 0) {
    lo = a.part_indptr[b];
    n = a.part_indptr[b + 1] - lo;
  } else {
    const int A = plan_alive_tokens(a.segs, a.seg_indptr, b);
    // same clamp as the attention kernels: never more partials than the grid had
    const int nAB = min((A + 15) / 16, a.S * a.split_blocks);
    n = (nAB + a.split_blocks - 1) / a.split_blocks;
    if (n == 1) return;  // the attention kernel wrote this sequence itself
    lo = b * a.S;
  }
  if (e >= HD) return;
  const int h = e / a.D, d = e % a.D;
  const size_t orow = (size_t(b) * a.R + r) * a.H + h;
  // running (M, L, O) in log2 units; a partial with a larger maximum rescales
  // what was folded so far, exactly as the two-pass form would weight it
  float M = -INFINITY, L = 0.f, O = 0.f;
  for (int i0 = 0; i0 < n; i0 += kUnroll) {
    float mi[kUnroll], li[kUnroll], oi[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      const bool in = i0 + k < n;
      const size_t pr = (size_t(lo + (in ? i0 + k : 0)) * a.R + r) * a.H + h;
      mi[k] = in ? a.m_part[pr] : -INFINITY;
      li[k] = in ? a.l_part[pr] : 0.f;
      oi[k] = in ? a.o_part[pr * a.D + d] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      if (mi[k] == -INFINITY) continue;  // empty partial: its o is never used
      const float m2 = mi[k] * kLog2e;
      if (m2 > M) {
        const float sc = M == -INFINITY ? 0.f : exp2f(M - m2);
        L *= sc;
        O *= sc;
        M = m2;
      }
      const float wi = exp2f(m2 - M);
      L = fmaf(wi, li[k], L);
      O = fmaf(wi, oi[k], O);
    }
  }
  const bool ok = L > 0.f;
  store_o(a.out, orow * a.D + d, ok ? O / L : 0.f, a.out_dtype);
  if (a.lse && d == 0) a.lse[orow] = ok ? (M + log2f(L)) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_merge_from_plan(const float* o_part, const float* m_part, const float* l_part,
                                  const msa_segment* segs, const int32_t* indptr, int32_t B,
                                  int32_t R, int32_t H, int32_t D, int32_t S,
                                  int32_t split_blocks, msa_dtype out_dtype, void* out,
                                  float* lse, hipStream_t stream) {
  MergeArgs a{o_part, m_part, l_part, nullptr, segs, indptr, S, split_blocks,
              B, R, H, D, out_dtype, out, lse};
  dim3 grid((H * D + kThreads - 1) / kThreads, R, B);
  hipLaunchKernelGGL(merge_kernel<1>, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_merge_indptr(const float* o_part, const float* m_part, const float* l_part,
                               const int32_t* part_indptr, int32_t B, int32_t R, int32_t H,
                               int32_t D, msa_dtype out_dtype, void* out, float* lse,
                               hipStream_t stream) {
  MergeArgs a{o_part, m_part, l_part, part_indptr, nullptr, nullptr, 0, 0,
              B, R, H, D, out_dtype, out, lse};
  dim3 grid((H * D + kThreads - 1) / kThreads, R, B);
  hipLaunchKernelGGL(merge_kernel<0>, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace msa
