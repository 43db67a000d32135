// a5: log-sum-exp merge of attention partials.
//
// The MSA pseudocode (P1, "Core method 1: MSA") adds up per-segment
// attention results, each scaled by a per-segment normaliser that the pages
// do not define.  It is read here as the log-sum-exp weight, which makes the
// stitched result equal to attention over the union of the keys:
//   M = max_i m_i,  w_i = exp(m_i - M) (0 for an empty partial),
//   L = sum_i w_i l_i,  out = sum_i w_i o_i / L,  lse = M + ln L.
// The combination order is fixed (below), so the result is deterministic
// run to run; mathematically it does not depend on the order.
//
// One workgroup covers 256/NG consecutive (head, d) elements of one
// (sequence, row) with 256 threads: thread (group j, element e) folds
// partials j, j+NG, j+2NG, ... of element e with a running maximum, and the
// NG group states of an element are then combined in LDS in group order.
// The merge is bound by how many loads are in flight, not by arithmetic:
// one thread per element folding all of a sequence's partials (69 per
// sequence on the 131k-token batch) kept too few loads outstanding (9.5 us
// for 9 MB of partials).  NG follows the split count (1 up to 4 partials per
// sequence, 2 up to 16, 4 up to 32, else 8): more groups than partials only
// multiply workgroups that have nothing to do.
#include "msa_internal.h"

namespace msa {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;  // a thread's partials loaded together
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ void store_o(void* out, size_t idx, float v, msa_dtype dt) {
  if (dt == MSA_BF16)
    static_cast<uint16_t*>(out)[idx] = f32_to_bf16(v);
  else
    static_cast<float*>(out)[idx] = v;
}

// mode 0: partials [indptr[b], indptr[b+1]); mode 1: derived from the plan;
// mode 2: as mode 0, but a sequence with one partial is skipped (the
// attention kernel wrote it)
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

// (M, L, O) <- (M, L, O) (+) (m2, l2, o2), log2 units; an empty state has
// M = -inf and contributes nothing
__device__ __forceinline__ void fold(float& M, float& L, float& O, float m2, float l2, float o2) {
  if (m2 == -INFINITY) return;
  if (m2 > M) {
    const float sc = M == -INFINITY ? 0.f : exp2f(M - m2);
    L *= sc;
    O *= sc;
    M = m2;
  }
  const float w = exp2f(m2 - M);
  L = fmaf(w, l2, L);
  O = fmaf(w, o2, O);
}

template <int MODE, int NG>
__global__ void __launch_bounds__(kThreads) merge_kernel(MergeArgs a) {
  constexpr int kGroups = NG, kElems = kThreads / NG;
  __shared__ float sM[kGroups][kElems], sL[kGroups][kElems], sO[kGroups][kElems];
  const int b = blockIdx.z, r = blockIdx.y;
  const int el = threadIdx.x % kElems, grp = threadIdx.x / kElems;
  const int e = blockIdx.x * kElems + el;
  const int HD = a.H * a.D;
  int lo, n;
  if (MODE != 1) {
    lo = a.part_indptr[b];
    n = a.part_indptr[b + 1] - lo;
    if (MODE == 2 && n <= 1) return;
  } else {
    const int A = plan_alive_tokens(a.segs, a.seg_indptr, b);
    // same clamp as the attention kernels: never more partials than the grid had
    const int nAB = min((A + 15) / 16, a.S * a.split_blocks);
    n = (nAB + a.split_blocks - 1) / a.split_blocks;
    if (n == 1) return;  // the attention kernel wrote this sequence itself
    lo = b * a.S;
  }
  const bool valid = e < HD;
  const int ec = valid ? e : 0;
  const int h = ec / a.D, d = ec % a.D;
  const size_t stride = size_t(a.R) * a.H;  // between consecutive partials' (row, head)
  const size_t first = (size_t(lo) * a.R + r) * a.H + h;
  // this thread's partials: grp, grp + 8, ... in order, with a running maximum
  float M = -INFINITY, L = 0.f, O = 0.f;
  for (int i0 = grp; i0 < n; i0 += kGroups * kUnroll) {
    float mi[kUnroll], li[kUnroll], oi[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      const int i = i0 + k * kGroups;
      const bool in = valid && i < n;
      const size_t pr = first + size_t(in ? i : 0) * stride;
      mi[k] = in ? a.m_part[pr] : -INFINITY;
      li[k] = in ? a.l_part[pr] : 0.f;
      oi[k] = in ? a.o_part[pr * a.D + d] : 0.f;  // used only if m_i > -inf
    }
#pragma unroll
    for (int k = 0; k < kUnroll; ++k)
      fold(M, L, O, mi[k] == -INFINITY ? -INFINITY : mi[k] * kLog2e, li[k], oi[k]);
  }
  sM[grp][el] = M;
  sL[grp][el] = L;
  sO[grp][el] = O;
  __syncthreads();
  if (grp != 0 || !valid) return;
  // combine the groups in order (deterministic run to run)
#pragma unroll
  for (int j = 1; j < kGroups; ++j) fold(M, L, O, sM[j][el], sL[j][el], sO[j][el]);
  const size_t orow = (size_t(b) * a.R + r) * a.H + h;
  const bool ok = L > 0.f;
  store_o(a.out, orow * a.D + d, ok ? O / L : 0.f, a.out_dtype);
  if (a.lse && d == 0) a.lse[orow] = ok ? (M + log2f(L)) * kLn2 : -INFINITY;
}

template <int MODE>
hipError_t launch_ng(const MergeArgs& a, int groups, hipStream_t stream) {
  const int HD = a.H * a.D;
  switch (groups) {
    case 1: hipLaunchKernelGGL((merge_kernel<MODE, 1>), dim3((HD + 255) / 256, a.R, a.B), dim3(kThreads), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((merge_kernel<MODE, 2>), dim3((HD + 127) / 128, a.R, a.B), dim3(kThreads), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((merge_kernel<MODE, 4>), dim3((HD + 63) / 64, a.R, a.B), dim3(kThreads), 0, stream, a); break;
    default: hipLaunchKernelGGL((merge_kernel<MODE, 8>), dim3((HD + 31) / 32, a.R, a.B), dim3(kThreads), 0, stream, a); break;
  }
  return hipGetLastError();
}

int groups_for(int partials) { return partials <= 4 ? 1 : partials <= 16 ? 2 : partials <= 32 ? 4 : 8; }

}  // namespace

hipError_t launch_merge_from_plan(const float* o_part, const float* m_part, const float* l_part,
                                  const msa_segment* segs, const int32_t* indptr, int32_t B,
                                  int32_t R, int32_t H, int32_t D, int32_t S,
                                  int32_t split_blocks, msa_dtype out_dtype, void* out,
                                  float* lse, hipStream_t stream) {
  MergeArgs a{o_part, m_part, l_part, nullptr, segs, indptr, S, split_blocks,
              B, R, H, D, out_dtype, out, lse};
  return launch_ng<1>(a, groups_for(S), stream);
}

hipError_t launch_merge_indptr(const float* o_part, const float* m_part, const float* l_part,
                               const int32_t* part_indptr, int32_t B, int32_t R, int32_t H,
                               int32_t D, msa_dtype out_dtype, void* out, float* lse,
                               hipStream_t stream) {
  MergeArgs a{o_part, m_part, l_part, part_indptr, nullptr, nullptr, 0, 0,
              B, R, H, D, out_dtype, out, lse};
  // the partial counts are on the device: four groups of partials
  return launch_ng<0>(a, 4, stream);
}

hipError_t launch_merge_block(const float* o_part, const float* m_part, const float* l_part,
                              const int32_t* part_indptr, int32_t B, int32_t H, int32_t D,
                              int32_t parts_per_seq, msa_dtype out_dtype, void* out, float* lse,
                              hipStream_t stream) {
  MergeArgs a{o_part, m_part, l_part, part_indptr, nullptr, nullptr, 0, 0,
              B, 1, H, D, out_dtype, out, lse};
  return launch_ng<2>(a, groups_for(parts_per_seq), stream);
}

}  // namespace msa
