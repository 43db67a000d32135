// a3 + a4 for the (dtype, head_dim) pairs the specialised kernels are not
// built for: decode in float32 with D 128, prefill in bfloat16 with D 64 and
// in float32 with D 64 or 128.
//
// Same result as the other kernels (multi_segment_attention, P1 "Core
// method 1: MSA" pseudocode and the paragraph after it: attention over the
// sequence's alive keys in logical order, the split's partial stitched by
// log-sum-exp), written plainly on the vector ALU in float32: one workgroup
// per (query row, KV head, sequence x split) holds the G query heads of its
// KV head and walks the split's segments in chunks of up to 64 consecutive
// tokens of one segment.  Per chunk: scores (one key and one head per
// thread), the online softmax per head (a wavefront per head), then O += P V
// with one (head, d) element per thread and pass.  Decode is the one-row
// case without a causal mask; a prefill row sees the keys at logical
// positions up to its own.  These shapes carry no throughput target; the
// kernel follows the other kernels' plan walk, split rule, cut at the grid's
// capacity and partial layout, so the same workspace and merge serve it.
#include <climits>

#include "msa_internal.h"

namespace msa {
namespace {

constexpr int kGThreads = 256;
constexpr int kGChunk = 64;  // tokens per chunk (one wavefront of keys)
constexpr int kGBlk = 16;
constexpr float kGLn2 = 0.69314718055994530942f;

template <typename T>
__device__ __forceinline__ float load_elt(const T* p);
template <>
__device__ __forceinline__ float load_elt<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_elt<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

template <typename T>
__device__ __forceinline__ void store_elt(T* p, float v);
template <>
__device__ __forceinline__ void store_elt<float>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void store_elt<uint16_t>(uint16_t* p, float v) { *p = f32_to_bf16(v); }

// largest i in [lo, hi) with segs[i].alive_token_start <= x (segs[lo] does)
__device__ __forceinline__ int g_search_segment(const msa_segment* segs, int lo, int hi, int x) {
  while (hi - lo > 1) {
    const int step = (hi - lo + kGThreads - 1) / kGThreads;
    const int idx = lo + int(threadIdx.x) * step;
    const bool pred = idx < hi && segs[idx].alive_token_start <= x;
    const int cnt = __syncthreads_count(pred);
    lo = lo + (cnt - 1) * step;
    hi = min(hi, lo + step);
  }
  return lo;
}

template <typename T, int D, int G>
__global__ void __launch_bounds__(kGThreads) generic_attend_kernel(GenericParams p) {
  __shared__ float q_lds[G][D];
  __shared__ float p_lds[G][kGChunk];  // scores, then weights
  __shared__ float m_lds[G], l_lds[G], a_lds[G];
  __shared__ int32_t kpos_lds[kGChunk];  // logical position of each key of the chunk (-1: absent)

  const int row = blockIdx.x, g = blockIdx.y;
  const int b = blockIdx.z / p.S, s = blockIdx.z % p.S;
  const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
  const int TS = p.split_blocks;  // blocks per split

  // ---- this split's alive-block range (the other kernels' rule) ----------
  const int s0 = p.indptr[b], s1 = p.indptr[b + 1];
  int A = 0;
  if (s1 > s0) {
    const msa_segment last = p.segs[s1 - 1];
    A = last.alive_token_start + last.num_tokens;
  }
  const int nAB_all = (A + kGBlk - 1) / kGBlk;
  const int nAB = min(nAB_all, p.S * TS);
  if (nAB_all > nAB && s == 0 && g == 0 && row == 0 && tid == 0 && p.dev_error)
    atomicOr(p.dev_error, MSA_DEVERR_TRUNCATED);
  const int Sb = (nAB + TS - 1) / TS;
  if (s > 0 && s >= Sb) return;  // split 0 of a sequence without keys writes O = 0 below
  const int j0 = Sb > 0 ? int(int64_t(s) * nAB / Sb) : 0;
  const int j1 = Sb > 0 ? int(int64_t(s + 1) * nAB / Sb) : 0;
  const int tok_lo = j0 * kGBlk, tok_hi = min(j1 * kGBlk, A);  // alive-token range of the split

  // ---- the G query rows of this KV head ----------------------------------
  const size_t q_row = (size_t(b) * p.C + row) * p.Hq + size_t(g) * G;
  const T* q = static_cast<const T*>(p.q) + q_row * D;
  for (int i = tid; i < G * D; i += kGThreads) q_lds[i / D][i % D] = load_elt<T>(q + i);
  if (tid < G) {
    m_lds[tid] = -INFINITY;
    l_lds[tid] = 0.f;
  }
  const int my_pos = p.q_pos0 ? p.q_pos0[b] + row : INT_MAX;  // decode: every key is visible
  const float c = p.scale_log2;

  // O accumulators: thread tid owns elements e = tid + k * 256 of [G][D]
  constexpr int kPer = (G * D + kGThreads - 1) / kGThreads;
  float o[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) o[k] = 0.f;

  const size_t tok_stride = p.head_major ? size_t(D) : size_t(p.Hkv) * D;  // elements
  const size_t blk_stride = size_t(p.Hkv) * D * kGBlk;
  const size_t head_off = p.head_major ? size_t(g) * D * kGBlk : size_t(g) * D;
  const T* kbase = static_cast<const T*>(p.k_pool) + head_off;
  const T* vbase = static_cast<const T*>(p.v_pool) + head_off;
  __syncthreads();

  if (tok_lo < tok_hi) {
    const int sf = tok_lo == 0 ? s0 : g_search_segment(p.segs, s0, s1, tok_lo);
    for (int si = sf; si < s1; ++si) {
      const msa_segment sg = p.segs[si];
      if (sg.alive_token_start >= tok_hi) break;
      // tokens of this segment inside the split
      const int t_lo = max(0, tok_lo - sg.alive_token_start);
      const int t_hi = min(sg.num_tokens, tok_hi - sg.alive_token_start);
      const bool in_pool = sg.phys_block >= 0 && sg.num_blocks >= 0 &&
                           int64_t(sg.phys_block) + sg.num_blocks <= p.P &&
                           sg.num_tokens <= sg.num_blocks * kGBlk;
      for (int t0 = t_lo; t0 < t_hi; t0 += kGChunk) {
        const int n = min(kGChunk, t_hi - t0);
        // keys of the chunk: logical position, or -1 where absent / not visible
        if (tid < kGChunk) {
          const int pos = sg.logical_block * kGBlk + t0 + tid;
          kpos_lds[tid] = (in_pool && tid < n && pos <= my_pos) ? pos : -1;
        }
        __syncthreads();
        // ---- scores: thread = (key, head), G/4 passes over the heads -------
        for (int hk = tid; hk < G * kGChunk; hk += kGThreads) {
          const int h = hk / kGChunk, kk = hk % kGChunk;
          float sc = -INFINITY;
          if (kpos_lds[kk] >= 0) {
            const int t = t0 + kk;
            const T* krow = kbase + size_t(sg.phys_block + t / kGBlk) * blk_stride + size_t(t % kGBlk) * tok_stride;
            float acc = 0.f;
#pragma unroll 8
            for (int d = 0; d < D; ++d) acc = fmaf(q_lds[h][d], load_elt<T>(krow + d), acc);
            sc = acc;
          }
          p_lds[h][kk] = sc;
        }
        __syncthreads();
        // ---- online softmax: wavefront w takes heads w, w + 4 --------------
        for (int h = w; h < G; h += kGThreads / kWave) {
          const float sc = p_lds[h][lane];
          const float cmax = wave_max(sc);
          const float m_old = m_lds[h];
          const float m_new = fmaxf(m_old, cmax);
          const float pw = m_new == -INFINITY ? 0.f : exp2f((sc - m_new) * c);
          const float alpha = (m_old == -INFINITY) ? 0.f : exp2f((m_old - m_new) * c);
          const float lsum = wave_sum(pw);
          p_lds[h][lane] = pw;
          if (lane == 0) {
            l_lds[h] = l_lds[h] * alpha + lsum;
            m_lds[h] = m_new;
            a_lds[h] = alpha;
          }
        }
        __syncthreads();
        // ---- O = O * alpha + P V -------------------------------------------
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
          const int e = tid + k * kGThreads;
          if (e < G * D) {
            const int h = e / D, d = e % D;
            float acc = o[k] * a_lds[h];
            for (int kk = 0; kk < n; ++kk) {
              if (kpos_lds[kk] < 0) continue;
              const int t = t0 + kk;
              const T* vrow = vbase + size_t(sg.phys_block + t / kGBlk) * blk_stride + size_t(t % kGBlk) * tok_stride;
              acc = fmaf(p_lds[h][kk], load_elt<T>(vrow + d), acc);
            }
            o[k] = acc;
          }
        }
        __syncthreads();
      }
    }
  }

  // ---- write: the output itself, or this split's partial ------------------
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int e = tid + k * kGThreads;
    if (e >= G * D) continue;
    const int h = e / D, d = e % D;
    const float L = l_lds[h];
    if (Sb <= 1) {
      store_elt<T>(static_cast<T*>(p.out) + (q_row + h) * D + d, L > 0.f ? o[k] / L : 0.f);
    } else {
      const size_t n = size_t(b) * p.S + s;
      p.o_part[((n * p.C + row) * p.Hq + size_t(g) * G + h) * D + d] = o[k];
    }
  }
  if (tid < G) {
    const int h = tid;
    const float L = l_lds[h], M = m_lds[h];
    if (Sb <= 1) {
      if (p.lse) p.lse[q_row + h] = L > 0.f ? (M * c + log2f(L)) * kGLn2 : -INFINITY;
    } else {
      const size_t n = size_t(b) * p.S + s;
      const size_t r = (n * p.C + row) * p.Hq + size_t(g) * G + h;
      p.m_part[r] = (L > 0.f) ? M * c * kGLn2 : -INFINITY;
      p.l_part[r] = L;
    }
  }
}

template <typename T, int D>
hipError_t launch_gd(const GenericParams& p, hipStream_t stream) {
  dim3 grid(p.C, p.Hkv, p.B * p.S);
  switch (p.Hq / p.Hkv) {
    case 1: hipLaunchKernelGGL((generic_attend_kernel<T, D, 1>), grid, dim3(kGThreads), 0, stream, p); break;
    case 2: hipLaunchKernelGGL((generic_attend_kernel<T, D, 2>), grid, dim3(kGThreads), 0, stream, p); break;
    case 4: hipLaunchKernelGGL((generic_attend_kernel<T, D, 4>), grid, dim3(kGThreads), 0, stream, p); break;
    case 8: hipLaunchKernelGGL((generic_attend_kernel<T, D, 8>), grid, dim3(kGThreads), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool generic_supported(msa_dtype dtype, int32_t D, int32_t G) {
  const bool g_ok = G == 1 || G == 2 || G == 4 || G == 8;
  return g_ok && (dtype == MSA_F32 || dtype == MSA_BF16) && (D == 64 || D == 128);
}

hipError_t launch_generic(const GenericParams& p, hipStream_t stream) {
  if (p.dtype == MSA_F32) {
    if (p.D == 64) return launch_gd<float, 64>(p, stream);
    if (p.D == 128) return launch_gd<float, 128>(p, stream);
  } else if (p.dtype == MSA_BF16) {
    if (p.D == 64) return launch_gd<uint16_t, 64>(p, stream);
    if (p.D == 128) return launch_gd<uint16_t, 128>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace msa
