// a2 + a3: MSA decode over the alive-token stream of a segment plan.
//
// multi_segment_attention for one decode query per sequence (P1, "Core
// method 1: MSA" pseudocode; P2, Key Results: one kernel over many disjoint
// KV segments).  Decode is bandwidth-bound (it reads every resident K/V
// row once per generated token; P3, "解决什么真问题", item 2), so both
// kernels here are built around the HBM stream: decode_kernel on the VALU,
// and, for grouped-query bf16 with G 4 or 8, decode_mfma_kernel (further
// below), which moves the G-head contractions onto matrix cores so that
// the VALU does not cap the stream.  This comment describes decode_kernel;
// the frame (grid, split rule, segment walk, merge) is shared.
//
// Grid: (split s, KV head g, sequence b); 256 threads = 4 wavefronts.
//   * The sequence's alive blocks, in logical order, are numbered
//     0..nAB-1 (block j holds alive tokens [16j, 16j+16)).  The sequence
//     uses Sb = ceil(nAB / T) splits that share the blocks evenly: split s
//     owns [s*nAB/Sb, (s+1)*nAB/Sb).  The workgroup finds the segment holding its
//     first block with a workgroup-parallel search over alive_token_start,
//     then expands its segments into a per-block physical id list in LDS.
//     Consecutive segments are folded into one running softmax state in
//     registers; partials exist only per split, never per segment.
//   * Each wavefront takes tiles of 4 blocks (64 tokens), interleaved with
//     the other wavefronts.  K rows are loaded with coalesced 16-byte loads
//     (4 rows of 256 B per instruction for bf16, D=128), staged through LDS
//     with an XOR swizzle, and read back one token per lane; the G query
//     heads of the KV head (GQA group) are broadcast from LDS, so each K/V
//     row is read from HBM once for all G heads.  Scores use v_dot2 on bf16
//     pairs with fp32 accumulation.
//   * Online softmax per wavefront: wave max by DPP + cross-row shuffles,
//     exp2 with the scale folded into log2 units; the weights go through
//     LDS and are broadcast to the PV loop, in which each lane owns a slice
//     of D and accumulates fp32 for all G heads.  K/V rows of masked tokens
//     (padding past ctx_len, blocks outside the split) lie outside their
//     block's buffer descriptor and read as zero, so NaN-poisoned slots
//     cannot leak into a product.
//   * At the end the 4 wavefront states are merged in LDS; a sequence with
//     one split writes O and LSE directly, otherwise the split writes its
//     (m, l, o) partial for the merge kernel.
#include <type_traits>

#include "msa_internal.h"

namespace msa {
namespace {

constexpr int kThreads = 256;
constexpr int kNW = kThreads / kWave;
constexpr int kTileTok = 64;      // tokens per wavefront tile (4 blocks of 16)
constexpr int kBlk = 16;          // block size the kernels are built for
constexpr int kMaxSplitBlocks = 512;
constexpr int kCUs = 256;  // compute units of an MI355X
constexpr float kLn2 = 0.69314718055994530942f;

template <typename KV, int D>
struct Geo {
  static constexpr int ES = sizeof(KV);
  static constexpr int ROW = D * ES;              // bytes of one head's row
  static constexpr int CH = ROW / 16;             // 16-byte chunks per row
  static constexpr int SW = CH < 16 ? CH : 16;    // LDS swizzle period
  static constexpr int RPI = kWave / CH;          // rows per 16-byte load instruction
  static constexpr int NL = kTileTok / RPI;       // load instructions per tile (K or V)
  static constexpr int LPB = kBlk / RPI;          // load instructions per block
  static constexpr int EPC = 16 / ES;             // elements per 16-byte chunk
  static constexpr int NPAT = SW > RPI ? SW / RPI : 1;  // distinct swizzle patterns of K writes
  static_assert(CH <= 16 && kBlk % RPI == 0, "row layout");
};

// Buffer resource for one KV block of one head: base = the block's first
// row, num_records = rows that may be read * row stride.  Buffer loads
// outside num_records return zero in hardware, so evicted blocks, blocks
// past the split and padding rows past ctx_len need no branch and no
// select, and can never touch memory outside the pool.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kBufferFlags = 0x00020000;  // raw (untyped) dword access, gfx9 family

__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const char* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, int(bytes), kBufferFlags);
}

// K/V rows are streamed: each byte is read once per call (all G query heads
// of a KV head share one workgroup), so the loads carry the non-temporal
// hint and do not displace reusable lines in L2 and the Infinity Cache.
constexpr int kStreamPolicy = 2;  // cache-policy bits: nt
__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, kStreamPolicy);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint4 load16_cached(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float dot_chunk(uint4 q, uint4 k, float acc, uint16_t) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.x),
                                        __builtin_bit_cast(bf16x2_t, k.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.y),
                                        __builtin_bit_cast(bf16x2_t, k.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.z),
                                        __builtin_bit_cast(bf16x2_t, k.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.w),
                                        __builtin_bit_cast(bf16x2_t, k.w), acc, false);
  return acc;
}

__device__ __forceinline__ float dot_chunk(uint4 q, uint4 k, float acc, float) {
  acc = fmaf(__uint_as_float(q.x), __uint_as_float(k.x), acc);
  acc = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), acc);
  acc = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), acc);
  acc = fmaf(__uint_as_float(q.w), __uint_as_float(k.w), acc);
  return acc;
}

template <typename KV>
__device__ __forceinline__ void unpack_chunk(uint4 x, float* v);
template <>
__device__ __forceinline__ void unpack_chunk<uint16_t>(uint4 x, float* v) {
  v[0] = bf16lo_to_f32(x.x); v[1] = bf16hi_to_f32(x.x);
  v[2] = bf16lo_to_f32(x.y); v[3] = bf16hi_to_f32(x.y);
  v[4] = bf16lo_to_f32(x.z); v[5] = bf16hi_to_f32(x.z);
  v[6] = bf16lo_to_f32(x.w); v[7] = bf16hi_to_f32(x.w);
}
template <>
__device__ __forceinline__ void unpack_chunk<float>(uint4 x, float* v) {
  v[0] = __uint_as_float(x.x); v[1] = __uint_as_float(x.y);
  v[2] = __uint_as_float(x.z); v[3] = __uint_as_float(x.w);
}

// G consecutive floats from LDS with the widest reads available
template <int G>
__device__ __forceinline__ void read_weights(const float* src, float* pw) {
  if constexpr (G % 4 == 0) {
#pragma unroll
    for (int i = 0; i < G; i += 4) {
      const float4 t = *reinterpret_cast<const float4*>(src + i);
      pw[i] = t.x; pw[i + 1] = t.y; pw[i + 2] = t.z; pw[i + 3] = t.w;
    }
  } else if constexpr (G == 2) {
    const float2 t = *reinterpret_cast<const float2*>(src);
    pw[0] = t.x; pw[1] = t.y;
  } else {
    pw[0] = src[0];
  }
}

template <typename KV>
__device__ __forceinline__ void store_out(void* out, size_t idx, float v);
template <>
__device__ __forceinline__ void store_out<uint16_t>(void* out, size_t idx, float v) {
  static_cast<uint16_t*>(out)[idx] = f32_to_bf16(v);
}
template <>
__device__ __forceinline__ void store_out<float>(void* out, size_t idx, float v) {
  static_cast<float*>(out)[idx] = v;
}

// Largest i in [lo, hi) with segs[i].alive_token_start <= x, given that
// segs[lo] satisfies it.  Workgroup-uniform; all THREADS threads of the
// workgroup must call it.
template <int THREADS>
__device__ __forceinline__ int wg_search_segment_n(const msa_segment* segs, int lo, int hi, int x) {
  while (hi - lo > 1) {
    const int step = (hi - lo + THREADS - 1) / THREADS;
    const int idx = lo + int(threadIdx.x) * step;
    const bool pred = idx < hi && segs[idx].alive_token_start <= x;
    const int cnt = __syncthreads_count(pred);
    lo = lo + (cnt - 1) * step;
    hi = min(hi, lo + step);
  }
  return lo;
}

template <typename KV, int D, int G>
__global__ void __launch_bounds__(kThreads, 2) decode_kernel(DecodeParams p) {
  using GE = Geo<KV, D>;
  constexpr int ROW = GE::ROW, CH = GE::CH, SW = GE::SW, EPC = GE::EPC;

  // K tiles; during set-up the same bytes hold the staged segment list, and
  // at the end the per-wavefront states for the cross-wave merge.
  __shared__ __align__(16) uint8_t k_lds[kNW][kTileTok * ROW];
  __shared__ __align__(16) float p_lds[kNW][kTileTok][G];
  __shared__ __align__(16) uint8_t q_lds[G * ROW];
  __shared__ int32_t blk_phys[kMaxSplitBlocks];
  static_assert(sizeof(k_lds) >= 3 * (kMaxSplitBlocks + 1) * sizeof(int32_t), "staging");
  static_assert(sizeof(k_lds) >= (kNW * G * D + 2 * kNW * G) * sizeof(float), "merge");

  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  // the wavefront index is wave-uniform; say so, or everything derived from
  // it (tile indices, buffer descriptors) is treated as divergent
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int T = p.split_blocks;

  const int s0 = p.indptr[b], s1 = p.indptr[b + 1];
  // staged segment list: first block, physical id and block count of each
  int32_t* st_start = reinterpret_cast<int32_t*>(&k_lds[0][0]);
  int32_t* st_phys = st_start + kMaxSplitBlocks + 1;
  int32_t* st_nblk = st_phys + kMaxSplitBlocks + 1;
  __shared__ int32_t st_alive;
  auto stage = [&](int sf, int n) {
    for (int i = tid; i < n; i += kThreads) {
      const msa_segment sg = p.segs[sf + i];
      st_start[i] = sg.alive_token_start / kBlk;
      // the plan never emits a segment outside the pool; a foreign one is dropped
      const bool in_pool = sg.phys_block >= 0 && sg.num_blocks >= 0 &&
                           int64_t(sg.phys_block) + sg.num_blocks <= p.P;
      st_phys[i] = in_pool ? sg.phys_block : -1;
      st_nblk[i] = in_pool ? sg.num_blocks : 0;
      if (sf + i == s1 - 1) st_alive = sg.alive_token_start + sg.num_tokens;
    }
  };
  // A split holds at most T blocks, so at most T segments: when the
  // sequence has no more, the first split stages the whole list at once and
  // takes the alive length from its last segment (one dependent round trip
  // to memory fewer than reading the last segment first)
  const bool staged = s == 0 && s1 > s0 && s1 - s0 <= T;
  int A = 0;
  if (staged) {
    stage(s0, s1 - s0);
    __syncthreads();
    A = st_alive;
  } else if (s1 > s0) {
    const msa_segment last = p.segs[s1 - 1];
    A = last.alive_token_start + last.num_tokens;
  }
  // a plan with more alive tokens than max_ctx_len promised is cut at the
  // grid, and the cut is reported (once per sequence)
  const int nAB_all = (A + kBlk - 1) / kBlk;
  const int nAB = min(nAB_all, p.S * T);
  if (nAB_all > nAB && s == 0 && g == 0 && tid == 0 && p.dev_error)
    atomicOr(p.dev_error, MSA_DEVERR_TRUNCATED);
  const int Sb = (nAB + T - 1) / T;
  if (s >= Sb) {
    if (s == 0 && p.S == 1) {  // no alive token at all: O = 0, LSE = -inf
      for (int i = tid; i < G * D; i += kThreads) {
        const int h = g * G + i / D;
        store_out<KV>(p.out, (size_t(b) * p.Hq + h) * D + i % D, 0.f);
        if (p.lse && i % D == 0) p.lse[size_t(b) * p.Hq + h] = -INFINITY;
      }
    }
    return;
  }
  // the sequence's Sb splits share its nAB blocks evenly (each <= T blocks)
  const int j0 = int(int64_t(s) * nAB / Sb);
  const int nblk = int(int64_t(s + 1) * nAB / Sb) - j0;
  const int last_tokens = min(kBlk, A - kBlk * (nAB - 1));  // tokens in the final alive block

  // ---- expand this split's segments into per-block physical ids ----------
  // (the first split starts at the sequence's first segment: no search)
  // (staged: sf = s0 and ns <= s1 - s0, all of it in LDS already)
  const int sf = j0 == 0 ? s0 : wg_search_segment_n<kThreads>(p.segs, s0, s1, j0 * kBlk);
  const int ns = min(nblk, s1 - sf);
  if (!staged) stage(sf, ns);
  {  // this KV head's G query rows -> LDS (contiguous G*ROW bytes)
    const uint8_t* qsrc = static_cast<const uint8_t*>(p.q) + (size_t(b) * p.Hq + size_t(g) * G) * ROW;
    for (int i = tid; i < G * CH; i += kThreads)
      *reinterpret_cast<uint4*>(q_lds + i * 16) = *reinterpret_cast<const uint4*>(qsrc + i * 16);
  }
  __syncthreads();
  for (int jj = tid; jj < nblk; jj += kThreads) {
    const int j = j0 + jj;
    int lo = 0, hi = ns;  // largest i with st_start[i] <= j
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (st_start[mid] <= j) lo = mid; else hi = mid;
    }
    const int off = j - st_start[lo];
    blk_phys[jj] = (st_phys[lo] >= 0 && off >= 0 && off < st_nblk[lo]) ? st_phys[lo] + off : -1;
  }
  __syncthreads();

  // ---- main loop: one 64-token tile (4 blocks) per wavefront per step ----
  // Loads: instruction c of a tile covers rows c*RPI .. c*RPI+RPI-1 (all in
  // block c/LPB), each lane one 16-byte chunk.  The block's base address is
  // wave-uniform (scalar registers); the per-lane offset is fixed for the
  // whole kernel, so no vector address arithmetic happens in the loop.
  // bytes between the slots of one head in a block, between blocks, and
  // from a block's start to this KV head's first row, for the token-major
  // [P, bs, Hkv, D] or the head-major [P, Hkv, bs, D] pool
  const size_t tok_stride = p.head_major ? size_t(ROW) : size_t(p.Hkv) * ROW;
  const size_t blk_stride = size_t(p.Hkv) * ROW * kBlk;
  const size_t head_off = p.head_major ? size_t(g) * ROW * kBlk : size_t(g) * ROW;
  const char* kbase = static_cast<const char*>(p.k_pool) + head_off;
  const char* vbase = static_cast<const char*>(p.v_pool) + head_off;
  // (rows of a block are tok_stride apart; a row's ROW bytes never cross
  // into the next row's range, so row-granular num_records is exact)
  const int lrow = lane / CH, lch = lane % CH;
  // per-lane byte offsets inside a block, one per load of the block
  uint32_t voff[GE::LPB];
#pragma unroll
  for (int ci = 0; ci < GE::LPB; ++ci)
    voff[ci] = uint32_t((ci * GE::RPI + lrow) * tok_stride + lch * 16);
  uint8_t* kt = &k_lds[w][0];
  float* pt = &p_lds[w][0][0];
  // LDS byte offsets of this lane's K chunk, one per swizzle pattern; load c
  // adds c*RPI*ROW on top (an immediate)
  uint32_t kwo[GE::NPAT];
#pragma unroll
  for (int cm = 0; cm < GE::NPAT; ++cm) {
    const int r = cm * GE::RPI + lrow;
    kwo[cm] = uint32_t(lrow * ROW + ((lch ^ (r % SW)) * 16));
  }

  float m_run[G], l_lane[G], o[G][EPC];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = -INFINITY;
    l_lane[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPC; ++e) o[h][e] = 0.f;
  }

  const int ntiles = (nblk + 3) / 4;
  const int last_local = nAB - 1 - j0;  // local index of the sequence's final block

  // wave-uniform physical block ids and readable row counts of tile ti
  auto tile_blocks = [&](int ti, int* ph, int* rows) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int jj = ti * 4 + k;
      ph[k] = __builtin_amdgcn_readfirstlane(jj < nblk ? blk_phys[min(jj, kMaxSplitBlocks - 1)] : -1);
      rows[k] = ph[k] < 0 ? 0 : (jj == last_local ? last_tokens : kBlk);
    }
  };
  auto load_tile = [&](const char* base, const int* ph, const int* rows, uint4* r) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const __amdgpu_buffer_rsrc_t rs =
          block_rsrc(base + size_t(ph[k] < 0 ? 0 : ph[k]) * blk_stride, uint32_t(rows[k] * tok_stride));
#pragma unroll
      for (int ci = 0; ci < GE::LPB; ++ci) r[k * GE::LPB + ci] = load16(rs, voff[ci]);
    }
  };

  uint4 kreg[GE::NL], vreg[GE::NL];
  int ph[4], rows[4];
  int ti = w;
  tile_blocks(ti, ph, rows);
  // K strictly before V, here and in the loop: the loop top then only waits
  // for the K loads (vmcnt counts in issue order) while V stays in flight
  __builtin_amdgcn_sched_barrier(0);
  load_tile(kbase, ph, rows, kreg);
  __builtin_amdgcn_sched_barrier(0);
  load_tile(vbase, ph, rows, vreg);
  __builtin_amdgcn_sched_barrier(0);
  for (; ti < ntiles; ti += kNW) {
    // K tile -> LDS, XOR-swizzled so the one-token-per-lane reads are
    // conflict-free
#pragma unroll
    for (int c = 0; c < GE::NL; ++c)
      *reinterpret_cast<uint4*>(kt + kwo[c % GE::NPAT] + c * GE::RPI * ROW) = kreg[c];
    __builtin_amdgcn_wave_barrier();
    // phase fences: without them the scheduler overlaps the next tile's
    // loads with this tile's live registers and runs out of VGPRs
    __builtin_amdgcn_sched_barrier(0);
    const int tn = ti + kNW;
    int phn[4], rowsn[4];
    tile_blocks(tn, phn, rowsn);
    // next K in flight during this tile (past the last tile the descriptors
    // have no readable rows: the loads return zeros and touch no memory)
    load_tile(kbase, phn, rowsn, kreg);
    __builtin_amdgcn_sched_barrier(0);

    // token validity for the one-token-per-lane score phase
    const int kb = lane / kBlk, slot = lane % kBlk;
    const int rows_l = kb == 0 ? rows[0] : kb == 1 ? rows[1] : kb == 2 ? rows[2] : rows[3];
    const bool tok_ok = slot < rows_l;

    // scores.  The query rows are re-read from LDS (broadcast) every tile: an
    // opaque offset keeps the compiler from hoisting G*D values into registers.
    int qoff = 0;
    asm volatile("" : "+v"(qoff));
    const uint8_t* qt = q_lds + qoff;
    float sc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) sc[h] = 0.f;
#pragma unroll 2
    for (int c = 0; c < CH; ++c) {
      const uint4 kc = *reinterpret_cast<const uint4*>(kt + lane * ROW + ((c ^ (lane % SW)) * 16));
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const uint4 qc = *reinterpret_cast<const uint4*>(qt + h * ROW + c * 16);
        sc[h] = dot_chunk(qc, kc, sc[h], KV());
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) sc[h] = tok_ok ? sc[h] * p.scale_log2 : -INFINITY;

    // online softmax (log2 units), one wavefront-wide max per head
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float m_new = fmaxf(m_run[h], wave_max(sc[h]));
      float alpha = 1.f, pw = 0.f;
      if (m_new != -INFINITY) {
        alpha = exp2f(m_run[h] - m_new);
        pw = exp2f(sc[h] - m_new);
      }
      m_run[h] = m_new;
      l_lane[h] = l_lane[h] * alpha + pw;
#pragma unroll
      for (int e = 0; e < EPC; ++e) o[h][e] *= alpha;
      pt[lane * G + h] = pw;
    }
    __builtin_amdgcn_wave_barrier();

    // PV: this lane's EPC elements of D for the rows its V loads covered
#pragma unroll
    for (int c = 0; c < GE::NL; ++c) {
      const int r = c * GE::RPI + lrow;
      float v[GE::EPC];
      unpack_chunk<KV>(vreg[c], v);
      float pw[G];
      read_weights<G>(pt + r * G, pw);
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < EPC; ++e) o[h][e] = fmaf(pw[h], v[e], o[h][e]);
      // keep each chunk's weight reads and unpacking next to its FMAs;
      // hoisting all of them would need more registers than the file has
      if (c % 2 == 1) __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_sched_barrier(0);
    load_tile(vbase, phn, rowsn, vreg);  // next V in flight during the next scores
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      ph[k] = phn[k];
      rows[k] = rowsn[k];
    }
    __builtin_amdgcn_wave_barrier();
  }

  // ---- merge the 4 wavefront states --------------------------------------
  float l_w[G];
#pragma unroll
  for (int h = 0; h < G; ++h) l_w[h] = wave_sum(l_lane[h]);
  // lanes with the same chunk hold partial sums over different rows
#pragma unroll
  for (int x = CH; x < kWave; x <<= 1)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPC; ++e) o[h][e] += __shfl_xor(o[h][e], x);
  __syncthreads();
  float* mo = reinterpret_cast<float*>(&k_lds[0][0]);  // [kNW][G][D]
  float* mm = mo + kNW * G * D;                        // [kNW][G]
  float* ml = mm + kNW * G;
  if (lrow == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPC; ++e) mo[(w * G + h) * D + lch * EPC + e] = o[h][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      mm[w * G + h] = m_run[h];
      ml[w * G + h] = l_w[h];
    }
  }
  __syncthreads();
  for (int i = tid; i < G * D; i += kThreads) {
    const int hh = i / D, d = i % D;
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < kNW; ++k) M = fmaxf(M, mm[k * G + hh]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int k = 0; k < kNW; ++k) {
        const float mk = mm[k * G + hh];
        const float wt = mk == -INFINITY ? 0.f : exp2f(mk - M);
        L = fmaf(wt, ml[k * G + hh], L);
        O = fmaf(wt, mo[(k * G + hh) * D + d], O);
      }
    }
    const int h = g * G + hh;
    if (Sb == 1) {
      store_out<KV>(p.out, (size_t(b) * p.Hq + h) * D + d, L > 0.f ? O / L : 0.f);
      if (p.lse && d == 0) p.lse[size_t(b) * p.Hq + h] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
    } else {
      const size_t n = size_t(b) * p.S + s;
      p.o_part[(n * p.Hq + h) * D + d] = O;
      if (d == 0) {
        p.m_part[n * p.Hq + h] = M == -INFINITY ? -INFINITY : M * kLn2;
        p.l_part[n * p.Hq + h] = L;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Grouped-query bf16 decode with D 128 and G in {4, 8}: the G query heads of a
// KV head against the keys of a tile form a real [G x 128] x [128 x 64]
// contraction, and so does P x V.  On the VALU these cost 2G multiply-adds
// per K/V element, which at G 8 limits the kernel well below the HBM stream;
// on v_mfma_f32_16x16x32_bf16 (heads padded to 16 rows) they are a few
// hundred cycles per 32 KB tile, so the loads set the pace.  Same grid,
// split rule, segment walk and cross-wavefront merge as decode_kernel.
//
// Per wavefront and 64-token tile (4 blocks):
//   S[key][head] = K Q^T: A = K (lane l: key l%16 of block kg, d 32 ds +
//     8(l/16) .. +7), B = Q^T (lane l: head l%16, same d), C: lane l holds
//     head l%16 for keys 16 kg + 4(l/16) + r.
//   online softmax per head over those 16 values x the 4 lanes of the head
//   O[head][d] += P V: A = P, exactly the lane's own weights (k-slots are
//     keys 16(2ks + s/4) + 4(l/16) + s%4), B = V from LDS with the gfx950
//     transpose read (4 keys x 1 d per lane per read).
// Loads: V reaches the wavefront's LDS tile by DMA, every instruction four
// whole 256-byte rows (16 lanes per row) with the streaming hint; each
// 16-byte chunk c of key k lands in slot c ^ (2k mod 16) of the key's row,
// which keeps the transpose reads free of bank conflicts.  Whole rows matter:
// the same data fetched as four 64-byte pieces per row from four
// instructions (which a streaming load never merges) took 88 against 80 us
// on the 32 x 4k batch with cold caches.  K comes either straight from HBM
// into the A operand registers (16 keys x 64 B per instruction, default
// cache policy so the two halves of each 128-byte line meet in the cache),
// or, when the grid holds at most one workgroup per CU (KDMA: the extra
// 64 KB of LDS then costs no occupancy), by DMA in whole rows like V
// (chunk c of key k in slot c ^ k), read back as operands: 78 against 80 us
// cold on the 32 x 4k batch, while on many-split grids the halved occupancy
// costs more than the rows gain.
// K(t+1) is loaded during softmax and PV of tile t, V(t+1) during QK(t+1).

typedef __bf16 mbf16x8_t __attribute__((ext_vector_type(8)));
typedef float mf32x4_t __attribute__((ext_vector_type(4)));
typedef short ms16x4_t __attribute__((ext_vector_type(4)));
typedef float mf32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 mbf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kMD = 128, kMRow = 256;
constexpr int kMTile = kTileTok * kMRow;  // bytes of a K or V tile (16 KB)
constexpr int kMBlock = kBlk * kMRow;     // one block's 16 rows of one head in a tile (4 KB)

__device__ __forceinline__ mbf16x8_t m_as_bf16x8(uint4 x) { return __builtin_bit_cast(mbf16x8_t, x); }
__device__ __forceinline__ uint32_t m_cvt_pk_bf16(float a, float b) {
  const mf32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, mbf16x2_t));
}
// gfx950 transpose LDS load: within each 16-lane group, lane i receives
// element i%4 of the 8-byte words addressed by lanes i/4, i/4+4, i/4+8 and
// i/4+12 of the group
__device__ __forceinline__ uint2 m_read_tr16(const uint8_t* lds_ptr) {
  const ms16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) ms16x4_t*)(lds_ptr));
  return __builtin_bit_cast(uint2, v);
}

template <int G, bool KDMA>
__global__ void __launch_bounds__(kThreads, KDMA ? 1 : 2) decode_mfma_kernel(DecodeParams p) {
  static_assert(G == 4 || G == 8, "heads padded to 16 MFMA rows");
  constexpr int D = kMD;
  // per-wavefront V tile; during set-up the same bytes hold the staged
  // segment list, and at the end the per-wavefront states for the merge
  __shared__ __align__(16) uint8_t v_lds[kNW][kMTile];
  // KDMA: per-wavefront K tile, rows landed whole by DMA
  __shared__ __align__(16) uint8_t k_lds[KDMA ? kNW : 1][KDMA ? kMTile : 16];
  __shared__ __align__(16) int32_t blk_phys[kMaxSplitBlocks];
  static_assert(sizeof(v_lds) >= 3 * (kMaxSplitBlocks + 1) * sizeof(int32_t), "staging");
  static_assert(sizeof(v_lds) >= (kNW * G * D + 2 * kNW * G) * sizeof(float), "merge");

  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int T = p.split_blocks;
  const int hl = lane % 16, q4 = lane / 16;

  // Q^T operand (lane l: head l%16, zero past G, d 32 ds + 8(l/16)): issued
  // first, so its round trip overlaps the plan reads below
  uint4 qop[4];
  {
    const uint8_t* qsrc = static_cast<const uint8_t*>(p.q) + (size_t(b) * p.Hq + size_t(g) * G + hl) * kMRow;
#pragma unroll
    for (int ds = 0; ds < 4; ++ds)
      qop[ds] = hl < G ? *reinterpret_cast<const uint4*>(qsrc + (4 * ds + q4) * 16) : make_uint4(0, 0, 0, 0);
  }

  const int s0 = p.indptr[b], s1 = p.indptr[b + 1];
  // staged segment list: first block, physical id and block count of each
  int32_t* st_start = reinterpret_cast<int32_t*>(&v_lds[0][0]);
  int32_t* st_phys = st_start + kMaxSplitBlocks + 1;
  int32_t* st_nblk = st_phys + kMaxSplitBlocks + 1;
  __shared__ int32_t st_alive;
  auto stage = [&](int sf, int n) {
    for (int i = tid; i < n; i += kThreads) {
      const msa_segment sg = p.segs[sf + i];
      st_start[i] = sg.alive_token_start / kBlk;
      const bool in_pool = sg.phys_block >= 0 && sg.num_blocks >= 0 &&
                           int64_t(sg.phys_block) + sg.num_blocks <= p.P;
      st_phys[i] = in_pool ? sg.phys_block : -1;
      st_nblk[i] = in_pool ? sg.num_blocks : 0;
      if (sf + i == s1 - 1) st_alive = sg.alive_token_start + sg.num_tokens;
    }
  };
  // A split holds at most T blocks, so at most T segments.  When the
  // sequence has no more than that, the first split stages its whole list
  // at once and takes the alive length from its last segment: one dependent
  // round trip to memory fewer than reading the last segment first.
  const bool staged = s == 0 && s1 > s0 && s1 - s0 <= T;
  int A = 0;
  if (staged) {
    stage(s0, s1 - s0);
    __syncthreads();
    A = st_alive;
  } else if (s1 > s0) {
    const msa_segment last = p.segs[s1 - 1];
    A = last.alive_token_start + last.num_tokens;
  }
  const int nAB_all = (A + kBlk - 1) / kBlk;
  const int nAB = min(nAB_all, p.S * T);
  if (nAB_all > nAB && s == 0 && g == 0 && tid == 0 && p.dev_error)
    atomicOr(p.dev_error, MSA_DEVERR_TRUNCATED);
  const int Sb = (nAB + T - 1) / T;
  if (s >= Sb) {
    if (s == 0 && p.S == 1) {  // no alive token at all: O = 0, LSE = -inf
      for (int i = tid; i < G * D; i += kThreads) {
        const int h = g * G + i / D;
        store_out<uint16_t>(p.out, (size_t(b) * p.Hq + h) * D + i % D, 0.f);
        if (p.lse && i % D == 0) p.lse[size_t(b) * p.Hq + h] = -INFINITY;
      }
    }
    return;
  }
  const int j0 = int(int64_t(s) * nAB / Sb);
  const int nblk = int(int64_t(s + 1) * nAB / Sb) - j0;
  const int last_tokens = min(kBlk, A - kBlk * (nAB - 1));

  // ---- expand this split's segments into per-block physical ids ----------
  {
    // the first split starts at the sequence's first segment: no search
    const int sf = j0 == 0 ? s0 : wg_search_segment_n<kThreads>(p.segs, s0, s1, j0 * kBlk);
    // (staged: sf = s0 and ns <= s1 - s0, all of it in LDS already)
    const int ns = min(nblk, s1 - sf);
    if (!staged) {
      stage(sf, ns);
      __syncthreads();
    }
    for (int jj = tid; jj < nblk; jj += kThreads) {
      const int j = j0 + jj;
      int lo = 0, hi = ns;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (st_start[mid] <= j) lo = mid; else hi = mid;
      }
      const int off = j - st_start[lo];
      blk_phys[jj] = (st_phys[lo] >= 0 && off >= 0 && off < st_nblk[lo]) ? st_phys[lo] + off : -1;
    }
    __syncthreads();  // staging dead from here on: the V tiles may overwrite it
  }

  // slot, block and KV-head strides of the token-major or head-major pool
  const size_t tok_stride = p.head_major ? size_t(kMRow) : size_t(p.Hkv) * kMRow;
  const size_t blk_stride = size_t(p.Hkv) * kMRow * kBlk;
  const size_t head_off = p.head_major ? size_t(g) * kMRow * kBlk : size_t(g) * kMRow;
  const char* kbase = static_cast<const char*>(p.k_pool) + head_off;
  const char* vbase = static_cast<const char*>(p.v_pool) + head_off;
  // K operand loads: lane offset inside a block for d step ds (adds 64 B each)
  const uint32_t k_voff = uint32_t(hl * tok_stride + q4 * 16);
  // row DMAs: instruction i of a block covers keys 4i .. 4i+3, lane l key
  // 4i + l/16 and its 16-byte slot l%16
  const int kq = lane / 16, slot = lane % 16;
  uint8_t* vt = &v_lds[w][0];
  uint8_t* kt = &k_lds[KDMA ? w : 0][0];
  // transpose-read word of lane l (j = l%16) for PV step (block, dg): key
  // 4(l/16) + j/4, d = 16 dg + 4(j%4) .. +3, i.e. chunk 2dg + (j%4)/2
  const int vr_key = 4 * q4 + hl / 4;
  const int vr_base = vr_key * kMRow + 8 * (hl % 2);
  auto vrow_off = [&](int dg) { return vr_base + 16 * ((2 * dg + (hl % 4) / 2) ^ ((2 * vr_key) & 15)); };

  mf32x4_t o[8];
#pragma unroll
  for (int dg = 0; dg < 8; ++dg) o[dg] = mf32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_lane = 0.f;
  const float c = p.scale_log2;

  const int ntiles = (nblk + 3) / 4;
  const int last_local = nAB - 1 - j0;
  // wave-uniform physical ids and readable row counts of tile ti's 4 blocks
  // (one 16-byte LDS read; tiles past the split get empty ranges)
  auto tile_blocks = [&](int ti, int* ph, int* rows) {
    int4 v = make_int4(-1, -1, -1, -1);
    if (ti < ntiles) v = *reinterpret_cast<const int4*>(&blk_phys[min(ti * 4, kMaxSplitBlocks - 4)]);
    const int pv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) {
      const int jj = ti * 4 + kg;
      ph[kg] = __builtin_amdgcn_readfirstlane(jj < nblk ? pv[kg] : -1);
      rows[kg] = ph[kg] < 0 ? 0 : (jj == last_local ? last_tokens : kBlk);
    }
  };
  auto rsrc_of = [&](const char* base, int ph, int rows) {
    return block_rsrc(base + size_t(ph < 0 ? 0 : ph) * blk_stride, uint32_t(rows * tok_stride));
  };
  uint4 kreg[4][4];
  auto issue_k = [&](const int* ph, const int* rows) {
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) {
      const __amdgpu_buffer_rsrc_t r = rsrc_of(kbase, ph[kg], rows[kg]);
      if constexpr (KDMA) {
        // chunk slot ^ key of key 4i + kq into slot `slot` of its row
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = 4 * i + kq;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              r, (__attribute__((address_space(3))) void*)(kt + kg * kMBlock + i * 4 * kMRow), 16,
              uint32_t(key * tok_stride + 16 * (slot ^ key)), 0, 0, kStreamPolicy);
        }
      } else {
        // default cache policy: each 128-byte line of a key row arrives as
        // two 64-byte pieces from two loads, which must meet in the cache
#pragma unroll
        for (int ds = 0; ds < 4; ++ds) kreg[kg][ds] = load16_cached(r, k_voff + ds * 64);
      }
    }
  };
  auto issue_v = [&](const int* ph, const int* rows) {
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) {
      const __amdgpu_buffer_rsrc_t r = rsrc_of(vbase, ph[kg], rows[kg]);
      // chunk slot ^ (2 key mod 16) of key 4i + kq into slot `slot` of its row
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 4 * i + kq;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            r, (__attribute__((address_space(3))) void*)(vt + kg * kMBlock + i * 4 * kMRow), 16,
            uint32_t(key * tok_stride + 16 * (slot ^ ((2 * key) & 15))), 0, 0, kStreamPolicy);
      }
    }
  };

  // Streaming wavefronts.  With one workgroup per CU on a grid that fills
  // most of the chip, the DRAM is oversubscribed and three wavefronts' loads
  // in flight per CU move the same bytes a little sooner than four (cold,
  // the 32 x 4k batch, two sessions: 73.5 / 74.1 against 75.3 / 74.8 us;
  // head-major pools unchanged within noise); at two workgroups per CU four
  // stay better (the 131k-token batch with this kernel: 200 against 197 us
  // with three).  The idle wavefront joins the merge with an empty state.
  const int nw_act =
      KDMA && int64_t(gridDim.x) * gridDim.y * gridDim.z >= 3 * kCUs / 4 ? kNW - 1 : kNW;
  int ti = w < nw_act ? w : ntiles;
  int ph[4], rows[4], phn[4], rowsn[4];
  tile_blocks(ti, ph, rows);
  issue_k(ph, rows);
  issue_v(ph, rows);
  for (; ti < ntiles; ti += nw_act) {
    if constexpr (KDMA) {
      // K(t) has landed once at most the 16 V DMAs of this tile are in
      // flight; then the A operands come from the K tile (slot c ^ key)
      asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
#pragma unroll
      for (int kg = 0; kg < 4; ++kg)
#pragma unroll
        for (int ds = 0; ds < 4; ++ds)
          kreg[kg][ds] = *reinterpret_cast<const uint4*>(kt + kg * kMBlock + hl * kMRow +
                                                         16 * ((4 * ds + q4) ^ hl));
    }
    // ---- S = K Q^T for the tile's 4 blocks ------------------------------
    mf32x4_t sc[4];
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) {
      sc[kg] = mf32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ds = 0; ds < 4; ++ds)
        sc[kg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(m_as_bf16x8(kreg[kg][ds]),
                                                         m_as_bf16x8(qop[ds]), sc[kg], 0, 0, 0);
    }
    // next tile's K is in flight during softmax and PV of this one (KDMA:
    // once this tile's operand reads have returned)
    tile_blocks(ti + nw_act, phn, rowsn);
    if constexpr (KDMA) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    issue_k(phn, rowsn);

    // ---- mask rows that do not exist (padding past ctx_len, missing blocks)
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) {
      if (rows[kg] < kBlk) {
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[kg][r] = 4 * q4 + r < rows[kg] ? sc[kg][r] : -INFINITY;
      }
    }
    // ---- online softmax per head (lane l%16), lazy rescale ----------------
    float mx = -INFINITY;
#pragma unroll
    for (int kg = 0; kg < 4; ++kg)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[kg][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const bool bump = (mx - m_run) * c > 8.f;
    const float m_use = bump ? mx : m_run;
    const float nm = m_use == -INFINITY ? 0.f : -m_use * c;
    const float alpha = (m_use == m_run) ? 1.f : __builtin_amdgcn_exp2f((m_run - m_use) * c);
    if (__builtin_amdgcn_ballot_w64(bump) != 0) {
      // O rows are heads 4(l/16) + r: fetch those heads' factors
      float ar[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * q4 + r);
#pragma unroll
      for (int dg = 0; dg < 8; ++dg)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[dg][r] *= ar[r];
    }
    m_run = m_use;
    float pw[4][4];
    float lsum = 0.f;
#pragma unroll
    for (int kg = 0; kg < 4; ++kg)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pw[kg][r] = __builtin_amdgcn_exp2f(fmaf(sc[kg][r], c, nm));
        lsum += pw[kg][r];
      }
    l_lane = l_lane * alpha + lsum;

    // ---- O += P V ----------------------------------------------------------
    // V(t) has landed once at most the 16 K loads of the next tile are still
    // in flight.  Written out: the compiler's own tracking of LDS DMA was
    // seen to let a transpose read run ahead of this wait.
    asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint4 pop = make_uint4(m_cvt_pk_bf16(pw[2 * ks][0], pw[2 * ks][1]),
                                   m_cvt_pk_bf16(pw[2 * ks][2], pw[2 * ks][3]),
                                   m_cvt_pk_bf16(pw[2 * ks + 1][0], pw[2 * ks + 1][1]),
                                   m_cvt_pk_bf16(pw[2 * ks + 1][2], pw[2 * ks + 1][3]));
#pragma unroll
      for (int dg = 0; dg < 8; ++dg) {
        // k-slots 0..3: block 2ks, rows 4(l/16)+0..3; 4..7: block 2ks+1
        const uint8_t* u0 = vt + (2 * ks) * kMBlock + vrow_off(dg);
        const uint2 lo2 = m_read_tr16(u0);
        const uint2 hi2 = m_read_tr16(u0 + kMBlock);
        const uint4 vop = make_uint4(lo2.x, lo2.y, hi2.x, hi2.y);
        o[dg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(m_as_bf16x8(pop), m_as_bf16x8(vop), o[dg],
                                                        0, 0, 0);
      }
    }
    // the V tile is free once its transpose reads have returned: next V in
    // flight during the next QK
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    issue_v(phn, rowsn);
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) {
      ph[kg] = phn[kg];
      rows[kg] = rowsn[kg];
    }
  }

  // ---- merge the 4 wavefront states --------------------------------------
  const float l_w = l_lane + __shfl_xor(l_lane, 16);
  const float l_h = l_w + __shfl_xor(l_w, 32);
  // no DMA may land in the tiles once they hold the merge states
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  float* mo = reinterpret_cast<float*>(&v_lds[0][0]);  // [kNW][G][D]
  float* mm = mo + kNW * G * D;                        // [kNW][G]
  float* ml = mm + kNW * G;
#pragma unroll
  for (int dg = 0; dg < 8; ++dg)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * q4 + r;
      if (h < G) mo[(w * G + h) * D + dg * 16 + hl] = o[dg][r];
    }
  if (q4 == 0 && hl < G) {
    mm[w * G + hl] = m_run;
    ml[w * G + hl] = l_h;
  }
  __syncthreads();
  for (int i = tid; i < G * D; i += kThreads) {
    const int hh = i / D, d = i % D;
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < kNW; ++k) M = fmaxf(M, mm[k * G + hh]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int k = 0; k < kNW; ++k) {
        const float mk = mm[k * G + hh];
        const float wt = mk == -INFINITY ? 0.f : exp2f((mk - M) * c);
        L = fmaf(wt, ml[k * G + hh], L);
        O = fmaf(wt, mo[(k * G + hh) * D + d], O);
      }
    }
    const int h = g * G + hh;
    const float Mc = M * c;  // log2 units
    if (Sb == 1) {
      store_out<uint16_t>(p.out, (size_t(b) * p.Hq + h) * D + d, L > 0.f ? O / L : 0.f);
      if (p.lse && d == 0) p.lse[size_t(b) * p.Hq + h] = L > 0.f ? (Mc + log2f(L)) * kLn2 : -INFINITY;
    } else {
      const size_t n = size_t(b) * p.S + s;
      p.o_part[(n * p.Hq + h) * D + d] = O;
      if (d == 0) {
        p.m_part[n * p.Hq + h] = M == -INFINITY ? -INFINITY : Mc * kLn2;
        p.l_part[n * p.Hq + h] = L;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// decode_block_kernel: the matrix-core decode with one workgroup per work
// item that streams whole KV blocks, all KV heads at once.
//
// In the token-major pool a block of K (or V) is one contiguous 32 KB run
// (16 slots x Hkv heads x 256 B).  The per-KV-head kernels above read one
// head's 256-byte pieces of it, 2 KB apart, at times unrelated to the other
// heads' workgroups; here eight wavefronts, one per KV head, pull the eight
// pieces of every row within a few hundred cycles, so the DRAM sees the
// whole block.  A streaming probe of the two orders (same bytes, no
// attention math, cold caches) moved 6.5 against 4.1-5.8 TB/s on the 32 x 4k
// batch and 6.9 against 3.9-5.6 TB/s on the 131k-token batch.
//
//   * Each wavefront owns one KV head and a two-stage ring of (K, V) blocks
//     of that head (4 KB each) in LDS, filled by DMA in whole 256-byte rows
//     (16 lanes per row, the slot swizzles of decode_mfma_kernel).  Block
//     j+1 is requested before block j is waited for, so two blocks per
//     wavefront are in flight; the ring is wavefront-private, so the loop
//     has no barrier.  128 KB of ring: one workgroup per CU.
//   * S = K Q^T per block on v_mfma_f32_16x16x32_bf16: the 16 columns of a
//     tile are (sequence, query head) pairs; the lane's four weights are
//     exactly the A operand of v_mfma_f32_16x16x16_bf16 for O += P V (k =
//     the block's 16 keys).
//   * Work items.  A private item is a split of one sequence's alive-block
//     stream.  With prefix sharing on, sequences whose first segment starts
//     at logical block 0 on the same physical block hold the same blocks up
//     to the shortest such segment (full blocks only); when two or more do,
//     that common prefix becomes shared items, each attending for up to
//     kBShareTiles * 16 / G member sequences at once (one column tile per 16
//     / G members), so the group's prefix is streamed once per sub-group
//     instead of once per member, and the members' private items start
//     after it.  Every item writes one partial per sequence it serves, and
//     a sequence's partials are merged by log-sum-exp like any split's.
//   * The split length, on the device: every workgroup reads all B
//     sequences' plan ends (and first segments, with sharing) and picks the
//     smallest T (at least kBMinSplit blocks) for which the items number at
//     most `target` (one workgroup per CU) and the partials fit the
//     workspace; the host knows only max_ctx_len, not the eviction rate,
//     the length mix or the sharing.  Exclusive scans number items and
//     partials; workgroup i takes item i, and workgroup 0 publishes the
//     partial ranges for the merge.
// ---------------------------------------------------------------------------
constexpr int kBThreads = 512;  // one wavefront per KV head
constexpr int kBHkv = kBThreads / kWave;
constexpr int kBMinSplit = 8;   // blocks: shorter splits cost more set-up than they balance
constexpr int kBShareTiles = 2;  // column tiles of a shared item
constexpr int kBMinShare = 8;   // a common prefix shorter than this is not shared

// inclusive prefix sum over the 64 lanes with DPP row shifts and row
// broadcasts (no LDS round trips): shifts 1, 2, 4, 8 scan each row of 16
// lanes, then lane 15 is added to row 1 (and row 3), lane 31 to rows 2, 3
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

__device__ __forceinline__ int wave_sum(int v) {
  return __builtin_amdgcn_readlane(wave_incl_scan(v), kWave - 1);
}

// sums of two values per thread over the workgroup (red: 2 kBHkv ints)
__device__ __forceinline__ void block_sum2(int u, int v, int* red, int& su, int& sv) {
  u = wave_sum(u);
  v = wave_sum(v);
  if ((threadIdx.x & (kWave - 1)) == 0) {
    red[threadIdx.x / kWave] = u;
    red[kBHkv + threadIdx.x / kWave] = v;
  }
  __syncthreads();
  su = sv = 0;
#pragma unroll
  for (int i = 0; i < kBHkv; ++i) {
    su += red[i];
    sv += red[kBHkv + i];
  }
  __syncthreads();
}

// exclusive prefix sums of three values per thread over the workgroup, and
// their totals (red: 3 kBHkv ints of LDS)
__device__ __forceinline__ void block_excl_scan3(int u, int v, int x, int* red, int& eu, int& ev, int& ex,
                                                 int& tu, int& tv, int& tx) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const int a = wave_incl_scan(u), b = wave_incl_scan(v), c = wave_incl_scan(x);
  if (lane == kWave - 1) {
    red[w] = a;
    red[kBHkv + w] = b;
    red[2 * kBHkv + w] = c;
  }
  __syncthreads();
  int ba = 0, bb = 0, bc = 0;
  tu = tv = tx = 0;
#pragma unroll
  for (int i = 0; i < kBHkv; ++i) {
    const int ra = red[i], rb = red[kBHkv + i], rc = red[2 * kBHkv + i];
    ba += i < w ? ra : 0;
    bb += i < w ? rb : 0;
    bc += i < w ? rc : 0;
    tu += ra;
    tv += rb;
    tx += rc;
  }
  __syncthreads();
  eu = ba + a - u;
  ev = bb + b - v;
  ex = bc + c - x;
}

// largest i in [lo, hi) with segs[i].alive_token_start <= x (the starts
// ascend, segs[lo] starts at or before x), for a whole workgroup: with at
// most 2 segments per thread every start is loaded in one round trip and the
// answer is lo + (how many start at or before x) - 1.  Longer lists take the
// narrowing search, which reads far fewer bytes (at 16 per thread, 4k-segment
// lists: the 131k-token batch's expansion took 5.6 against 4.0 us).  red:
// kBHkv ints of LDS.
__device__ __forceinline__ int wg_search_segment_wide(const msa_segment* segs, int lo, int hi, int x, int* red) {
  if (hi - lo > 2 * kBThreads) return wg_search_segment_n<kBThreads>(segs, lo, hi, x);
  int cnt = 0;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int idx = lo + k * kBThreads + int(threadIdx.x);
    if (k * kBThreads < hi - lo) cnt += idx < hi && segs[idx].alive_token_start <= x;
  }
  cnt = wave_sum(cnt);
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = cnt;
  __syncthreads();
  int total = 0;
#pragma unroll
  for (int i = 0; i < kBHkv; ++i) total += red[i];
  __syncthreads();
  return lo + total - 1;
}

// largest i in [0, n) with a[i] <= x (a ascending, a[0] <= x)
__device__ __forceinline__ int lds_upper(const int32_t* a, int n, int x) {
  int lo = 0, hi = n;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

struct BlockItemLds {
  int32_t alive[kDecodeBlockMaxSeq];       // alive tokens per sequence
  int32_t key[kDecodeBlockMaxSeq + 4];     // first segment's physical block (sharing), else -1
  int32_t fb[kDecodeBlockMaxSeq + 4];      // full blocks of the first segment
  int32_t lc[kDecodeBlockMaxSeq];          // shared prefix blocks (0: none)
  int32_t sub[kDecodeBlockMaxSeq];         // sub-group id: leader * 64 + rank / members-per-item
  int32_t rank[kDecodeBlockMaxSeq];        // rank among the sequences of its group
  int32_t pfirst[kDecodeBlockMaxSeq + 1];  // first partial of each sequence
  int32_t ifirst[kDecodeBlockMaxSeq + 1];  // first private item of each sequence
  int32_t sfirst[kDecodeBlockMaxSeq + 1];  // first shared item of each sub-group head
  int32_t red[3 * kBHkv];
  int32_t mem[16];   // this item's sequences
  int32_t pidx[16];  // their partial index (-1: the item writes the output itself)
};

template <int G, int NT>
__device__ __forceinline__ void block_stream(const DecodeParams& p, int nmem, const int32_t* mem,
                                             const int32_t* pidx, int nblk, const int32_t* blk_phys,
                                             int last_local, int last_tokens,
                                             uint8_t (*kv_lds)[2][kBHkv][kMBlock]) {
  constexpr int D = kMD;
  constexpr int kMPT = 16 / G;  // member sequences per column tile
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int g = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int hl = lane % 16, q4 = lane / 16;

  // Q^T operand of tile t (lane l: column l%16 = member t*kMPT + (l%16)/G,
  // query head g*G + (l%16)%G; zero past the members; d 32 ds + 8(l/16))
  uint4 qop[NT][4];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int m = t * kMPT + hl / G;
    const bool on = m < nmem;
    const size_t row = on ? (size_t(mem[m]) * p.Hq + size_t(g) * G + hl % G) : 0;
    const uint8_t* qsrc = static_cast<const uint8_t*>(p.q) + row * kMRow;
#pragma unroll
    for (int ds = 0; ds < 4; ++ds)
      qop[t][ds] = on ? *reinterpret_cast<const uint4*>(qsrc + (4 * ds + q4) * 16) : make_uint4(0, 0, 0, 0);
  }

  const size_t tok_stride = p.head_major ? size_t(kMRow) : size_t(p.Hkv) * kMRow;
  const size_t blk_stride = size_t(p.Hkv) * kMRow * kBlk;
  const size_t head_off = p.head_major ? size_t(g) * kMRow * kBlk : size_t(g) * kMRow;
  const char* kbase = static_cast<const char*>(p.k_pool) + head_off;
  const char* vbase = static_cast<const char*>(p.v_pool) + head_off;
  const int kq = lane / 16, slot = lane % 16;
  // transpose-read word of lane l for d group dg: key 4(l/16) + (l%16)/4,
  // d = 16 dg + 4(l%4) .. +3 (see decode_mfma_kernel)
  const int vr_key = 4 * q4 + hl / 4;
  const int vr_base = vr_key * kMRow + 8 * (hl % 2);
  auto vrow_off = [&](int dg) { return vr_base + 16 * ((2 * dg + (hl % 4) / 2) ^ ((2 * vr_key) & 15)); };
  const int k_off = hl * kMRow;  // + 16 ((4 ds + q4) ^ hl)

  // (K, V) of block jj of the item into ring stage jj % 2: the wave-uniform
  // physical id and readable rows (past the item or a dropped segment: an
  // empty range, so the DMAs land zeros)
  auto issue = [&](int jj) {
    const int ph = jj < nblk ? __builtin_amdgcn_readfirstlane(blk_phys[jj]) : -1;
    const int rows = ph < 0 ? 0 : (jj == last_local ? last_tokens : kBlk);
    const size_t boff = size_t(ph < 0 ? 0 : ph) * blk_stride;
    const uint32_t nrec = uint32_t(rows * tok_stride);
    const __amdgpu_buffer_rsrc_t rk = block_rsrc(kbase + boff, nrec);
    const __amdgpu_buffer_rsrc_t rv = block_rsrc(vbase + boff, nrec);
    uint8_t* kt = &kv_lds[jj & 1][0][g][0];
    uint8_t* vt = &kv_lds[jj & 1][1][g][0];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = 4 * i + kq;  // K: chunk slot ^ key into slot `slot`
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)(kt + i * 4 * kMRow),
                                               16, uint32_t(key * tok_stride + 16 * (slot ^ key)), 0, 0,
                                               kStreamPolicy);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = 4 * i + kq;  // V: chunk slot ^ (2 key mod 16) into slot `slot`
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (__attribute__((address_space(3))) void*)(vt + i * 4 * kMRow),
                                               16, uint32_t(key * tok_stride + 16 * (slot ^ ((2 * key) & 15))),
                                               0, 0, kStreamPolicy);
    }
    return rows;
  };

  mf32x4_t o[NT][8];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int dg = 0; dg < 8; ++dg) o[t][dg] = mf32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run[NT], l_lane[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    m_run[t] = -INFINITY;
    l_lane[t] = 0.f;
  }
  const float c = p.scale_log2;

  int rows = issue(0);
  for (int jj = 0; jj < nblk; ++jj) {
    // block jj+1 into the other stage, whose reads of block jj-1 have
    // returned (the wait at the end of the previous step)
    const int rows_next = issue(jj + 1);
    // block jj has landed once at most the 8 DMAs of block jj+1 are in flight
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    const uint8_t* kt = &kv_lds[jj & 1][0][g][0];
    const uint8_t* vt = &kv_lds[jj & 1][1][g][0];
    uint4 kr[4];
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) kr[ds] = *reinterpret_cast<const uint4*>(kt + k_off + 16 * ((4 * ds + q4) ^ hl));
    uint2 vr[8];
#pragma unroll
    for (int dg = 0; dg < 8; ++dg) vr[dg] = m_read_tr16(vt + vrow_off(dg));
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      // ---- S = K Q^T: lane l holds column l%16, keys 4(l/16) .. +3 --------
      mf32x4_t sc = mf32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ds = 0; ds < 4; ++ds)
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(m_as_bf16x8(kr[ds]), m_as_bf16x8(qop[t][ds]), sc, 0, 0, 0);
      if (rows < kBlk) {
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[r] = 4 * q4 + r < rows ? sc[r] : -INFINITY;
      }
      // ---- online softmax per column, lazy rescale -------------------------
      float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const bool bump = (mx - m_run[t]) * c > 8.f;
      const float m_use = bump ? mx : m_run[t];
      const float nm = m_use == -INFINITY ? 0.f : -m_use * c;
      const float alpha = (m_use == m_run[t]) ? 1.f : __builtin_amdgcn_exp2f((m_run[t] - m_use) * c);
      if (__builtin_amdgcn_ballot_w64(bump) != 0) {
        // O rows are columns 4(l/16) + r: fetch those columns' factors
        float ar[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * q4 + r);
#pragma unroll
        for (int dg = 0; dg < 8; ++dg)
#pragma unroll
          for (int r = 0; r < 4; ++r) o[t][dg][r] *= ar[r];
      }
      m_run[t] = m_use;
      float pw[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) pw[r] = __builtin_amdgcn_exp2f(fmaf(sc[r], c, nm));
      l_lane[t] = l_lane[t] * alpha + ((pw[0] + pw[1]) + (pw[2] + pw[3]));
      // ---- O += P V ---------------------------------------------------------
      const ms16x4_t pop = __builtin_bit_cast(ms16x4_t, make_uint2(m_cvt_pk_bf16(pw[0], pw[1]),
                                                                   m_cvt_pk_bf16(pw[2], pw[3])));
#pragma unroll
      for (int dg = 0; dg < 8; ++dg)
        o[t][dg] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pop, __builtin_bit_cast(ms16x4_t, vr[dg]),
                                                             o[t][dg], 0, 0, 0);
    }
    // this stage is refilled by the next step's DMA: its reads must be back
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    rows = rows_next;
  }
  // no DMA may be left in flight when the workgroup ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- write: column hh of tile t is member t*kMPT + hh/G, head hh%G -------
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float l_w = l_lane[t] + __shfl_xor(l_lane[t], 16);
    const float l_h = l_w + __shfl_xor(l_w, 32);  // column hl's sum over the item
    float lr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) lr[r] = __shfl(l_h, 4 * q4 + r);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int hh = 4 * q4 + r, m = t * kMPT + hh / G;
      if (m < nmem) {
        const int b = mem[m], pi = pidx[m];
        const size_t h = size_t(g) * G + hh % G;
#pragma unroll
        for (int dg = 0; dg < 8; ++dg) {
          const int d = dg * 16 + hl;
          if (pi < 0)
            store_out<uint16_t>(p.out, (size_t(b) * p.Hq + h) * D + d, lr[r] > 0.f ? o[t][dg][r] / lr[r] : 0.f);
          else if (pi < p.block_parts)
            p.o_part[(size_t(pi) * p.Hq + h) * D + d] = o[t][dg][r];
        }
      }
    }
    const int m = t * kMPT + hl / G;
    if (q4 == 0 && m < nmem) {
      const int b = mem[m], pi = pidx[m];
      const size_t h = size_t(g) * G + hl % G;
      const float Mc = m_run[t] * c;  // log2 units
      if (pi < 0) {
        if (p.lse) p.lse[size_t(b) * p.Hq + h] = l_h > 0.f ? (Mc + log2f(l_h)) * kLn2 : -INFINITY;
      } else if (pi < p.block_parts) {
        p.m_part[size_t(pi) * p.Hq + h] = m_run[t] == -INFINITY ? -INFINITY : Mc * kLn2;
        p.l_part[size_t(pi) * p.Hq + h] = l_h;
      }
    }
  }
}

template <int G>
__global__ void __launch_bounds__(kBThreads, 1) decode_block_kernel(DecodeParams p) {
  static_assert(G == 4 || G == 8, "heads padded to 16 MFMA rows");
  constexpr int D = kMD;
  constexpr int kMPI = kBShareTiles * 16 / G;  // member sequences per shared item
  // [stage][K, V][wavefront] blocks of one head; during set-up the same
  // bytes hold the staged segment list
  __shared__ __align__(16) uint8_t kv_lds[2][2][kBHkv][kMBlock];
  __shared__ __align__(16) int32_t blk_phys[kMaxSplitBlocks];
  __shared__ __align__(16) BlockItemLds sh;
  static_assert(sizeof(kv_lds) >= 3 * (kMaxSplitBlocks + 1) * sizeof(int32_t), "staging");

  const int tid = threadIdx.x;
  const int B = p.B, id = blockIdx.x;
  const bool share = p.block_share != 0;

  // ---- per sequence: alive tokens, first segment ---------------------------
  // thread t holds sequences [i0, i1)
  const int per = (B + kBThreads - 1) / kBThreads;
  const int i0 = min(B, tid * per), i1 = min(B, i0 + per);
  int cut = 0;
  for (int i = i0; i < i1; ++i) {
    const int a0 = p.indptr[i], a1 = p.indptr[i + 1];
    int A = 0, key = -1, fb = 0;
    if (a1 > a0) {
      const msa_segment l = p.segs[a1 - 1];
      A = max(0, l.alive_token_start + l.num_tokens);
      if (share) {
        const msa_segment f = p.segs[a0];
        if (f.logical_block == 0 && f.phys_block >= 0 && f.num_blocks > 0 &&
            int64_t(f.phys_block) + f.num_blocks <= p.P) {
          key = f.phys_block;
          fb = min(f.num_tokens / kBlk, f.num_blocks);
        }
      }
    }
    const int nb = (A + kBlk - 1) / kBlk;
    const int nbc = min(nb, p.cap_blocks);
    cut |= nb > nbc;
    sh.alive[i] = A;
    sh.key[i] = key;
    sh.fb[i] = min(fb, nbc);
  }
  if (tid < 4 && B + tid < kDecodeBlockMaxSeq + 4) {
    sh.key[B + tid] = -1;
    sh.fb[B + tid] = 0;
  }
  __syncthreads();
  // ---- sharing: groups of equal first physical block, their common prefix --
  // Each sequence's group is summed over the batch by NP threads, one slice
  // of the batch each, whose partial sums meet in LDS (the ring bytes are
  // free until the items start): with one thread per sequence the scan was
  // one wavefront's serial loop over the whole batch.
  if (share) {
    const int Bc = B <= 64 ? 64 : (B <= 128 ? 128 : 256);  // B <= kDecodeBlockMaxShareSeq
    const int NP = kBThreads / Bc;
    const int i = tid % Bc, part = tid / Bc;
    const int span = ((B + NP - 1) / NP + 3) & ~3;  // whole int4 reads per slice
    const int jlo = part * span, jhi = min(B, jlo + span);
    int size = 0, rank = 0, lead = B, lmin = INT_MAX;
    const int key = i < B ? sh.key[i] : -1;
    if (key >= 0) {
      // four sequences per LDS read (the arrays are padded with key -1)
      for (int j4 = jlo; j4 < jhi; j4 += 4) {
        const int4 k4 = *reinterpret_cast<const int4*>(&sh.key[j4]);
        const int4 f4 = *reinterpret_cast<const int4*>(&sh.fb[j4]);
        const int kk[4] = {k4.x, k4.y, k4.z, k4.w}, ff[4] = {f4.x, f4.y, f4.z, f4.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int j = j4 + u;
          const bool same = kk[u] == key;
          size += same;
          rank += same && j < i;
          lead = same ? min(lead, j) : lead;
          lmin = same ? min(lmin, ff[u]) : lmin;
        }
      }
    }
    int4* part_sum = reinterpret_cast<int4*>(&kv_lds[0][0][0][0]);  // [NP][Bc]
    part_sum[part * Bc + i] = make_int4(size, rank, lead, lmin);
    __syncthreads();
    if (part == 0 && i < B) {
      int lc = 0, sub = -1;
      if (key >= 0) {
        for (int q = 1; q < NP; ++q) {
          const int4 v = part_sum[q * Bc + i];
          size += v.x;
          rank += v.y;
          lead = min(lead, v.z);
          lmin = min(lmin, v.w);
        }
        if (size >= 2 && lmin >= kBMinShare) {
          lc = lmin;
          sub = lead * 64 + rank / kMPI;
        }
      }
      sh.lc[i] = lc;
      sh.sub[i] = sub;
      sh.rank[i] = rank;
    }
  } else {
    for (int i = i0; i < i1; ++i) {
      sh.lc[i] = 0;
      sh.sub[i] = -1;
      sh.rank[i] = 0;
    }
  }
  __syncthreads();
  // members join sub-groups in index order: the head is rank 0 of its sub-group
  auto is_head = [&](int i) { return sh.lc[i] > 0 && sh.rank[i] % kMPI == 0; };
  // items at split length T: private ones of a sequence, shared ones of a
  // sub-group (counted at its head); each is one partial per sequence served
  auto nbc_of = [&](int i) { return min((sh.alive[i] + kBlk - 1) / kBlk, p.cap_blocks); };
  auto priv_items = [&](int i, int T) {
    const int rest = nbc_of(i) - sh.lc[i];
    return rest > 0 ? (rest + T - 1) / T : (sh.lc[i] == 0 ? 1 : 0);
  };
  auto shared_items = [&](int lc, int T) { return lc > 0 ? (lc + T - 1) / T : 0; };
  int heads_mask = 0;  // bit k: sequence i0 + k heads its sub-group (per <= 2)
  for (int i = i0; i < i1; ++i)
    if (is_head(i)) heads_mask |= 1 << (i - i0);
  int T = p.split_blocks;
  if (p.block_auto) {
    // blocks actually read, and the ranges they come in (a sequence with no
    // alive block counts as one range: it is one item at any T)
    int wsum = 0, ranges = 0;
    for (int i = i0; i < i1; ++i) {
      const int rest = nbc_of(i) - sh.lc[i];
      wsum += max(rest, 0);
      ranges += rest > 0 || sh.lc[i] == 0;
      if ((heads_mask >> (i - i0)) & 1) {
        wsum += sh.lc[i];
        ranges += 1;
      }
    }
    int W, NR;
    block_sum2(wsum, ranges, sh.red, W, NR);
    const int target = p.block_target;
    // smallest T in [lo, hi] with at most target items and the partials
    // within the workspace; both counts fall as T grows.  A round tests
    // eight points, one per wavefront, each summing over all sequences in
    // its own lanes, and returns which of them fit.
    const int w = tid / kWave, lane = tid & (kWave - 1);
    auto fits = [&](int cand) {
      int it = 0, pa = 0;
      for (int i = lane; i < B; i += kWave) {
        const int pv = priv_items(i, cand), sv = shared_items(sh.lc[i], cand);
        it += pv + (is_head(i) ? sv : 0);
        pa += pv + sv;
      }
      it = wave_sum(it);
      pa = wave_sum(pa);
      if (lane == 0) sh.red[w] = it <= target && pa <= p.block_parts;
      __syncthreads();
      int bits = 0;
#pragma unroll
      for (int k = 0; k < kBHkv; ++k) bits |= (sh.red[k] != 0) << k;
      __syncthreads();
      return bits;
    };
    int lo = min(max(kBMinSplit, (W + target - 1) / target), kMaxSplitBlocks);
    int hi = kMaxSplitBlocks;  // always fits: the host sized grid and workspace for it
    // A range of r blocks makes ceil(r / T) <= r / T + 1 items, so every T
    // >= W / (target - NR) meets the item bound; unless the partial bound
    // binds, the answer lies in [lo, that].  A first round tests eight
    // points ending there; then [lo, hi] narrows with hi known to fit.
    const int slack = target - NR;
    const int ha = min(max(slack > 0 ? (W + slack - 1) / slack : kMaxSplitBlocks, lo), kMaxSplitBlocks);
    if (ha < hi) {
      const int bits = fits(lo + ((ha - lo) * (w + 1)) / kBHkv);
      if (bits != 0) {
        const int k = __builtin_ctz(bits);
        hi = lo + ((ha - lo) * (k + 1)) / kBHkv;
        lo = k == 0 ? lo : lo + ((ha - lo) * k) / kBHkv + 1;
      } else {
        lo = ha + 1;
      }
    }
    while (lo < hi) {
      const int bits = fits(lo + ((hi - lo) * (w + 1)) / 9);
      if (bits != 0) {
        const int k = __builtin_ctz(bits);
        const int nhi = lo + ((hi - lo) * (k + 1)) / 9;
        lo = k == 0 ? lo : lo + ((hi - lo) * k) / 9 + 1;
        hi = nhi;
      } else {
        lo = lo + ((hi - lo) * 8) / 9 + 1;
      }
    }
    T = lo;
  }
  // ---- number items and partials -------------------------------------------
  {
    int pv_mine = 0, sv_mine = 0, pa_mine = 0;
    for (int i = i0; i < i1; ++i) {
      const int pv = priv_items(i, T), sv = shared_items(sh.lc[i], T);
      pv_mine += pv;
      sv_mine += ((heads_mask >> (i - i0)) & 1) ? sv : 0;
      pa_mine += pv + sv;
    }
    int np, ns, npa;
    int rp, rs, ra;
    block_excl_scan3(pv_mine, sv_mine, pa_mine, sh.red, rp, rs, ra, np, ns, npa);
    for (int i = i0; i < i1; ++i) {
      const int pv = priv_items(i, T), sv = shared_items(sh.lc[i], T);
      sh.ifirst[i] = rp;
      sh.sfirst[i] = np + rs;  // shared items follow the private ones
      sh.pfirst[i] = ra;
      rp += pv;
      rs += ((heads_mask >> (i - i0)) & 1) ? sv : 0;
      ra += pv + sv;
    }
    if (tid == 0) {
      sh.ifirst[B] = np;
      sh.sfirst[B] = np + ns;
      sh.pfirst[B] = npa;
    }
  }
  const bool any_cut = __syncthreads_or(cut) != 0;
  const int n_items = sh.sfirst[B], n_parts = sh.pfirst[B];
  if (id == 0) {
    // the merge reads these; clamped to the workspace so that it can never
    // read a partial outside it (the sizing rule keeps n_parts within it)
    for (int i = tid; i <= B; i += kBThreads) p.part_indptr[i] = min(sh.pfirst[i], p.block_parts);
    if (tid == 0 && p.dev_error && (any_cut || n_items > int(gridDim.x) || n_parts > p.block_parts))
      atomicOr(p.dev_error, MSA_DEVERR_TRUNCATED);
  }
  if (id >= n_items || n_parts > p.block_parts) return;

  // ---- this item: its sequences, their partials, its blocks ---------------
  int nmem, j0, nblk, last_local, last_tokens;
  bool shared_item;
  if (id < sh.ifirst[B]) {
    // private item s of sequence b: blocks [lc + s*rest/Sp, ...)
    shared_item = false;
    const int b = lds_upper(sh.ifirst, B, id);
    const int Sp = max(1, sh.ifirst[b + 1] - sh.ifirst[b]), s = min(id - sh.ifirst[b], Sp - 1);
    const int A = sh.alive[b], nbc = nbc_of(b), lc = sh.lc[b];
    const int rest = nbc - lc;
    nmem = 1;
    if (tid == 0) {
      sh.mem[0] = b;
      // one partial in all: the item writes the output itself
      sh.pidx[0] = sh.pfirst[b + 1] - sh.pfirst[b] == 1 ? -1 : sh.pfirst[b] + s;
    }
    if (rest <= 0) {
      nblk = 0;  // no alive block at all (a sequence with a shared prefix always has rest > 0 here)
      j0 = 0;
    } else {
      j0 = lc + int(int64_t(s) * rest / Sp);
      nblk = lc + int(int64_t(s + 1) * rest / Sp) - j0;
    }
    last_local = nbc - 1 - j0;
    last_tokens = nbc > 0 ? min(kBlk, A - kBlk * (nbc - 1)) : 0;
    if (nblk > 0) {
      // expand the item's segments into per-block physical ids
      const int s0 = p.indptr[b], s1 = p.indptr[b + 1];
      const int sf = j0 == 0 ? s0 : wg_search_segment_wide(p.segs, s0, s1, j0 * kBlk, sh.red);
      const int ns = min(nblk, s1 - sf);
      int32_t* st_start = reinterpret_cast<int32_t*>(&kv_lds[0][0][0][0]);
      int32_t* st_phys = st_start + kMaxSplitBlocks + 1;
      int32_t* st_nblk = st_phys + kMaxSplitBlocks + 1;
      for (int i = tid; i < ns; i += kBThreads) {
        const msa_segment sg = p.segs[sf + i];
        st_start[i] = sg.alive_token_start / kBlk;
        const bool in_pool = sg.phys_block >= 0 && sg.num_blocks >= 0 &&
                             int64_t(sg.phys_block) + sg.num_blocks <= p.P;
        st_phys[i] = in_pool ? sg.phys_block : -1;
        st_nblk[i] = in_pool ? sg.num_blocks : 0;
      }
      __syncthreads();
      for (int jj = tid; jj < nblk; jj += kBThreads) {
        const int j = j0 + jj;
        const int lo = lds_upper(st_start, ns, j);
        const int off = j - st_start[lo];
        blk_phys[jj] = (st_phys[lo] >= 0 && off >= 0 && off < st_nblk[lo]) ? st_phys[lo] + off : -1;
      }
    }
  } else {
    // shared item s of the sub-group headed by sequence hd: blocks
    // [s*lc/Ss, (s+1)*lc/Ss) of the common prefix, all in the first segment
    shared_item = true;
    const int hd = lds_upper(sh.sfirst, B, id);
    const int lc = sh.lc[hd], sub = sh.sub[hd];
    const int Ss = max(1, (lc + T - 1) / T), s = min(id - sh.sfirst[hd], Ss - 1);
    j0 = int(int64_t(s) * lc / Ss);
    nblk = int(int64_t(s + 1) * lc / Ss) - j0;
    last_local = -1;  // full blocks only
    last_tokens = kBlk;
    // the members, in index order: slot rank % kMPI
    int mine = 0;
    for (int j = hd + tid; j < B; j += kBThreads) {
      if (sh.sub[j] == sub) {
        const int slot = sh.rank[j] % kMPI;
        sh.mem[slot] = j;
        sh.pidx[slot] = sh.pfirst[j + 1] - sh.pfirst[j] == 1 ? -1 : sh.pfirst[j] + priv_items(j, T) + s;
        ++mine;
      }
    }
    const int ph0 = sh.key[hd] + j0;
    for (int jj = tid; jj < nblk; jj += kBThreads) blk_phys[jj] = ph0 + jj;
    nmem = __syncthreads_count(mine);
  }
  __syncthreads();  // staging dead from here on: the ring may overwrite it

  if (nblk == 0) {  // no alive token at all: O = 0, LSE = -inf
    const int b = sh.mem[0];
    for (int i = tid; i < p.Hq * D; i += kBThreads) {
      store_out<uint16_t>(p.out, size_t(b) * p.Hq * D + i, 0.f);
      if (p.lse && i % D == 0) p.lse[size_t(b) * p.Hq + i / D] = -INFINITY;
    }
    return;
  }
  if (shared_item)
    block_stream<G, kBShareTiles>(p, nmem, sh.mem, sh.pidx, nblk, blk_phys, last_local, last_tokens, kv_lds);
  else
    block_stream<G, 1>(p, nmem, sh.mem, sh.pidx, nblk, blk_phys, last_local, last_tokens, kv_lds);
}

template <typename KV, int D, int G>
hipError_t launch_t(const DecodeParams& p, hipStream_t stream) {
  dim3 grid(p.S, p.Hkv, p.B);
  // The MFMA kernel whenever it is built for the shape (bf16, D 128, G 4 or
  // 8): the VALU kernel is compute-bound at G 8 and, with whole-row V
  // loads in the MFMA kernel, also slower at G 4 (cold caches: 84 against
  // 80 us on the 32 x 4k batch, 254 against 241 us on the lognormal batch,
  // 199 against ~190 us on the 131k-token layout with 32 query heads).
  // A caller may also ask for one kernel explicitly (msa_decode_kernel); the
  // API has checked that the matrix-core kernel exists for the shape.
  bool mfma = false;
  if constexpr (std::is_same<KV, uint16_t>::value && D == kMD && (G == 4 || G == 8))
    mfma = p.kernel != MSA_DECODE_VECTOR;
  if (mfma) {
    if constexpr (std::is_same<KV, uint16_t>::value && D == kMD && (G == 4 || G == 8)) {
      // K by row DMA when the grid is at most one workgroup per CU, where
      // its extra LDS costs no occupancy
      if (int64_t(p.S) * p.Hkv * p.B <= kCUs)
        hipLaunchKernelGGL((decode_mfma_kernel<G, true>), grid, dim3(kThreads), 0, stream, p);
      else
        hipLaunchKernelGGL((decode_mfma_kernel<G, false>), grid, dim3(kThreads), 0, stream, p);
    }
  } else {
    hipLaunchKernelGGL((decode_kernel<KV, D, G>), grid, dim3(kThreads), 0, stream, p);
  }
  return hipGetLastError();
}

template <typename KV, int D>
hipError_t launch_g(const DecodeParams& p, hipStream_t stream) {
  if constexpr (std::is_same<KV, uint16_t>::value && D == kMD) {
    if (p.use_block) {
      if (p.Hq / p.Hkv == 4)
        hipLaunchKernelGGL((decode_block_kernel<4>), dim3(p.nwg), dim3(kBThreads), 0, stream, p);
      else
        hipLaunchKernelGGL((decode_block_kernel<8>), dim3(p.nwg), dim3(kBThreads), 0, stream, p);
      return hipGetLastError();
    }
  }
  switch (p.Hq / p.Hkv) {
    case 1: return launch_t<KV, D, 1>(p, stream);
    case 2: return launch_t<KV, D, 2>(p, stream);
    case 4: return launch_t<KV, D, 4>(p, stream);
    case 8: return launch_t<KV, D, 8>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool decode_supported(msa_dtype dtype, int32_t D, int32_t G) {
  const bool g_ok = G == 1 || G == 2 || G == 4 || G == 8;
  if (dtype == MSA_BF16) return g_ok && (D == 64 || D == 128);
  if (dtype == MSA_F32) return g_ok && (D == 64 || D == 128);  // D 128: the generic kernel
  return false;
}

SplitPlan decode_split(int32_t B, int32_t Hkv, int32_t max_ctx_len, int32_t block_size,
                       int32_t split_blocks) {
  SplitPlan sp;
  const int64_t nbm = (int64_t(max_ctx_len) + block_size - 1) / block_size;
  int64_t T = split_blocks;
  if (T <= 0) {
    // Splits of at most 128 blocks (2048 tokens): long enough that the
    // per-split set-up and partial write are small next to its 8 MB of K/V
    // per KV head (bf16, D 128), short enough that a few long contexts in a
    // skewed batch do not leave most CUs idle.  Short batches get shorter
    // splits (down to 32 blocks) so the grid still covers the chip.  When
    // the (sequence, KV head) pairs alone cover the 256 CUs the cap is 192
    // blocks: the grid is sized by the longest context, so shorter splits
    // mostly add workgroups with nothing to do and partials to merge (the
    // 64-sequence lognormal batch: 249 against 261 us at 120 blocks; the
    // 4-sequence 131k batch, 32 pairs, is best at 120-136 blocks).
    const int64_t pairs = int64_t(B) * Hkv;
    const int64_t cap = pairs >= 256 ? 192 : 128;
    T = (nbm * pairs + 511) / 512;
    T = ((T + 15) / 16) * 16;
    if (T < 32) T = 32;
    if (T > cap) T = cap;
    // When the (sequence, KV head) pairs alone fill the 256 CUs and no
    // context exceeds 256 blocks, one split per pair needs no merge at all
    // (77 against 81 us with two splits on the 32 x 4k batch).
    if (pairs >= 256 && nbm <= 256) T = nbm > 0 ? nbm : 1;
    // Workgroup ids go round-robin to the 8 XCDs, so with a split count that
    // is a multiple of 8 split s of every (sequence, KV head) lands on XCD
    // s mod 8; on the 131k-token batch (equal-length sequences) that cost
    // 283 against 218 us.  Shorten the splits until the count is not.
    while (T > 32 && ((nbm + T - 1) / T) % 8 == 0) T -= 8;
  }
  sp.split_blocks = int32_t(T);
  sp.S = int32_t(nbm == 0 ? 1 : (nbm + T - 1) / T);
  return sp;
}

bool decode_matrix_supported(msa_dtype dtype, int32_t D, int32_t G) {
  return dtype == MSA_BF16 && D == kMD && (G == 4 || G == 8);
}

int32_t decode_max_split_blocks() { return kMaxSplitBlocks; }

bool decode_block_supported(msa_dtype dtype, int32_t D, int32_t Hkv, int32_t G, int32_t B) {
  return dtype == MSA_BF16 && D == kMD && Hkv == kBHkv && (G == 4 || G == 8) && B >= 1 &&
         B <= kDecodeBlockMaxSeq;
}

int32_t decode_block_target(int32_t B) { return kCUs > 2 * B ? kCUs : 2 * B; }

// Workgroups and partials of the block kernel.  A sequence's alive blocks
// (at most cap) come in at most two ranges, a shared prefix and the rest, so
// at split length T there are at most cap * B / T + 2B items and as many
// partials.  The device rule keeps the items within target and the partials
// within its capacity whenever some T <= kMaxSplitBlocks does, and T =
// kMaxSplitBlocks always does with these sizes; a caller's T sizes both.
BlockSizes decode_block_sizes(int32_t B, int32_t cap_blocks, int32_t split_blocks) {
  const int64_t work = int64_t(cap_blocks) * B;
  BlockSizes z;
  if (split_blocks > 0) {
    z.items = z.parts = (work + split_blocks - 1) / split_blocks + 2 * int64_t(B);
  } else {
    const int64_t at_max = (work + kMaxSplitBlocks - 1) / kMaxSplitBlocks;
    const int64_t target = decode_block_target(B);
    z.items = (at_max > target ? at_max : target) + 2 * int64_t(B);
    z.parts = (at_max > 2 * target ? at_max : 2 * target) + 2 * int64_t(B);
  }
  return z;
}

bool decode_block_shares(int32_t B) { return B >= 2 && B <= kDecodeBlockMaxShareSeq; }

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  if (p.dtype == MSA_BF16) {
    if (p.D == 128) return launch_g<uint16_t, 128>(p, stream);
    if (p.D == 64) return launch_g<uint16_t, 64>(p, stream);
  } else if (p.dtype == MSA_F32) {
    if (p.D == 64) return launch_g<float, 64>(p, stream);
    if (p.D == 128) {
      // float32 rows of 512 bytes do not fit the vector kernel's load
      // layout: the generic kernel, one query row
      GenericParams gp{};
      gp.q = p.q;
      gp.q_pos0 = nullptr;
      gp.C = 1;
      gp.k_pool = p.k_pool;
      gp.v_pool = p.v_pool;
      gp.P = p.P;
      gp.segs = p.segs;
      gp.indptr = p.indptr;
      gp.B = p.B;
      gp.Hq = p.Hq;
      gp.Hkv = p.Hkv;
      gp.D = p.D;
      gp.head_major = p.head_major;
      gp.dtype = p.dtype;
      gp.scale_log2 = p.scale_log2;
      gp.split_blocks = p.split_blocks;
      gp.S = p.S;
      gp.dev_error = p.dev_error;
      gp.out = p.out;
      gp.lse = p.lse;
      gp.o_part = p.o_part;
      gp.m_part = p.m_part;
      gp.l_part = p.l_part;
      return launch_generic(gp, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace msa
