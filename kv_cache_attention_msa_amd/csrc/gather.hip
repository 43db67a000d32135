// Gather-then-attend baseline: the detour MSA avoids.
//
// Without a multi-segment kernel, attention over a fragmented cache first
// copies the surviving K/V blocks into one contiguous buffer and then runs a
// contiguous kernel over it (P1, "Core method 1: MSA": the gather + attention
// slow path; P2, Key Results: MSA against gathering).  This file provides that
// copy so the two paths can be timed on the same inputs with the same
// attention kernel: the dense pool it writes holds sequence b's alive block
// j at block b*blocks_per_seq + j, and the plan it writes has one segment per
// sequence covering them.
//
// Grid: (dense block j, sequence b); 256 threads copy one K block and one V
// block ([16, Hkv, D] each, contiguous in both pools) with 16-byte
// non-temporal loads and stores.  Workgroup (0, b) also writes sequence b's
// dense segment and workgroup (0, 0) the indptr.
#include "msa_internal.h"

namespace msa {
namespace {

constexpr int kThreads = 256;
constexpr int kBlk = 16;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(kThreads) gather_kernel(GatherParams p) {
  const int j = blockIdx.x, b = blockIdx.y;
  const int s0 = p.indptr[b], s1 = p.indptr[b + 1];
  int A = 0;
  if (s1 > s0) {
    const msa_segment last = p.segs[s1 - 1];
    A = last.alive_token_start + last.num_tokens;
  }
  const int nAB = min((A + kBlk - 1) / kBlk, p.blocks_per_seq);
  if (j == 0 && threadIdx.x == 0) {
    msa_segment d;
    d.seq = b;
    d.logical_block = 0;
    d.phys_block = b * p.blocks_per_seq;
    d.num_blocks = nAB;
    d.num_tokens = min(A, nAB * kBlk);
    d.alive_token_start = 0;
    p.dense_segs[b] = d;
    if (b == 0)
      for (int i = 0; i <= p.B; ++i) p.dense_indptr[i] = i;
  }
  if (j >= nAB) return;
  // segment holding alive block j: largest i with alive_token_start <= 16 j
  int lo = s0, hi = s1;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.segs[mid].alive_token_start <= j * kBlk) lo = mid; else hi = mid;
  }
  const msa_segment sg = p.segs[lo];
  const int phys = sg.phys_block + (j - sg.alive_token_start / kBlk);
  if (phys < 0 || phys >= p.P) return;  // a foreign plan: leave the dense block as is
  const size_t n16 = p.block_bytes / 16;
  const u32x4_t* ks = reinterpret_cast<const u32x4_t*>(static_cast<const char*>(p.k_pool) + size_t(phys) * p.block_bytes);
  const u32x4_t* vs = reinterpret_cast<const u32x4_t*>(static_cast<const char*>(p.v_pool) + size_t(phys) * p.block_bytes);
  const size_t dst = size_t(b) * p.blocks_per_seq + j;
  u32x4_t* kd = reinterpret_cast<u32x4_t*>(static_cast<char*>(p.dense_k) + dst * p.block_bytes);
  u32x4_t* vd = reinterpret_cast<u32x4_t*>(static_cast<char*>(p.dense_v) + dst * p.block_bytes);
  for (size_t i = threadIdx.x; i < n16; i += kThreads) {
    const u32x4_t k = __builtin_nontemporal_load(ks + i);
    const u32x4_t v = __builtin_nontemporal_load(vs + i);
    __builtin_nontemporal_store(k, kd + i);
    __builtin_nontemporal_store(v, vd + i);
  }
}

}  // namespace

hipError_t launch_gather(const GatherParams& p, hipStream_t stream) {
  dim3 grid(p.blocks_per_seq, p.B);
  hipLaunchKernelGGL(gather_kernel, grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace msa
