// a1: segment plan on the device.
//
// split_into_contiguous_segments (P1, "Core method 1: MSA" pseudocode and the
// paragraph after it): the alive blocks of each sequence are cut into
// maximal runs that are consecutive both in logical index and in physical
// id; the hole an evicted block leaves always breaks a run.
//
// Two launches, one workgroup per sequence each:
//   count  -- number of segment starts per sequence + data-error flags
//   write  -- prefix of the counts -> seg_indptr; every block that ENDS a
//             run writes that run's whole record, so each record has exactly
//             one writer and no cross-workgroup coordination is needed.
// For small batches each write workgroup sums the counts before its own
// sequence itself (B reads each, cheaper than a launch).  Above kDirectMaxB
// sequences that would be B^2 reads in all, so a one-workgroup scan launch
// between the two computes every record offset, seg_indptr and the error
// word once, and each write workgroup reads only its own offset.
// A block l "is alive" iff alive[b][l] != 0 and its physical id is in
// [0, P); an out-of-range id is reported and the block treated as evicted,
// so no consumer of the plan can be sent outside the pool.
#include "msa_internal.h"

namespace msa {
namespace {

constexpr int kPlanThreads = 256;
constexpr int kScanThreads = 1024;
constexpr int kDirectMaxB = 1024;  // above this many sequences the scan launch runs
constexpr int kPerThread = 4;  // consecutive blocks per thread per chunk
constexpr int kChunk = kPlanThreads * kPerThread;

struct SeqView {
  const int32_t* trow;
  const uint8_t* arow;
  int32_t n_tok;
  int32_t nb;
};

__device__ __forceinline__ SeqView seq_view(const PlanParams& p, int b, int& flags) {
  SeqView v;
  v.trow = p.table + size_t(b) * p.max_blocks;
  v.arow = p.alive + size_t(b) * p.max_blocks;
  int32_t n = p.ctx_len[b];
  const int32_t lim = p.max_blocks * p.bs;  // host checked it fits in int32
  if (n < 0 || n > lim) {
    flags |= MSA_DEVERR_CTX_RANGE;
    n = n < 0 ? 0 : lim;
  }
  v.n_tok = n;
  v.nb = (n + p.bs - 1) / p.bs;
  return v;
}

// a block's alive flag and table entry, read together whatever their
// values (the row pointers do not depend on ctx_len, so these loads need not
// wait for it); blocks outside the row read as dead
struct Raw {
  uint8_t a;
  int32_t ph;
};
__device__ __forceinline__ Raw load_raw(const PlanParams& p, const SeqView& v, int l) {
  Raw r = {0, -1};
  if (l >= 0 && l < p.max_blocks) {
    r.a = v.arow[l];
    r.ph = v.trow[l];
  }
  return r;
}

// alive-and-valid predicate on block l's raw values; phys is meaningful only
// when it returns true
__device__ __forceinline__ bool live(const PlanParams& p, const SeqView& v, int l, Raw r,
                                     int32_t& phys, int& flags) {
  if (l < 0 || l >= v.nb || r.a == 0) return false;
  if (r.ph < 0 || r.ph >= p.P) {
    flags |= MSA_DEVERR_PHYS_RANGE;
    return false;
  }
  phys = r.ph;
  return true;
}

// Inclusive prefix over the 64 lanes of a wavefront with DPP (no LDS round
// trips): row shifts by 1, 2, 4, 8 scan each 16-lane row, then lane 15 is
// folded into rows 1 and 3 and lane 31 into rows 2 and 3.  Lanes a shift
// leaves without a source take the identity.
template <typename Op>
__device__ __forceinline__ int dpp_scan(int x, int ident, Op op) {
  x = op(x, __builtin_amdgcn_update_dpp(ident, x, 0x111, 0xf, 0xf, false));  // row_shr:1
  x = op(x, __builtin_amdgcn_update_dpp(ident, x, 0x112, 0xf, 0xf, false));  // row_shr:2
  x = op(x, __builtin_amdgcn_update_dpp(ident, x, 0x114, 0xf, 0xf, false));  // row_shr:4
  x = op(x, __builtin_amdgcn_update_dpp(ident, x, 0x118, 0xf, 0xf, false));  // row_shr:8
  x = op(x, __builtin_amdgcn_update_dpp(ident, x, 0x142, 0xa, 0xf, false));  // row_bcast:15
  x = op(x, __builtin_amdgcn_update_dpp(ident, x, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return x;
}
struct AddOp {
  __device__ int operator()(int a, int b) const { return a + b; }
};
struct OrOp {
  __device__ int operator()(int a, int b) const { return a | b; }
};
struct MaxOp {
  __device__ int operator()(int a, int b) const { return max(a, b); }
};

// workgroup sum of x and OR of y, both returned to every thread (red: two
// ints per wavefront of LDS)
__device__ __forceinline__ void block_sum_or(int x, int y, int* red, int& sum, int& any) {
  x = __builtin_amdgcn_readlane(dpp_scan(x, 0, AddOp()), kWave - 1);
  y = __builtin_amdgcn_readlane(dpp_scan(y, 0, OrOp()), kWave - 1);
  constexpr int nw = kPlanThreads / kWave;
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) {
    red[w] = x;
    red[nw + w] = y;
  }
  __syncthreads();
  sum = 0;
  any = 0;
#pragma unroll
  for (int i = 0; i < nw; ++i) {
    sum += red[i];
    any |= red[nw + i];
  }
}

__global__ void __launch_bounds__(kPlanThreads) plan_count_kernel(PlanParams p) {
  __shared__ int red[2 * (kPlanThreads / kWave)];
  const int b = blockIdx.x;
  int flags = 0;
  const SeqView v = seq_view(p, b, flags);
  int starts = 0;
  // the raw loads come before the test against nb, so the first ones go out
  // together with the ctx_len load
  for (int l = threadIdx.x; l < p.max_blocks; l += kPlanThreads) {
    const Raw r = load_raw(p, v, l), rp = load_raw(p, v, l - 1);
    if (l >= v.nb) break;
    int32_t ph = 0, pp = 0;
    if (live(p, v, l, r, ph, flags)) {
      int dummy = 0;  // the previous block's flags are counted by its own thread
      const bool cont = live(p, v, l - 1, rp, pp, dummy) && pp + 1 == ph;
      starts += cont ? 0 : 1;
    }
  }
  int total, f;
  block_sum_or(starts, flags, red, total, f);
  if (threadIdx.x == 0) {
    p.ws[b] = total;
    p.ws[p.B + b] = f;
  }
}

// Inclusive block scan of three values: two sums and a max.
struct Scan3 {
  int a, t, m;
};

__device__ __forceinline__ Scan3 block_exclusive_scan3(Scan3 v, Scan3* lds, Scan3& total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  Scan3 inc;
  inc.a = dpp_scan(v.a, 0, AddOp());
  inc.t = dpp_scan(v.t, 0, AddOp());
  inc.m = dpp_scan(v.m, -1, MaxOp());
  __syncthreads();
  if (lane == kWave - 1) lds[w] = inc;
  __syncthreads();
  Scan3 pre = {0, 0, -1};
  total = {0, 0, -1};
  for (int i = 0; i < kPlanThreads / kWave; ++i) {
    const Scan3 s = lds[i];
    if (i < w) {
      pre.a += s.a;
      pre.t += s.t;
      pre.m = max(pre.m, s.m);
    }
    total.a += s.a;
    total.t += s.t;
    total.m = max(total.m, s.m);
  }
  // exclusive = prefix of earlier waves + inclusive within wave - own value;
  // the max part is kept inclusive-of-earlier-lanes only.
  Scan3 ex;
  ex.a = pre.a + inc.a - v.a;
  ex.t = pre.t + inc.t - v.t;
  const int prev_m = __shfl_up(inc.m, 1);
  ex.m = max(pre.m, lane > 0 ? prev_m : -1);
  return ex;
}

__global__ void __launch_bounds__(kPlanThreads) plan_write_kernel(PlanParams p) {
  __shared__ int red[2 * (kPlanThreads / kWave)];
  __shared__ Scan3 scan_lds[kPlanThreads / kWave];
  const int b = blockIdx.x;

  // this thread's first blocks (and their neighbours): loaded before the
  // offset reduction below, so the two memory round trips overlap
  int dummy = 0;  // flags were gathered by the count pass
  const SeqView v = seq_view(p, b, dummy);
  Raw r0[kPerThread + 2];
#pragma unroll
  for (int k = 0; k < kPerThread + 2; ++k)
    r0[k] = load_raw(p, v, threadIdx.x * kPerThread - 1 + k);

  // offset of this sequence's records: from the scan launch, or summed here
  // (workgroup 0 then also publishes the totals)
  int off;
  if (p.scanned) {
    off = p.ws[2 * p.B + b];
  } else {
    int before = 0, all = 0, fl = 0;
    for (int i = threadIdx.x; i < p.B; i += kPlanThreads) {
      const int c = p.ws[i];
      if (i < b) before += c;
      all += c;
      fl |= p.ws[p.B + i];
    }
    int unused;
    block_sum_or(before, 0, red, off, unused);
    const int count_b = p.ws[b];
    if (threadIdx.x == 0) p.indptr[b + 1] = min(off + count_b, p.cap);
    if (b == 0) {
      int total, flags;
      block_sum_or(all, fl, red, total, flags);
      if (threadIdx.x == 0) {
        p.indptr[0] = 0;
        p.dev_error[0] = flags | (total > p.cap ? MSA_DEVERR_CAPACITY : 0);
      }
    }
  }

  Scan3 carry = {0, 0, -1};
  for (int base = 0; base < v.nb; base += kChunk) {
    const int l0 = base + threadIdx.x * kPerThread;
    Raw r[kPerThread + 2];  // blocks l0-1 .. l0+kPerThread
#pragma unroll
    for (int k = 0; k < kPerThread + 2; ++k) r[k] = base == 0 ? r0[k] : load_raw(p, v, l0 - 1 + k);
    bool a[kPerThread];
    int32_t ph[kPerThread];
    int tok[kPerThread];
    bool st[kPerThread];
    int32_t prev_ph = 0;
    bool prev_a = live(p, v, l0 - 1, r[0], prev_ph, dummy);
    Scan3 mine = {0, 0, -1};
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      const int l = l0 + k;
      ph[k] = 0;
      a[k] = live(p, v, l, r[k + 1], ph[k], dummy);
      st[k] = a[k] && !(prev_a && prev_ph + 1 == ph[k]);
      tok[k] = a[k] ? min(p.bs, v.n_tok - l * p.bs) : 0;
      mine.a += st[k] ? 1 : 0;
      mine.t += tok[k];
      if (st[k]) mine.m = l;
      prev_a = a[k];
      prev_ph = ph[k];
    }
    int32_t next_ph = 0;
    const bool next_a = live(p, v, l0 + kPerThread, r[kPerThread + 1], next_ph, dummy);

    Scan3 total;
    const Scan3 ex = block_exclusive_scan3(mine, scan_lds, total);
    int run_cnt = carry.a + ex.a;
    int run_tok = carry.t + ex.t;
    int run_start = max(carry.m, ex.m);
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      run_cnt += st[k] ? 1 : 0;
      run_tok += tok[k];
      if (st[k]) run_start = l0 + k;
      if (!a[k]) continue;
      const bool nxt_a = (k + 1 < kPerThread) ? a[k + 1] : next_a;
      const int32_t nxt_ph = (k + 1 < kPerThread) ? ph[k + 1] : next_ph;
      const bool ends = !(nxt_a && nxt_ph == ph[k] + 1);
      if (!ends) continue;
      const int l = l0 + k;
      const int nblk = l - run_start + 1;
      const int ntok = (nblk - 1) * p.bs + tok[k];
      const int rec = off + run_cnt - 1;
      if (rec < p.cap) {
        msa_segment s;
        s.seq = b;
        s.logical_block = run_start;
        s.phys_block = ph[k] - (nblk - 1);
        s.num_blocks = nblk;
        s.num_tokens = ntok;
        s.alive_token_start = run_tok - ntok;
        p.segs[rec] = s;
      }
    }
    carry.a += total.a;
    carry.t += total.t;
    carry.m = max(carry.m, total.m);
    __syncthreads();
  }
}

// One workgroup: exclusive prefix of the B segment counts.  Thread t owns the
// contiguous sequences [t*per, t*per + per); its local sums are scanned
// across the workgroup, then it writes its sequences' record offsets
// (unclamped, for the write pass), seg_indptr (clamped to the capacity) and,
// from thread 0, the error word.
__global__ void __launch_bounds__(kScanThreads) plan_scan_kernel(PlanParams p) {
  __shared__ int wsum[kScanThreads / kWave];
  __shared__ int wor[kScanThreads / kWave];
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const int per = (p.B + kScanThreads - 1) / kScanThreads;
  const int lo = min(p.B, int(threadIdx.x) * per), hi = min(p.B, lo + per);
  int sum = 0, fl = 0;
  for (int i = lo; i < hi; ++i) {
    sum += p.ws[i];
    fl |= p.ws[p.B + i];
  }
  int inc = sum;
  for (int o = 1; o < kWave; o <<= 1) {
    const int t = __shfl_up(inc, o);
    if (lane >= o) inc += t;
  }
  int wfl = fl;
  for (int o = 32; o > 0; o >>= 1) wfl |= __shfl_xor(wfl, o);
  if (lane == kWave - 1) wsum[w] = inc;
  if (lane == 0) wor[w] = wfl;
  __syncthreads();
  int run = inc - sum, total = 0, flags = 0;
  for (int i = 0; i < kScanThreads / kWave; ++i) {
    if (i < w) run += wsum[i];
    total += wsum[i];
    flags |= wor[i];
  }
  for (int i = lo; i < hi; ++i) {
    p.ws[2 * p.B + i] = run;
    run += p.ws[i];
    p.indptr[i + 1] = min(run, p.cap);
  }
  if (threadIdx.x == 0) {
    p.indptr[0] = 0;
    p.dev_error[0] = flags | (total > p.cap ? MSA_DEVERR_CAPACITY : 0);
  }
}

}  // namespace

bool plan_uses_scan(int32_t B) { return B > kDirectMaxB; }

hipError_t launch_plan(const PlanParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(plan_count_kernel, dim3(p.B), dim3(kPlanThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.scanned) {
    hipLaunchKernelGGL(plan_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(plan_write_kernel, dim3(p.B), dim3(kPlanThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace msa
