// a2 + a4: MSA chunked prefill over the alive-token stream of a segment plan.
//
// multi_segment_attention for a chunk of query rows (P1, "Core method 1:
// MSA" pseudocode; P1 "3. 自适应分块调度器": prefill runs in chunks whose
// KV is already in the pool).  Row i of sequence b sits at logical position
// q_pos0[b] + i and sees the alive keys at logical positions <= its own.
// This is a dense contraction, so QK^T and PV run on bf16 MFMA
// (v_mfma_f32_32x32x16_bf16) with fp32 accumulation.
//
// Workgroup = (query-position tile, KV head g, sequence b [, split s]),
// eight wavefronts.  The G query heads of KV head g are stacked: each
// wavefront owns one 32-row tile (one head, 32 consecutive positions), so
// every K/V tile staged in LDS is used by all G heads (GQA reuse) and by
// all 256/G positions of the workgroup.
//
// Per 64-key tile and wavefront (one lane = one query row throughout):
//   S^T[key][row] = K[key][:] . Q[row][:]     A = K from LDS (operand-order
//                                             DMA units), B = Q in VGPRs
//   online softmax over the lane's 32 keys + the other half-wave's 32
//   O^T[d][row] += V^T[d][key] . P^T[key][row] A = V^T read from the V tile
//                                             with the gfx950 transpose load
//                                             (ds_read_b64_tr_b16), B = P in
//                                             VGPRs: exactly the lane's own S
//                                             accumulators rounded to bf16
// Keys come from the sequence's segments in logical order: the workgroup
// expands its segments into per-block (physical offset, logical id, rows)
// lists in LDS, 256 blocks (64 tiles) at a time.  Tiles reach LDS by DMA
// (buffer_load ... lds) through per-block buffer descriptors whose
// num_records covers only the rows that exist, so missing blocks and padding
// rows past ctx_len land as zeros (and are masked); tiles straddling the
// causal diagonal are masked per element by logical position.
//
// Schedule: wavefronts w and w+4 share a SIMD, and one wavefront cannot
// overlap its own exponentials with its own MFMAs, while two wavefronts
// overlap them almost fully.  So the two halves of the workgroup alternate:
// while wavefronts 0-3 run the matrix half of a step (QK of the next tile,
// PV of this one), wavefronts 4-7 run the softmax half, and the other way
// round in the next half-step; a barrier ends every half-step.  The lone
// matrix-half wavefront of a SIMD is kept fed by reading half of its V
// operands during its preceding softmax half.  Four K/V stages in LDS.
#include "msa_internal.h"

namespace msa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kD = 128;            // head dim built
constexpr int kRow = kD * 2;       // bytes per K/V row of one head (bf16)
constexpr int kBlk = 16;           // tokens per block
constexpr int kTK = 64;            // keys per tile (4 blocks)
constexpr int kTileBytes = kTK * kRow;  // one K or V tile in LDS (16 KB)
constexpr int kUnit = 1024;             // one LDS DMA unit: 16 keys of a block x 64 B of d
constexpr int kStages = 4;              // K and V tiles resident or in flight
constexpr int kChunkBlocks = 256;  // blocks expanded into LDS at a time
constexpr int kMaxSplitBlocks = 1 << 20;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr int kBufferFlags = 0x00020000;
constexpr int kXcds = 8;  // accelerator complex dies on MI355X, one L2 each

// Eight wavefronts per workgroup (two per SIMD) and one workgroup per CU:
// every K/V tile staged in LDS feeds 8 x 32 query rows, one 32-row tile per
// wavefront.
template <int G>
struct PGeo {
  static constexpr int WAVES = 8;
  static constexpr int THREADS = WAVES * kWave;
  static constexpr int NPOS = 256 / G;          // query positions per workgroup
  static constexpr int UPW = 16 / WAVES;        // DMA units of a K (and a V) tile per wavefront
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), kBufferFlags);
}
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 x) { return __builtin_bit_cast(bf16x8_t, x); }

// Wavefront-wide LDS DMA (gfx950 buffer_load_dwordx4 ... lds): lane i loads
// 16 bytes at byte offset voff of the buffer and the data lands in LDS at
// lds_addr + 16*i, without passing through VGPRs.  Lanes outside the
// descriptor's range write zeros.  Completion is counted by vmcnt; the
// compiler does not track these, so the tile loop waits for them itself.
// The LDS address goes through M0, which the compiler treats as reserved
// (it warns that the clobber is ignored): nothing else in this kernel uses
// M0 -- in the generated code every M0 write is one of these.
__device__ __forceinline__ void dma16(u32x4_t rsrc, uint32_t lds_addr, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(lds_addr), "v"(voff), "s"(rsrc) : "memory", "m0");
}
// LDS byte address of a pointer into __shared__ memory
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return uint32_t(size_t((const __attribute__((address_space(3))) uint8_t*)(p)));
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));
// gfx950 transpose LDS load: within each 16-lane group, lane i receives
// element i%4 of the 8-byte words addressed by lanes i/4, i/4+4, i/4+8 and
// i/4+12 of the group
__device__ __forceinline__ uint2 ds_read_tr16(const uint8_t* lds_ptr) {
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4_t*)(lds_ptr));
  return __builtin_bit_cast(uint2, v);
}

// max of x over lanes l and l ^ 32: gfx950's v_permlane32_swap exchanges the
// two halves of the wavefront in one VALU instruction, keeping the LDS
// permute unit's latency out of the per-tile softmax chain
__device__ __forceinline__ float max_halves(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, uint32_t(r[0])), __builtin_bit_cast(float, uint32_t(r[1])));
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Largest i in [lo, hi) with segs[i].alive_token_start <= x (segs[lo] does).
template <int THREADS>
__device__ __forceinline__ int wg_search_segment(const msa_segment* segs, int lo, int hi, int x) {
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

template <int G>
__global__ void __launch_bounds__((PGeo<G>::THREADS), (PGeo<G>::WAVES / 4))
    prefill_kernel(PrefillParams p) {
  using PG = PGeo<G>;
  constexpr int RT = 1;  // 32-row tiles per wavefront
  constexpr int THREADS = PG::THREADS, NPOS = PG::NPOS;

  // K and V tiles in MFMA-operand order (see the DMA unit layout below),
  // four stages each: K(k+1) and V(k) being read by the two halves of the
  // workgroup, the later tiles landing or in flight
  __shared__ __align__(16) uint8_t k_lds[kStages][kTileBytes];
  __shared__ __align__(16) uint8_t v_lds[kStages][kTileBytes];
  __shared__ int32_t blk_rows[kChunkBlocks];  // rows present (0 = block missing)
  __shared__ int32_t blk_lpos[kChunkBlocks];  // logical block id
  __shared__ uint2 blk_off[kChunkBlocks];     // byte offset of the block in a pool (64-bit)
  // segment staging for the chunk expansion; it only lives between chunks,
  // when no K tile is in LDS and no DMA is in flight, so it shares the
  // second K buffer
  static_assert(4 * (kChunkBlocks + 1) * sizeof(int32_t) <= sizeof(k_lds[1]), "staging");
  int32_t* st_start = reinterpret_cast<int32_t*>(&k_lds[1][0]);
  int32_t* st_phys = st_start + (kChunkBlocks + 1);
  int32_t* st_nblk = st_phys + (kChunkBlocks + 1);
  int32_t* st_lblk = st_nblk + (kChunkBlocks + 1);

  // XCD-aware order: consecutive workgroup ids go round-robin to the 8 XCDs
  // (each with its own L2).  Remap so that the workgroups one XCD receives
  // are whole runs of position tiles of the same (sequence, KV head, split):
  // they stream the same K/V tiles, which then hit in that XCD's L2.
  int ptile, g, bz;
  {
    const int gx = gridDim.x, gy = gridDim.y;
    const int n = gx * gy * gridDim.z;
    const int n8 = n / kXcds * kXcds;
    const int lin = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
    const int r = lin < n8 ? (lin % kXcds) * (n8 / kXcds) + lin / kXcds : lin;
    ptile = r % gx;
    g = (r / gx) % gy;
    bz = r / (gx * gy);
  }
  const int b = bz / p.S, s = bz % p.S;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int half = lane / 32, lr = lane % 32;
  const int C = p.C;
  const int p0 = ptile * NPOS;        // first position (row index in the chunk)
  const int q0 = p.q_pos0[b];
  // the wavefront's RT row tiles: global tile index w*RT + r -> (head, 32
  // consecutive positions); a lane owns one row of each
  int pt[RT], h[RT], my_row[RT], my_qpos[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const int rt = w * RT + r;
    pt[r] = rt / G;                   // 32-position sub-tile
    h[r] = g * G + rt % G;            // query head
    my_row[r] = p0 + pt[r] * 32 + lr;  // this lane's row in the chunk
    my_qpos[r] = q0 + my_row[r];      // its logical position
  }
  const int wg_qmin = q0 + p0;
  const int wg_qmax = q0 + min(p0 + NPOS, C) - 1;

  // ---- this split's alive-block range -----------------------------------
  const int s0 = p.indptr[b], s1 = p.indptr[b + 1];
  int A = 0;
  if (s1 > s0) {
    const msa_segment last = p.segs[s1 - 1];
    A = last.alive_token_start + last.num_tokens;
  }
  const int T = p.split_blocks;
  // more alive tokens than max_ctx_len promised: cut at the grid, reported
  // once per sequence
  const int nAB_all = (A + kBlk - 1) / kBlk;
  const int nAB = min(nAB_all, p.S * T);
  if (nAB_all > nAB && s == 0 && g == 0 && ptile == 0 && tid == 0 && p.dev_error)
    atomicOr(p.dev_error, MSA_DEVERR_TRUNCATED);
  const int Sb = (nAB + T - 1) / T;
  // a split past this sequence's keys has nothing to contribute (split 0 of
  // a sequence without keys still writes O = 0, LSE = -inf below)
  if (s > 0 && s >= Sb) return;
  // the sequence's Sb splits share its nAB blocks evenly (each <= T blocks);
  // a sequence without alive keys (Sb = 0) has an empty key range
  const int j_begin = Sb > 0 ? int(int64_t(s) * nAB / Sb) : 0;
  const int j_end = Sb > 0 ? int(int64_t(s + 1) * nAB / Sb) : 0;
  const int last_tokens = min(kBlk, A - kBlk * (nAB - 1));

  // ---- Q of this lane's row into MFMA B-operand registers ----------------
  // rows past the chunk read as zero (descriptor covers only existing rows)
  uint4 qop[RT][kD / 16];
  {
    const size_t row_bytes = size_t(p.Hq) * kRow;
    const int nrows = max(0, min(NPOS, C - p0));
    const char* qb = static_cast<const char*>(p.q) + (size_t(b) * C + p0) * row_bytes;
    const __amdgpu_buffer_rsrc_t qr = rsrc(qb, uint32_t(nrows * row_bytes));
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const uint32_t off = uint32_t((pt[r] * 32 + lr) * row_bytes + size_t(h[r]) * kRow + half * 16);
#pragma unroll
      for (int k = 0; k < kD / 16; ++k) qop[r][k] = bload16(qr, off + k * 32);
    }
    // consume Q here: the compiler's wait for these loads then sits before
    // the first tile DMA instead of inside the tile pipeline, where it would
    // also wait for DMAs still in flight
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int k = 0; k < kD / 16; ++k)
        asm volatile("" ::"v"(qop[r][k].x), "v"(qop[r][k].y), "v"(qop[r][k].z), "v"(qop[r][k].w));
  }

  f32x16_t acc_o[RT][kD / 32];
  float m_run[RT], l_lane[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
#pragma unroll
    for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc_o[r][dt][i] = 0.f;
    m_run[r] = -INFINITY;
    l_lane[r] = 0.f;
  }

  // slot, block and KV-head strides of the token-major [P, bs, Hkv, D] or
  // head-major [P, Hkv, bs, D] pool
  const size_t tok_stride = p.head_major ? size_t(kRow) : size_t(p.Hkv) * kRow;
  const size_t blk_stride = size_t(p.Hkv) * kRow * kBlk;
  const size_t head_off = p.head_major ? size_t(g) * kRow * kBlk : size_t(g) * kRow;
  const char* kbase = static_cast<const char*>(p.k_pool) + head_off;
  const char* vbase = static_cast<const char*>(p.v_pool) + head_off;

  // ---- LDS tile layout --------------------------------------------------
  // A tile (64 keys = 4 blocks) is 16 DMA units of 1 KB; unit u covers block
  // u/4 (16 keys) and a 64-byte quarter u%4 of the head dimension.  The
  // bytes of a unit are placed so that the MFMA operand reads are lane-linear
  // (conflict-free, immediate offsets):
  //   K unit (block b, quarter c): slot i holds key i%16 of block b, 16-B d
  //     chunk 4c + i/16.  The A operand of QK step (kb2, k) for lane l is key
  //     32 kb2 + l%32, d chunk 2k + l/32, i.e. unit (2 kb2 + bit4(l), k/2),
  //     slot l%16 + 16 (2 (k%2) + bit5(l)).
  //   V unit (block t, quarter dt): two 512-byte halves h, one per
  //     transpose read; 8-byte slot L of half h holds key 8h + 4(L/32) +
  //     (L%16)/4 of block t, d = 32 dt + 16((L/16)%2) + 4(L%4) .. +3, the word
  //     lane L of the read must point at.  DMA lane i writes slots 2(i%32)
  //     and 2(i%32)+1 of half i/32: 8 consecutive d of one key.
  // Wavefront w loads units UPW*w .. UPW*w+UPW-1 of both K and V, all from
  // block UPW*w/4; quarter q of a block adds 64 bytes to both global offsets.
  constexpr int UPW = PG::UPW;
  static_assert(UPW == 2, "DMA split: two units of each tile per wavefront");
  const int u0 = UPW * w, q0u = u0 % 4;
  const uint32_t k_voff0 = uint32_t((lane % 16) * tok_stride + (4 * q0u + lane / 16) * 16);
  const int vkey = 8 * (lane / 32) + 4 * ((lane % 32) / 16) + (lane % 8) / 2;
  const int vd = 16 * (((lane % 32) / 8) % 2) + 8 * (lane % 2);
  const uint32_t v_voff0 = uint32_t(vkey * tok_stride + 2 * (32 * q0u + vd));
  const uint32_t dma_dst = uint32_t(u0 * kUnit);
  // operand-read offsets of this lane
  const int k_lane_off = 4096 * ((lane >> 4) & 1) + 16 * (lane % 16) + 256 * (lane >> 5);
  const int v_lane_off = 8 * lane;

  bool done = false;
  for (int cb = j_begin; cb < j_end && !done; cb += kChunkBlocks) {
    const int nblk = min(kChunkBlocks, j_end - cb);
    // ---- expand the segments covering blocks [cb, cb+nblk) ---------------
    __syncthreads();  // previous chunk's lists are no longer read
    const int sf = wg_search_segment<THREADS>(p.segs, s0, s1, cb * kBlk);
    const int ns = min(nblk, s1 - sf);
    for (int i = tid; i < ns; i += THREADS) {
      const msa_segment sg = p.segs[sf + i];
      const bool in_pool = sg.phys_block >= 0 && sg.num_blocks >= 0 &&
                           int64_t(sg.phys_block) + sg.num_blocks <= p.P;
      st_start[i] = sg.alive_token_start / kBlk;
      st_phys[i] = in_pool ? sg.phys_block : -1;
      st_nblk[i] = in_pool ? sg.num_blocks : 0;
      st_lblk[i] = sg.logical_block;
    }
    __syncthreads();
    for (int jj = tid; jj < nblk; jj += THREADS) {
      const int j = cb + jj;
      int lo = 0, hi = ns;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (st_start[mid] <= j) lo = mid; else hi = mid;
      }
      const int off = j - st_start[lo];
      const bool ok = st_phys[lo] >= 0 && off >= 0 && off < st_nblk[lo];
      const uint64_t bo = ok ? uint64_t(st_phys[lo] + off) * blk_stride : 0;
      blk_off[jj] = make_uint2(uint32_t(bo), uint32_t(bo >> 32));
      blk_lpos[jj] = st_lblk[lo] + off;
      blk_rows[jj] = !ok ? 0 : (j == nAB - 1 ? last_tokens : kBlk);
    }
    __syncthreads();

    const int ntiles = (nblk + 3) / 4;
    // Each wavefront loads whole units of one block of every tile, so its
    // buffer descriptor is wave-uniform by construction.
    const int my_blk = u0 / 4;
    // Per-tile bookkeeping in registers, lane t <-> tile t of the chunk: the
    // pool offset and row count of the block this wavefront loads for tile
    // t (read back with v_readlane, no LDS round trip in the tile loop), and
    // two wave masks: tiles at or past the last row of the workgroup, and
    // tiles that need the per-element mask (padding rows or the diagonal).
    static_assert(kChunkBlocks == 4 * kWave, "one tile of the chunk per lane");
    uint32_t t_off_lo, t_off_hi;
    int t_rows;
    uint64_t past_mask, mask_mask;
    {
      const int jl = lane * 4 + my_blk;
      const bool in = jl < nblk;
      const uint2 off = blk_off[jl];
      t_off_lo = in ? off.x : 0u;
      t_off_hi = in ? off.y : 0u;
      t_rows = in ? blk_rows[jl] : 0;
      const int jt = lane * 4;
      bool full = jt + 3 < nblk;
      int lp_last = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int jj = min(jt + k, nblk - 1);
        full = full && blk_rows[jj] == kBlk;
        lp_last = blk_lpos[jj];
      }
      const bool past = lane >= ntiles || blk_lpos[min(jt, nblk - 1)] * kBlk > wg_qmax;
      const bool need = !full || lp_last * kBlk + kBlk - 1 > wg_qmin;
      past_mask = __builtin_amdgcn_ballot_w64(past);
      mask_mask = __builtin_amdgcn_ballot_w64(need);
    }
    // buffer descriptor of this wavefront's block of tile ti; tiles past the
    // chunk get an empty range, so their DMA writes zeros and reads nothing
    auto tile_desc = [&](const char* base, int ti) {
      const int tl = min(ti, kWave - 1);
      const uint32_t lo = __builtin_amdgcn_readlane(t_off_lo, tl);
      const uint32_t hi = __builtin_amdgcn_readlane(t_off_hi, tl);
      const int rows = ti < kWave ? __builtin_amdgcn_readlane(t_rows, tl) : 0;
      const uint64_t a = reinterpret_cast<uint64_t>(base) + ((uint64_t(hi) << 32) | lo);
      const u32x4_t r = {uint32_t(a), uint32_t(a >> 32) & 0xffffu, uint32_t(rows * tok_stride),
                         uint32_t(kBufferFlags)};
      return r;
    };
    // UPW DMAs each: this wavefront's units of the tile into stage ti % 3
    auto issue_k = [&](int ti) {
      const u32x4_t r = tile_desc(kbase, ti);
      const uint32_t dst = lds_addr(&k_lds[ti % kStages][0]) + dma_dst;
#pragma unroll
      for (int i = 0; i < UPW; ++i) dma16(r, dst + i * kUnit, k_voff0 + 64 * i);
    };
    auto issue_v = [&](int ti) {
      const u32x4_t r = tile_desc(vbase, ti);
      const uint32_t dst = lds_addr(&v_lds[ti % kStages][0]) + dma_dst;
#pragma unroll
      for (int i = 0; i < UPW; ++i) dma16(r, dst + i * kUnit, v_voff0 + 64 * i);
    };
    // the DMAs of this wavefront's last two loop iterations (2 x 2*UPW) may
    // stay in flight; everything older has landed in LDS
    auto wait_older = [] { asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); };
    // only the DMAs of this wavefront's last loop iteration may stay in flight
    auto wait_last = [] { asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); };
    // The matrix half of a step: S^T = K Q^T for the 2 x 32 keys of the K
    // tile at kt (QK of the next tile) and O^T += V^T P^T for the V tile at
    // vt0 (PV of this tile).  The first eight PV MFMAs use the V operands
    // the softmax half already read (vpre); their 256+ cycles cover the K
    // operand reads, which then run two MFMAs ahead, followed by the other
    // half of the V reads.  One wavefront per SIMD issues these MFMAs while
    // the other runs its softmax, so this half runs at raised priority.
    auto mphase = [&](const uint8_t* kt, const uint8_t* vt0, f32x16_t* sacc, const uint4* pp,
                      const uint2* vpre) {
      __builtin_amdgcn_s_setprio(1);
      uint4 ka[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int kb2 = j / 8, k = j % 8;
        ka[j] = *reinterpret_cast<const uint4*>(kt + k_lane_off + 8192 * kb2 + 1024 * (k / 2) + 512 * (k % 2));
      }
      uint2 va[16];
      const uint8_t* vt = vt0 + v_lane_off;
#pragma unroll
      for (int j = 8; j < 16; ++j) {
        const int t = j / 4, dt = j % 4;
        const uint8_t* vb0 = vt + (t * 4 + dt) * kUnit;
        va[2 * (j - 8)] = ds_read_tr16(vb0);
        va[2 * (j - 8) + 1] = ds_read_tr16(vb0 + kUnit / 2);
      }
      // PV steps 0..7 on the V operands read during the softmax half
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int t = j / 4, dt = j % 4;
        const uint4 a = make_uint4(vpre[2 * j].x, vpre[2 * j].y, vpre[2 * j + 1].x, vpre[2 * j + 1].y);
        acc_o[0][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(pp[t]), acc_o[0][dt], 0, 0, 0);
      }
      const f32x16_t zero = {};
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int kb2 = j / 8, k = j % 8;
        sacc[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka[j]), as_bf16x8(qop[0][k]),
                                                            k == 0 ? zero : sacc[kb2], 0, 0, 0);
      }
#pragma unroll
      for (int j = 8; j < 16; ++j) {
        const int t = j / 4, dt = j % 4;
        const uint4 a = make_uint4(va[2 * (j - 8)].x, va[2 * (j - 8)].y, va[2 * (j - 8) + 1].x, va[2 * (j - 8) + 1].y);
        acc_o[0][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(pp[t]), acc_o[0][dt], 0, 0, 0);
      }
      // order: 2 K reads; then each of 30 MFMAs (PV 0..7, QK 0..15, PV 8..13)
      // followed by one read (K 2..15, then the 16 halves of V steps 8..15);
      // PV 14..15
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
      for (int i = 0; i < 30; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_s_setprio(0);
    };

    // The softmax half of a step for tile j: the V operands of PV steps
    // 0..7 of tile j are read into vpre first (the LDS is otherwise idle for
    // this wavefront here), then mask (padding or diagonal tiles), running
    // max with lazy rescaling, weights rounded to bf16 into the P operand,
    // row sums.
    auto softmax = [&](int j, f32x16_t* sc, uint4* pp, uint2* vpre) {
      {
        const uint8_t* vt = &v_lds[j % kStages][0] + v_lane_off;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int t = i / 4, dt = i % 4;
          const uint8_t* vb0 = vt + (t * 4 + dt) * kUnit;
          vpre[2 * i] = ds_read_tr16(vb0);
          vpre[2 * i + 1] = ds_read_tr16(vb0 + kUnit / 2);
        }
      }
      if ((mask_mask >> j) & 1) {
        int lp[4], rw[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int jj = j * 4 + k;
          lp[k] = jj < nblk ? blk_lpos[jj] : 0x07ffffff;
          rw[k] = jj < nblk ? blk_rows[jj] : 0;
        }
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kb2 * 32 + 8 * (i / 4) + 4 * half + (i % 4);
            const int kblk = key / kBlk, slot = key % kBlk;
            const int kpos = lp[kblk] * kBlk + slot;
            const bool vis = slot < rw[kblk] && kpos <= my_qpos[0];
            sc[kb2][i] = vis ? sc[kb2][i] : -INFINITY;
          }
      }
      const float c = p.scale_log2;
      float mx = -INFINITY;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[kb2][i]);
      mx = max_halves(mx);
      // Lazy rescaling: a row keeps its reference max m_run until the true
      // max exceeds it by more than 2^8 in the exponent; the weights are then
      // at most 256 (harmless for fp32 sums and for bf16's relative
      // precision) and the accumulator rescale is skipped in almost every
      // tile.  The LSE stays exact: it is m_run*scale + log2(sum).
      const bool bump = (mx - m_run[0]) * c > 8.f;  // true on the first visible key
      const float m_use = bump ? mx : m_run[0];
      const float nm = m_use == -INFINITY ? 0.f : -m_use * c;
      const float alpha = (m_use == m_run[0]) ? 1.f : __builtin_amdgcn_exp2f((m_run[0] - m_use) * c);
      if (__builtin_amdgcn_ballot_w64(bump) != 0) {
#pragma unroll
        for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc_o[0][dt][i] *= alpha;
      }
      m_run[0] = m_use;
      // four partial sums per row keep the additions out of one long chain
      float lsum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pv[e] = __builtin_amdgcn_exp2f(fmaf(sc[t / 2][8 * (t % 2) + e], c, nm));
          lsum[e % 4] += pv[e];
        }
        pp[t] = make_uint4(cvt_pk_bf16(pv[0], pv[1]), cvt_pk_bf16(pv[2], pv[3]),
                           cvt_pk_bf16(pv[4], pv[5]), cvt_pk_bf16(pv[6], pv[7]));
      }
      l_lane[0] = l_lane[0] * alpha + ((lsum[0] + lsum[1]) + (lsum[2] + lsum[3]));
    };

    // Ping-pong schedule.  Wavefronts w and w+4 share a SIMD; group A
    // (w < 4) and group B (w >= 4) alternate between the matrix half of a
    // step (QK of tile k+1 and PV of tile k, MFMA only) and the softmax half
    // (VALU only), so that each SIMD's matrix core runs one wavefront's
    // MFMAs while its VALU runs the other's exponentials.  A barrier ends
    // every half-step; B runs the same loop as A one half-step later:
    //   half-step 2k:   A: QK(k+1) + PV(k)    B: softmax(k)
    //   half-step 2k+1: A: softmax(k+1)       B: QK(k+1) + PV(k)
    // K(k+1) and V(k) are read in half-steps 2k and 2k+1, and half of V(k+1)
    // in advance by A's softmax half in 2k+1.  Iteration k sends the DMAs of
    // K(k+4) and V(k+3) into the stages of K(k) and V(k-1), last read in
    // half-step 2k-1 (A issues them at the start of 2k, B of 2k+1).  Every
    // tile needs all eight wavefronts' DMA units, so the waits are set by
    // the other group's barriers: before the barrier that ends its matrix
    // half a wavefront waits for all but its last two iterations' DMAs,
    // before the one that ends its softmax half for all but its last one.
    // Then K(k+1) and V(k) (iteration k-3) have landed for every wavefront
    // before half-step 2k, and V(k+1) (iteration k-2) before 2k+1: B passes
    // that barrier at the end of its iteration k-1, A in the middle of its
    // iteration k.  Tiles past the workgroup's last row are never processed.
    const int n_eff = past_mask == 0 ? kWave : min(ntiles, int(__builtin_ctzll(past_mask)));
    if (n_eff == 0) {
      done = true;
      continue;
    }
    done = n_eff < ntiles;
    const bool grp_b = w >= 4;
    issue_k(0);
    issue_v(0);
    issue_k(1);
    issue_k(2);
    issue_v(1);
    issue_k(3);
    issue_v(2);
    wait_older();  // K(0), V(0), K(1) have landed
    __syncthreads();
    f32x16_t sc[2];
    uint4 pp[4];
    uint2 vpre[16];
    {
      const f32x16_t zero = {};
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int k = 0; k < kD / 16; ++k) {
          const uint4 a = *reinterpret_cast<const uint4*>(
              &k_lds[0][0] + k_lane_off + 8192 * kb2 + 1024 * (k / 2) + 512 * (k % 2));
          sc[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(qop[0][k]),
                                                            k == 0 ? zero : sc[kb2], 0, 0, 0);
        }
    }
    // A: softmax(0), barrier.  B: barrier, softmax(0), barrier.  Every
    // wavefront has read K(0) before the first DMA rewrites its stage.
    if (grp_b) __syncthreads();
    softmax(0, sc, pp, vpre);
    __builtin_amdgcn_sched_barrier(0);
    wait_last();  // B: the prologue's V(1), which A reads in half-step 1
    __syncthreads();
    for (int k = 0; k < n_eff; ++k) {
      issue_k(k + 4);
      issue_v(k + 3);
      mphase(&k_lds[(k + 1) % kStages][0], &v_lds[k % kStages][0], sc, pp, vpre);
      // keep the matrix half's MFMAs on this side of the barrier
      __builtin_amdgcn_sched_barrier(0);
      wait_older();
      __syncthreads();
      if (k + 1 < n_eff) softmax(k + 1, sc, pp, vpre);
      __builtin_amdgcn_sched_barrier(0);
      wait_last();
      __syncthreads();
    }
    // A ends one half-step earlier: its last barrier pairs with B's last
    if (!grp_b) __syncthreads();
    // no DMA may still write into a stage (the next chunk's staging shares
    // one) once the workgroup leaves this chunk
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  // ---- finish: combine the two half-waves' sums, write O and LSE --------
  // the row index is rebuilt from the logical position the mask kept live
  // through the tile loop (an opaque copy stops the compiler from folding it
  // back to the original, which it would then keep live -- in scratch)
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    int qp = my_qpos[r];
    asm volatile("" : "+v"(qp));
    my_row[r] = qp - q0;
  }
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const float L = l_lane[r] + __shfl_xor(l_lane[r], 32);
    if (my_row[r] >= C) continue;
    if (Sb <= 1) {
      const bool ok = L > 0.f;
      const float inv = ok ? 1.f / L : 0.f;
      uint16_t* out = static_cast<uint16_t*>(p.out) + ((size_t(b) * C + my_row[r]) * p.Hq + h[r]) * kD;
#pragma unroll
      for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d = dt * 32 + 8 * i + 4 * half;
          uint2 v;
          v.x = cvt_pk_bf16(acc_o[r][dt][4 * i] * inv, acc_o[r][dt][4 * i + 1] * inv);
          v.y = cvt_pk_bf16(acc_o[r][dt][4 * i + 2] * inv, acc_o[r][dt][4 * i + 3] * inv);
          *reinterpret_cast<uint2*>(out + d) = v;
        }
      if (p.lse && half == 0)
        p.lse[(size_t(b) * C + my_row[r]) * p.Hq + h[r]] =
            ok ? (m_run[r] * p.scale_log2 + log2f(L)) * kLn2 : -INFINITY;
    } else {
      const size_t n = size_t(b) * p.S + s;
      const size_t row = (n * C + my_row[r]) * p.Hq + h[r];
      float* o = p.o_part + row * kD;
#pragma unroll
      for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d = dt * 32 + 8 * i + 4 * half;
          *reinterpret_cast<float4*>(o + d) = make_float4(acc_o[r][dt][4 * i], acc_o[r][dt][4 * i + 1],
                                                          acc_o[r][dt][4 * i + 2], acc_o[r][dt][4 * i + 3]);
        }
      if (half == 0) {
        p.m_part[row] = (L > 0.f) ? m_run[r] * p.scale_log2 * kLn2 : -INFINITY;
        p.l_part[row] = L;
      }
    }
  }
}

template <int G>
hipError_t launch_g(const PrefillParams& p, hipStream_t stream) {
  using PG = PGeo<G>;
  dim3 grid((p.C + PG::NPOS - 1) / PG::NPOS, p.Hkv, p.B * p.S);
  hipLaunchKernelGGL((prefill_kernel<G>), grid, dim3(PG::THREADS), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

bool prefill_supported(msa_dtype dtype, int32_t D, int32_t G) {
  // bf16 D 128 on the matrix cores (this file); the other pairs of {bf16,
  // f32} x {64, 128} on the generic kernel
  return (dtype == MSA_BF16 && D == kD && (G == 1 || G == 2 || G == 4 || G == 8)) ||
         generic_supported(dtype, D, G);
}

int32_t prefill_max_split_blocks() { return kMaxSplitBlocks; }

SplitPlan prefill_split(int32_t B, int32_t C, int32_t Hq, int32_t Hkv, int32_t max_ctx_len,
                        int32_t block_size, int32_t split_blocks) {
  SplitPlan sp;
  const int64_t nbm = (int64_t(max_ctx_len) + block_size - 1) / block_size;
  const int G = Hkv > 0 ? Hq / Hkv : 1;
  const int npos = 256 / (G > 0 ? G : 1);
  const int64_t wgs = int64_t((C + npos - 1) / npos) * Hkv * B;
  int64_t T = split_blocks;
  if (T <= 0) {
    // split the key stream only when the grid alone cannot fill the chip
    // (one workgroup per CU on 256 CUs); never below 64 blocks per split
    int64_t S = wgs >= 256 ? 1 : (256 + wgs - 1) / wgs;
    T = nbm > 0 ? (nbm + S - 1) / S : 1;
    if (T < 64) T = 64;
  }
  if (T < 1) T = 1;
  sp.split_blocks = int32_t(T > kMaxSplitBlocks ? kMaxSplitBlocks : T);
  sp.S = int32_t(nbm == 0 ? 1 : (nbm + sp.split_blocks - 1) / sp.split_blocks);
  if (sp.S < 1) sp.S = 1;
  return sp;
}

int32_t prefill_chunk_rows(int32_t B, int32_t Hq, int32_t Hkv, int32_t remaining,
                           int32_t max_rows, int32_t compute_units) {
  const int G = Hq / Hkv;
  const int64_t npos = 256 / G;  // query positions per workgroup
  const int64_t cus = compute_units > 0 ? compute_units : 256;
  const int64_t cap = min(int64_t(remaining), int64_t(max_rows));
  // smallest whole number of position tiles whose (tile, KV head, sequence)
  // workgroups cover every compute unit at one workgroup per unit; below it
  // the key stream has to be split (partials + merge), above it throughput
  // is flat while every chunk waits longer
  const int64_t per_tile = int64_t(Hkv) * B;
  const int64_t tiles = (cus + per_tile - 1) / per_tile;
  int64_t C = tiles * npos;
  if (C >= cap) return int32_t(cap);
  // a tail shorter than one position tile rides along with this chunk
  if (remaining - C < npos && remaining <= max_rows) return remaining;
  return int32_t(C);
}

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
  if (p.dtype != MSA_BF16 || p.D != kD) {
    GenericParams gp{};
    gp.q = p.q;
    gp.q_pos0 = p.q_pos0;
    gp.C = p.C;
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
  switch (p.Hq / p.Hkv) {
    case 1: return launch_g<1>(p, stream);
    case 2: return launch_g<2>(p, stream);
    case 4: return launch_g<4>(p, stream);
    case 8: return launch_g<8>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace msa
