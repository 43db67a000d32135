// Internal declarations shared by the HIP translation units of libmsa.
// Device helpers (bf16 conversion, wavefront reductions) and the launchers
// that the C ABI in api.hip calls after validating its arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/msa.h"

namespace msa {

constexpr int kWave = 64;  // CDNA wavefront width

// ---------------------------------------------------------------------------
// bf16 <-> f32 (bf16 is the upper half of an IEEE binary32)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16lo_to_f32(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// Round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return uint32_t(f32_to_bf16(lo)) | (uint32_t(f32_to_bf16(hi)) << 16);
}

// ---------------------------------------------------------------------------
// wavefront reductions (all lanes receive the result)
// ---------------------------------------------------------------------------
// Within a 16-lane row: DPP row rotations and quad permutes, fused into the
// ALU op by the compiler.  Across rows: ds_swizzle-free cross-lane moves via
// __shfl_xor (ds_bpermute).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int kDppQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;

__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f<kDppQuadXor1>(x));
  x = fmaxf(x, dpp_f<kDppQuadXor2>(x));
  x = fmaxf(x, dpp_f<kDppRowRor4>(x));
  x = fmaxf(x, dpp_f<kDppRowRor8>(x));
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
  x += dpp_f<kDppQuadXor1>(x);
  x += dpp_f<kDppQuadXor2>(x);
  x += dpp_f<kDppRowRor4>(x);
  x += dpp_f<kDppRowRor8>(x);
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

// ---------------------------------------------------------------------------
// launch parameter blocks
// ---------------------------------------------------------------------------
struct PlanParams {
  const int32_t* table;
  const uint8_t* alive;
  const int32_t* ctx_len;
  int32_t B, max_blocks, bs, P;
  msa_segment* segs;
  int32_t cap;
  int32_t* indptr;
  int32_t* dev_error;
  int32_t* ws;  // [3*B]: per-sequence segment counts, error flags, record offsets
  int32_t scanned;  // 1: a scan launch wrote the offsets, indptr and dev_error
};

struct DecodeParams {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  int32_t P;
  const msa_segment* segs;
  const int32_t* indptr;
  int32_t B, Hq, Hkv, D;
  int32_t head_major;    // pool layout: 0 = [P, bs, Hkv, D], 1 = [P, Hkv, bs, D]
  msa_dtype dtype;
  float scale_log2;      // softmax scale * log2(e)
  int32_t split_blocks;  // blocks per split
  int32_t S;             // splits per sequence in the grid
  int32_t kernel;        // msa_decode_kernel: automatic, vector or matrix-core kernel
  int32_t* dev_error;    // nullable: MSA_DEVERR_TRUNCATED is ORed in
  // block kernel (one workgroup per split streaming whole KV blocks)
  int32_t use_block;     // 1: decode_block_kernel over nwg workgroups
  int32_t nwg;           // its grid
  int32_t block_auto;    // 1: split length from the device rule, 0: split_blocks
  int32_t block_target;  // workgroups the device rule aims at
  int32_t block_parts;   // partials the workspace holds
  int32_t block_share;   // 1: common prefixes of sequences are streamed once per sub-group
  int32_t cap_blocks;    // alive blocks a sequence may use (S * split_blocks)
  int32_t* part_indptr;  // [B+1] first partial of each sequence (written by workgroup 0)
  void* out;
  float* lse;
  float* o_part;  // [B*S, Hq, D]
  float* m_part;  // [B*S, Hq]  natural-log units
  float* l_part;  // [B*S, Hq]
};

struct PrefillParams {
  const void* q;
  const int32_t* q_pos0;
  int32_t C;
  const void* k_pool;
  const void* v_pool;
  int32_t P;
  const msa_segment* segs;
  const int32_t* indptr;
  int32_t B, Hq, Hkv, D;
  msa_dtype dtype;       // bf16 D 128: the matrix-core kernel; else the generic kernel
  int32_t head_major;    // pool layout: 0 = [P, bs, Hkv, D], 1 = [P, Hkv, bs, D]
  float scale_log2;
  int32_t split_blocks;  // 0 = no split
  int32_t S;
  int32_t* dev_error;    // nullable: MSA_DEVERR_TRUNCATED is ORed in
  void* out;
  float* lse;
  float* o_part;  // [B*S, C, Hq, D]
  float* m_part;  // [B*S, C, Hq]
  float* l_part;
};

// the generic (vector-ALU, float32) kernel: decode is C = 1 with no q_pos0
struct GenericParams {
  const void* q;
  const int32_t* q_pos0;  // nullable: decode (every alive key is visible)
  int32_t C;
  const void* k_pool;
  const void* v_pool;
  int32_t P;
  const msa_segment* segs;
  const int32_t* indptr;
  int32_t B, Hq, Hkv, D;
  int32_t head_major;
  msa_dtype dtype;
  float scale_log2;
  int32_t split_blocks;
  int32_t S;
  int32_t* dev_error;
  void* out;
  float* lse;
  float* o_part;  // [B*S, C, Hq, D]
  float* m_part;  // [B*S, C, Hq]
  float* l_part;
};

struct GatherParams {
  const void* k_pool;
  const void* v_pool;
  int32_t P;
  const msa_segment* segs;
  const int32_t* indptr;
  int32_t B;
  int32_t blocks_per_seq;  // dense blocks reserved per sequence
  size_t block_bytes;      // bytes of one pool block (16 * Hkv * D * element size)
  void* dense_k;
  void* dense_v;
  msa_segment* dense_segs;  // [B]
  int32_t* dense_indptr;    // [B+1]
};

// Decode/prefill work split, shared by the workspace-size functions and the
// launches so both always agree.
struct SplitPlan {
  int32_t split_blocks;
  int32_t S;
};
SplitPlan decode_split(int32_t B, int32_t Hkv, int32_t max_ctx_len, int32_t block_size,
                       int32_t split_blocks);
SplitPlan prefill_split(int32_t B, int32_t C, int32_t Hq, int32_t Hkv, int32_t max_ctx_len,
                        int32_t block_size, int32_t split_blocks);

bool decode_supported(msa_dtype dtype, int32_t D, int32_t G);
bool decode_matrix_supported(msa_dtype dtype, int32_t D, int32_t G);
int32_t decode_max_split_blocks();
// block kernel: shapes it is built for, its split rule's target, its grid
// and partial capacity, and when it shares common prefixes
constexpr int kDecodeBlockMaxSeq = 512;
constexpr int kDecodeBlockMaxShareSeq = 256;
struct BlockSizes {
  int64_t items, parts;
};
bool decode_block_supported(msa_dtype dtype, int32_t D, int32_t Hkv, int32_t G, int32_t B);
int32_t decode_block_target(int32_t B);
BlockSizes decode_block_sizes(int32_t B, int32_t cap_blocks, int32_t split_blocks);
bool decode_block_shares(int32_t B);
int32_t prefill_max_split_blocks();
bool prefill_supported(msa_dtype dtype, int32_t D, int32_t G);
int32_t prefill_chunk_rows(int32_t B, int32_t Hq, int32_t Hkv, int32_t remaining,
                           int32_t max_rows, int32_t compute_units);

// true if the plan of B sequences takes the three-launch form (scan launch)
bool plan_uses_scan(int32_t B);
hipError_t launch_plan(const PlanParams& p, hipStream_t stream);
hipError_t launch_decode(const DecodeParams& p, hipStream_t stream);
hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream);
hipError_t launch_gather(const GatherParams& p, hipStream_t stream);
// (dtype, head_dim) pairs outside the specialised kernels: decode float32 D
// 128, prefill bfloat16 D 64 and float32 D 64 / 128
bool generic_supported(msa_dtype dtype, int32_t D, int32_t G);
hipError_t launch_generic(const GenericParams& p, hipStream_t stream);
// Merge of decode/prefill split partials; the partial count of each sequence
// is derived from the plan (same rule as the attention launch).
hipError_t launch_merge_from_plan(const float* o_part, const float* m_part, const float* l_part,
                                  const msa_segment* segs, const int32_t* indptr, int32_t B,
                                  int32_t R, int32_t H, int32_t D, int32_t S,
                                  int32_t split_blocks, msa_dtype out_dtype, void* out,
                                  float* lse, hipStream_t stream);
// Merge of caller-described partials (msa_merge_partials).
hipError_t launch_merge_indptr(const float* o_part, const float* m_part, const float* l_part,
                               const int32_t* part_indptr, int32_t B, int32_t R, int32_t H,
                               int32_t D, msa_dtype out_dtype, void* out, float* lse,
                               hipStream_t stream);
// Merge after the decode block kernel: partial ranges from its part_indptr;
// a sequence with one partial was written by the attention kernel itself.
// parts_per_seq: the expected partials per sequence (sets the group count).
hipError_t launch_merge_block(const float* o_part, const float* m_part, const float* l_part,
                              const int32_t* part_indptr, int32_t B, int32_t H, int32_t D,
                              int32_t parts_per_seq, msa_dtype out_dtype, void* out, float* lse,
                              hipStream_t stream);

// Number of alive tokens of sequence b according to the plan (device).
__device__ __forceinline__ int32_t plan_alive_tokens(const msa_segment* segs, const int32_t* indptr,
                                                     int32_t b) {
  const int32_t s0 = indptr[b], s1 = indptr[b + 1];
  if (s1 <= s0) return 0;
  const msa_segment last = segs[s1 - 1];
  return last.alive_token_start + last.num_tokens;
}

}  // namespace msa
