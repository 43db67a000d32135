// C ABI of libmsa: argument validation, workspace carving, launches.
// Every entry point checks what the host can check before it enqueues
// anything, and returns a negative msa_status on the first problem.
#include <math.h>
#include <stdint.h>

#include "msa_internal.h"

using namespace msa;

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct PartLayout {
  size_t o_off, m_off, l_off, total;
};

// partials for N splits, R rows, H heads, D dims: o [N,R,H,D], m and l [N,R,H]
inline PartLayout part_layout(int64_t N, int64_t R, int64_t H, int64_t D) {
  PartLayout L;
  L.o_off = 0;
  L.m_off = align_up(size_t(N * R * H * D) * sizeof(float));
  L.l_off = L.m_off + align_up(size_t(N * R * H) * sizeof(float));
  L.total = L.l_off + align_up(size_t(N * R * H) * sizeof(float));
  return L;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline int from_hip(hipError_t e) { return e == hipSuccess ? MSA_OK : MSA_ERR_DEVICE; }

// shape checks common to decode and prefill
int check_attn_shape(const void* q, const void* k_pool, const void* v_pool, int32_t P,
                     int32_t block_size, const msa_segment* segs, const int32_t* seg_indptr,
                     int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t max_ctx_len,
                     msa_dtype dtype, float scale, int32_t split_blocks, const void* out) {
  if (!q || !k_pool || !v_pool || !segs || !seg_indptr || !out) return MSA_ERR_INVALID_ARG;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || P <= 0 || max_ctx_len < 0 || block_size <= 0)
    return MSA_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return MSA_ERR_INVALID_ARG;
  if (split_blocks < 0) return MSA_ERR_INVALID_ARG;
  if (isnan(scale) || isinf(scale)) return MSA_ERR_INVALID_ARG;
  if (dtype != MSA_F32 && dtype != MSA_BF16) return MSA_ERR_UNSUPPORTED;
  if (block_size != 16) return MSA_ERR_UNSUPPORTED;
  if (B > 65535 || Hkv > 65535) return MSA_ERR_UNSUPPORTED;  // grid y/z limits
  return MSA_OK;
}

// The decode kernel a call runs: true for the block kernel.  Automatic
// choice: the block kernel for up to 256 sequences (the range in which it
// looks for shared prefixes) holding at least 6144 blocks in all, unless
// one workgroup per (sequence, KV head) already fills the chip with no
// split (every context within 256 blocks):
// there the per-head kernel needs no merge and no device-side set-up, and
// wins (32 x 4k tokens, cold: 75.5 against 85 us).  Elsewhere the block
// kernel's whole-block stream wins: 4 x 131k tokens 179 against 197 us, 64
// lognormal contexts with shared prefixes 201 against 245 us.
bool decode_uses_block(msa_decode_kernel kernel, msa_dtype dtype, int32_t B, int32_t Hq,
                       int32_t Hkv, int32_t D, int32_t max_ctx_len, int32_t block_size) {
  if (kernel == MSA_DECODE_BLOCK) return true;
  if (kernel != MSA_DECODE_AUTO) return false;
  if (!decode_block_supported(dtype, D, Hkv, Hq / Hkv, B) || B > kDecodeBlockMaxShareSeq) return false;
  const int64_t nbm = (int64_t(max_ctx_len) + block_size - 1) / block_size;
  // Its 256 items must be long enough to pay for the block kernel's set-up
  // and merge: below 24 blocks per item on a fully alive batch the per-head
  // kernel is faster (cold, headline recipe at 128k tokens or less: batch
  // 1 x 32k 32.5 against 35.4 us, 1 x 64k 48.5 against 54.4, 2 x 32k 46.2
  // against 52.8; at 6144 blocks the two are within 2% either way, above it
  // the block kernel wins or ties).
  if (int64_t(B) * nbm < 24 * 256) return false;
  return !(int64_t(B) * Hkv >= 256 && nbm <= 256);
}

// block kernel workspace: its partial capacity, then the per-sequence
// partial ranges
struct BlockLayout {
  PartLayout parts;
  size_t indptr_off, total;
  BlockSizes n;
};
inline BlockLayout block_layout(int32_t B, int32_t Hq, int32_t D, int32_t cap_blocks,
                                int32_t split_blocks) {
  BlockLayout L;
  L.n = decode_block_sizes(B, cap_blocks, split_blocks);
  L.parts = part_layout(L.n.parts, 1, Hq, D);
  L.indptr_off = L.parts.total;
  L.total = L.indptr_off + align_up(size_t(B + 1) * sizeof(int32_t));
  return L;
}

inline float resolve_scale(float scale, int32_t D) {
  return scale > 0.f ? scale : 1.0f / sqrtf(float(D));
}

constexpr float kLog2e = 1.44269504088896340736f;

}  // namespace

extern "C" {

int msa_version(void) { return MSA_VERSION; }

int msa_attention_supported(int prefill, msa_dtype dtype, int32_t head_dim, int32_t group_size,
                            int32_t block_size) {
  if (block_size != 16) return 0;
  return (prefill ? prefill_supported(dtype, head_dim, group_size)
                  : decode_supported(dtype, head_dim, group_size)) ? 1 : 0;
}

const char* msa_status_string(int status) {
  switch (status) {
    case MSA_OK: return "MSA_OK";
    case MSA_ERR_INVALID_ARG: return "MSA_ERR_INVALID_ARG: invalid argument";
    case MSA_ERR_UNSUPPORTED: return "MSA_ERR_UNSUPPORTED: configuration not built";
    case MSA_ERR_CAPACITY: return "MSA_ERR_CAPACITY: workspace or output too small";
    case MSA_ERR_DEVICE: return "MSA_ERR_DEVICE: HIP runtime error";
  }
  return "unknown msa status";
}

// ---------------------------------------------------------------------------
// per sequence: segment count, error flags, record offset
size_t msa_plan_workspace_size(int32_t B) { return B > 0 ? align_up(size_t(B) * 3 * sizeof(int32_t)) : 0; }

int msa_plan_segments(const int32_t* block_table, const uint8_t* alive, const int32_t* ctx_len,
                      int32_t B, int32_t max_blocks, int32_t block_size, int32_t num_phys_blocks,
                      msa_segment* segs, int32_t seg_capacity, int32_t* seg_indptr,
                      int32_t* dev_error, void* workspace, size_t workspace_bytes, void* stream) {
  if (!block_table || !alive || !ctx_len || !seg_indptr || !dev_error || !workspace)
    return MSA_ERR_INVALID_ARG;
  if (B <= 0 || max_blocks <= 0 || block_size <= 0 || num_phys_blocks <= 0 || seg_capacity < 0)
    return MSA_ERR_INVALID_ARG;
  if (seg_capacity > 0 && !segs) return MSA_ERR_INVALID_ARG;
  if (int64_t(max_blocks) * block_size > INT32_MAX) return MSA_ERR_INVALID_ARG;
  if (int64_t(B) * max_blocks > INT32_MAX) return MSA_ERR_INVALID_ARG;
  if (B > 2147483647 / 2) return MSA_ERR_INVALID_ARG;
  if (workspace_bytes < msa_plan_workspace_size(B)) return MSA_ERR_CAPACITY;
  PlanParams p;
  p.table = block_table;
  p.alive = alive;
  p.ctx_len = ctx_len;
  p.B = B;
  p.max_blocks = max_blocks;
  p.bs = block_size;
  p.P = num_phys_blocks;
  p.segs = segs;
  p.cap = seg_capacity;
  p.indptr = seg_indptr;
  p.dev_error = dev_error;
  p.ws = static_cast<int32_t*>(workspace);
  p.scanned = plan_uses_scan(B) ? 1 : 0;
  return from_hip(launch_plan(p, as_stream(stream)));
}

// ---------------------------------------------------------------------------
size_t msa_decode_workspace_size(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                 int32_t max_ctx_len, int32_t block_size, int32_t split_blocks) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || block_size <= 0 || max_ctx_len < 0) return 0;
  const SplitPlan sp = decode_split(B, Hkv, max_ctx_len, block_size, split_blocks);
  size_t need = sp.S <= 1 ? 0 : part_layout(int64_t(B) * sp.S, 1, Hq, D).total;
  // the block kernel may run for this shape (the dtype is not an argument)
  if (Hq % Hkv == 0 && decode_block_supported(MSA_BF16, D, Hkv, Hq / Hkv, B)) {
    const BlockLayout L = block_layout(B, Hq, D, sp.S * sp.split_blocks, split_blocks);
    if (L.total > need) need = L.total;
  }
  return need;
}

int msa_decode_ex(const void* q, const void* k_pool, const void* v_pool, int32_t num_phys_blocks,
                  int32_t block_size, const msa_segment* segs, const int32_t* seg_indptr,
                  int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t max_ctx_len,
                  msa_dtype dtype, float scale, int32_t split_blocks, void* out, float* lse_out,
                  void* workspace, size_t workspace_bytes, msa_kv_layout kv_layout,
                  msa_decode_kernel kernel, int32_t* dev_error, void* stream) {
  int st = check_attn_shape(q, k_pool, v_pool, num_phys_blocks, block_size, segs, seg_indptr, B,
                            Hq, Hkv, D, max_ctx_len, dtype, scale, split_blocks, out);
  if (st != MSA_OK) return st;
  if (kv_layout != MSA_LAYOUT_NHD && kv_layout != MSA_LAYOUT_HND) return MSA_ERR_INVALID_ARG;
  if (kernel != MSA_DECODE_AUTO && kernel != MSA_DECODE_VECTOR && kernel != MSA_DECODE_MATRIX &&
      kernel != MSA_DECODE_BLOCK)
    return MSA_ERR_INVALID_ARG;
  if (!decode_supported(dtype, D, Hq / Hkv)) return MSA_ERR_UNSUPPORTED;
  if (kernel == MSA_DECODE_MATRIX && !decode_matrix_supported(dtype, D, Hq / Hkv))
    return MSA_ERR_UNSUPPORTED;
  if (kernel == MSA_DECODE_BLOCK && !decode_block_supported(dtype, D, Hkv, Hq / Hkv, B))
    return MSA_ERR_UNSUPPORTED;
  if (split_blocks > decode_max_split_blocks()) return MSA_ERR_INVALID_ARG;
  const SplitPlan sp = decode_split(B, Hkv, max_ctx_len, block_size, split_blocks);
  const size_t need = msa_decode_workspace_size(B, Hq, Hkv, D, max_ctx_len, block_size, split_blocks);
  if (need > 0 && (!workspace || workspace_bytes < need)) return MSA_ERR_CAPACITY;

  DecodeParams p{};
  p.q = q;
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.P = num_phys_blocks;
  p.segs = segs;
  p.indptr = seg_indptr;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.D = D;
  p.head_major = kv_layout == MSA_LAYOUT_HND ? 1 : 0;
  p.dtype = dtype;
  p.scale_log2 = resolve_scale(scale, D) * kLog2e;
  p.split_blocks = sp.split_blocks;
  p.S = sp.S;
  p.kernel = kernel;
  p.dev_error = dev_error;
  p.out = out;
  p.lse = lse_out;
  p.o_part = p.m_part = p.l_part = nullptr;
  p.use_block = 0;
  p.part_indptr = nullptr;
  p.cap_blocks = sp.S * sp.split_blocks;
  if (decode_uses_block(kernel, dtype, B, Hq, Hkv, D, max_ctx_len, block_size)) {
    const BlockLayout L = block_layout(B, Hq, D, p.cap_blocks, split_blocks);
    if (L.n.items > INT32_MAX || L.n.parts > INT32_MAX) return MSA_ERR_UNSUPPORTED;
    char* ws = static_cast<char*>(workspace);
    p.use_block = 1;
    p.nwg = int32_t(L.n.items);
    p.block_auto = split_blocks == 0 ? 1 : 0;
    p.block_target = decode_block_target(B);
    p.block_parts = int32_t(L.n.parts);
    p.block_share = decode_block_shares(B) ? 1 : 0;
    p.o_part = reinterpret_cast<float*>(ws + L.parts.o_off);
    p.m_part = reinterpret_cast<float*>(ws + L.parts.m_off);
    p.l_part = reinterpret_cast<float*>(ws + L.parts.l_off);
    p.part_indptr = reinterpret_cast<int32_t*>(ws + L.indptr_off);
    hipError_t e = launch_decode(p, as_stream(stream));
    if (e != hipSuccess) return MSA_ERR_DEVICE;
    const int64_t per_seq = (L.n.items - B + B - 1) / B;
    e = launch_merge_block(p.o_part, p.m_part, p.l_part, p.part_indptr, B, Hq, D,
                           int32_t(per_seq < 1 ? 1 : per_seq), dtype, out, lse_out,
                           as_stream(stream));
    return e == hipSuccess ? MSA_OK : MSA_ERR_DEVICE;
  }
  if (sp.S > 1) {
    const PartLayout L = part_layout(int64_t(B) * sp.S, 1, Hq, D);
    char* ws = static_cast<char*>(workspace);
    p.o_part = reinterpret_cast<float*>(ws + L.o_off);
    p.m_part = reinterpret_cast<float*>(ws + L.m_off);
    p.l_part = reinterpret_cast<float*>(ws + L.l_off);
  }
  hipError_t e = launch_decode(p, as_stream(stream));
  if (e != hipSuccess) return MSA_ERR_DEVICE;
  if (sp.S > 1) {
    e = launch_merge_from_plan(p.o_part, p.m_part, p.l_part, segs, seg_indptr, B, 1, Hq, D, sp.S,
                               sp.split_blocks, dtype, out, lse_out, as_stream(stream));
    if (e != hipSuccess) return MSA_ERR_DEVICE;
  }
  return MSA_OK;
}

int msa_decode(const void* q, const void* k_pool, const void* v_pool, int32_t num_phys_blocks,
               int32_t block_size, const msa_segment* segs, const int32_t* seg_indptr, int32_t B,
               int32_t Hq, int32_t Hkv, int32_t D, int32_t max_ctx_len, msa_dtype dtype,
               float scale, int32_t split_blocks, void* out, float* lse_out, void* workspace,
               size_t workspace_bytes, int32_t* dev_error, void* stream) {
  return msa_decode_ex(q, k_pool, v_pool, num_phys_blocks, block_size, segs, seg_indptr, B, Hq,
                       Hkv, D, max_ctx_len, dtype, scale, split_blocks, out, lse_out, workspace,
                       workspace_bytes, MSA_LAYOUT_NHD, MSA_DECODE_AUTO, dev_error, stream);
}

// ---------------------------------------------------------------------------
size_t msa_prefill_workspace_size(int32_t B, int32_t C, int32_t Hq, int32_t Hkv, int32_t D,
                                  int32_t max_ctx_len, int32_t block_size, int32_t split_blocks) {
  if (B <= 0 || C <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || block_size <= 0 || max_ctx_len < 0)
    return 0;
  const SplitPlan sp = prefill_split(B, C, Hq, Hkv, max_ctx_len, block_size, split_blocks);
  if (sp.S <= 1) return 0;
  return part_layout(int64_t(B) * sp.S, C, Hq, D).total;
}

int msa_prefill_chunk_ex(const void* q, int32_t C, const int32_t* q_pos0, const void* k_pool,
                         const void* v_pool, int32_t num_phys_blocks, int32_t block_size,
                         const msa_segment* segs, const int32_t* seg_indptr, int32_t B,
                         int32_t Hq, int32_t Hkv, int32_t D, int32_t max_ctx_len, msa_dtype dtype,
                         float scale, int32_t split_blocks, void* out, float* lse_out,
                         void* workspace, size_t workspace_bytes, msa_kv_layout kv_layout,
                         int32_t* dev_error, void* stream) {
  int st = check_attn_shape(q, k_pool, v_pool, num_phys_blocks, block_size, segs, seg_indptr, B,
                            Hq, Hkv, D, max_ctx_len, dtype, scale, split_blocks, out);
  if (st != MSA_OK) return st;
  if (kv_layout != MSA_LAYOUT_NHD && kv_layout != MSA_LAYOUT_HND) return MSA_ERR_INVALID_ARG;
  if (!q_pos0 || C <= 0) return MSA_ERR_INVALID_ARG;
  if (!prefill_supported(dtype, D, Hq / Hkv)) return MSA_ERR_UNSUPPORTED;
  if (split_blocks > prefill_max_split_blocks()) return MSA_ERR_INVALID_ARG;
  const SplitPlan sp = prefill_split(B, C, Hq, Hkv, max_ctx_len, block_size, split_blocks);
  // grid z is (sequence, split); the split merge's grid y is the chunk row
  if (int64_t(B) * sp.S > 65535 || (sp.S > 1 && C > 65535)) return MSA_ERR_UNSUPPORTED;
  const size_t need =
      msa_prefill_workspace_size(B, C, Hq, Hkv, D, max_ctx_len, block_size, split_blocks);
  if (need > 0 && (!workspace || workspace_bytes < need)) return MSA_ERR_CAPACITY;

  PrefillParams p{};
  p.q = q;
  p.q_pos0 = q_pos0;
  p.dtype = dtype;
  p.C = C;
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.P = num_phys_blocks;
  p.segs = segs;
  p.indptr = seg_indptr;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.D = D;
  p.head_major = kv_layout == MSA_LAYOUT_HND ? 1 : 0;
  p.scale_log2 = resolve_scale(scale, D) * kLog2e;
  p.split_blocks = sp.split_blocks;
  p.S = sp.S;
  p.dev_error = dev_error;
  p.out = out;
  p.lse = lse_out;
  p.o_part = p.m_part = p.l_part = nullptr;
  if (sp.S > 1) {
    const PartLayout L = part_layout(int64_t(B) * sp.S, C, Hq, D);
    char* ws = static_cast<char*>(workspace);
    p.o_part = reinterpret_cast<float*>(ws + L.o_off);
    p.m_part = reinterpret_cast<float*>(ws + L.m_off);
    p.l_part = reinterpret_cast<float*>(ws + L.l_off);
  }
  hipError_t e = launch_prefill(p, as_stream(stream));
  if (e != hipSuccess) return MSA_ERR_DEVICE;
  if (sp.S > 1) {
    e = launch_merge_from_plan(p.o_part, p.m_part, p.l_part, segs, seg_indptr, B, C, Hq, D, sp.S,
                               sp.split_blocks, dtype, out, lse_out, as_stream(stream));
    if (e != hipSuccess) return MSA_ERR_DEVICE;
  }
  return MSA_OK;
}

int msa_prefill_chunk(const void* q, int32_t C, const int32_t* q_pos0, const void* k_pool,
                      const void* v_pool, int32_t num_phys_blocks, int32_t block_size,
                      const msa_segment* segs, const int32_t* seg_indptr, int32_t B, int32_t Hq,
                      int32_t Hkv, int32_t D, int32_t max_ctx_len, msa_dtype dtype, float scale,
                      int32_t split_blocks, void* out, float* lse_out, void* workspace,
                      size_t workspace_bytes, int32_t* dev_error, void* stream) {
  return msa_prefill_chunk_ex(q, C, q_pos0, k_pool, v_pool, num_phys_blocks, block_size, segs,
                              seg_indptr, B, Hq, Hkv, D, max_ctx_len, dtype, scale, split_blocks,
                              out, lse_out, workspace, workspace_bytes, MSA_LAYOUT_NHD, dev_error,
                              stream);
}

int32_t msa_prefill_chunk_rows(int32_t B, int32_t Hq, int32_t Hkv, int32_t remaining_tokens,
                               int32_t max_rows, int32_t compute_units) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || remaining_tokens < 0 || max_rows <= 0)
    return MSA_ERR_INVALID_ARG;
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return MSA_ERR_UNSUPPORTED;
  if (remaining_tokens == 0) return 0;
  return prefill_chunk_rows(B, Hq, Hkv, remaining_tokens, max_rows, compute_units);
}

// ---------------------------------------------------------------------------
int msa_merge_partials(const float* o_part, const float* m_part, const float* l_part,
                       const int32_t* part_indptr, int32_t B, int32_t R, int32_t H, int32_t D,
                       msa_dtype out_dtype, void* out, float* lse_out, void* stream) {
  if (!o_part || !m_part || !l_part || !part_indptr || !out) return MSA_ERR_INVALID_ARG;
  if (B <= 0 || R <= 0 || H <= 0 || D <= 0) return MSA_ERR_INVALID_ARG;
  if (out_dtype != MSA_F32 && out_dtype != MSA_BF16) return MSA_ERR_UNSUPPORTED;
  if (B > 65535 || R > 65535) return MSA_ERR_UNSUPPORTED;
  if (int64_t(H) * D > INT32_MAX) return MSA_ERR_INVALID_ARG;
  return from_hip(launch_merge_indptr(o_part, m_part, l_part, part_indptr, B, R, H, D, out_dtype,
                                      out, lse_out, as_stream(stream)));
}

int msa_gather_alive(const void* k_pool, const void* v_pool, int32_t num_phys_blocks,
                     int32_t block_size, const msa_segment* segs, const int32_t* seg_indptr,
                     int32_t B, int32_t Hkv, int32_t D, msa_dtype dtype, int32_t blocks_per_seq,
                     void* dense_k, void* dense_v, msa_segment* dense_segs,
                     int32_t* dense_indptr, void* stream) {
  if (!k_pool || !v_pool || !segs || !seg_indptr || !dense_k || !dense_v || !dense_segs ||
      !dense_indptr)
    return MSA_ERR_INVALID_ARG;
  if (B <= 0 || Hkv <= 0 || D <= 0 || num_phys_blocks <= 0 || blocks_per_seq <= 0)
    return MSA_ERR_INVALID_ARG;
  if (dtype != MSA_F32 && dtype != MSA_BF16) return MSA_ERR_UNSUPPORTED;
  if (block_size != 16) return MSA_ERR_UNSUPPORTED;
  if (B > 65535) return MSA_ERR_UNSUPPORTED;
  const size_t esz = dtype == MSA_BF16 ? 2 : 4;
  const size_t block_bytes = size_t(block_size) * size_t(Hkv) * size_t(D) * esz;
  if (block_bytes % 16 != 0) return MSA_ERR_UNSUPPORTED;
  if (int64_t(B) * blocks_per_seq > INT32_MAX) return MSA_ERR_INVALID_ARG;
  GatherParams p;
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.P = num_phys_blocks;
  p.segs = segs;
  p.indptr = seg_indptr;
  p.B = B;
  p.blocks_per_seq = blocks_per_seq;
  p.block_bytes = block_bytes;
  p.dense_k = dense_k;
  p.dense_v = dense_v;
  p.dense_segs = dense_segs;
  p.dense_indptr = dense_indptr;
  return from_hip(launch_gather(p, as_stream(stream)));
}

}  // extern "C"
