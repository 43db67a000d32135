// msa_decode without a caller workspace: the split partials live in a
// file-scope device array instead, for callers that cannot allocate device
// memory at call time (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).  The kernels are msa_decode's own.
//
// The array is a __device__ symbol: every GPU the library runs on holds its
// own copy for the life of the process.  Its device address is looked up
// once per device with hipGetSymbolAddress (with that device current) and
// kept; host code never passes the symbol itself to a kernel, since on the
// host it only names a host-side stand-in.  Calls on one GPU share the
// array: calls that overlap in time on that GPU (other streams, other host
// threads) race on it and must be ordered by the caller.
#include <mutex>

#include "msa_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;  // the array's size: 32 MiB
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of this device's copy of the array (looked up on the
// device's first call), or nullptr if the lookup failed.
void* scratch_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" {

size_t msa_decode_noalloc_capacity(void) { return kScratchBytes; }

int msa_decode_noalloc(const void* q, const void* k_pool, const void* v_pool,
                       int32_t num_phys_blocks, int32_t block_size, const msa_segment* segs,
                       const int32_t* seg_indptr, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                       int32_t max_ctx_len, msa_dtype dtype, float scale, int32_t split_blocks,
                       void* out, float* lse_out, int32_t* dev_error, void* stream) {
  // the same checks msa_decode makes, before anything touches the device
  if (!q || !k_pool || !v_pool || !segs || !seg_indptr || !out) return MSA_ERR_INVALID_ARG;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || num_phys_blocks <= 0 || max_ctx_len < 0 ||
      block_size <= 0 || split_blocks < 0 || Hq % Hkv != 0)
    return MSA_ERR_INVALID_ARG;
  const size_t need =
      msa_decode_workspace_size(B, Hq, Hkv, D, max_ctx_len, block_size, split_blocks);
  if (need > kScratchBytes) return MSA_ERR_CAPACITY;
  void* ws = nullptr;
  if (need > 0) {
    ws = scratch_for_current_device();
    if (ws == nullptr) return MSA_ERR_DEVICE;
  }
  return msa_decode(q, k_pool, v_pool, num_phys_blocks, block_size, segs, seg_indptr, B, Hq, Hkv,
                    D, max_ctx_len, dtype, scale, split_blocks, out, lse_out, ws, need, dev_error,
                    stream);
}

}  // extern "C"
