// a2 + a4: MSA chunked prefill (placeholder until the MFMA kernel lands).
#include "msa_internal.h"

namespace msa {

bool prefill_supported(msa_dtype, int32_t, int32_t) { return false; }
int32_t prefill_max_split_blocks() { return 512; }

SplitPlan prefill_split(int32_t, int32_t, int32_t, int32_t, int32_t, int32_t, int32_t split_blocks) {
  SplitPlan sp;
  sp.split_blocks = split_blocks;
  sp.S = 1;
  return sp;
}

hipError_t launch_prefill(const PrefillParams&, hipStream_t) { return hipErrorInvalidValue; }

}  // namespace msa
