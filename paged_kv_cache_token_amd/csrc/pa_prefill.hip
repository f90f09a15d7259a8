// pa_prefill.hip -- matrix-core causal prefill over the paged cache (in progress).
#include "pa_internal.h"

namespace pa {

int prefill_tile_tokens(int group) { return 128 / group; }

int prefill_work_capacity(int num_seqs, int total_q_tokens, int group) {
  const int t = prefill_tile_tokens(group);
  return total_q_tokens / t + num_seqs + 1;
}

hipError_t launch_prefill(const PrefillArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace pa
