// Chunked prefill on the matrix cores: the head-dim-128 instances of pa_prefill.h, and the
// dispatch to the 64- and 80-dim ones (pa_prefill_d64.hip, pa_prefill_d80.hip).
#include "pa_prefill.h"

namespace pa {

hipError_t launch_prefill_mfma(DT dt, bool kv8, int head_dim, int block_size, bool split_p,
                               const PrefillParams& p, int grid, hipStream_t st) {
  if (head_dim == 64) return launch_prefill_mfma_d64(dt, kv8, block_size, split_p, p, grid, st);
  if (head_dim == 80) return launch_prefill_mfma_d80(dt, kv8, block_size, split_p, p, grid, st);
  if (head_dim != 128) return hipErrorInvalidValue;
  return launch_prefill_d<128>(dt, kv8, block_size, split_p, p, grid, st);
}

}  // namespace pa
