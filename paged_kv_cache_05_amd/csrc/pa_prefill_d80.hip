// Chunked prefill on the matrix cores at head dim 80: the 128-dim instances of pa_prefill.h with
// rows of 80 stored dims (dims 80 .. 127 zero in registers and LDS, never loaded or stored).
#include "pa_prefill.h"

namespace pa {

hipError_t launch_prefill_mfma_d80(DT dt, bool kv8, int block_size, bool split_p,
                                   const PrefillParams& p, int grid, hipStream_t st) {
  return launch_prefill_d<128, 80>(dt, kv8, block_size, split_p, p, grid, st);
}

}  // namespace pa
