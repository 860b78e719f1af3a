// Chunked prefill on the matrix cores: the head-dim-64 instances of pa_prefill.h (the head
// size of GPT-OSS-style models, the subject of "GPT-OSS显存管理技巧：PagedAttention机制解析"
// (yongjin360.com)).
#include "pa_prefill.h"

namespace pa {

hipError_t launch_prefill_mfma_d64(DT dt, bool kv8, int block_size, bool split_p,
                                   const PrefillParams& p, int grid, hipStream_t st) {
  return launch_prefill_d<64>(dt, kv8, block_size, split_p, p, grid, st);
}

}  // namespace pa
