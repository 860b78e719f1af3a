// Vector-ALU paged decode over an 8-bit E4M3 cache (f16 / bf16 queries): the 128-dim
// instances, and the dispatch to the 64 / 80 / 256-dim ones (pa_decode_valu_fp8_dims.hip).
#include "pa_decode_valu.h"

namespace pa {

hipError_t launch_decode_valu_fp8(DT dt, int head_dim, int block_size, int heads_per_wg,
                                  bool stream_kv, const DecodeParams& p, int grid, hipStream_t st) {
  if (head_dim != 128)
    return launch_decode_valu_fp8_dims(dt, head_dim, block_size, heads_per_wg, stream_kv, p, grid, st);
  if (dt == DT::F16) return launch_bs<DT::F16, DT::FP8, 128>(block_size, heads_per_wg, stream_kv, p, grid, st);
  if (dt == DT::BF16) return launch_bs<DT::BF16, DT::FP8, 128>(block_size, heads_per_wg, stream_kv, p, grid, st);
  return hipErrorInvalidValue;
}
}  // namespace pa
