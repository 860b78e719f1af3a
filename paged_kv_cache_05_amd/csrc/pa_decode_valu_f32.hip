// Vector-ALU paged decode, fp32 queries and cache; also the dispatch over element types.
#include "pa_decode_valu.h"

namespace pa {

hipError_t launch_decode_valu(DT dt, int head_dim, int block_size, int heads_per_wg,
                              bool stream_kv, const DecodeParams& p, int grid, hipStream_t st) {
  if (dt == DT::F16) return launch_decode_valu_f16(head_dim, block_size, heads_per_wg, stream_kv, p, grid, st);
  if (dt == DT::BF16) return launch_decode_valu_bf16(head_dim, block_size, heads_per_wg, stream_kv, p, grid, st);
  if (dt != DT::F32) return hipErrorInvalidValue;
  if (head_dim == 64) return launch_bs<DT::F32, DT::F32, 64>(block_size, heads_per_wg, stream_kv, p, grid, st);
  if (head_dim == 128) return launch_bs<DT::F32, DT::F32, 128>(block_size, heads_per_wg, stream_kv, p, grid, st);
  return hipErrorInvalidValue;
}
}  // namespace pa
