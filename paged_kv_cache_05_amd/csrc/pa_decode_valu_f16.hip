// Vector-ALU paged decode, f16 queries and cache (head dims 64, 80, 128, 256).
#include "pa_decode_valu.h"

namespace pa {

hipError_t launch_decode_valu_f16(int head_dim, int block_size, int heads_per_wg, bool stream_kv,
                                 const DecodeParams& p, int grid, hipStream_t st) {
  switch (head_dim) {
    case 64: return launch_bs<DT::F16, DT::F16, 64>(block_size, heads_per_wg, stream_kv, p, grid, st);
    case 80: return launch_bs<DT::F16, DT::F16, 80>(block_size, heads_per_wg, stream_kv, p, grid, st);
    case 128: return launch_bs<DT::F16, DT::F16, 128>(block_size, heads_per_wg, stream_kv, p, grid, st);
    case 256: return launch_bs<DT::F16, DT::F16, 256>(block_size, heads_per_wg, stream_kv, p, grid, st);
  }
  return hipErrorInvalidValue;
}
}  // namespace pa
