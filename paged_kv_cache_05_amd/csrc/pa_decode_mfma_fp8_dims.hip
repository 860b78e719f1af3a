// Matrix-core paged decode over 8-bit E4M3 caches at head dims 64, 80 and 256: instantiations of
// pa_decode_mfma.h (head dim 128 is in pa_decode_mfma_fp8.hip).  A 64-dim token row is 64
// bytes, so one 1 KiB wave load carries all 16 rows of a chunk's K and each lane takes one
// 4-byte piece of a V row; a 256-dim row is four loads' worth; 80-dim rows (80 bytes) run
// through the 128-dim products with the padding dims zero.
#include "pa_decode_mfma.h"

namespace pa {

hipError_t launch_decode_mfma_fp8_dims(DT dt, int head_dim, int block_size, int heads_per_wg,
                                       bool stream_kv, const DecodeParams& p, int grid,
                                       hipStream_t st) {
  switch (head_dim) {
    case 64:
      if (dt == DT::F16) return launch_bs<DT::F16, DT::FP8, 64>(block_size, heads_per_wg, stream_kv, p, grid, st);
      if (dt == DT::BF16) return launch_bs<DT::BF16, DT::FP8, 64>(block_size, heads_per_wg, stream_kv, p, grid, st);
      break;
    case 80:   // the 128-dim products on rows of 80 stored dims
      if (dt == DT::F16) return launch_bs<DT::F16, DT::FP8, 128, 80>(block_size, heads_per_wg, stream_kv, p, grid, st);
      if (dt == DT::BF16) return launch_bs<DT::BF16, DT::FP8, 128, 80>(block_size, heads_per_wg, stream_kv, p, grid, st);
      break;
    case 256:
      if (dt == DT::F16) return launch_bs<DT::F16, DT::FP8, 256>(block_size, heads_per_wg, stream_kv, p, grid, st);
      if (dt == DT::BF16) return launch_bs<DT::BF16, DT::FP8, 256>(block_size, heads_per_wg, stream_kv, p, grid, st);
      break;
    default: break;
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
