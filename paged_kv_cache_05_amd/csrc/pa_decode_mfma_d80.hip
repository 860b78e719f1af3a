// Matrix-core paged decode over 16-bit caches at head dim 80: the 128-dim instantiations of
// pa_decode_mfma.h with rows of 80 stored dims (dims 80 .. 127 zero in registers and LDS, never
// loaded or stored), in a translation unit of their own.
#include "pa_decode_mfma.h"

namespace pa {

hipError_t launch_decode_mfma_d80(DT dt, int block_size, int heads_per_wg, bool stream_kv,
                                  const DecodeParams& p, int grid, hipStream_t st) {
  switch (dt) {
    case DT::F16: return launch_bs<DT::F16, DT::F16, 128, 80>(block_size, heads_per_wg, stream_kv, p, grid, st);
    case DT::BF16: return launch_bs<DT::BF16, DT::BF16, 128, 80>(block_size, heads_per_wg, stream_kv, p, grid, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
