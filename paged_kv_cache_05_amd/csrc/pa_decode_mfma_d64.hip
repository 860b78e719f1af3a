// Matrix-core paged decode over 16-bit caches at head dim 64: instantiations of
// pa_decode_mfma.h in a translation unit of their own (built in parallel with the others).
#include "pa_decode_mfma.h"

namespace pa {

hipError_t launch_decode_mfma_d64(DT dt, int block_size, int heads_per_wg, bool stream_kv,
                                  const DecodeParams& p, int grid, hipStream_t st) {
  switch (dt) {
    case DT::F16: return launch_bs<DT::F16, DT::F16, 64>(block_size, heads_per_wg, stream_kv, p, grid, st);
    case DT::BF16: return launch_bs<DT::BF16, DT::BF16, 64>(block_size, heads_per_wg, stream_kv, p, grid, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
