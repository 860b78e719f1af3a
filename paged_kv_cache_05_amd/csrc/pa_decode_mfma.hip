// Matrix-core paged decode over 16-bit caches: instantiations of pa_decode_mfma.h.
#include "pa_decode_mfma.h"

namespace pa {

hipError_t launch_decode_mfma(DT dt, int head_dim, int block_size, int heads_per_wg,
                              bool stream_kv, const DecodeParams& p, int grid, hipStream_t st) {
  if (head_dim != 128) return hipErrorInvalidValue;
  switch (dt) {
    case DT::F16: return launch_bs<DT::F16, DT::F16>(block_size, heads_per_wg, stream_kv, p, grid, st);
    case DT::BF16: return launch_bs<DT::BF16, DT::BF16>(block_size, heads_per_wg, stream_kv, p, grid, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
