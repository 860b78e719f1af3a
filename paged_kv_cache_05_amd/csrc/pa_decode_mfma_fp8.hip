// Matrix-core paged decode over 8-bit E4M3 caches (16-bit queries and output): the head-dim-128
// instantiations of pa_decode_mfma.h, and the dispatch to the 64-, 80- and 256-dim ones.  K/V codes are converted to the query type in registers (exactly), so
// grouped query heads share each K/V byte as in the 16-bit kernel.
#include "pa_decode_mfma.h"

namespace pa {

hipError_t launch_decode_mfma_fp8(DT dt, int head_dim, int block_size, int heads_per_wg,
                                  bool stream_kv, const DecodeParams& p, int grid, hipStream_t st) {
  if (head_dim == 64 || head_dim == 80 || head_dim == 256)
    return launch_decode_mfma_fp8_dims(dt, head_dim, block_size, heads_per_wg, stream_kv, p, grid, st);
  if (head_dim != 128) return hipErrorInvalidValue;
  switch (dt) {
    case DT::F16: return launch_bs<DT::F16, DT::FP8, 128>(block_size, heads_per_wg, stream_kv, p, grid, st);
    case DT::BF16: return launch_bs<DT::BF16, DT::FP8, 128>(block_size, heads_per_wg, stream_kv, p, grid, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
