// Matrix-core paged decode over 16-bit caches: the head-dim-128 instantiations of
// pa_decode_mfma.h, and the dispatch to the 64-, 80- and 256-dim ones (pa_decode_mfma_d64.hip,
// pa_decode_mfma_d80.hip, pa_decode_mfma_d256.hip).
#include "pa_decode_mfma.h"

namespace pa {

hipError_t launch_decode_mfma_d80(DT dt, int block_size, int heads_per_wg, bool stream_kv,
                                  const DecodeParams& p, int grid, hipStream_t st);

hipError_t launch_decode_mfma(DT dt, int head_dim, int block_size, int heads_per_wg,
                              bool stream_kv, const DecodeParams& p, int grid, hipStream_t st) {
  if (head_dim == 64) return launch_decode_mfma_d64(dt, block_size, heads_per_wg, stream_kv, p, grid, st);
  if (head_dim == 80) return launch_decode_mfma_d80(dt, block_size, heads_per_wg, stream_kv, p, grid, st);
  if (head_dim == 256) return launch_decode_mfma_d256(dt, block_size, heads_per_wg, stream_kv, p, grid, st);
  if (head_dim != 128) return hipErrorInvalidValue;
  switch (dt) {
    case DT::F16: return launch_bs<DT::F16, DT::F16, 128>(block_size, heads_per_wg, stream_kv, p, grid, st);
    case DT::BF16: return launch_bs<DT::BF16, DT::BF16, 128>(block_size, heads_per_wg, stream_kv, p, grid, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
