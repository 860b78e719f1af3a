// Vector-ALU paged decode over an 8-bit E4M3 cache at head dims 64, 80 and 256 (f16 / bf16
// queries): instantiations of pa_decode_valu.h, in a translation unit of their own so they
// compile in parallel with the 128-dim ones.
#include "pa_decode_valu.h"

namespace pa {

hipError_t launch_decode_valu_fp8_dims(DT dt, int head_dim, int block_size, int heads_per_wg,
                                       bool stream_kv, const DecodeParams& p, int grid,
                                       hipStream_t st) {
  auto by_dim = [&](auto dt_tag) -> hipError_t {
    constexpr DT T = decltype(dt_tag)::value;
    switch (head_dim) {
      case 64: return launch_bs<T, DT::FP8, 64>(block_size, heads_per_wg, stream_kv, p, grid, st);
      case 80: return launch_bs<T, DT::FP8, 80>(block_size, heads_per_wg, stream_kv, p, grid, st);
      case 256: return launch_bs<T, DT::FP8, 256>(block_size, heads_per_wg, stream_kv, p, grid, st);
    }
    return hipErrorInvalidValue;
  };
  if (dt == DT::F16) return by_dim(std::integral_constant<DT, DT::F16>{});
  if (dt == DT::BF16) return by_dim(std::integral_constant<DT, DT::BF16>{});
  return hipErrorInvalidValue;
}
}  // namespace pa
