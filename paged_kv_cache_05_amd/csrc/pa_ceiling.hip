// Read-only bandwidth probe: the rate at which the GPU streams bytes it only reads, either as
// one contiguous run or as whole tiles at scattered places (the access pattern of paged decode,
// where every (block, KV head) tile is a contiguous 4-8 KiB run somewhere in the pool).  It does
// no arithmetic beyond an XOR of the words it reads, so it sets the ceiling that the decode
// kernels' achieved bandwidth is compared with.  Decode is bound by memory bandwidth (UltraLAB
// summary of Kwon et al. (xasun.com) §三, compute-pattern row and FAQ), so this ceiling, not the
// matrix or vector units, is what its kernels are measured against.
//
// Loads are the decode's: 16 bytes per lane, non-temporal, one wave instruction moving 1 KiB.
// Each wave takes 4 tiles and issues all their loads before consuming any (16 loads per lane
// in flight for 4 KiB tiles), then writes one XOR word per tile.
#include "pa_common.h"

namespace pa {
namespace {

constexpr int kTilesPerWave = 4;

template <int LPT>   // 16-byte loads per lane per tile: the tile is LPT KiB
__global__ __launch_bounds__(256) void read_tiles_kernel(const char* __restrict__ base,
                                                         const int32_t* __restrict__ ids,
                                                         int num_tiles, long base_tiles,
                                                         uint32_t* __restrict__ xor_out) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const long t0 = ((long)blockIdx.x * 4 + wave) * kTilesPerWave;
  long id[kTilesPerWave];
  bool ok[kTilesPerWave];
#pragma unroll
  for (int k = 0; k < kTilesPerWave; ++k) {
    const long t = t0 + k;
    long b = t;
    if (ids != nullptr) b = t < num_tiles ? ids[t] : -1;
    ok[k] = t < num_tiles && b >= 0 && b < base_tiles;
    id[k] = ok[k] ? b : 0;    // a skipped tile reads tile 0 and reports 0
  }
  uint4 v[kTilesPerWave][LPT];
#pragma unroll
  for (int k = 0; k < kTilesPerWave; ++k)
#pragma unroll
    for (int i = 0; i < LPT; ++i)
      v[k][i] = load_stream(base + (id[k] * LPT + i) * 1024 + lane * 16);
#pragma unroll
  for (int k = 0; k < kTilesPerWave; ++k) {
    uint32_t x = 0;
#pragma unroll
    for (int i = 0; i < LPT; ++i) x ^= v[k][i].x ^ v[k][i].y ^ v[k][i].z ^ v[k][i].w;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) x ^= (uint32_t)__shfl_xor((int)x, off);
    const long t = t0 + k;
    if (lane == 0 && t < num_tiles) xor_out[t] = ok[k] ? x : 0u;
  }
}

}  // namespace

hipError_t launch_read_tiles(const void* base, long base_tiles, int tile_bytes,
                             const int32_t* ids, int num_tiles, uint32_t* xor_out,
                             hipStream_t st) {
  const long grid = ((long)num_tiles + 4 * kTilesPerWave - 1) / (4 * kTilesPerWave);
  const char* b = reinterpret_cast<const char*>(base);
  switch (tile_bytes) {
    case 1024: hipLaunchKernelGGL(read_tiles_kernel<1>, dim3(grid), dim3(256), 0, st, b, ids, num_tiles, base_tiles, xor_out); break;
    case 2048: hipLaunchKernelGGL(read_tiles_kernel<2>, dim3(grid), dim3(256), 0, st, b, ids, num_tiles, base_tiles, xor_out); break;
    case 4096: hipLaunchKernelGGL(read_tiles_kernel<4>, dim3(grid), dim3(256), 0, st, b, ids, num_tiles, base_tiles, xor_out); break;
    case 8192: hipLaunchKernelGGL(read_tiles_kernel<8>, dim3(grid), dim3(256), 0, st, b, ids, num_tiles, base_tiles, xor_out); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
