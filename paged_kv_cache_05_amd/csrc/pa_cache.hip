// KV-cache writers: reshape_and_cache (store each new token at its slot), copy_blocks
// (copy-on-write of whole blocks) and swap_blocks (whole blocks between the GPU pool and a
// pinned host pool).  All are pure data movement in 16-byte vectors; bits are
// copied unchanged.
//
// reshape_and_cache: each decode step appends the new token's K/V to the cache
// (PyTorch-CUDA-v2.9 PagedAttention page (jsqmd.com), paged-memory section and serving
// workflow).  Token i goes to block slot/bs, offset slot%bs, every KV head.
// copy_blocks: shared blocks are reference-counted and copied before a write (UltraLAB
// summary of Kwon et al. (xasun.com) §一 and §二, sharing item).
// swap_blocks: a preempted sequence's blocks move to a CPU block pool and back (same page,
// §二: block pools on both GPU and CPU; recovery by swapping).
// reshape_and_cache into an 8-bit cache quantizes instead of copying: the cache element type
// is a serving choice (kv_cache_dtype in the vLLM configuration of yongjin360.com, §3.2).
#include "pa_common.h"

namespace pa {
namespace {

// One workgroup per token; threads stride over the token's num_kv_heads * row_vecs vectors.
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const uint4* __restrict__ key, const uint4* __restrict__ value, uint4* __restrict__ kc,
    uint4* __restrict__ vc, const int64_t* __restrict__ slots, int row_vecs, int block_size,
    int64_t num_slots, int num_kv_heads) {
  const int i = blockIdx.x;
  const int64_t slot = slots[i];
  if (slot < 0 || slot >= num_slots) return;   // padding, or out of the pool
  const int64_t b = slot / block_size;
  const int off = (int)(slot - b * block_size);
  const int total = num_kv_heads * row_vecs;
  const uint4* ks = key + (size_t)i * total;
  const uint4* vs = value + (size_t)i * total;
  for (int v = threadIdx.x; v < total; v += blockDim.x) {
    const int h = v / row_vecs, j = v - h * row_vecs;
    const size_t dst = ((size_t)(b * num_kv_heads + h) * block_size + off) * row_vecs + j;
    kc[dst] = ks[v];
    vc[dst] = vs[v];
  }
}

// reshape_and_cache into an 8-bit E4M3 cache: each 16-byte vector of a 16-bit source row (8
// elements) becomes 8 bytes of the cache row: x * (1 / scale) in fp32, clamped to +-448,
// rounded to nearest-even.
template <DT dt>
__global__ __launch_bounds__(256) void reshape_and_cache_fp8_kernel(
    const uint4* __restrict__ key, const uint4* __restrict__ value, uint2* __restrict__ kc,
    uint2* __restrict__ vc, const int64_t* __restrict__ slots, int row_vecs, int block_size,
    int64_t num_slots, int num_kv_heads, float k_inv, float v_inv) {
  static_assert(Elem<dt>::kPerVec == 8, "16-bit source elements");
  const int i = blockIdx.x;
  const int64_t slot = slots[i];
  if (slot < 0 || slot >= num_slots) return;   // padding, or out of the pool
  const int64_t b = slot / block_size;
  const int off = (int)(slot - b * block_size);
  const int total = num_kv_heads * row_vecs;
  const uint4* ks = key + (size_t)i * total;
  const uint4* vs = value + (size_t)i * total;
  for (int v = threadIdx.x; v < total; v += blockDim.x) {
    const int h = v / row_vecs, j = v - h * row_vecs;
    const size_t dst = ((size_t)(b * num_kv_heads + h) * block_size + off) * row_vecs + j;
    float f[8];
    Elem<dt>::unpack(ks[v], f);
    kc[dst] = make_uint2(fp8_pack4(f[0] * k_inv, f[1] * k_inv, f[2] * k_inv, f[3] * k_inv),
                         fp8_pack4(f[4] * k_inv, f[5] * k_inv, f[6] * k_inv, f[7] * k_inv));
    Elem<dt>::unpack(vs[v], f);
    vc[dst] = make_uint2(fp8_pack4(f[0] * v_inv, f[1] * v_inv, f[2] * v_inv, f[3] * v_inv),
                         fp8_pack4(f[4] * v_inv, f[5] * v_inv, f[6] * v_inv, f[7] * v_inv));
  }
}

constexpr int kCopyUnroll = 4;
constexpr int kCopyVecsPerWg = 256 * kCopyUnroll;

// Whole-block copies between two pools (the same pool for copy-on-write, the GPU pool and a
// pinned host pool for swapping).  grid.x = pairs * 2 (K, V) * chunks; each workgroup copies up
// to 16 KiB of one block with four independent 16-byte loads per lane.
__global__ __launch_bounds__(256) void block_copy_kernel(const uint4* __restrict__ src_k,
                                                         const uint4* __restrict__ src_v,
                                                         uint4* __restrict__ dst_k,
                                                         uint4* __restrict__ dst_v,
                                                         const int64_t* __restrict__ mapping,
                                                         int64_t block_vecs, int chunks,
                                                         int src_blocks, int dst_blocks,
                                                         const int32_t* __restrict__ count) {
  const int chunk = blockIdx.x % chunks;
  const int which = (blockIdx.x / chunks) & 1;
  const int pair = blockIdx.x / (2 * chunks);
  // the pair's ids are read together with the device-made count (the mapping always holds
  // as many rows as the grid has pairs), saving one dependent round trip
  const int64_t src = mapping[2 * pair], dst = mapping[2 * pair + 1];
  if (count != nullptr && pair >= *count) return;   // pair count produced on the device
  if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) return;
  const uint4* s = (which ? src_v : src_k) + src * block_vecs;
  uint4* d = (which ? dst_v : dst_k) + dst * block_vecs;
  const int64_t v0 = (int64_t)chunk * kCopyVecsPerWg + threadIdx.x;
  uint4 r[kCopyUnroll];
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t v = v0 + u * 256;
    if (v < block_vecs) r[u] = s[v];
  }
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t v = v0 + u * 256;
    if (v < block_vecs) d[v] = r[u];
  }
}

}  // namespace

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* kc, void* vc,
                                    const int64_t* slots, int num_tokens, int row_vecs,
                                    int block_size, int num_blocks, int num_kv_heads,
                                    hipStream_t st) {
  if (num_tokens <= 0) return hipSuccess;
  hipLaunchKernelGGL(reshape_and_cache_kernel, dim3(num_tokens), dim3(256), 0, st,
                     (const uint4*)key, (const uint4*)value, (uint4*)kc, (uint4*)vc, slots,
                     row_vecs, block_size, (int64_t)num_blocks * block_size, num_kv_heads);
  return hipGetLastError();
}

hipError_t launch_reshape_and_cache_fp8(DT dt, const void* key, const void* value, void* kc,
                                        void* vc, const int64_t* slots, int num_tokens,
                                        int head_dim, int block_size, int num_blocks,
                                        int num_kv_heads, float k_inv, float v_inv,
                                        hipStream_t st) {
  if (num_tokens <= 0) return hipSuccess;
  const int row_vecs = head_dim / 8;   // 16-byte source vectors per head row
  const int64_t num_slots = (int64_t)num_blocks * block_size;
  if (dt == DT::BF16)
    hipLaunchKernelGGL(reshape_and_cache_fp8_kernel<DT::BF16>, dim3(num_tokens), dim3(256), 0, st,
                       (const uint4*)key, (const uint4*)value, (uint2*)kc, (uint2*)vc, slots,
                       row_vecs, block_size, num_slots, num_kv_heads, k_inv, v_inv);
  else if (dt == DT::F16)
    hipLaunchKernelGGL(reshape_and_cache_fp8_kernel<DT::F16>, dim3(num_tokens), dim3(256), 0, st,
                       (const uint4*)key, (const uint4*)value, (uint2*)kc, (uint2*)vc, slots,
                       row_vecs, block_size, num_slots, num_kv_heads, k_inv, v_inv);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_block_copy(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                             const int64_t* mapping, int num_pairs, int64_t block_vecs,
                             int src_blocks, int dst_blocks, hipStream_t st,
                             const int32_t* count) {
  if (num_pairs <= 0) return hipSuccess;
  const int chunks = (int)((block_vecs + kCopyVecsPerWg - 1) / kCopyVecsPerWg);
  const int64_t grid = (int64_t)num_pairs * 2 * chunks;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(block_copy_kernel, dim3((unsigned)grid), dim3(256), 0, st,
                     (const uint4*)src_k, (const uint4*)src_v, (uint4*)dst_k, (uint4*)dst_v,
                     mapping, block_vecs, chunks, src_blocks, dst_blocks, count);
  return hipGetLastError();
}

}  // namespace pa
