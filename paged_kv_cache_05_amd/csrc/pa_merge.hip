// Split-KV merge: combine per-partition (max, denominator, normalised output) triples of one
// (sequence, query head) into the final output by their log-sum-exp weights:
//   M = max_p m_p,  w_p = l_p * 2^(m_p - M),  out = sum_p w_p o_p / sum_p w_p
// (m is kept in base-2 units because the decode kernels pre-scale scores by log2(e)).
// Splitting a sequence's tokens over workgroups is how long contexts use the whole GPU; the
// pages only hint at page-level parallelism over cores ("PagedAttention技术：加速GPT推理的利器"
// (yunthe.com) §1.2 and §1.3).
//
// One wave per (sequence, head); each lane owns head_dim/64 consecutive output elements.
// Partitions are summed in index order, so the result is deterministic.
#include "pa_common.h"

namespace pa {
namespace {

template <DT dt> __device__ __forceinline__ void store_elem(void* out, size_t i, float v);
template <> __device__ __forceinline__ void store_elem<DT::F32>(void* out, size_t i, float v) {
  reinterpret_cast<float*>(out)[i] = v;
}
template <> __device__ __forceinline__ void store_elem<DT::F16>(void* out, size_t i, float v) {
  reinterpret_cast<uint16_t*>(out)[i] = (uint16_t)f16_bits(v);
}
template <> __device__ __forceinline__ void store_elem<DT::BF16>(void* out, size_t i, float v) {
  reinterpret_cast<uint16_t*>(out)[i] = (uint16_t)bf16_bits(v);
}

template <DT dt, int D>
__global__ __launch_bounds__(256) void merge_kernel(const MergeParams p) {
  constexpr int DPL = (D + kWave - 1) / kWave;   // dims per lane (80 dims: lanes 0..39 busy)
  static_assert(D % DPL == 0, "whole lanes");
  const int lane = threadIdx.x & (kWave - 1);
  const bool act = lane * DPL < D;
  const int idx = blockIdx.x * 4 + threadIdx.x / kWave;   // s * num_heads + h
  if (idx >= p.num_seqs * p.num_heads) return;
  const int s = idx / p.num_heads;
  const int n = min(p.context_lens[s], p.max_blocks_per_seq * p.block_size);
  if (n <= 0) return;
  const int np = (n + p.partition - 1) / p.partition;
  if (np <= 1) return;  // written directly by the decode kernel

  const float2* ml = reinterpret_cast<const float2*>(p.ws_ml) + (size_t)idx * p.max_parts;
  const float* po = p.ws_o + (size_t)idx * p.max_parts * D + (act ? lane * DPL : 0);

  float M = -INFINITY;
  for (int i = lane; i < np; i += kWave) M = fmaxf(M, ml[i].x);
  M = group_max<kWave>(M);
  const float ms = safe_max(M);

  float L = 0.0f, acc[DPL] = {};
  for (int i0 = 0; i0 < np; i0 += kWave) {
    float w = 0.0f;
    if (i0 + lane < np) {
      const float2 v = ml[i0 + lane];
      w = v.y * fast_exp2(v.x - ms);
    }
    const int cnt = min(kWave, np - i0);
    // eight partitions per step: their loads are issued together, then accumulated in
    // partition order (the order, and so the result, does not depend on the unrolling)
    constexpr int U = 8;
    for (int j0 = 0; j0 < cnt; j0 += U) {
      float v[U][DPL];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = min(j0 + u, cnt - 1);   // in-bounds; surplus slots get weight 0 below
        const float* src = po + (size_t)(i0 + j) * D;
#pragma unroll
        for (int e = 0; e < DPL; ++e) v[u][e] = src[e];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (j0 + u < cnt) {
          const float wj = __builtin_bit_cast(
              float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), j0 + u));
          L += wj;
#pragma unroll
          for (int e = 0; e < DPL; ++e) acc[e] = fmaf(wj, v[u][e], acc[e]);
        }
      }
    }
  }
  if (!act) return;
  const float inv = 1.0f / L;
  const size_t obase = (size_t)idx * D + lane * DPL;
#pragma unroll
  for (int e = 0; e < DPL; ++e) store_elem<dt>(p.out, obase + e, acc[e] * inv);
}

template <DT dt>
hipError_t launch_d(int d, const MergeParams& p, hipStream_t st) {
  const int grid = (p.num_seqs * p.num_heads + 3) / 4;
  if (grid == 0) return hipSuccess;
  switch (d) {
    case 64: hipLaunchKernelGGL((merge_kernel<dt, 64>), dim3(grid), dim3(256), 0, st, p); break;
    case 80: hipLaunchKernelGGL((merge_kernel<dt, 80>), dim3(grid), dim3(256), 0, st, p); break;
    case 128: hipLaunchKernelGGL((merge_kernel<dt, 128>), dim3(grid), dim3(256), 0, st, p); break;
    case 256: hipLaunchKernelGGL((merge_kernel<dt, 256>), dim3(grid), dim3(256), 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(DT dt, int head_dim, const MergeParams& p, hipStream_t st) {
  switch (dt) {
    case DT::F32: return launch_d<DT::F32>(head_dim, p, st);
    case DT::F16: return launch_d<DT::F16>(head_dim, p, st);
    case DT::BF16: return launch_d<DT::BF16>(head_dim, p, st);
    default: break;
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
