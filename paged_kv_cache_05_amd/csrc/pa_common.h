// Shared device helpers and internal launcher declarations for libpa (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------------------
// Element types.  Every kernel moves data in 16-byte vectors (one global_load_dwordx4 per
// lane) and computes in fp32.
// ---------------------------------------------------------------------------------------
enum class DT { F32, F16, BF16, FP8 };   // FP8: OCP E4M3 ("FN"), cache element only

template <DT> struct Elem;

template <> struct Elem<DT::F32> {
  static constexpr int kBytes = 4;
  static constexpr int kPerVec = 4;
  __device__ __forceinline__ static void unpack(const uint4 v, float* f) {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  }
  __device__ __forceinline__ static uint4 pack(const float* f) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                      __float_as_uint(f[3]));
  }
};

__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}
__device__ __forceinline__ uint32_t f16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);  // v_cvt_f16_f32: nearest-even
}

template <> struct Elem<DT::F16> {
  static constexpr int kBytes = 2;
  static constexpr int kPerVec = 8;
  __device__ __forceinline__ static void unpack(const uint4 v, float* f) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = f16_lo(w[i]);
      f[2 * i + 1] = f16_hi(w[i]);
    }
  }
  __device__ __forceinline__ static uint4 pack(const float* f) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = f16_bits(f[2 * i]) | (f16_bits(f[2 * i + 1]) << 16);
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
};

// bfloat16 is the top half of an fp32 bit pattern.
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;  // NaN stays a quiet NaN
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;          // round to nearest, ties to even
}

template <> struct Elem<DT::BF16> {
  static constexpr int kBytes = 2;
  static constexpr int kPerVec = 8;
  __device__ __forceinline__ static void unpack(const uint4 v, float* f) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  __device__ __forceinline__ static uint4 pack(const float* f) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = bf16_bits(f[2 * i]) | (bf16_bits(f[2 * i + 1]) << 16);
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
};

// 8-bit E4M3 cache elements (OCP "FN" encoding: bias 7, max 448, no infinities).  gfx950's
// v_cvt_pk_f32_fp8 / v_cvt_pk_fp8_f32 use this encoding; the conversion to 8 bits rounds to
// nearest-even and turns values past 464 into NaN, so writers clamp to +-448 first.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
template <> struct Elem<DT::FP8> {
  static constexpr int kBytes = 1;
  static constexpr int kPerVec = 16;
  __device__ __forceinline__ static void unpack(const uint4 v, float* f) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(w[i], false);
      const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8(w[i], true);
      f[4 * i] = lo[0];
      f[4 * i + 1] = lo[1];
      f[4 * i + 2] = hi[0];
      f[4 * i + 3] = hi[1];
    }
  }
};

// Saturate to the largest finite E4M3 magnitude; NaN passes through (and encodes as NaN).
__device__ __forceinline__ float fp8_saturate(float y) {
  return y > 448.0f ? 448.0f : (y < -448.0f ? -448.0f : y);
}
// four floats -> four E4M3 codes in one word (byte i = element i)
__device__ __forceinline__ uint32_t fp8_pack4(float a, float b, float c, float d) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_pk_fp8_f32(fp8_saturate(a), fp8_saturate(b), w, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(fp8_saturate(c), fp8_saturate(d), w, true);
  return w;
}

// ---------------------------------------------------------------------------------------
// Cross-lane reductions inside groups of N consecutive lanes (N = 1, 8, 16, 32).  Every step
// pairs each lane with one partner and adds (or maxes) the two values; since a + b and b + a
// round identically, all lanes of a group end with the same bits.
// ---------------------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i inside each 8-lane half row
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i inside each 16-lane row

template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp<kDppXor1>(x);
  if constexpr (N >= 4) x += dpp<kDppXor2>(x);
  if constexpr (N >= 8) x += dpp<kDppHalfMirror>(x);
  if constexpr (N >= 16) x += dpp<kDppMirror>(x);
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  if constexpr (N >= 64) x += __shfl_xor(x, 32);
  return x;
}

template <int N>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (N >= 2) x = fmaxf(x, dpp<kDppXor1>(x));
  if constexpr (N >= 4) x = fmaxf(x, dpp<kDppXor2>(x));
  if constexpr (N >= 8) x = fmaxf(x, dpp<kDppHalfMirror>(x));
  if constexpr (N >= 16) x = fmaxf(x, dpp<kDppMirror>(x));
  if constexpr (N >= 32) x = fmaxf(x, __shfl_xor(x, 16));
  if constexpr (N >= 64) x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max(a, b) of two permlane-swap results as one v_max_f32.  fmaxf would first pass each
// operand through a canonicalising v_max (x, x), since the compiler cannot tell that a
// permlane output is no signalling NaN; these values are scores, -inf or NaNs that arithmetic
// produced, for which v_max_f32 alone gives the same result.  Only for operands written by a
// permlane swap: inline asm gets no hazard wait states from the compiler, and a VALU read right
// after a permlane swap needs none, while one right after an MFMA would.
__device__ __forceinline__ float max_of_swapped(uint32_t a, uint32_t b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Max over the four lanes l, l^16, l^32, l^48 (one query row of an MFMA output).  Each
// permlane swap leaves, in every lane, its own value and its partner's (lane ^ 32, then
// lane ^ 16) in the two results, whichever result holds which.
__device__ __forceinline__ float row_max4(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  x = max_of_swapped(a[0], a[1]);
  const uint32_t w = __float_as_uint(x);
  const auto b = __builtin_amdgcn_permlane16_swap(w, w, false, false);
  return max_of_swapped(b[0], b[1]);
}

// max of four values that vector-ALU instructions wrote (products, selects; never MFMA results,
// for the reason given at max_of_swapped), as v_max3_f32 + v_max_f32
__device__ __forceinline__ float max4_valu(float a, float b, float c, float d) {
  float r, t;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(t) : "v"(a), "v"(b), "v"(c));
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(t), "v"(d));
  return r;
}

// max(m, row_max4(x)), the last step one v_max3_f32 (m: a value the vector ALUs wrote, such
// as a running max, never an MFMA result)
__device__ __forceinline__ float row_max4_with(float m, float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  x = max_of_swapped(a[0], a[1]);
  const uint32_t w = __float_as_uint(x);
  const auto b = __builtin_amdgcn_permlane16_swap(w, w, false, false);
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(m), "v"(b[0]), "v"(b[1]));
  return r;
}

// Streaming 16-byte load: K/V tiles are read exactly once per call, so they are fetched with
// the non-temporal hint and do not displace reusable lines in the caches.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const void* ptr) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(ptr));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Split partials (fp32 normalised outputs of a partition) are written with the non-temporal
// hint: stored the ordinary way they cost the matrix-core decode ~3% on long GQA contexts
// (timing-only copies without the stores), written this way ~1-2% (the merge that reads them
// back right after is not slower).
typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_stream(float* ptr, float a, float b, float c, float d) {
  __builtin_nontemporal_store((f32x4_t){a, b, c, d}, reinterpret_cast<f32x4_t*>(ptr));
}

// K/V tile load: streaming by default; an ordinary (cache-allocating) load when the caller
// says blocks are shared by several sequences of the call, so later readers hit in L2.
template <bool STREAM>
__device__ __forceinline__ uint4 load_kv(const void* ptr) {
  if constexpr (STREAM) return load_stream(ptr);
  else return *reinterpret_cast<const uint4*>(ptr);
}

// Column e (0..7) of a 4x8 tile of 16-bit values held as 4 rows r[j] (row j = token j, word q
// = dims 2q, 2q+1): the 4 tokens' values of dim e, two per word, token order preserved.
__device__ __forceinline__ uint2 tile_column(const uint4 (&r)[4], int e) {
  const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
  auto word = [&](const uint4& v) -> uint32_t {
    const int q = e >> 1;
    return q == 0 ? v.x : q == 1 ? v.y : q == 2 ? v.z : v.w;
  };
  return make_uint2(__builtin_amdgcn_perm(word(r[1]), word(r[0]), sel),
                    __builtin_amdgcn_perm(word(r[3]), word(r[2]), sel));
}

// Softmax running state uses base-2 exponents: scores are pre-multiplied by log2(e).
// A running max of -inf means "no token seen"; exp2(x - safe(m)) is then 0 for every x
// that is itself -inf and the state stays empty.
__device__ __forceinline__ float safe_max(float m) { return m == -INFINITY ? 0.0f : m; }

// ---------------------------------------------------------------------------------------
// Launch parameters shared by the decode kernels (all sizes validated on the host).
// ---------------------------------------------------------------------------------------
struct DecodeParams {
  void* out;
  const void* q;
  const void* kc;
  const void* vc;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* ws_ml;   // [S][Hq][max_parts][2] (running max in log2 units, denominator)
  float* ws_o;    // [S][Hq][max_parts][D] normalised partial outputs
  int32_t num_seqs, num_heads, num_kv_heads, group;   // group = num_heads / num_kv_heads
  int32_t head_chunks;       // query-head chunks per KV head handled by separate workgroups
  int32_t max_blocks_per_seq, num_blocks;
  int32_t partition;         // tokens per partition (multiple of 16)
  int32_t max_parts;         // partitions a full table can hold
  int32_t parts_per_wg;      // consecutive partitions one matrix-core workgroup walks (1, 2, 4)
  float scale_log2;          // scale * log2(e) (times the key scale of an 8-bit cache)
  float v_scale;             // value scale of an 8-bit cache (1 otherwise)
};

struct MergeParams {
  void* out;
  const int32_t* context_lens;
  const float* ws_ml;
  const float* ws_o;
  int32_t num_seqs, num_heads, max_blocks_per_seq, block_size, partition, max_parts;
};

struct PrefillParams {
  void* out;                        // [T][Hq][D]
  const void* q;                    // [T][Hq][D]
  const void* kc;
  const void* vc;
  const int32_t* block_tables;
  const int32_t* query_start_loc;   // [S + 1]
  const int32_t* context_lens;      // [S], the chunk included
  int32_t num_seqs, num_heads, num_kv_heads, group;
  int32_t max_blocks_per_seq, num_blocks, max_query_len;
  int32_t row_tiles;                // workgroups per (sequence, KV head): ceil(max_query_len * G / 128)
  float scale_log2;                 // |scale| * log2(e), at least FLT_MIN (so it is > 0)
  uint32_t q_sign;                  // 0x80008000 when scale < 0: query signs are flipped instead
  // Key splits: each (sequence, KV head, row tile) is also cut into kv_splits workgroups over
  // key tiles [k * split_tiles, (k + 1) * split_tiles).  With kv_splits > 1 a token whose keys
  // span several splits gets per-split (max, denominator, normalised output) triples in
  // ws_ml / ws_o ([token][head][kv_splits] like the decode partitions) and tok_len[token] =
  // its position + 1 (0: leave the row to the prefill kernel or unwritten); the decode merge
  // kernel then combines them.
  int32_t kv_splits, split_tiles;
  int32_t num_tokens;               // rows of the workspace arrays (writes past them are skipped)
  int32_t* tok_len;
  float* ws_ml;
  float* ws_o;
  float v_scale;                    // value-pool scale of an E4M3 cache (1 for 16-bit pools)
};

// host-side launchers (return hipSuccess or the launch error)
hipError_t launch_decode_valu(DT dt, int head_dim, int block_size, int heads_per_wg,
                              bool stream_kv, const DecodeParams& p, int grid, hipStream_t st);
hipError_t launch_decode_valu_f16(int head_dim, int block_size, int heads_per_wg, bool stream_kv,
                                  const DecodeParams& p, int grid, hipStream_t st);
hipError_t launch_decode_valu_bf16(int head_dim, int block_size, int heads_per_wg, bool stream_kv,
                                   const DecodeParams& p, int grid, hipStream_t st);
hipError_t launch_decode_valu_fp8(DT dt, int head_dim, int block_size, int heads_per_wg,
                                  bool stream_kv, const DecodeParams& p, int grid, hipStream_t st);
hipError_t launch_decode_valu_fp8_dims(DT dt, int head_dim, int block_size, int heads_per_wg,
                                       bool stream_kv, const DecodeParams& p, int grid,
                                       hipStream_t st);
hipError_t launch_reshape_and_cache_fp8(DT dt, const void* key, const void* value, void* kc,
                                        void* vc, const int64_t* slots, int num_tokens,
                                        int head_dim, int block_size, int num_blocks,
                                        int num_kv_heads, float k_inv, float v_inv,
                                        hipStream_t st);
hipError_t launch_decode_mfma(DT dt, int head_dim, int block_size, int heads_per_wg,
                              bool stream_kv, const DecodeParams& p, int grid, hipStream_t st);
hipError_t launch_decode_mfma_d64(DT dt, int block_size, int heads_per_wg, bool stream_kv,
                                  const DecodeParams& p, int grid, hipStream_t st);
hipError_t launch_decode_mfma_d256(DT dt, int block_size, int heads_per_wg, bool stream_kv,
                                   const DecodeParams& p, int grid, hipStream_t st);
hipError_t launch_decode_mfma_fp8(DT dt, int head_dim, int block_size, int heads_per_wg,
                                  bool stream_kv, const DecodeParams& p, int grid, hipStream_t st);
hipError_t launch_decode_mfma_fp8_dims(DT dt, int head_dim, int block_size, int heads_per_wg,
                                       bool stream_kv, const DecodeParams& p, int grid,
                                       hipStream_t st);
hipError_t launch_prefill_mfma(DT dt, bool kv8, int head_dim, int block_size, bool split_p,
                               const PrefillParams& p, int grid, hipStream_t st);
hipError_t launch_prefill_mfma_d64(DT dt, bool kv8, int block_size, bool split_p,
                                   const PrefillParams& p, int grid, hipStream_t st);
hipError_t launch_prefill_mfma_d80(DT dt, bool kv8, int block_size, bool split_p,
                                   const PrefillParams& p, int grid, hipStream_t st);
hipError_t launch_merge(DT dt, int head_dim, const MergeParams& p, hipStream_t st);
hipError_t launch_reshape_and_cache(const void* key, const void* value, void* kc, void* vc,
                                    const int64_t* slots, int num_tokens, int row_vecs,
                                    int block_size, int num_blocks, int num_kv_heads,
                                    hipStream_t st);
// `count` (device, optional): only pairs below *count are copied (num_pairs bounds the grid)
hipError_t launch_block_copy(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                             const int64_t* mapping, int num_pairs, int64_t block_vecs,
                             int src_blocks, int dst_blocks, hipStream_t st,
                             const int32_t* count = nullptr);

// read-only bandwidth probe (pa_read_tiles); ids may be null (tile t is tile t)
hipError_t launch_read_tiles(const void* base, long base_tiles, int tile_bytes,
                             const int32_t* ids, int num_tiles, uint32_t* xor_out,
                             hipStream_t st);

struct EngineState {           // block-engine state kept on the device (all caller-owned)
  int32_t* tables;             // [num_seqs][max_blocks_per_seq]
  int32_t* context_lens;       // [num_seqs]
  int32_t* ref_counts;         // [num_blocks]
  int32_t* free_stack;         // [num_blocks]; entries below *free_top are free blocks
  int32_t* free_top;           // [1]
  int32_t num_seqs, max_blocks_per_seq, block_size, num_blocks;
};
hipError_t launch_append_slots(const EngineState& e, const int32_t* seq_ids, int n,
                               int64_t* slots, int64_t* pairs, int32_t* num_pairs,
                               int32_t* status, hipStream_t st);
hipError_t launch_fork(const EngineState& e, const int32_t* parent_child, int n, hipStream_t st);
hipError_t launch_free_seqs(const EngineState& e, const int32_t* seq_ids, int n, hipStream_t st);
hipError_t launch_block_hashes(const int32_t* tokens, const int32_t* num_tokens, int num_seqs,
                               int max_tokens, int block_size, uint64_t* hashes, hipStream_t st);

}  // namespace pa
