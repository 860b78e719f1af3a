#pragma once
// Paged decode attention for grouped-query attention on the matrix cores (gfx950): the kernel
// template, for head dims D = 64, 128 and 256.  pa_decode_mfma.hip (D = 128),
// pa_decode_mfma_d64.hip and pa_decode_mfma_d256.hip instantiate it for 16-bit caches,
// pa_decode_mfma_fp8.hip for 8-bit E4M3 caches at D = 128 (in parallel translation units).
//
// When G query heads share one KV head (the pages note that GQA/MQA shrinks the per-token KV
// cache: UltraLAB summary of Kwon et al. (xasun.com), boundary note after §八), the G queries
// against one K/V tile form two small dense products, S = Q K^T and O += P V.  They run on the
// matrix cores; the decode stays bound by HBM (about 4 flop per KV byte at G = 4), and the
// matrix cores take the multiply-adds off the vector ALUs.
//
// Tiling.  A wave consumes one 16-token chunk per step: a block of 16, a slice of a larger
// block, or two blocks of 8 (then K loads 0-1 and lanes 0-31 of the V loads read the first).
//   Scores: S^T[16 tokens x 16 cols] = K_chunk[16 x D] * Q^T[D x 16], D/32 (2, 4, 8)
//     v_mfma_f32_16x16x32 ops.  Column n holds query head n mod GT (heads are replicated when
//     GT < 16).  A operand (K): lane l holds K[token l%16][32kc + 8(l/16) .. +8]; B operand
//     (Q^T): lane l holds Q[head (l%16) mod GT][same 8 dims].  Result: lane l, register i holds
//     the score of token 4(l/16)+i for head (l%16) mod GT.
//   Output: O[16 rows x 16 cols] += P[16 x 16 tokens] * V[16 tokens x 16 cols], two
//     v_mfma_f32_16x16x16 ops per column group e = 0 .. D/16-1, column n meaning dim
//     (D/16) n + e.  The A operand (P) of lane l is head (l%16) mod GT at tokens 4(l/16) .. +4:
//     exactly the four scores the lane already holds, so P never moves between lanes.  The B
//     operand needs four tokens of one column per lane: lane l loads dims (D/16)(l%16) .. of
//     tokens 4(l/16) .. +4 (the 16 lanes of a token group cover whole rows) and transposes the
//     4 x D/16 16-bit tile in registers with v_perm_b32 (8-bit rows: the codes are gathered by
//     byte permutes first, then converted two at a time straight into operand order).
//   P is split into a 16-bit high part and a 16-bit remainder (two MFMAs per column group), so
//   the probabilities keep about 16 significant bits instead of the 8 of one bfloat16.
// Softmax state: a running reference point per head, shared by the four lanes holding that head
// (two permlane swaps per chunk for the chunk max); accumulators are rescaled only when
// some head's max passes its reference point by more than 2^8.
// Partitions.  A workgroup walks parts_per_wg consecutive partitions of one (sequence, KV head)
// (the host picks up to ~1024 tokens' worth when the grid stays large; one partition otherwise).
// Wave w takes chunks w, w+4, ... of the whole run, so with partitions of a multiple of 128
// tokens every wave holds the same number of chunks of each full partition.  When a wave has
// consumed its last chunk of a partition it leaves its state in that partition's LDS slot once
// the loads of its next chunk are issued (two chunks stay in flight); the last wave to finish
// the workgroup merges every partition's partial, so no wave waits for another.  The query and
// table prologue is paid once per workgroup.
#include <type_traits>

#include "pa_common.h"

namespace pa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

template <DT dt> struct Mfma;
template <> struct Mfma<DT::BF16> {
  __device__ __forceinline__ static f32x4 mma32(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  __device__ __forceinline__ static f32x4 mma16(uint2 a, uint2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                    __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
  }
  // values of the low and high 16-bit halves of a packed word
  __device__ __forceinline__ static float lo(uint32_t w) { return __uint_as_float(w << 16); }
  __device__ __forceinline__ static float hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
  __device__ __forceinline__ static uint32_t pack2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
  }
};
template <> struct Mfma<DT::F16> {
  __device__ __forceinline__ static f32x4 mma32(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                 __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ __forceinline__ static f32x4 mma16(uint2 a, uint2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
  }
  __device__ __forceinline__ static float lo(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
  }
  __device__ __forceinline__ static float hi(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
  }
  __device__ __forceinline__ static uint32_t pack2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, f16x2));
  }
};

constexpr float kLazy = 8.0f;   // running-max slack (log2 units): probabilities < 256

// Four E4M3 codes (one word) as four 16-bit values of the query type, two words.  Exact: every
// E4M3 value (3 mantissa bits, 2^-9 .. 448) is representable in bfloat16 and in fp16.  One
// scaled packed conversion per two codes, with scale 1 (gfx950 converts E4M3 pairs straight to
// 16-bit pairs; checked bit for bit against the convert-to-fp32-then-round path on every pair
// of codes, NaN included).
template <class M>
__device__ __forceinline__ uint2 fp8x4_to_16bit(uint32_t w) {
  if constexpr (std::is_same_v<M, Mfma<DT::BF16>>) {
    return make_uint2(
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)));
  } else {
    return make_uint2(
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true)));
  }
}

// The two 16-bit values of dim e (byte e % 4 of word e / 4) of four tokens' E4M3 rows, in
// token order: x01 / x23 hold the bytes k, k+1 (k = e & 2) of tokens 0, 1 / 2, 3 interleaved
// (one v_perm_b32 each, shared by dims k and k+1), and one scaled packed conversion of a half
// word turns two codes into two 16-bit values.  Gathering the codes before converting takes
// half the permutes of transposing the converted 16-bit values.
template <class M>
__device__ __forceinline__ uint32_t fp8x2_to_16bit(uint32_t w, bool hi) {
  if constexpr (std::is_same_v<M, Mfma<DT::BF16>>) {
    return hi ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true))
              : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  } else {
    return hi ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true))
              : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
  }
}

// 8-byte K/V load (rows of an 8-bit cache), streaming or cache-allocating like load_kv
template <bool STREAM>
__device__ __forceinline__ uint2 load_kv8(const void* ptr) {
  typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
  if constexpr (STREAM) {
    const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(ptr));
    return make_uint2(v.x, v.y);
  } else {
    return *reinterpret_cast<const uint2*>(ptr);
  }
}

// 4-byte K/V load (V pieces of an 8-bit cache at D = 64), streaming or cache-allocating
template <bool STREAM>
__device__ __forceinline__ uint32_t load_kv4(const void* ptr) {
  if constexpr (STREAM) return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(ptr));
  else return *reinterpret_cast<const uint32_t*>(ptr);
}

// W consecutive 32-bit words (W = 1, 2 or a multiple of 4) in the fewest loads
template <int W, bool STREAM>
__device__ __forceinline__ void load_words(uint32_t (&w)[W], const char* ptr) {
  if constexpr (W == 1) {
    w[0] = load_kv4<STREAM>(ptr);
  } else if constexpr (W == 2) {
    const uint2 v = load_kv8<STREAM>(ptr);
    w[0] = v.x;
    w[1] = v.y;
  } else {
    static_assert(W % 4 == 0, "whole 16-byte vectors");
#pragma unroll
    for (int i = 0; i < W / 4; ++i) {
      const uint4 v = load_kv<STREAM>(ptr + 16 * i);
      w[4 * i] = v.x;
      w[4 * i + 1] = v.y;
      w[4 * i + 2] = v.z;
      w[4 * i + 3] = v.w;
    }
  }
}

// Column e of a 4 x 2W tile of 16-bit values held as 4 rows of W words (row j = token j, word q
// = dims 2q, 2q+1): the 4 tokens' values of dim e, two per word, token order preserved.
template <int W>
__device__ __forceinline__ uint2 tile_column_words(const uint32_t (&r)[4][W], int e) {
  const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
  const int q = e >> 1;
  return make_uint2(__builtin_amdgcn_perm(r[1][q], r[0][q], sel),
                    __builtin_amdgcn_perm(r[3][q], r[2][q], sel));
}

// Raw chunk buffers: K as NK 16-byte loads of whole token rows, V as this lane's 4 token rows
// of D/16 dims, VW 32-bit words each (16-bit or 8-bit cache elements).
template <int NK, int VW> struct ChunkBuf { uint4 k[NK]; uint32_t v[4][VW]; };

// LDS slots for the per-partition wave states: at most 32 KiB, so 4, 2 or 1 partitions per
// workgroup (heads per workgroup x head dim up to 512, 1024, 2048).
constexpr int mfma_slots(int gt, int d) { return 2048 / (gt * d) >= 4 ? 4 : 2048 / (gt * d); }

// With an 8-bit cache the kernel is asked for three workgroups per CU: the compiler then fits it
// in <= 168 registers (three waves per SIMD, no spills), and the extra wave hides the loads of
// the shorter 8-bit chunks.  The 16-bit instances are built with their MFMA accumulators in
// ordinary VGPRs (176-180 registers, two waves per SIMD); asked for three waves they spill 7-10
// values and ran GQA long-context batches 13% slower.
// DP: the head dim of the queries, outputs and pools.  It equals D, except for heads of 80 dims,
// which run through the 128-dim products (D = 128, DP = 80) with dims 80 .. 127 zero in
// registers and LDS: they are never loaded or stored, add nothing to a score and give output
// dims that are dropped.
template <DT dt, DT kt, int D, int BS, int GT, bool STREAM, int DP = D>
__global__ __launch_bounds__(256, kt == DT::FP8 ? 3 : 1) void decode_mfma_kernel(const DecodeParams p) {
  static_assert(D == 64 || D == 128 || D == 256, "head dim");
  static_assert(DP == D || (D == 128 && DP == 80), "stored head dim: as computed, or 80 in 128");
  constexpr bool PAD = DP != D;
  constexpr int EB = 2;            // query / output element bytes
  constexpr bool K8 = kt == DT::FP8;
  constexpr int EBK = K8 ? 1 : 2;  // cache element bytes
  constexpr int ROW = D * EBK;     // token row in bytes
  constexpr int KC = D / 32;       // 32-dim depth steps of the score product
  constexpr int KCOL = D / 8;      // 16-byte columns (8 dims of 16-bit values) of a K row
  constexpr int DPL = D / 16;      // output dims per lane: column groups of O
  constexpr int NK = 16 * ROW / 1024;   // 1-KiB K loads per 16-token chunk
  constexpr int TPL = 1024 / ROW;  // token rows per K load
  constexpr int LPR = ROW / 16;    // lanes per token row in a K load
  constexpr int VW = DPL * EBK / 4;     // 32-bit words of this lane's piece of a V row
  // Stored rows (PAD): ROWP bytes, a chunk's 16 K rows one contiguous run of 16 ROWP bytes
  // loaded as 16-byte pieces (PPR a row), NKL loads of 64 pieces, the last one partial.
  constexpr int ROWP = DP * EBK;
  constexpr int PPR = ROWP / 16;
  constexpr int NKL = PAD ? (16 * PPR + 63) / 64 : NK;
  constexpr int KCE = PAD ? (DP + 31) / 32 : KC;   // depth steps that hold stored dims
  using Chunk = ChunkBuf<NKL, VW>;
  constexpr int CPB = BS >= 16 ? BS / 16 : 1;   // 16-token chunks per block
  constexpr int BPC = BS >= 16 ? 1 : 16 / BS;   // blocks per chunk (2 for 8-token blocks)
  static_assert(BS % 16 == 0 || BS == 8, "block size must be 8 or a multiple of 16");
  using M = Mfma<dt>;
  static_assert(GT == 4 || GT == 8 || GT == 16, "heads per workgroup");
  static_assert(GT * D <= 2048, "the partition slots must fit 32 KiB of LDS");

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform
  const int lr = lane & 15, kg = lane >> 4;

  // Workgroups are dealt round-robin to the 8 XCDs (id mod 8); the partition-group index is the
  // slowest grid index so every XCD gets an even share of (sequence, head) units.
  const int units = p.num_seqs * p.num_kv_heads * p.head_chunks;
  const int pg = blockIdx.x / units;
  const int unit = blockIdx.x - pg * units;
  const int hc = unit % (p.num_kv_heads * p.head_chunks);
  const int s = unit / (p.num_kv_heads * p.head_chunks);
  const int g = hc / p.head_chunks;
  const int h0 = g * p.group + (hc % p.head_chunks) * GT;
  const int p0 = pg * p.parts_per_wg;   // first partition of this workgroup
  // Workgroups past a sequence's last partition leave before any vector load (as in the
  // vector-ALU kernel); partition 0 always has work.
  if (p0 > 0) {
    const int n0 = min(p.context_lens[s], p.max_blocks_per_seq * BS);
    if (p0 * p.partition >= n0) return;
  }

  // Loads independent of the context length first (their latency overlaps the read of
  // context_lens): the Q^T operand and the table entries of this wave's first 64 chunks
  // (entries past the sequence's end are loaded but never used; all lie inside the row).
  const size_t q_row0 = ((size_t)s * p.num_heads + h0) * DP;
  const int32_t* table = p.block_tables + (size_t)s * p.max_blocks_per_seq;
  const int ch_begin = p0 * (p.partition / 16);
  uint4 qb[KC];  // Q^T operand (unscaled 16-bit values): chunk kc holds Q[h][32kc + 8kg .. +8]
  {
    const char* qp = (const char*)p.q + (q_row0 + (size_t)(lr % GT) * DP) * EB;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      if constexpr (PAD)
        qb[kc] = kc < KCE && 32 * kc + 8 * kg < DP
                     ? *reinterpret_cast<const uint4*>(qp + (32 * kc + 8 * kg) * EB)
                     : make_uint4(0, 0, 0, 0);
      else
        qb[kc] = *reinterpret_cast<const uint4*>(qp + (32 * kc + 8 * kg) * EB);
    }
  }
  // table entries of chunk ch: its block, or its two 8-token blocks (the second lies past the
  // table row when the row length is odd)
  auto fetch_entries = [&](int ch, int& e0, int& e1) {
    if constexpr (BPC == 1) {
      if (ch < p.max_blocks_per_seq * CPB) e0 = table[ch / CPB];
    } else {
      if (2 * ch < p.max_blocks_per_seq) e0 = table[2 * ch];
      if (2 * ch + 1 < p.max_blocks_per_seq) e1 = table[2 * ch + 1];
    }
  };
  int ent_first = -1, ent_first1 = -1;
  fetch_entries(ch_begin + wave + 4 * lane, ent_first, ent_first1);

  int n = p.context_lens[s];
  n = min(n, p.max_blocks_per_seq * BS);
  const int nparts = n > 0 ? (n + p.partition - 1) / p.partition : 1;
  if (p0 >= nparts) return;
  if (n <= 0) {  // empty context: the output is defined as zero
    if (threadIdx.x < GT * DP / 8)
      *reinterpret_cast<uint4*>((char*)p.out + (q_row0 * EB) + threadIdx.x * 16) =
          make_uint4(0, 0, 0, 0);
    return;
  }

  float m_run = -INFINITY;  // running max (log2 units) of head lr % GT
  float l_run = 0.0f;       // this lane's share of that head's denominator
  f32x4 acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int np_wg = min(nparts, p0 + p.parts_per_wg) - p0;   // partitions of this workgroup
  const int t_end = min(n, (p0 + np_wg) * p.partition);
  const int ch_end = (t_end + 15) / 16;
  const int Q = p.partition / 64;   // a wave's chunks in each full partition (used if np_wg > 1)
  const size_t head_off = (size_t)g * BS * DP;
  const size_t block_stride = (size_t)p.num_kv_heads * BS * DP;
  const int v_off = (4 * kg * DP + DPL * lr) * EBK;   // V rows: token 4kg (+j), dims DPL lr ..
  const bool v_live = !PAD || DPL * lr < DP;          // this lane's V dims are stored ones

  // K arrives coalesced (load i, lane l: token TPL i + l / LPR, 16-byte piece l % LPR -- each
  // load instruction reads whole rows) and is re-laid out through a wave-private LDS tile of 16
  // tokens x KCOL columns into the MFMA operand layout (token l%16, columns 4kc + l/16).
  // Loading the operand layout straight from HBM would cut every row into 64-byte pieces per
  // instruction, which measured ~15% slower at D = 128.  Slot of (token t, column c) is
  // KCOL t + (c xor swz(t)), swz(t) = t (t / 2 with 8 columns): writes and operand reads both
  // touch 16 distinct 16-byte bank groups per 16 lanes.
  __shared__ uint4 s_k[4][16 * KCOL];
  uint4* kst = s_k[wave];
  auto kslot = [](int t, int c) { return KCOL * t + (c ^ (KCOL >= 16 ? t : t >> 1)); };
  if constexpr (PAD) {
    // columns DP / 8 .. 4 KCE - 1 are read by the last depth step but hold no stored dims:
    // zero them once (the wave's own tile; nothing else writes them)
    constexpr int ZC = 4 * KCE - DP / 8;
    for (int z = lane; z < 16 * ZC; z += kWave)
      kst[kslot(z & 15, DP / 8 + z / 16)] = make_uint4(0, 0, 0, 0);
  }

  auto load_chunk = [&](Chunk& c, int phys0, int phys1, int ch) {
    const size_t el0 = (size_t)phys0 * block_stride + head_off + (size_t)(ch % CPB) * 16 * DP;
    // K: load i reads 1 KiB = TPL token rows, lane l 16 bytes of it
    const char* kp0 = (const char*)p.kc + el0 * EBK + lane * 16;
    const char* kp1 = kp0;
    const char* vp = (const char*)p.vc + el0 * EBK + v_off;
    if constexpr (BPC == 2) {
      // tokens 0-7 in block phys0, 8-15 in phys1 (at offsets 0-7 there)
      const size_t el1 = (size_t)phys1 * block_stride + head_off;
      kp1 = (const char*)p.kc + el1 * EBK + lane * 16 - 8 * ROWP;
      if (kg >= 2) vp = (const char*)p.vc + el1 * EBK + v_off - 8 * ROWP;
    }
    if constexpr (PAD) {
      // piece q = 64 i + lane of the chunk's 16 contiguous stored rows: token q / PPR; pieces
      // past the 16 rows are not loaded
#pragma unroll
      for (int i = 0; i < NKL; ++i) {
        const int q = 64 * i + lane;
        c.k[i] = make_uint4(0, 0, 0, 0);
        if (q < 16 * PPR) c.k[i] = load_kv<STREAM>((q / PPR < 8 ? kp0 : kp1) + 1024 * i);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (v_live) {
          load_words<VW, STREAM>(c.v[j], vp + j * ROWP);
        } else {
#pragma unroll
          for (int w = 0; w < VW; ++w) c.v[j][w] = 0;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < NK; ++i)   // token TPL i + lane / LPR: tokens 8-15 of an 8-token pair in phys1
        c.k[i] = load_kv<STREAM>((TPL * i + lane / LPR < 8 ? kp0 : kp1) + 1024 * i);
#pragma unroll
      for (int j = 0; j < 4; ++j) load_words<VW, STREAM>(c.v[j], vp + j * ROW);
    }
  };
  // End of partition p0 + k for this wave: it leaves its state (running max, denominator,
  // unnormalised outputs) in the partition's LDS slot and starts the next partition afresh.
  // Slots are never reused within a workgroup (the host gives a workgroup at most NBUF
  // partitions: 4, 2, 1 at 4, 8, 16 heads, 32 KiB of slots each), so no wave waits for another:
  // the last wave to finish the workgroup merges every partition (see the end of the kernel).
  constexpr int NBUF = mfma_slots(GT, D);
  __shared__ float s_o[NBUF][4][GT][D];
  __shared__ float s_m[NBUF][4][GT], s_l[NBUF][4][GT];
  __shared__ int s_done;
  if (threadIdx.x == 0) s_done = 0;
  __syncthreads();
  auto flush = [&](int k) {
    // this wave's denominator per head: sum the four token groups
    float lt = l_run + __shfl_xor(l_run, 16);
    lt += __shfl_xor(lt, 32);
    if (kg * 4 < GT) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < DPL; ++e) s_o[k][wave][kg * 4 + i][DPL * lr + e] = acc[e][i];
    }
    if (lane < GT) {
      s_m[k][wave][lane] = m_run;
      s_l[k][wave][lane] = lt;
    }
    m_run = -INFINITY;
    l_run = 0.0f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  // A consumed chunk that ends one of the workgroup's non-final partitions (those are full: Q
  // chunks per wave, Q even) leaves that partition pending; settle() flushes it right after the
  // next chunk's loads are issued.  Such a chunk has an odd index in the wave's run (Q even), so
  // it is always the second of an unrolled pair below, and every 64-chunk table block starts on
  // an even index: settling at the top of each pair, of each block and before a lone last chunk
  // is enough.
  int pending = -1;
  int left = Q, kpart = 0;   // this wave's chunks left in partition p0 + kpart
  auto settle = [&]() {
    if (pending >= 0) {
      flush(pending);
      pending = -1;
    }
  };

  // okm: bit b set when the chunk's block b has a valid id (both bits for blocks >= 16); this
  // lane's tokens 4kg .. 4kg+3 lie in block kg/2 of an 8-token pair
  auto consume = [&](Chunk& c, int ch, int okm) {
    const bool ok = ((okm >> (BPC == 1 ? 0 : kg >> 1)) & 1) != 0;
    if constexpr (PAD) {
      // piece q = 64 i + lane: token q / PPR, 16 bytes at q % PPR of its stored row -- 8
      // 16-bit dims (column q % PPR), or 16 codes that become columns 2 (q % PPR) and +1
#pragma unroll
      for (int i = 0; i < NKL; ++i) {
        const int q = 64 * i + lane;
        if (q < 16 * PPR) {
          const int t = q / PPR, j = q % PPR;
          if constexpr (K8) {
            const uint2 a = fp8x4_to_16bit<M>(c.k[i].x), b = fp8x4_to_16bit<M>(c.k[i].y);
            const uint2 d = fp8x4_to_16bit<M>(c.k[i].z), e = fp8x4_to_16bit<M>(c.k[i].w);
            kst[kslot(t, 2 * j)] = make_uint4(a.x, a.y, b.x, b.y);
            kst[kslot(t, 2 * j + 1)] = make_uint4(d.x, d.y, e.x, e.y);
          } else {
            kst[kslot(t, j)] = c.k[i];
          }
        }
      }
    } else if constexpr (K8) {
      // lane l of load i holds 16 codes: token TPL i + l / LPR, dims 16 (l % LPR) .. +15, which
      // become the 16-bit columns 2 (l % LPR) and 2 (l % LPR) + 1 of that token
#pragma unroll
      for (int i = 0; i < NK; ++i) {
        const int t = TPL * i + lane / LPR, c0 = 2 * (lane % LPR);
        const uint2 a = fp8x4_to_16bit<M>(c.k[i].x), b = fp8x4_to_16bit<M>(c.k[i].y);
        const uint2 d = fp8x4_to_16bit<M>(c.k[i].z), e = fp8x4_to_16bit<M>(c.k[i].w);
        kst[kslot(t, c0)] = make_uint4(a.x, a.y, b.x, b.y);
        kst[kslot(t, c0 + 1)] = make_uint4(d.x, d.y, e.x, e.y);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NK; ++i) kst[kslot(TPL * i + lane / LPR, lane % LPR)] = c.k[i];
    }
    uint4 kop[KCE];
#pragma unroll
    for (int kc = 0; kc < KCE; ++kc) kop[kc] = kst[kslot(lr, 4 * kc + kg)];
    f32x4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < KCE; ++kc) st = M::mma32(kop[kc], qb[kc], st);
    const int tok0 = ch * 16 + 4 * kg;   // token of register j is tok0 + j
    const bool full = okm == 3 && (ch * 16 + 16 <= t_end);
    float sv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) sv[j] = st[j] * p.scale_log2;
    if (!full) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool valid = ok && (tok0 + j < t_end);
        sv[j] = valid ? sv[j] : -INFINITY;
        if (!valid) {   // masked rows may hold NaN
#pragma unroll
          for (int w = 0; w < VW; ++w) c.v[j][w] = 0;
        }
      }
    }
    // chunk max per head over the four token groups (lanes l, l^16, l^32, l^48), with
    // permlane swaps on the vector ALUs rather than LDS round trips
    const float mn = row_max4_with(m_run, max4_valu(sv[0], sv[1], sv[2], sv[3]));
    // Lazy reference point: it moves only when a head's max exceeds it by more than kLazy
    // (always on the first live chunk, from -inf), so probabilities stay below 2^kLazy and the
    // rescale -- four cross-lane shuffles and 4 D/16 multiplies -- runs on few chunks instead of on
    // every chunk that sets a new max.  Any reference point gives the same o / l.
    const bool grow = mn > m_run + kLazy;
    if (__any(grow)) {
      const float alpha = grow ? fast_exp2(m_run - mn) : 1.0f;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = __shfl(alpha, (kg * 4 + i) % GT);
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[e][i] *= a;
      }
      m_run = grow ? mn : m_run;
    }
    const float ms = safe_max(m_run);
    float pv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      pv[j] = fast_exp2(sv[j] - ms);
      l_run += pv[j];
    }
    // 16-bit high parts of the probabilities (two per word, token 4kg + j in half j % 2), then
    // the 16-bit remainders p - high: packed round-to-nearest-even conversions, one instruction
    // per pair (the probabilities are finite and non-negative)
    const uint32_t h01 = M::pack2(pv[0], pv[1]), h23 = M::pack2(pv[2], pv[3]);
    const uint2 phi = make_uint2(h01, h23);
    const uint2 plo = make_uint2(M::pack2(pv[0] - M::lo(h01), pv[1] - M::hi(h01)),
                                 M::pack2(pv[2] - M::lo(h23), pv[3] - M::hi(h23)));
    if constexpr (K8) {
      // word w of row j holds the codes of dims DPL lr + 4w .. +3 of token 4kg + j
#pragma unroll
      for (int w = 0; w < VW; ++w) {
#pragma unroll
        for (int k = 0; k < 4; k += 2) {
          const uint32_t sel = k == 0 ? 0x05010400u : 0x07030602u;
          const uint32_t x01 = __builtin_amdgcn_perm(c.v[1][w], c.v[0][w], sel);
          const uint32_t x23 = __builtin_amdgcn_perm(c.v[3][w], c.v[2][w], sel);
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            const int e = 4 * w + k + b;
            const uint2 bv = make_uint2(fp8x2_to_16bit<M>(x01, b), fp8x2_to_16bit<M>(x23, b));
            acc[e] = M::mma16(phi, bv, acc[e]);
            acc[e] = M::mma16(plo, bv, acc[e]);
          }
        }
      }
    } else {
      uint32_t vb[4][DPL / 2];   // this lane's 4 V rows (dims DPL lr ..) as 16-bit values
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int w = 0; w < VW; ++w) vb[j][w] = c.v[j][w];
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        const uint2 bv = tile_column_words<DPL / 2>(vb, e);
        acc[e] = M::mma16(phi, bv, acc[e]);
        acc[e] = M::mma16(plo, bv, acc[e]);
      }
    }
    // a countdown, not a division by the runtime Q: full partitions hold Q chunks per wave
    if (np_wg > 1 && --left == 0) {
      left = Q;
      if (kpart < np_wg - 1) pending = kpart;
      ++kpart;
    }
  };

  // chunks of this wave: ch_begin + wave + 4*i; table entries fetched 64 at a time, one per
  // lane, and broadcast with readlane (the first 64 were fetched above)
  for (int base = ch_begin + wave; base < ch_end; base += 4 * kWave) {
    const int cnt = min(kWave, (ch_end - base + 3) / 4);
    int ent = ent_first, ent1 = ent_first1;
    if (base != ch_begin + wave) {
      ent = ent1 = -1;
      if (lane < cnt) fetch_entries(base + 4 * lane, ent, ent1);
    }
    // ids of chunk i's block(s); a bad id reads block 0 and its tokens are masked
    int ph0, ph1;
    auto phys_of = [&](int i, int& okm) {
      const int b0 = __builtin_amdgcn_readlane(ent, i);
      const bool ok0 = (unsigned)b0 < (unsigned)p.num_blocks;
      ph0 = ok0 ? b0 : 0;
      if constexpr (BPC == 1) {
        okm = ok0 ? 3 : 0;
        ph1 = ph0;
      } else {
        const int b1 = __builtin_amdgcn_readlane(ent1, i);
        const bool ok1 = (unsigned)b1 < (unsigned)p.num_blocks;
        ph1 = ok1 ? b1 : 0;
        okm = (ok0 ? 1 : 0) | (ok1 ? 2 : 0);
      }
    };
    // Two register buffers, steady-state loads unconditional (see the vector-ALU kernel).  A
    // scheduling barrier after each chunk's load issue keeps the intended order: without it
    // the compiler moved the next chunk's LDS stores of K -- and the wait for its K loads that
    // they need -- above the current chunk's products, so the chunk after next was issued only
    // once the next one had arrived (about 1.5 chunks in flight instead of 2).
    Chunk ca, cb;
    int oka, okb;
    phys_of(0, oka);
    load_chunk(ca, ph0, ph1, base);
    __builtin_amdgcn_sched_barrier(0);
    settle();
    int i = 0;
    for (; i + 2 < cnt; i += 2) {
      phys_of(i + 1, okb);
      load_chunk(cb, ph0, ph1, base + 4 * (i + 1));
      __builtin_amdgcn_sched_barrier(0);
      settle();
      consume(ca, base + 4 * i, oka);
      phys_of(i + 2, oka);
      load_chunk(ca, ph0, ph1, base + 4 * (i + 2));
      __builtin_amdgcn_sched_barrier(0);
      consume(cb, base + 4 * (i + 1), okb);
    }
    if (i + 1 < cnt) {
      phys_of(i + 1, okb);
      load_chunk(cb, ph0, ph1, base + 4 * (i + 1));
      __builtin_amdgcn_sched_barrier(0);
      settle();
      consume(ca, base + 4 * i, oka);
      consume(cb, base + 4 * (i + 1), okb);
    } else {
      settle();   // the loop's last pair may have ended a partition; no load is left to overlap
      consume(ca, base + 4 * i, oka);
    }
  }
  settle();
  flush(np_wg - 1);   // the workgroup's final partition (possibly partial, possibly empty here)

  // The last of the four waves to get here merges every partition of the workgroup into its
  // partial (or into the output when the sequence has one partition).  Each wave's LDS writes
  // complete before it counts itself in.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  int before = 0;
  if (lane == 0) before = atomicAdd(&s_done, 1);
  before = __builtin_amdgcn_readfirstlane(before);
  if (before != 3) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  constexpr int CPH = DP / 8;   // 8-dim pieces of a head's (stored) output
  for (int t = lane; t < np_wg * GT * CPH; t += kWave) {
    const int k = t / (GT * CPH), h = (t / CPH) % GT, cc = t % CPH;
    float Mx = s_m[k][0][h];
#pragma unroll
    for (int w = 1; w < 4; ++w) Mx = fmaxf(Mx, s_m[k][w][h]);
    const float ms = safe_max(Mx);
    float L = 0.0f, O[8] = {};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      // waves hold unnormalised sums relative to their own max: rescale both to M
      const float wt = fast_exp2(s_m[k][w][h] - ms);
      L = fmaf(wt, s_l[k][w][h], L);
#pragma unroll
      for (int e = 0; e < 8; ++e) O[e] = fmaf(wt, s_o[k][w][h][cc * 8 + e], O[e]);
    }
    const float inv = p.v_scale / L;   // an 8-bit cache's value scale factors out of the sum
#pragma unroll
    for (int e = 0; e < 8; ++e) O[e] *= inv;
    const size_t qrow = q_row0 + (size_t)h * DP;
    if (nparts == 1) {
      *reinterpret_cast<uint4*>((char*)p.out + (qrow + cc * 8) * EB) = Elem<dt>::pack(O);
    } else {
      const size_t slot = ((size_t)s * p.num_heads + h0 + h) * p.max_parts + p0 + k;
      float* po = p.ws_o + slot * DP + cc * 8;
      store_stream(po, O[0], O[1], O[2], O[3]);
      store_stream(po + 4, O[4], O[5], O[6], O[7]);
      if (cc == 0) *reinterpret_cast<float2*>(p.ws_ml + slot * 2) = make_float2(Mx, L);
    }
  }
}




template <DT dt, DT kt, int D, int BS, bool ST, int DP = D>
hipError_t launch_gt(int gt, const DecodeParams& p, int grid, hipStream_t st) {
  // the kernel holds LDS slots for mfma_slots(gt, D) partitions (and 16 heads need D <= 128)
  if (gt * D > 2048 || p.parts_per_wg < 1 || p.parts_per_wg > mfma_slots(gt, D))
    return hipErrorInvalidValue;
  switch (gt) {
    case 4: hipLaunchKernelGGL((decode_mfma_kernel<dt, kt, D, BS, 4, ST, DP>), dim3(grid), dim3(256), 0, st, p); break;
    case 8: hipLaunchKernelGGL((decode_mfma_kernel<dt, kt, D, BS, 8, ST, DP>), dim3(grid), dim3(256), 0, st, p); break;
    case 16:
      if constexpr (D <= 128) {
        hipLaunchKernelGGL((decode_mfma_kernel<dt, kt, D, BS, 16, ST, DP>), dim3(grid), dim3(256), 0, st, p);
        break;
      }
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <DT dt, DT kt, int D, int DP = D>
hipError_t launch_bs(int bs, int gt, bool sk, const DecodeParams& p, int grid, hipStream_t st) {
  auto go = [&](auto bs_tag) -> hipError_t {
    constexpr int BS = decltype(bs_tag)::value;
    return sk ? launch_gt<dt, kt, D, BS, true, DP>(gt, p, grid, st) : launch_gt<dt, kt, D, BS, false, DP>(gt, p, grid, st);
  };
  switch (bs) {
    case 8: return go(std::integral_constant<int, 8>{});
    case 16: return go(std::integral_constant<int, 16>{});
    case 32: return go(std::integral_constant<int, 32>{});
    case 64: return go(std::integral_constant<int, 64>{});
    case 128: return go(std::integral_constant<int, 128>{});
  }
  return hipErrorInvalidValue;
}

}  // namespace
}  // namespace pa
