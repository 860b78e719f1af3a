#pragma once
// Paged decode attention for grouped-query attention on the matrix cores (gfx950): the kernel
// template.  pa_decode_mfma.hip instantiates it for 16-bit caches, pa_decode_mfma_fp8.hip for
// 8-bit E4M3 caches (in parallel translation units).
//
// When G query heads share one KV head (the pages note that GQA/MQA shrinks the per-token KV
// cache: UltraLAB summary of Kwon et al. (xasun.com), boundary note after §八), the G queries
// against one K/V tile form two small dense products, S = Q K^T and O += P V.  They run on the
// matrix cores; the decode stays bound by HBM (about 4 flop per KV byte at G = 4), and the
// matrix cores take the multiply-adds off the vector ALUs.
//
// Tiling.  A wave consumes one 16-token chunk per step: a block of 16, a slice of a larger
// block, or two blocks of 8 (then K loads 0-1 and lanes 0-31 of the V loads read the first).
//   Scores: S^T[16 tokens x 16 cols] = K_chunk[16 x 128] * Q^T[128 x 16], four
//     v_mfma_f32_16x16x32 ops.  Column n holds query head n mod GT (heads are replicated when
//     GT < 16).  A operand (K): lane l holds K[token l%16][32kc + 8(l/16) .. +8]; B operand
//     (Q^T): lane l holds Q[head (l%16) mod GT][same 8 dims].  Result: lane l, register i holds
//     the score of token 4(l/16)+i for head (l%16) mod GT.
//   Output: O[16 rows x 16 cols] += P[16 x 16 tokens] * V[16 tokens x 16 cols], eight
//     v_mfma_f32_16x16x16 ops per column group e = 0..7, column n meaning dim 8n + e.  The A
//     operand (P) of lane l is head (l%16) mod GT at tokens 4(l/16) .. +4: exactly the four
//     scores the lane already holds, so P never moves between lanes.  The B operand needs four
//     tokens of one column per lane: lane l loads dims 8(l%16) .. +8 of tokens 4(l/16) .. +4
//     (each load instruction reads four whole 256-byte rows) and transposes the 4x8 16-bit
//     tile in registers with v_perm_b32.
//   P is split into a 16-bit high part and a 16-bit remainder (two MFMAs per column group), so
//   the probabilities keep about 16 significant bits instead of the 8 of one bfloat16.
// Softmax state: a running reference point per head, shared by the four lanes holding that head
// (two permlane swaps per chunk for the chunk max); accumulators are rescaled only when
// some head's max passes its reference point by more than 2^8.
// Partitions, wave interleaving, prefetch and the final merge follow the vector-ALU kernel.
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
  __device__ __forceinline__ static uint32_t bits(float f) { return bf16_bits(f); }
  __device__ __forceinline__ static float value(uint32_t b) { return __uint_as_float(b << 16); }
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
  __device__ __forceinline__ static uint32_t bits(float f) { return f16_bits(f); }
  __device__ __forceinline__ static float value(uint32_t b) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
  }
  __device__ __forceinline__ static uint32_t pack2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, f16x2));
  }
};

constexpr float kLazy = 8.0f;   // running-max slack (log2 units): probabilities < 256

// Four E4M3 codes (one word) as four 16-bit values of the query type, two words.  Exact: every
// E4M3 value (3 mantissa bits, 2^-9 .. 448) is representable in bfloat16 and in fp16.
template <class M>
__device__ __forceinline__ uint2 fp8x4_to_16bit(uint32_t w) {
  const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  return make_uint2(M::pack2(lo[0], lo[1]), M::pack2(hi[0], hi[1]));
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

// Raw chunk buffers: 16-bit cache (K: 4 loads of 4 token rows; V: this lane's 4 rows of 8
// dims) or 8-bit cache (K: 2 loads of 8 token rows; V: 4 rows of 8 dims, 8 bytes each).
struct Chunk16 { uint4 k[4]; uint4 v[4]; };
struct Chunk8 { uint4 k[2]; uint2 v[4]; };

// With an 8-bit cache the kernel is asked for three workgroups per CU: the compiler then fits it
// in <= 168 registers (three waves per SIMD, no spills), and the extra wave hides the loads of
// the shorter 8-bit chunks (GQA long, E4M3: 163-171 -> 133-140 us).  The 16-bit instances keep
// the compiler's own choice (224-232 registers, two waves): three waves measured within +-2%.
template <DT dt, DT kt, int BS, int GT, bool STREAM>
__global__ __launch_bounds__(256, kt == DT::FP8 ? 3 : 1) void decode_mfma_kernel(const DecodeParams p) {
  constexpr int D = 128;
  constexpr int EB = 2;            // query / output element bytes
  constexpr bool K8 = kt == DT::FP8;
  constexpr int EBK = K8 ? 1 : 2;  // cache element bytes
  constexpr int ROW = D * EBK;     // token row: 256 bytes (16-bit cache) or 128 (8-bit)
  using Chunk = std::conditional_t<K8, Chunk8, Chunk16>;
  constexpr int CPB = BS >= 16 ? BS / 16 : 1;   // 16-token chunks per block
  constexpr int BPC = BS >= 16 ? 1 : 16 / BS;   // blocks per chunk (2 for 8-token blocks)
  static_assert(BS % 16 == 0 || BS == 8, "block size must be 8 or a multiple of 16");
  using M = Mfma<dt>;
  static_assert(GT == 4 || GT == 8 || GT == 16, "heads per workgroup");

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform
  const int lr = lane & 15, kg = lane >> 4;

  // Workgroups are dealt round-robin to the 8 XCDs (id mod 8); the partition index is the
  // slowest grid index so every XCD gets an even share of (sequence, head) units.
  const int units = p.num_seqs * p.num_kv_heads * p.head_chunks;
  const int part = blockIdx.x / units;
  const int unit = blockIdx.x - part * units;
  const int hc = unit % (p.num_kv_heads * p.head_chunks);
  const int s = unit / (p.num_kv_heads * p.head_chunks);
  const int g = hc / p.head_chunks;
  const int h0 = g * p.group + (hc % p.head_chunks) * GT;
  // Workgroups past a sequence's last partition leave before any vector load (as in the
  // vector-ALU kernel); partition 0 always has work.
  if (part > 0) {
    const int n0 = min(p.context_lens[s], p.max_blocks_per_seq * BS);
    if (part * p.partition >= n0) return;
  }

  // Loads independent of the context length first (their latency overlaps the read of
  // context_lens): the Q^T operand and the table entries of this wave's first 64 chunks
  // (entries past the sequence's end are loaded but never used; all lie inside the row).
  const size_t q_row0 = ((size_t)s * p.num_heads + h0) * D;
  const int32_t* table = p.block_tables + (size_t)s * p.max_blocks_per_seq;
  const int ch_begin = part * (p.partition / 16);
  uint4 qb[4];  // Q^T operand (unscaled 16-bit values): chunk kc holds Q[h][32kc + 8kg .. +8]
  {
    const char* qp = (const char*)p.q + (q_row0 + (size_t)(lr % GT) * D) * EB;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
      qb[kc] = *reinterpret_cast<const uint4*>(qp + (32 * kc + 8 * kg) * EB);
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
  if (part >= nparts) return;
  if (n <= 0) {  // empty context: the output is defined as zero
    if (threadIdx.x < GT * 16)
      *reinterpret_cast<uint4*>((char*)p.out + (q_row0 * EB) + threadIdx.x * 16) =
          make_uint4(0, 0, 0, 0);
    return;
  }

  float m_run = -INFINITY;  // running max (log2 units) of head lr % GT
  float l_run = 0.0f;       // this lane's share of that head's denominator
  f32x4 acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int t_end = min(n, (part + 1) * p.partition);
  const int ch_end = (t_end + 15) / 16;
  const size_t head_off = (size_t)g * BS * D;
  const size_t block_stride = (size_t)p.num_kv_heads * BS * D;
  const int v_off = (4 * kg * D + 8 * lr) * EBK;   // V rows: token 4kg (+j), dims 8lr..

  // K arrives coalesced (load i, lane l: token 4i + l/16, 16-byte column l%16 -- each load
  // instruction reads four whole rows) and is re-laid out through a wave-private 4 KiB LDS tile
  // into the MFMA operand layout (token l%16, columns 4kc + l/16).  Loading the operand layout
  // straight from HBM would cut every row into 64-byte pieces per instruction, which measured
  // ~15% slower.  Slot of (token t, column c) is 16t + (c xor t): writes and operand reads both
  // touch 16 distinct 16-byte bank groups per 16 lanes.
  __shared__ uint4 s_k[4][256];
  uint4* kst = s_k[wave];

  auto load_chunk = [&](Chunk& c, int phys0, int phys1, int ch) {
    const size_t el0 = (size_t)phys0 * block_stride + head_off + (size_t)(ch % CPB) * 16 * D;
    // K: load i reads 1 KiB = 1024 / ROW token rows (4 or 8), lane l 16 bytes of it
    constexpr int NK = K8 ? 2 : 4;
    constexpr int TPL = 1024 / ROW;   // token rows per K load
    const char* kp0 = (const char*)p.kc + el0 * EBK + lane * 16;
    const char* kp1 = kp0;
    const char* vp = (const char*)p.vc + el0 * EBK + v_off;
    if constexpr (BPC == 2) {
      // tokens 0-7 in block phys0, 8-15 in phys1 (at offsets 0-7 there)
      const size_t el1 = (size_t)phys1 * block_stride + head_off;
      kp1 = (const char*)p.kc + el1 * EBK + lane * 16 - 8 * ROW;
      if (kg >= 2) vp = (const char*)p.vc + el1 * EBK + v_off - 8 * ROW;
    }
#pragma unroll
    for (int i = 0; i < NK; ++i) c.k[i] = load_kv<STREAM>((i * TPL < 8 ? kp0 : kp1) + 1024 * i);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (K8) c.v[j] = load_kv8<STREAM>(vp + j * ROW);
      else c.v[j] = load_kv<STREAM>(vp + j * ROW);
    }
  };
  // okm: bit b set when the chunk's block b has a valid id (both bits for blocks >= 16); this
  // lane's tokens 4kg .. 4kg+3 lie in block kg/2 of an 8-token pair
  auto consume = [&](Chunk& c, int ch, int okm) {
    const bool ok = ((okm >> (BPC == 1 ? 0 : kg >> 1)) & 1) != 0;
    if constexpr (K8) {
      // lane l of load i holds 16 codes: token 8i + l/8, dims 16(l%8) .. +15, which become the
      // 16-bit columns 2(l%8) and 2(l%8)+1 of that token
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int t = 8 * i + (lane >> 3), c0 = 2 * (lane & 7);
        const uint2 a = fp8x4_to_16bit<M>(c.k[i].x), b = fp8x4_to_16bit<M>(c.k[i].y);
        const uint2 d = fp8x4_to_16bit<M>(c.k[i].z), e = fp8x4_to_16bit<M>(c.k[i].w);
        kst[16 * t + (c0 ^ t)] = make_uint4(a.x, a.y, b.x, b.y);
        kst[16 * t + ((c0 + 1) ^ t)] = make_uint4(d.x, d.y, e.x, e.y);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) kst[16 * (4 * i + kg) + (lr ^ (4 * i + kg))] = c.k[i];
    }
    uint4 kop[4];
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) kop[kc] = kst[16 * lr + ((4 * kc + kg) ^ lr)];
    f32x4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) st = M::mma32(kop[kc], qb[kc], st);
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
          if constexpr (K8) c.v[j] = make_uint2(0, 0);
          else c.v[j] = make_uint4(0, 0, 0, 0);
        }
      }
    }
    // chunk max per head over the four token groups (lanes l, l^16, l^32, l^48), with
    // permlane swaps on the vector ALUs rather than LDS round trips
    const float bm = row_max4(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
    // Lazy reference point: it moves only when a head's max exceeds it by more than kLazy
    // (always on the first live chunk, from -inf), so probabilities stay below 2^kLazy and the
    // rescale -- four cross-lane shuffles and 32 multiplies -- runs on few chunks instead of on
    // every chunk that sets a new max.  Any reference point gives the same o / l.
    const float mn = fmaxf(m_run, bm);
    const bool grow = mn > m_run + kLazy;
    if (__any(grow)) {
      const float alpha = grow ? fast_exp2(m_run - mn) : 1.0f;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = __shfl(alpha, (kg * 4 + i) % GT);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e][i] *= a;
      }
      m_run = grow ? mn : m_run;
    }
    const float ms = safe_max(m_run);
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float pj = fast_exp2(sv[j] - ms);
      l_run += pj;
      hi[j] = M::bits(pj);
      lo[j] = M::bits(pj - M::value(hi[j]));
    }
    const uint2 phi = make_uint2(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16));
    const uint2 plo = make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
    uint4 vb[4];   // this lane's 4 V rows (dims 8lr .. +8) as 16-bit values
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (K8) {
        const uint2 a = fp8x4_to_16bit<M>(c.v[j].x), b = fp8x4_to_16bit<M>(c.v[j].y);
        vb[j] = make_uint4(a.x, a.y, b.x, b.y);
      } else {
        vb[j] = c.v[j];
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint2 bv = tile_column(vb, e);
      acc[e] = M::mma16(phi, bv, acc[e]);
      acc[e] = M::mma16(plo, bv, acc[e]);
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
    int i = 0;
    for (; i + 2 < cnt; i += 2) {
      phys_of(i + 1, okb);
      load_chunk(cb, ph0, ph1, base + 4 * (i + 1));
      __builtin_amdgcn_sched_barrier(0);
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
      consume(ca, base + 4 * i, oka);
      consume(cb, base + 4 * (i + 1), okb);
    } else {
      consume(ca, base + 4 * i, oka);
    }
  }

  // this wave's denominator per head: sum the four token groups
  float lt = l_run + __shfl_xor(l_run, 16);
  lt += __shfl_xor(lt, 32);

  __shared__ float s_o[4][GT][D];
  __shared__ float s_m[4][GT], s_l[4][GT];
  if (kg * 4 < GT) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) s_o[wave][kg * 4 + i][8 * lr + e] = acc[e][i];
  }
  if (lane < GT) {
    s_m[wave][lane] = m_run;
    s_l[wave][lane] = lt;
  }
  __syncthreads();
  if (threadIdx.x < GT * 16) {
    const int h = threadIdx.x / 16, cc = threadIdx.x % 16;
    float Mx = s_m[0][h];
#pragma unroll
    for (int w = 1; w < 4; ++w) Mx = fmaxf(Mx, s_m[w][h]);
    const float ms = safe_max(Mx);
    float L = 0.0f, O[8] = {};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      // waves hold unnormalised sums relative to their own max: rescale both to M
      const float wt = fast_exp2(s_m[w][h] - ms);
      L = fmaf(wt, s_l[w][h], L);
#pragma unroll
      for (int e = 0; e < 8; ++e) O[e] = fmaf(wt, s_o[w][h][cc * 8 + e], O[e]);
    }
    const float inv = p.v_scale / L;   // an 8-bit cache's value scale factors out of the sum
#pragma unroll
    for (int e = 0; e < 8; ++e) O[e] *= inv;
    const size_t qrow = q_row0 + (size_t)h * D;
    if (nparts == 1) {
      *reinterpret_cast<uint4*>((char*)p.out + (qrow + cc * 8) * EB) = Elem<dt>::pack(O);
    } else {
      const size_t slot = ((size_t)s * p.num_heads + h0 + h) * p.max_parts + part;
      float* po = p.ws_o + slot * D + cc * 8;
      *reinterpret_cast<float4*>(po) = make_float4(O[0], O[1], O[2], O[3]);
      *reinterpret_cast<float4*>(po + 4) = make_float4(O[4], O[5], O[6], O[7]);
      if (cc == 0) *reinterpret_cast<float2*>(p.ws_ml + slot * 2) = make_float2(Mx, L);
    }
  }
}

template <DT dt, DT kt, int BS, bool ST>
hipError_t launch_gt(int gt, const DecodeParams& p, int grid, hipStream_t st) {
  switch (gt) {
    case 4: hipLaunchKernelGGL((decode_mfma_kernel<dt, kt, BS, 4, ST>), dim3(grid), dim3(256), 0, st, p); break;
    case 8: hipLaunchKernelGGL((decode_mfma_kernel<dt, kt, BS, 8, ST>), dim3(grid), dim3(256), 0, st, p); break;
    case 16: hipLaunchKernelGGL((decode_mfma_kernel<dt, kt, BS, 16, ST>), dim3(grid), dim3(256), 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <DT dt, DT kt>
hipError_t launch_bs(int bs, int gt, bool sk, const DecodeParams& p, int grid, hipStream_t st) {
  auto go = [&](auto bs_tag) -> hipError_t {
    constexpr int BS = decltype(bs_tag)::value;
    return sk ? launch_gt<dt, kt, BS, true>(gt, p, grid, st) : launch_gt<dt, kt, BS, false>(gt, p, grid, st);
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
