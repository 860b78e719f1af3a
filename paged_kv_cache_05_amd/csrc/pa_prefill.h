// Paged prefill attention on the matrix cores (gfx950): causal attention of a chunk of new
// tokens per sequence over the paged KV cache.
//
// Prefill is the compute-heavy phase before decoding (UltraLAB summary of Kwon et al.
// (xasun.com) §三, table row on the compute pattern), and serving engines may cut a long prompt
// into chunks (the chunked-prefill switch in the vLLM example on the PyTorch-CUDA-v2.9
// PagedAttention page, jsqmd.com).  Sequence s contributes L query rows; its n cached tokens
// already hold the chunk's own K/V (reshape_and_cache runs first), so chunk token i sits at
// position n - L + i and attends to positions 0 .. n - L + i, read block by block through the
// block table exactly as decode reads them.
//
// Head dims 64 and 128 (D below; the figures quote D = 128, the GPT-OSS-shaped D = 64 halves
// the depth steps and output blocks), and 80 (DP, the head dim of the queries, outputs and
// pools, below D): such rows run through the 128-dim products with dims DP .. 127 zero in
// registers and LDS -- they add nothing to a score and give output dims that are not stored.
//
// Work decomposition.  A workgroup (4 waves) owns 128 query rows of one (sequence, KV head):
// row r is chunk token r / G with query head kvh*G + r % G, so the G heads sharing a KV head
// share every K/V tile.  Each wave owns 32 rows.  Keys/values stream through LDS in tiles of
// 64 tokens, double-buffered: while the waves multiply tile k, every thread has tile k+1's
// loads in flight (four 16-byte rows of K and of V per thread) and stores them after its
// products.  One barrier per tile.
//
// Products, per wave and tile (v_mfma_f32_16x16x32, 16-bit operands, fp32 accumulation):
//   S^T[64 tokens x 32 rows] = K[64 x 128] Q^T[128 x 32]: 4 token blocks x 2 row blocks x 4
//     depth steps = 32 MFMAs.  A (K): lane l reads K[token 16j + l%16][dims 32c + 8(l/16) ..
//     +8] from LDS; B (Q^T): the wave's queries, held in registers for the whole loop.  Result:
//     lane l holds row 16n + l%16 at tokens 16j + 4(l/16) .. +4.
//   O^T[128 dims x 32 rows] += V^T[128 x 64] P^T[64 x 32]: 2 token halves x 8 dim blocks x 2
//     row blocks = 32 MFMAs.  The B operand (P^T) of lane l must be row l%16 at 8 tokens, which
//     are exactly 8 of the scores the lane already holds (tokens 4(l/16)+i of blocks 2h and
//     2h+1): the reduction order inside one MFMA is free, so P never moves between lanes.  The
//     A operand (V^T) needs 8 tokens of one dim per lane, so V is stored transposed in LDS, with
//     each dim row's tokens in the same order, making every A operand one 16-byte LDS read.
//   O^T keeps each query row in one lane column, so the softmax rescale of a row touches only
//   lanes that already hold that row's running max (no cross-lane traffic).
// With bfloat16 data, P is split into a 16-bit high part and remainder (two MFMAs per O^T
// product) so the probabilities keep about 16 significant bits; fp16 P keeps 11 bits in one.
//
// LDS layouts (16-byte chunks, swizzled so that the 8 lanes served per LDS cycle hit distinct
// banks on both the stores and the MFMA operand reads):
//   K tile  [64 tokens][D/8 chunks of 8 dims], chunk c of token t at slot c ^ (t & 15) (with
//           8 chunks, c ^ ((t ^ t/8) & 7), so rows t and t+8 of a 16-lane access differ).
//   V^T tile [128 dims][8 chunks of 8 token positions], chunk c of dim d at c ^ swz(d).
#pragma once

#include <type_traits>

#include "pa_common.h"

namespace pa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

template <DT dt> struct Mma;
template <> struct Mma<DT::BF16> {
  __device__ __forceinline__ static f32x4 mma(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static constexpr uint32_t kOnes = 0x3F803F80u;   // two bfloat16 ones
  __device__ __forceinline__ static uint32_t bits(float f) { return bf16_bits(f); }
  // E4M3 codes 0,1 (or 2,3) of a word as two bfloat16 values (exact), one instruction
  __device__ __forceinline__ static uint32_t fp8_lo(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  }
  __device__ __forceinline__ static uint32_t fp8_hi(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
  }
  // two values, nearest-even, in one v_cvt_pk_bf16_f32
  __device__ __forceinline__ static uint32_t pack2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
  }
};
template <> struct Mma<DT::F16> {
  __device__ __forceinline__ static f32x4 mma(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                 __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static constexpr uint32_t kOnes = 0x3C003C00u;   // two fp16 ones
  __device__ __forceinline__ static uint32_t bits(float f) { return f16_bits(f); }
  __device__ __forceinline__ static uint32_t fp8_lo(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
  }
  __device__ __forceinline__ static uint32_t fp8_hi(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
  }
  __device__ __forceinline__ static uint32_t pack2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, f16x2));
  }
};

constexpr int kTile = 64;        // KV tokens per LDS tile
constexpr int kRowsWave = 32;    // query rows per wave
constexpr int kRowsWG = 128;     // query rows per workgroup
constexpr float kLazy = 8.0f;    // running-max slack (log2 units): probabilities < 256

__device__ __forceinline__ int vswz(int d) { return (d ^ (d >> 3)) & 7; }

// With ON, the value as an opaque register: the compiler must take it as changed here, so the
// addresses derived from it are recomputed where they are used (one XOR each) instead of being
// hoisted out of the loop into a register apiece.  At head dim 64 (three waves per SIMD, 168
// registers) the hoisted addresses made the 16-bit instances spill 11-12 values; recomputed,
// they fit in 154-162 and the GPT-OSS-shaped prefill ran 6-11% faster.  At head dim 128 (two
// waves per SIMD) hoisting costs nothing, and recomputing made the 8-bit instances ~1% slower.
template <bool ON>
__device__ __forceinline__ int opaque(int v) {
  if constexpr (ON) asm volatile("" : "+v"(v));
  return v;
}

// Two workgroups per CU (two waves per SIMD, up to 256 registers) at D = 128.  At D = 64 the
// kernel is asked for three (168 registers): with the LDS addresses recomputed (opaque<>) every
// instance fits in 142-162 with no spills.
template <DT dt, int D, int BS, bool SPLIT_P, bool K8, int DP = D>
__global__ __launch_bounds__(256, D == 64 ? 3 : 2) void prefill_mfma_kernel(const PrefillParams p) {
  using M = Mma<dt>;
  static_assert(D == 64 || D == 128, "head dims 64 and 128");
  static_assert(DP <= D && DP % 16 == 0, "stored head dim: whole 16-dim output blocks");
  constexpr int kD = D;                     // head dim of the products
  constexpr int CHP = DP / 8;               // 16-byte chunks of a stored 16-bit row
  constexpr int kRow = kD * 2;              // bytes of a 16-bit token row
  constexpr int KC = kD / 32;               // 32-dim depth steps of the score product
  constexpr int NDB = kD / 16;              // 16-dim blocks of the output
  constexpr int CH = kD / 8;                // 16-byte chunks of a 16-bit row
  auto kswz = [](int t) { return CH == 16 ? (t & 15) : ((t ^ (t >> 3)) & 7); };
  // K8: E4M3 pools (128-byte token rows); the codes are widened to dt when a tile is stored in
  // LDS, so the products below are the 16-bit ones.  The key scale is folded into scale_log2 by
  // the host, the value scale into the final normalisation.
  constexpr int CROW = K8 ? DP : 2 * DP;    // bytes of one cached token row
  constexpr int CPIECE = K8 ? 8 : 16;       // bytes of a row one loader thread moves
  using Raw = std::conditional_t<K8, uint2, uint4>;
  static_assert(BS % 8 == 0, "a thread's 4 tokens must sit in one block");
  __shared__ uint4 s_k[2][kTile * CH];
  __shared__ uint4 s_v[2][kD * 8];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lr = lane & 15, lg = lane >> 4;

  // Work item.  Workgroups are dealt round-robin to the 8 XCDs (id mod 8).  Unit u =
  // (sequence, KV head) goes whole to XCD u mod 8 -- its row tiles and key splits, which read
  // the same K/V, share that XCD's L2 and run one after another -- and the units are dealt
  // round-robin, so every XCD gets the same KV heads of all sequences (units in contiguous
  // blocks per XCD would give an XCD whole sequences, whose work can differ several-fold).
  // Within a unit the last rows (longest causal range) come first, the key split fastest.
  const int KS = p.kv_splits;
  const int IPU = p.row_tiles * KS;                  // items per unit
  const int units = p.num_seqs * p.num_kv_heads;
  int unit, sub;
  if ((units & 7) == 0) {
    const int j = blockIdx.x >> 3;
    unit = (j / IPU) * 8 + (blockIdx.x & 7);
    sub = j - (j / IPU) * IPU;
  } else {
    unit = blockIdx.x / IPU;
    sub = blockIdx.x - unit * IPU;
  }
  const int ks = sub % KS;
  const int rt = p.row_tiles - 1 - sub / KS;
  const int kvh = unit % p.num_kv_heads;
  const int s = unit / p.num_kv_heads;

  const int q0 = p.query_start_loc[s];
  const int L_all = p.query_start_loc[s + 1] - q0;  // chunk length (sets the positions)
  const int L = min(L_all, p.max_query_len);        // rows this grid covers
  const int n = p.context_lens[s];
  const int G = p.group;
  const int rows = L * G;
  const int row0 = rt * kRowsWG;
  const bool fits = n >= L_all && n <= p.max_blocks_per_seq * BS;
  if (KS > 1 && kvh == 0 && rt == 0 && ks == 0) {
    // token lengths for the merge: position + 1 for the rows this grid covers; 0 for rows
    // written here directly (a chunk that does not fit: zeros) or left unwritten
    for (int t = tid; t < L_all && q0 + t < p.num_tokens; t += 256)
      p.tok_len[q0 + t] = (fits && t < L) ? n - L_all + t + 1 : 0;
  }
  if (L <= 0 || row0 >= rows) return;

  // element offset of row r's query / output vector
  auto row_off = [&](int r) -> size_t {
    const int t = r / G;
    return ((size_t)(q0 + t) * p.num_heads + kvh * G + (r - t * G)) * DP;
  };

  if (!fits) {  // the chunk does not fit its context: zeros (from the first key split)
    if (ks != 0) return;
    for (int idx = tid; idx < kRowsWG * CHP; idx += 256) {
      const int r = row0 + idx / CHP;
      if (r < rows)
        *reinterpret_cast<uint4*>((char*)p.out + row_off(r) * 2 + (idx % CHP) * 16) =
            make_uint4(0, 0, 0, 0);
    }
    return;
  }

  const int prefix = n - L_all;
  const int last_row = min(rows, row0 + kRowsWG) - 1;
  const int ntiles_all = (prefix + last_row / G + 1 + kTile - 1) / kTile;
  const int k_begin = ks * p.split_tiles;                     // this split's key tiles
  const int k_end = min(ntiles_all, k_begin + p.split_tiles);
  if (k_begin >= k_end) return;

  const int wrow0 = row0 + wave * kRowsWave;
  const bool wave_active = wrow0 < rows;
  const int w_kv_end = wave_active ? prefix + (min(rows, wrow0 + kRowsWave) - 1) / G + 1 : 0;
  const int w_kv_min = prefix + wrow0 / G;  // no row of the wave stops before this position

  // Q^T operand of the wave (16-bit values as stored) and the last position each of the
  // lane's two rows may attend to.  Rows past the chunk reuse the last row (never stored).
  uint4 qb[2][KC];
  int lim[2];
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2) {
    const int r = wrow0 + 16 * c2 + lr;
    const int rc = min(r, rows - 1);
    lim[c2] = prefix + rc / G;
    const char* qp = (const char*)p.q + row_off(rc) * 2;
#pragma unroll
    for (int c = 0; c < KC; ++c)
      qb[c2][c] = r < rows && 32 * c + 8 * lg < DP
                      ? *reinterpret_cast<const uint4*>(qp + (32 * c + 8 * lg) * 2)
                      : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      qb[c2][c].x ^= p.q_sign;
      qb[c2][c].y ^= p.q_sign;
      qb[c2][c].z ^= p.q_sign;
      qb[c2][c].w ^= p.q_sign;
    }
  }

  // Loader role: thread (tg, dc) moves tokens 4tg .. 4tg+3 of a tile, dims 8dc .. 8dc+7.  The
  // 16 lanes of each LDS write phase are two token groups (tg, tg+4, whose V^T rows use the
  // two 8-byte halves of a chunk) times 8 dim columns, so the transposed 8-byte writes land on
  // 16 distinct bank pairs; 8 lanes still cover 128 contiguous bytes of a K/V row.
  // With D = 64 the 16 x 8 (token group, dim column) pieces of a tile take the first 128
  // threads (waves 0 and 1); the others only multiply.
  const int p16 = tid >> 4, l16 = tid & 15;
  const int dc = CH == 16 ? ((l16 & 7) | ((p16 & 1) << 3)) : (l16 & 7);
  const int tg = CH == 16 ? (((p16 >> 1) & 3) | ((l16 >> 3) << 2) | ((p16 >> 3) << 3))
                          : (((p16 >> 1) & 3) | ((l16 >> 3) << 2) | ((p16 & 1) << 3));
  const bool loader = CH == 16 || tid < 128;   // wave-uniform
  // dims 8dc .. 8dc+7 are stored (below DP); the others are zero in LDS
  const bool dlive = DP == D || 8 * dc < DP;
  const int32_t* table = p.block_tables + (size_t)s * p.max_blocks_per_seq;
  const int nb_live = (n + BS - 1) / BS;
  const size_t head_off = (size_t)kvh * BS * CROW;
  const size_t blk_stride = (size_t)p.num_kv_heads * BS * CROW;
  auto entry = [&](int tile) -> int {
    const int page = (tile * kTile + 4 * tg) / BS;
    return (tile < k_end && page < nb_live) ? table[page] : -1;
  };
  Raw kr[4], vr[4];
  auto issue = [&](int tile, int ent) {
    const int t0 = tile * kTile + 4 * tg;
    // An id outside the pool (a broken table) is replaced by block 0, so no access leaves the
    // pools; slots past the context are never read.
    const size_t off = (size_t)((unsigned)ent < (unsigned)p.num_blocks ? ent : 0) * blk_stride +
                       head_off + (size_t)(t0 % BS) * CROW + dc * CPIECE;
    const char* kp = (const char*)p.kc + off;
    const char* vp = (const char*)p.vc + off;
    if (dlive && t0 + 3 < n) {   // the usual case: four live rows, unconditional loads
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        kr[i] = *reinterpret_cast<const Raw*>(kp + i * CROW);
        vr[i] = *reinterpret_cast<const Raw*>(vp + i * CROW);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool live = dlive && t0 + i < n;   // padded dims are never loaded
        Raw zk, zv;
        if constexpr (K8) {
          zk = zv = make_uint2(0, 0);
        } else {
          zk = zv = make_uint4(0, 0, 0, 0);
        }
        kr[i] = live ? *reinterpret_cast<const Raw*>(kp + i * CROW) : zk;
        vr[i] = live ? *reinterpret_cast<const Raw*>(vp + i * CROW) : zv;
      }
    }
  };
  // V^T position of this thread's tokens: token 32h + 16b + 4g + i sits at 32h + 8g + 4b + i,
  // so the 8 tokens one MFMA lane needs (4g+i of 16-token blocks 2h and 2h+1) are contiguous.
  const int v_chunk = 4 * (tg >> 3) + (tg & 3);
  const int v_half = (tg >> 2) & 1;
  // Swizzles split into a lane part and a compile-time part: the K chunk of the thread's token
  // 4tg + i is sk ^ i, the V^T chunk of its dim 8dc + e is sv ^ e; the score operand of lane
  // (lr, lg) at depth step c of token block j is klane ^ 4c (^ 2j mod 8 with 8 chunks a row);
  // the V^T operand of half h at dim block b is vlane[h] ^ (2b mod 8).
  const int sk = dc ^ kswz(4 * tg);
  const int sv = v_chunk ^ (dc & 7);
  const int klane = lg ^ (CH == 16 ? lr : ((lr & 7) ^ (lr >> 3)));
  const int vlane[2] = {lg ^ (lr & 7) ^ (lr >> 3), (4 + lg) ^ (lr & 7) ^ (lr >> 3)};
  // a loaded row piece as 8 values of dt (16 bytes): as loaded, or 8 E4M3 codes widened
  auto widen = [](const Raw& r) -> uint4 {
    if constexpr (K8) {
      return make_uint4(M::fp8_lo(r.x), M::fp8_hi(r.x), M::fp8_lo(r.y), M::fp8_hi(r.y));
    } else {
      return r;
    }
  };
  auto stash = [&](int buf) {
    const int skx = opaque<D == 64>(sk), svx = opaque<D == 64>(sv);
    uint4 kw[4], vw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kw[i] = widen(kr[i]);
      vw[i] = widen(vr[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 4 * tg + i;
      s_k[buf][t * CH + (skx ^ i)] = kw[i];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = 8 * dc + e;
      char* dst = reinterpret_cast<char*>(&s_v[buf][d * 8 + (svx ^ e)]) + 8 * v_half;
      *reinterpret_cast<uint2*>(dst) = tile_column(vw, e);
    }
  };

  f32x4 o[NDB][2];
#pragma unroll
  for (int dt2 = 0; dt2 < NDB; ++dt2) o[dt2][0] = o[dt2][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {-INFINITY, -INFINITY};  // running max of each row (log2 units)
  // Denominators on the matrix cores: ones^T P^T adds each row's probabilities exactly as
  // they enter O (16-bit parts included); every element of l_acc[c2] holds the row's sum.
  f32x4 l_acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  const uint4 ones = make_uint4(M::kOnes, M::kOnes, M::kOnes, M::kOnes);

  int ent_next = entry(k_begin + 1);
  if (loader) {
    issue(k_begin, entry(k_begin));
    stash(0);
  }
  __syncthreads();

  // The steps of one 32-token half h of the tile in LDS buffer `buf`:
  //   scores:  S^T = K Q^T (16 MFMAs)
  //   mask:    causal mask, only where the half reaches past some row's last position (a
  //            branch holding a scheduling barrier, so fully visible halves pay nothing)
  //   core:    row max (raw scores: scale > 0 commutes with max), lazy running max,
  //            probabilities exp2(s * scale_log2 - m) with one FMA each, packed as B operand
  //   rescale: O and l times alpha, only when some row's reference point moved (a branch)
  //   accumulate: l += ones^T P^T and O^T += V^T P^T on the matrix cores
  // Halves are software-pipelined inside the wave: the second half's score MFMAs sit in the
  // same basic block as the first half's softmax, and the first half's output MFMAs in the
  // same block as the second half's softmax, so the compiler's scheduler can let one wave keep
  // its matrix core and its vector ALU busy at once (the two halves are independent there;
  // the branches -- masking, rescale -- sit between those blocks).  Forcing a fixed
  // MFMA / VALU interleave with scheduling-group barriers measured much slower.
  using St = f32x4[2][2];   // [16-token block][row block]
  auto scores = [&](St& st, int buf, int h) {
    const int kl = opaque<D == 64>(klane);
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
      const int j = 2 * h + jb;
      st[jb][0] = st[jb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const uint4 a = s_k[buf][(16 * j + lr) * CH + (kl ^ (4 * c) ^ (CH == 16 ? 0 : (2 * j) & 7))];
        st[jb][0] = M::mma(a, qb[0][c], st[jb][0]);
        st[jb][1] = M::mma(a, qb[1][c], st[jb][1]);
      }
    }
  };
  auto mask = [&](St& st, int tstart) {
    if (tstart + 31 > w_kv_min) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (tstart + 16 * jb + 4 * lg + i > lim[c2]) st[jb][c2][i] = -INFINITY;
    }
  };
  // Lazy running max (log2 units): the reference point moves only when a row's max exceeds
  // it by more than kLazy, so probabilities stay below 2^kLazy and the O/l rescale runs only on
  // the few steps where some row's max jumps.  Any reference point gives the same o / l;
  // position 0, in every row's first half, makes the first step always move it from -inf.
  // Returns whether any row of the wave moved (alpha[c2] = its factor, 1 for the others).
  auto core = [&](St& st, uint4 (&ph)[2], uint4 (&pl)[2], float (&alpha)[2]) -> bool {
    bool any_grow = false;
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      float mx = -INFINITY;
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, st[jb][c2][i]);
      mx = row_max4(mx);
      const float ms = mx == -INFINITY ? -INFINITY : mx * p.scale_log2;
      const bool grow = ms > m_run[c2] + kLazy;
      const float m_new = grow ? ms : m_run[c2];
      alpha[c2] = grow ? fast_exp2(m_run[c2] - m_new) : 1.0f;
      m_run[c2] = m_new;
      any_grow |= grow;
      // a row with no key in this split yet keeps -inf: exp2(-inf) = 0, not NaN
      const float neg_m = m_new == -INFINITY ? 0.0f : -m_new;
      float pv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pv[e] = fast_exp2(fmaf(st[e >> 2][c2][e & 3], p.scale_log2, neg_m));
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        hw[e >> 1] = M::pack2(pv[e], pv[e + 1]);
        if constexpr (SPLIT_P) {
          const float r0 = pv[e] - __uint_as_float(hw[e >> 1] << 16);
          const float r1 = pv[e + 1] - __uint_as_float(hw[e >> 1] & 0xFFFF0000u);
          lw[e >> 1] = M::pack2(r0, r1);
        }
      }
      ph[c2] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      if constexpr (SPLIT_P) pl[c2] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    }
    return __any(any_grow);
  };
  auto rescale = [&](const float (&alpha)[2]) {
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      l_acc[c2] *= alpha[c2];
#pragma unroll
      for (int dt2 = 0; dt2 < NDB; ++dt2) o[dt2][c2] *= alpha[c2];
    }
  };
  auto accumulate = [&](const uint4 (&ph)[2], const uint4 (&pl)[2], int buf, int h) {
    const int vl = opaque<D == 64>(vlane[h]);
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      l_acc[c2] = M::mma(ones, ph[c2], l_acc[c2]);
      if constexpr (SPLIT_P) l_acc[c2] = M::mma(ones, pl[c2], l_acc[c2]);
    }
#pragma unroll
    for (int dt2 = 0; dt2 < NDB; ++dt2) {
      const int d = 16 * dt2 + lr;
      const uint4 a = s_v[buf][d * 8 + (vl ^ ((2 * dt2) & 7))];
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) o[dt2][c2] = M::mma(a, ph[c2], o[dt2][c2]);
      if constexpr (SPLIT_P) {
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) o[dt2][c2] = M::mma(a, pl[c2], o[dt2][c2]);
      }
    }
  };

  for (int k = k_begin; k < k_end; ++k) {
    const int buf = (k - k_begin) & 1;
    const bool more = k + 1 < k_end;
    const int ent_after = entry(k + 2);
    if (more && loader) issue(k + 1, ent_next);

    const int t0 = k * kTile;
    // A wave whose rows all end before this tile skips it; a second half past all of its rows
    // is masked whole (zero probabilities), which costs one idle half per wave at most.
    St st0, st1;
    uint4 ph0[2], pl0[2], ph1[2], pl1[2];
    float al0[2], al1[2];
    if (wave_active && t0 < w_kv_end) {   // wave-uniform
      scores(st0, buf, 0);
      mask(st0, t0);
      scores(st1, buf, 1);
      const bool g0 = core(st0, ph0, pl0, al0);
      mask(st1, t0 + 32);
      if (g0) rescale(al0);
      accumulate(ph0, pl0, buf, 0);
      const bool g1 = core(st1, ph1, pl1, al1);
      if (g1) rescale(al1);
      accumulate(ph1, pl1, buf, 1);
    }

    if (more && loader) stash(buf ^ 1);
    __syncthreads();
    ent_next = ent_after;
  }

  if (!wave_active) return;
  // Finalise: the four lanes holding a row add their denominators; lane l writes dims
  // 16b + 4(l/16) .. +4 of its rows.  A row whose keys all lie in one split is written here;
  // otherwise each split with keys for it writes its partial triple for the merge.
  const int split_len = p.split_tiles * kTile;
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2) {
    const float inv = p.v_scale / l_acc[c2][0];   // 1 for 16-bit pools
    const int r = wrow0 + 16 * c2 + lr;
    const int np = KS == 1 ? 1 : (lim[c2] + split_len) / split_len;   // splits holding its keys
    if (r < rows && np == 1 && ks == 0) {
      char* op = (char*)p.out + row_off(r) * 2;
#pragma unroll
      for (int dt2 = 0; dt2 < DP / 16; ++dt2) {   // stored dims only
        const f32x4 v = o[dt2][c2];
        const uint2 w2 = make_uint2(M::bits(v[0] * inv) | (M::bits(v[1] * inv) << 16),
                                    M::bits(v[2] * inv) | (M::bits(v[3] * inv) << 16));
        *reinterpret_cast<uint2*>(op + (16 * dt2 + 4 * lg) * 2) = w2;
      }
    } else if (r < rows && np > 1 && ks < np && q0 + r / G < p.num_tokens) {
      const size_t slot = (row_off(r) / DP) * KS + ks;
      float* po = p.ws_o + slot * DP;
#pragma unroll
      for (int dt2 = 0; dt2 < DP / 16; ++dt2) {
        const f32x4 v = o[dt2][c2];
        *reinterpret_cast<float4*>(po + 16 * dt2 + 4 * lg) =
            make_float4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
      }
      if (lg == 0) *reinterpret_cast<float2*>(p.ws_ml + 2 * slot) = make_float2(m_run[c2], l_acc[c2][0]);
    }
  }
}

template <DT dt, int D, int BS, bool SPLIT, bool K8, int DP>
hipError_t go(const PrefillParams& p, int grid, hipStream_t st) {
  hipLaunchKernelGGL((prefill_mfma_kernel<dt, D, BS, SPLIT, K8, DP>), dim3(grid), dim3(256), 0, st, p);
  return hipGetLastError();
}

// every instance of head dim D (stored head dim DP): query type, probability split, cache
// element, block size
template <int D, int DP = D>
hipError_t launch_prefill_d(DT dt, bool kv8, int block_size, bool split_p,
                            const PrefillParams& p, int grid, hipStream_t st) {
  auto by_bs = [&](auto dt_tag, auto split_tag, auto k8_tag) -> hipError_t {
    constexpr DT T = decltype(dt_tag)::value;
    constexpr bool SP = decltype(split_tag)::value;
    constexpr bool K8 = decltype(k8_tag)::value;
    switch (block_size) {
      case 8: return go<T, D, 8, SP, K8, DP>(p, grid, st);
      case 16: return go<T, D, 16, SP, K8, DP>(p, grid, st);
      case 32: return go<T, D, 32, SP, K8, DP>(p, grid, st);
      case 64: return go<T, D, 64, SP, K8, DP>(p, grid, st);
      case 128: return go<T, D, 128, SP, K8, DP>(p, grid, st);
    }
    return hipErrorInvalidValue;
  };
  auto by_kv = [&](auto dt_tag, auto split_tag) -> hipError_t {
    return kv8 ? by_bs(dt_tag, split_tag, std::true_type{})
               : by_bs(dt_tag, split_tag, std::false_type{});
  };
  using BF = std::integral_constant<DT, DT::BF16>;
  using HF = std::integral_constant<DT, DT::F16>;
  if (dt == DT::BF16)
    return split_p ? by_kv(BF{}, std::true_type{}) : by_kv(BF{}, std::false_type{});
  if (dt == DT::F16) return by_kv(HF{}, std::false_type{});
  return hipErrorInvalidValue;
}

}  // namespace
}  // namespace pa
