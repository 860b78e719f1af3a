#pragma once
// Paged decode attention on the vector ALUs (gfx950, wave64): the kernel template.  The
// per-element-type files pa_decode_valu_*.hip instantiate it (in parallel translation units).
//
// What is computed: for one query per (sequence, head), softmax-weighted sum of V over the
// sequence's cached tokens, with K/V fetched block by block through the block table (UltraLAB
// summary of Kwon et al. (xasun.com) §二, attention-algorithm item; scaled dot-product
// attention, "PagedAttention技术：加速GPT推理的利器" (yunthe.com) §1.1).
//
// Work decomposition.  One workgroup (4 waves) per (sequence, KV head, query-head chunk,
// partition of P tokens).  Splitting one sequence over partitions is what lets long contexts
// spread over all 256 CUs; the partial results are merged exactly by their log-sum-exp
// weights (pa_merge.hip).  A partition is cut into 16-token chunks; wave w takes chunks w,
// w+4, w+8, ...  A chunk is a slice of one block (blocks of 16 tokens and more) or two whole
// 8-token blocks, each with its own table entry.
//
// Data path for one chunk.  A (block, KV head) tile is block_size * head_dim contiguous
// elements.  One 16-byte load per lane moves 1 KiB per wave: with LPT = head_dim*elem/16 lanes
// per token row, a wave covers TPI = 64/LPT consecutive tokens per load instruction, fully
// coalesced.  Scores are reduced over the LPT lanes of a row with DPP; each row of lanes keeps
// its own online-softmax state (running max, denominator, partial output), so the loop has no
// cross-row traffic.  Rows and waves are merged once, at the end of the partition.
// The next chunk's K and V loads are issued before the current chunk is consumed.
#include <type_traits>

#include "pa_common.h"


namespace pa {
namespace {

template <DT dt, DT kt, int D, int BS, int GT>
struct ValuCfg {
  using E = Elem<kt>;                        // cache elements
  using Q = Elem<dt>;                        // query / output elements
  static constexpr int EPL = E::kPerVec;     // elements per lane per 16-byte vector
  static constexpr int QV = EPL / Q::kPerVec;  // query vectors per lane (2 for an 8-bit cache)
  static constexpr int VC = D / EPL;         // 16-byte vectors per token row
  // lanes per token row: VC rounded up to a power of two (rows of 80 or 96 dims leave the
  // last lanes of each row idle, so DPP reductions still run over a whole lane group)
  static constexpr int LPT = VC <= 8 ? 8 : VC <= 16 ? 16 : 32;
  static constexpr int TPI = kWave / LPT;    // tokens per wave load instruction
  static constexpr int NI = 16 / TPI;        // load instructions per 16-token chunk
  static constexpr int CPB = BS >= 16 ? BS / 16 : 1;   // chunks per block
  static constexpr int BPC = BS >= 16 ? 1 : 16 / BS;   // blocks per chunk (2 for 8-token blocks)
  static constexpr int ROW_BYTES = D * E::kBytes;
  static_assert(VC * EPL == D && VC >= 4 && VC <= 32, "row must be 4..32 whole vectors");
  static_assert(BS % 16 == 0 || BS == 8, "block size must be 8 or a multiple of 16");
  static_assert(TPI <= BS, "one load instruction must stay inside one block");
};

template <DT dt, DT kt, int D, int BS, int GT, bool STREAM>
__global__ __launch_bounds__(256) void decode_valu_kernel(const DecodeParams p) {
  using C = ValuCfg<dt, kt, D, BS, GT>;
  using E = typename C::E;
  using Q = typename C::Q;
  constexpr int EPL = C::EPL, LPT = C::LPT, TPI = C::TPI, NI = C::NI, CPB = C::CPB, QV = C::QV;
  constexpr int BPC = C::BPC;
  constexpr int VC = C::VC;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform
  const int row = lane / LPT;   // token slot inside one load instruction
  const int col = lane % LPT;   // 16-byte column of the token row
  const bool act = col < VC;    // idle padding lanes (VC < LPT) read column VC-1, weight 0
  const int colc = act ? col : VC - 1;

  // Workgroups are dealt round-robin to the 8 XCDs (id mod 8).  The partition index is the
  // slowest index of the work item so every XCD gets an even share of (sequence, KV head)
  // units; with it fastest, XCD k would receive only partition k.  When a KV head's query
  // heads take several workgroups (head chunks), those read the same K/V: their ids are 8
  // apart (id = 8 * (HC * j + chunk) + x), so they run on one XCD at about the same time and
  // the later ones find the tiles in that XCD's L2.  The grid is padded to a multiple of 8 HC;
  // padding items fall past the last partition and exit.
  const int HC = p.head_chunks;
  int chunk = 0, item = blockIdx.x;
  if (HC > 1) {
    const int y = blockIdx.x >> 3;
    chunk = y % HC;
    item = (y / HC) * 8 + (blockIdx.x & 7);
  }
  const int ukv = p.num_seqs * p.num_kv_heads;
  const int part = item / ukv;
  const int r = item - part * ukv;
  const int s = r / p.num_kv_heads;
  const int g = r - s * p.num_kv_heads;
  const int h0 = g * p.group + chunk * GT;
  // The grid holds every partition a full table could need, so workgroups past a sequence's
  // last partition are common (tables sized for long contexts, short sequences).  Such a
  // workgroup reads the length alone and leaves before issuing any vector load: with the
  // query and table loads below in flight it would have to wait for them before ending.
  // Partition 0 always has work, so it skips this check and keeps the early loads.
  if (part > 0) {
    const int n0 = min(p.context_lens[s], p.max_blocks_per_seq * BS);
    if (part * p.partition >= n0) return;
  }

  // Loads that do not depend on the context length go first, so their latency overlaps the
  // read of context_lens: the query rows and the table entries of this wave's first chunks
  // (entries past the sequence's end are loaded but never used; all lie inside the table row).
  const size_t q_row0 = ((size_t)s * p.num_heads + h0) * D;
  const int32_t* table = p.block_tables + (size_t)s * p.max_blocks_per_seq;
  const int ch_begin = part * (p.partition / 16);
  uint4 qraw[GT][QV];
#pragma unroll
  for (int h = 0; h < GT; ++h)
#pragma unroll
    for (int v = 0; v < QV; ++v)
      qraw[h][v] = *reinterpret_cast<const uint4*>(
          (const char*)p.q + (q_row0 + (size_t)h * D + colc * EPL) * Q::kBytes + 16 * v);
  // table entries of chunk ch: its block (blocks of >= 16 tokens), or its two blocks e0, e1
  // (8-token blocks; the second lies past the table row when the row length is odd)
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
    if (wave == 0 && row == 0 && act) {
      const float z[EPL] = {};
#pragma unroll
      for (int h = 0; h < GT; ++h)
#pragma unroll
        for (int v = 0; v < QV; ++v)
          *reinterpret_cast<uint4*>((char*)p.out + (q_row0 + (size_t)h * D + col * EPL) * Q::kBytes +
                                    16 * v) = Q::pack(z);
    }
    return;
  }

  // query, pre-scaled by scale*log2(e) (and the key scale of an 8-bit cache), as fp32
  float qf[GT][EPL];
#pragma unroll
  for (int h = 0; h < GT; ++h) {
#pragma unroll
    for (int v = 0; v < QV; ++v) Q::unpack(qraw[h][v], qf[h] + v * Q::kPerVec);
    if (!act) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) qf[h][e] = 0.0f;
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) qf[h][e] *= p.scale_log2;
  }

  float m[GT], l[GT], o[GT][EPL];
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[h][e] = 0.0f;
  }

  const int t_end = min(n, (part + 1) * p.partition);
  const int ch_end = (t_end + 15) / 16;
  const size_t head_off = (size_t)g * BS * D;               // elements
  const size_t block_stride = (size_t)p.num_kv_heads * BS * D;
  const int lane_off = (row * D + colc * EPL) * E::kBytes;   // bytes inside a 16-token chunk

  // address of this lane's first vector of chunk `ch` (physical block `phys`); with 8-token
  // blocks, of the chunk's half in block `phys`
  auto chunk_ptr = [&](const void* base, int phys, int ch) -> const char* {
    const size_t el = (size_t)phys * block_stride + head_off + (size_t)(ch % CPB) * 16 * D;
    return (const char*)base + el * E::kBytes + lane_off;
  };
  // load i covers chunk tokens i*TPI + row, inside the chunk's block i*TPI*BPC/16
  auto load_chunk = [&](uint4 (&kb)[NI], uint4 (&vb)[NI], int phys0, int phys1, int ch) {
    const char* kp0 = chunk_ptr(p.kc, phys0, ch);
    const char* vp0 = chunk_ptr(p.vc, phys0, ch);
    const char* kp1 = BPC == 1 ? kp0 : chunk_ptr(p.kc, phys1, ch);
    const char* vp1 = BPC == 1 ? vp0 : chunk_ptr(p.vc, phys1, ch);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int t = i * TPI, hb = BPC == 1 ? 0 : t / BS;
      kb[i] = load_kv<STREAM>((hb ? kp1 : kp0) + (t - hb * BS) * C::ROW_BYTES);
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int t = i * TPI, hb = BPC == 1 ? 0 : t / BS;
      vb[i] = load_kv<STREAM>((hb ? vp1 : vp0) + (t - hb * BS) * C::ROW_BYTES);
    }
  };
  // okm: bit b set when the chunk's block b has a valid id (both bits for blocks >= 16)
  auto consume = [&](const uint4 (&kb)[NI], const uint4 (&vb)[NI], int ch, int okm) {
    const int tok0 = ch * 16 + row;
    const bool full = okm == 3 && (ch * 16 + 16 <= t_end);
    auto ok_of = [&](int i) { return ((okm >> (BPC == 1 ? 0 : i * TPI / BS)) & 1) != 0; };
    float sc[NI][GT];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float kf[EPL];
      E::unpack(kb[i], kf);
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        float acc = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc = fmaf(qf[h][e], kf[e], acc);
        sc[i][h] = group_sum<LPT>(acc);
      }
      if (!full) {
        const bool valid = ok_of(i) && (tok0 + i * TPI < t_end);
#pragma unroll
        for (int h = 0; h < GT; ++h) sc[i][h] = valid ? sc[i][h] : -INFINITY;
      }
    }
    float pr[NI][GT];
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      float bm = sc[0][h];
#pragma unroll
      for (int i = 1; i < NI; ++i) bm = fmaxf(bm, sc[i][h]);
      const float mn = fmaxf(m[h], bm);
      const float ms = safe_max(mn);
      const float alpha = fast_exp2(m[h] - ms);
      float ps = 0.0f;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        pr[i][h] = fast_exp2(sc[i][h] - ms);
        ps += pr[i][h];
      }
      l[h] = l[h] * alpha + ps;
      m[h] = mn;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[h][e] *= alpha;
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float vf[EPL];
      E::unpack(vb[i], vf);
      if (!full) {
        const bool valid = ok_of(i) && (tok0 + i * TPI < t_end);
#pragma unroll
        for (int e = 0; e < EPL; ++e) vf[e] = valid ? vf[e] : 0.0f;  // masked slots may hold NaN
      }
#pragma unroll
      for (int h = 0; h < GT; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[h][e] = fmaf(pr[i][h], vf[e], o[h][e]);
    }
  };

  // chunks of this wave: ch_begin + wave + 4*i; their table entries are fetched 64 at a time,
  // one per lane, and broadcast with readlane (the first 64 were fetched above)
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
    // Two register buffers; in the steady state every iteration issues the next chunk's
    // loads unconditionally before consuming the current one, so the wait before a consume
    // covers only the older chunk (a conditional load would force a wait for everything).
    uint4 ka[NI], va[NI], kb[NI], vb[NI];
    int oka, okb;
    phys_of(0, oka);
    load_chunk(ka, va, ph0, ph1, base);
    int i = 0;
    for (; i + 2 < cnt; i += 2) {
      phys_of(i + 1, okb);
      load_chunk(kb, vb, ph0, ph1, base + 4 * (i + 1));
      consume(ka, va, base + 4 * i, oka);
      phys_of(i + 2, oka);
      load_chunk(ka, va, ph0, ph1, base + 4 * (i + 2));
      consume(kb, vb, base + 4 * (i + 1), okb);
    }
    if (i + 1 < cnt) {
      phys_of(i + 1, okb);
      load_chunk(kb, vb, ph0, ph1, base + 4 * (i + 1));
      consume(ka, va, base + 4 * i, oka);
      consume(kb, vb, base + 4 * (i + 1), okb);
    } else {
      consume(ka, va, base + 4 * i, oka);
    }
  }

  // merge the rows of each wave (xor-butterfly over lane groups)
#pragma unroll
  for (int off = LPT; off < kWave; off <<= 1) {
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      const float mp = __shfl_xor(m[h], off);
      const float lp = __shfl_xor(l[h], off);
      const float mn = fmaxf(m[h], mp);
      const float ms = safe_max(mn);
      const float a0 = fast_exp2(m[h] - ms), a1 = fast_exp2(mp - ms);
      l[h] = l[h] * a0 + lp * a1;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[h][e] = o[h][e] * a0 + __shfl_xor(o[h][e], off) * a1;
      m[h] = mn;
    }
  }

  // merge the 4 waves through LDS
  __shared__ float s_o[4][GT][D];
  __shared__ float s_m[4][GT], s_l[4][GT];
  if (row == 0 && act) {
#pragma unroll
    for (int h = 0; h < GT; ++h) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_o[wave][h][col * EPL + e] = o[h][e];
      if (col == 0) {
        s_m[wave][h] = m[h];
        s_l[wave][h] = l[h];
      }
    }
  }
  __syncthreads();
  if (threadIdx.x < GT * LPT && (int)(threadIdx.x % LPT) < VC) {
    const int h = threadIdx.x / LPT, cc = threadIdx.x % LPT;
    float M = s_m[0][h];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, s_m[w][h]);
    const float ms = safe_max(M);
    float L = 0.0f, O[EPL] = {};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      // waves hold unnormalised sums relative to their own max: rescale both to M
      const float wt = fast_exp2(s_m[w][h] - ms);
      L = fmaf(wt, s_l[w][h], L);
#pragma unroll
      for (int e = 0; e < EPL; ++e) O[e] = fmaf(wt, s_o[w][h][cc * EPL + e], O[e]);
    }
    const float inv = p.v_scale / L;   // an 8-bit cache's value scale factors out of the sum
#pragma unroll
    for (int e = 0; e < EPL; ++e) O[e] *= inv;
    const size_t qrow = q_row0 + (size_t)h * D;
    if (nparts == 1) {
#pragma unroll
      for (int v = 0; v < QV; ++v)
        *reinterpret_cast<uint4*>((char*)p.out + (qrow + cc * EPL) * Q::kBytes + 16 * v) =
            Q::pack(O + v * Q::kPerVec);
    } else {
      const size_t slot = ((size_t)s * p.num_heads + h0 + h) * p.max_parts + part;
      float* po = p.ws_o + slot * D + cc * EPL;
#pragma unroll
      for (int e = 0; e < EPL; e += 4)
        store_stream(po + e, O[e], O[e + 1], O[e + 2], O[e + 3]);
      if (cc == 0) *reinterpret_cast<float2*>(p.ws_ml + slot * 2) = make_float2(M, L);
    }
  }
}

// Heads per workgroup a (cache type, head dim) may use: each lane keeps EPL fp32 outputs per
// head, and past ~64 of them occupancy drops to one wave per SIMD (or registers spill).
template <DT kt, int D>
constexpr int max_heads_per_wg() {
  if constexpr (kt == DT::FP8 || D >= 256) return 2;
  else if constexpr (D == 80 || D == 96) return 4;
  else return 8;
}

template <DT dt, DT kt, int D, int BS, bool ST>
hipError_t launch_gt(int gt, const DecodeParams& p, int grid, hipStream_t st) {
  constexpr int kMax = max_heads_per_wg<kt, D>();
  if (gt > kMax) return hipErrorInvalidValue;
  switch (gt) {
    case 1: hipLaunchKernelGGL((decode_valu_kernel<dt, kt, D, BS, 1, ST>), dim3(grid), dim3(256), 0, st, p); break;
    case 2: hipLaunchKernelGGL((decode_valu_kernel<dt, kt, D, BS, 2, ST>), dim3(grid), dim3(256), 0, st, p); break;
    case 4:
      if constexpr (kMax >= 4) {
        hipLaunchKernelGGL((decode_valu_kernel<dt, kt, D, BS, 4, ST>), dim3(grid), dim3(256), 0, st, p);
        break;
      }
      return hipErrorInvalidValue;
    case 8:
      if constexpr (kMax >= 8) {
        hipLaunchKernelGGL((decode_valu_kernel<dt, kt, D, BS, 8, ST>), dim3(grid), dim3(256), 0, st, p);
        break;
      }
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <DT dt, DT kt, int D>
hipError_t launch_bs(int bs, int gt, bool stream_kv, const DecodeParams& p, int grid, hipStream_t st) {
  auto go = [&](auto bs_tag) -> hipError_t {
    constexpr int BS = decltype(bs_tag)::value;
    return stream_kv ? launch_gt<dt, kt, D, BS, true>(gt, p, grid, st)
                     : launch_gt<dt, kt, D, BS, false>(gt, p, grid, st);
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
