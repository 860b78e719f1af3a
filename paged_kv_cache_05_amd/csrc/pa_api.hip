// C ABI of libpa: argument checks, launch planning and dispatch.  Everything here runs on
// the host from host scalars only: no device memory is read, nothing synchronises, nothing
// is allocated.  Declarations and the contract of every entry point are in include/pa.h.
#include <algorithm>
#include <cmath>
#include <cstddef>

#include "pa_common.h"

namespace {

using pa::DT;

constexpr int32_t kVersion = 1 * 10000 + 0 * 100 + 0;
constexpr long kMinPartition = 256;      // tokens per split-KV partition, lower bound
constexpr long kMaxPartition = 2048;     // and upper bound
constexpr long kTargetWorkgroups = 2048; // 256 CUs x 8 resident 4-wave workgroups

// Element types of query / output / 16-bit-or-wider caches.
bool dtype_of(pa_dtype d, DT* out) {
  switch (d) {
    case PA_F32: *out = DT::F32; return true;
    case PA_F16: *out = DT::F16; return true;
    case PA_BF16: *out = DT::BF16; return true;
    default: break;
  }
  return false;
}
// Element types a pool may hold (the block copies move bytes of any of them).
bool pool_dtype_of(pa_dtype d, DT* out) {
  if (d == PA_FP8_E4M3) {
    *out = DT::FP8;
    return true;
  }
  return dtype_of(d, out);
}
int elem_bytes(DT d) { return d == DT::F32 ? 4 : d == DT::FP8 ? 1 : 2; }
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct Plan {
  int partition = 0;     // tokens per partition
  int max_parts = 1;
  size_t ws_ml_bytes = 0;
  size_t ws_bytes = 0;   // total workspace (0: single pass)
};

// Shape checks shared by every decode entry point.
pa_status check_shape(int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t BS, int32_t maxb,
                      int32_t partition_size) {
  if (S < 0 || Hq <= 0 || Hkv <= 0 || maxb <= 0 || partition_size < 0) return PA_ERR_BAD_SHAPE;
  if (Hq % Hkv != 0) return PA_ERR_BAD_SHAPE;
  if ((long)S * Hq > 0x7FFFFFFFL) return PA_ERR_BAD_SHAPE;   // (sequence, head) ids are int32
  if (D != 64 && D != 80 && D != 128 && D != 256) return PA_ERR_UNSUPPORTED;
  if (BS != 8 && BS != 16 && BS != 32 && BS != 64 && BS != 128) return PA_ERR_UNSUPPORTED;
  // partitions hold whole blocks and whole 16-token chunks
  if (partition_size > 0 && partition_size % std::max<int32_t>(BS, 16) != 0) return PA_ERR_BAD_SHAPE;
  if ((long)maxb * BS > (1L << 30)) return PA_ERR_BAD_SHAPE;
  return PA_OK;
}

// Split only as far as needed to give ~kTargetWorkgroups workgroups, since every extra
// workgroup repeats the table/query prologue and every split adds a merge; but never let one
// workgroup stream more than kMaxPartition tokens, which bounds the tail when lengths are
// skewed.  Measured on MI355X (Llama-7B-shaped batch of 256): 2048-token partitions beat 512 by
// ~3%; with few (sequence, KV head) units, small partitions are what fills the GPU.
int auto_partition(int32_t S, int32_t Hkv, int32_t BS, int32_t maxb) {
  const long cap = (long)maxb * BS;
  const long units = (long)S * Hkv;
  if (units <= 0) return 0;   // an empty batch: nothing to split
  const long parts = std::max(1L, (kTargetWorkgroups + units - 1) / units);
  long P = (cap + parts - 1) / parts;
  P = std::min<long>(std::max<long>(P, kMinPartition), kMaxPartition);
  const long q = std::max(32, (int)BS);   // partitions hold whole blocks
  P = (P + q - 1) / q * q;
  if (P >= cap) return 0;  // one pass
  return (int)P;
}

Plan make_plan(int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t BS, int32_t maxb,
               int32_t partition_size) {
  Plan pl;
  const long cap = (long)maxb * BS;
  int P = partition_size > 0 ? partition_size : auto_partition(S, Hkv, BS, maxb);
  if (P == 0 || P >= cap) {
    pl.partition = (int)((cap + 31) / 32 * 32);   // a single partition covers the table
    pl.max_parts = 1;
    return pl;
  }
  pl.partition = P;
  pl.max_parts = (int)((cap + P - 1) / P);
  const size_t units = (size_t)S * Hq * pl.max_parts;
  pl.ws_ml_bytes = align256(units * 2 * sizeof(float));
  pl.ws_bytes = pl.ws_ml_bytes + align256(units * D * sizeof(float));
  return pl;
}

bool mfma_eligible(DT dt, int D, int G, int partition) {
  return (dt == DT::F16 || dt == DT::BF16) && (D == 64 || D == 80 || D == 128 || D == 256) &&
         G % 4 == 0 && partition % 16 == 0;
}
// Head dim of the matrix-core products: 80-dim heads run through the 128-dim ones (padded).
int mfma_compute_dim(int D) { return D == 80 ? 128 : D; }

// Consecutive partitions one matrix-core workgroup walks.  Walking several pays the query and
// table prologue once per workgroup instead of once per partition, and each partition still
// gets its own partial.  It needs partitions of a multiple of 128 tokens (the same number of
// chunks per wave in each), at most as many as the kernel's 32 KiB of LDS slots hold (4, 2, 1
// for heads x head dim up to 512, 1024, 2048), and is used only while the grid keeps at least
// kTargetWorkgroups workgroups.  Up to
// kGroupTokens tokens per workgroup: measured on GQA long-context batches, single partitions of
// 1024 tokens stream faster (5.80 TB/s) than of 512 (5.60) or 2048 (5.72).
constexpr long kGroupTokens = 1024;
int mfma_parts_per_wg(int partition, int max_parts, long units, int heads_per_wg, int head_dim) {
  if (max_parts <= 1 || partition % 128 != 0) return 1;
  const int cap = std::min(4, 2048 / (heads_per_wg * head_dim));
  int ppw = 1;
  while (2 * ppw <= cap && 2L * ppw * partition <= kGroupTokens &&
         units * ((max_parts + 2 * ppw - 1) / (2 * ppw)) >= kTargetWorkgroups)
    ppw *= 2;
  return ppw;
}

// Query heads one workgroup serves.  The vector-ALU kernel keeps head_dim/64 .. head_dim/8
// fp32 outputs per lane per head, so wide heads get fewer per workgroup.
int heads_per_wg(bool mfma, int G, int D) {
  if (mfma) return G % 16 == 0 && D <= 128 ? 16 : G % 8 == 0 ? 8 : 4;
  const int cap = D >= 256 ? 2 : D == 80 ? 4 : 8;
  for (int gt = cap; gt > 1; gt /= 2)
    if (G % gt == 0) return gt;
  return 1;
}

// Grid of the vector-ALU decode: one workgroup per (partition, sequence, KV head, head chunk),
// padded to a multiple of 8 x head chunks for the kernel's XCD-aware numbering (the padding
// workgroups fall past the last partition and exit at once).
long valu_grid(long S, long Hkv, long HC, long parts) {
  long g = S * Hkv * HC * parts;
  if (HC > 1) g = (g + 8 * HC - 1) / (8 * HC) * (8 * HC);
  return g;
}

pa_status launch_status(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH; }

// Device block-engine state from the ABI arguments.
pa_status engine_of(int32_t* tables, int32_t* lens, int32_t* refs, int32_t* stack, int32_t* top,
                    int32_t num_seqs, int32_t maxb, int32_t bs, int32_t num_blocks,
                    bool needs_stack, pa::EngineState* e) {
  if (num_seqs < 0 || maxb <= 0 || bs <= 0 || num_blocks <= 0) return PA_ERR_BAD_SHAPE;
  if (!tables || !lens || !refs || (needs_stack && (!stack || !top))) return PA_ERR_NULL_PTR;
  e->tables = tables;
  e->context_lens = lens;
  e->ref_counts = refs;
  e->free_stack = stack;
  e->free_top = top;
  e->num_seqs = num_seqs;
  e->max_blocks_per_seq = maxb;
  e->block_size = bs;
  e->num_blocks = num_blocks;
  return PA_OK;
}

// Key-split plan of a prefill call.  Splitting is for grids too small to fill the GPU for
// long: below kPrefillTargetWG workgroups the keys are cut so that the grid reaches about
// that many, with at least kMinSplitTiles tiles per split (each split costs a partial write
// and a merge read per row).  An explicit kv_split (tokens, a multiple of 64) overrides it.
constexpr long kPrefillTargetWG = 2048;
constexpr long kPrefillSplitBelow = 1024;
constexpr long kMinSplitTiles = 8;

struct PrefillPlan {
  int kv_splits = 1, split_tiles = 0;
  long row_tiles = 0;
  size_t tok_bytes = 0, ml_bytes = 0, ws_bytes = 0;
};

pa_status prefill_plan(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                       int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                       int32_t max_query_len, int32_t num_tokens, int32_t kv_split,
                       PrefillPlan* pl) {
  if (kv_split < 0 || kv_split % 64 != 0) return PA_ERR_BAD_SHAPE;
  const long G = num_heads / num_kv_heads;
  pl->row_tiles = ((long)max_query_len * G + 127) / 128;
  const long cap_tiles = ((long)max_blocks_per_seq * block_size + 63) / 64;
  pl->split_tiles = (int)std::min<long>(cap_tiles, 0x7FFFFFFF);
  const long base = (long)num_seqs * num_kv_heads * pl->row_tiles;
  long st = cap_tiles;
  if (kv_split > 0) {
    st = kv_split / 64;
  } else if (base > 0 && base < kPrefillSplitBelow) {
    const long ks = std::min((kPrefillTargetWG + base - 1) / base, cap_tiles / kMinSplitTiles);
    if (ks > 1) st = (cap_tiles + ks - 1) / ks;
  }
  const long ks = (cap_tiles + st - 1) / st;
  if (ks <= 1) return PA_OK;
  if (num_tokens <= 0) return PA_ERR_BAD_SHAPE;   // splitting needs the token count
  pl->kv_splits = (int)ks;
  pl->split_tiles = (int)st;
  const size_t slots = (size_t)num_tokens * num_heads * ks;
  pl->tok_bytes = align256((size_t)num_tokens * sizeof(int32_t));
  pl->ml_bytes = align256(slots * 2 * sizeof(float));
  pl->ws_bytes = pl->tok_bytes + pl->ml_bytes + slots * (size_t)head_dim * sizeof(float);
  return PA_OK;
}

}  // namespace

extern "C" {

const char* pa_status_string(pa_status s) {
  switch (s) {
    case PA_OK: return "PA_OK";
    case PA_ERR_NULL_PTR: return "PA_ERR_NULL_PTR: a required pointer is NULL";
    case PA_ERR_BAD_SHAPE: return "PA_ERR_BAD_SHAPE: a size is invalid or inconsistent";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: unsupported head_dim, block_size, dtype or kernel";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: workspace missing or too small";
    case PA_ERR_LAUNCH: return "PA_ERR_LAUNCH: the HIP runtime rejected a kernel launch";
  }
  return "unknown pa_status";
}

int32_t pa_version(void) { return kVersion; }

int32_t pa_decode_auto_partition(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size,
                                 int32_t max_blocks_per_seq) {
  if (check_shape(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, 0) != PA_OK)
    return 0;
  return make_plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, 0).partition;
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size,
                                 int32_t max_blocks_per_seq, int32_t partition_size) {
  if (check_shape(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                  partition_size) != PA_OK)
    return 0;
  return make_plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, partition_size)
      .ws_bytes;
}

pa_status pa_decode_partitions(void* out, const void* query, const void* key_cache,
                               const void* value_cache, const int32_t* block_tables,
                               const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int32_t num_blocks, int32_t max_blocks_per_seq, float scale,
                               pa_dtype dtype, int32_t partition_size, void* workspace,
                               size_t workspace_bytes, pa_kernel kernel, uint32_t flags,
                               void* stream) {
  DT dt;
  if (!dtype_of(dtype, &dt)) return PA_ERR_UNSUPPORTED;
  pa_status st = check_shape(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                             max_blocks_per_seq, partition_size);
  if (st != PA_OK) return st;
  if (kernel != PA_KERNEL_AUTO && kernel != PA_KERNEL_VALU && kernel != PA_KERNEL_MFMA)
    return PA_ERR_UNSUPPORTED;
  if ((flags & ~PA_DECODE_SHARED_BLOCKS) != 0) return PA_ERR_UNSUPPORTED;
  if (dt == DT::F32 && head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PA_OK;
  if (num_blocks <= 0) return PA_ERR_BAD_SHAPE;
  if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens)
    return PA_ERR_NULL_PTR;
  if (!std::isfinite(scale)) return PA_ERR_BAD_SHAPE;

  const Plan pl = make_plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                            partition_size);
  if (pl.ws_bytes > 0 && (!workspace || workspace_bytes < pl.ws_bytes)) return PA_ERR_WORKSPACE;

  const int G = num_heads / num_kv_heads;
  const bool can_mfma = mfma_eligible(dt, head_dim, G, pl.partition);
  bool mfma = false;
  if (kernel == PA_KERNEL_MFMA) {
    if (!can_mfma) return PA_ERR_UNSUPPORTED;
    mfma = true;
  } else if (kernel == PA_KERNEL_AUTO) {
    mfma = can_mfma;
  }
  const int gt = heads_per_wg(mfma, G, head_dim);

  pa::DecodeParams p;
  p.out = out;
  p.q = query;
  p.kc = key_cache;
  p.vc = value_cache;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.ws_ml = pl.ws_bytes ? reinterpret_cast<float*>(workspace) : nullptr;
  p.ws_o = pl.ws_bytes ? reinterpret_cast<float*>((char*)workspace + pl.ws_ml_bytes) : nullptr;
  p.num_seqs = num_seqs;
  p.num_heads = num_heads;
  p.num_kv_heads = num_kv_heads;
  p.group = G;
  p.head_chunks = G / gt;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.num_blocks = num_blocks;
  p.partition = pl.partition;
  p.max_parts = pl.max_parts;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.v_scale = 1.0f;

  const long units = (long)num_seqs * num_kv_heads * p.head_chunks;
  p.parts_per_wg = mfma ? mfma_parts_per_wg(pl.partition, pl.max_parts, units, gt, mfma_compute_dim(head_dim)) : 1;
  const long grid = mfma ? units * ((pl.max_parts + p.parts_per_wg - 1) / p.parts_per_wg)
                        : valu_grid(num_seqs, num_kv_heads, p.head_chunks, pl.max_parts);
  if (grid > 0x7FFFFFFFL) return PA_ERR_BAD_SHAPE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  // K/V read by several workgroups (a shared prefix, or several head chunks of one KV head)
  // use cache-allocating loads, so the later readers find them in L2
  const bool stream_kv = (flags & PA_DECODE_SHARED_BLOCKS) == 0 && p.head_chunks == 1;
  const hipError_t e = mfma ? pa::launch_decode_mfma(dt, head_dim, block_size, gt, stream_kv, p, (int)grid, s)
                            : pa::launch_decode_valu(dt, head_dim, block_size, gt, stream_kv, p, (int)grid, s);
  return launch_status(e);
}

pa_status pa_decode_merge(void* out, const int32_t* context_lens, int32_t num_seqs,
                          int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t block_size, int32_t max_blocks_per_seq, pa_dtype dtype,
                          int32_t partition_size, const void* workspace, size_t workspace_bytes,
                          void* stream) {
  DT dt;
  if (!dtype_of(dtype, &dt)) return PA_ERR_UNSUPPORTED;
  pa_status st = check_shape(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                             max_blocks_per_seq, partition_size);
  if (st != PA_OK) return st;
  if (num_seqs == 0) return PA_OK;
  const Plan pl = make_plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                            partition_size);
  if (pl.max_parts <= 1) return PA_OK;   // nothing was split
  if (!out || !context_lens) return PA_ERR_NULL_PTR;
  if (!workspace || workspace_bytes < pl.ws_bytes) return PA_ERR_WORKSPACE;
  pa::MergeParams p;
  p.out = out;
  p.context_lens = context_lens;
  p.ws_ml = reinterpret_cast<const float*>(workspace);
  p.ws_o = reinterpret_cast<const float*>((const char*)workspace + pl.ws_ml_bytes);
  p.num_seqs = num_seqs;
  p.num_heads = num_heads;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.block_size = block_size;
  p.partition = pl.partition;
  p.max_parts = pl.max_parts;
  (void)hipGetLastError();
  return launch_status(pa::launch_merge(dt, head_dim, p, reinterpret_cast<hipStream_t>(stream)));
}

pa_status pa_decode_ex(void* out, const void* query, const void* key_cache,
                       const void* value_cache, const int32_t* block_tables,
                       const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                       int32_t num_blocks, int32_t max_blocks_per_seq, float scale,
                       pa_dtype dtype, int32_t partition_size, void* workspace,
                       size_t workspace_bytes, pa_kernel kernel, uint32_t flags, void* stream) {
  pa_status st = pa_decode_partitions(out, query, key_cache, value_cache, block_tables,
                                      context_lens, num_seqs, num_heads, num_kv_heads, head_dim,
                                      block_size, num_blocks, max_blocks_per_seq, scale, dtype,
                                      partition_size, workspace, workspace_bytes, kernel, flags,
                                      stream);
  if (st != PA_OK) return st;
  return pa_decode_merge(out, context_lens, num_seqs, num_heads, num_kv_heads, head_dim,
                         block_size, max_blocks_per_seq, dtype, partition_size, workspace,
                         workspace_bytes, stream);
}

pa_status pa_decode(void* out, const void* query, const void* key_cache, const void* value_cache,
                    const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                    int32_t num_blocks, int32_t max_blocks_per_seq, float scale, pa_dtype dtype,
                    int32_t partition_size, void* workspace, size_t workspace_bytes,
                    void* stream) {
  return pa_decode_ex(out, query, key_cache, value_cache, block_tables, context_lens, num_seqs,
                      num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                      max_blocks_per_seq, scale, dtype, partition_size, workspace,
                      workspace_bytes, PA_KERNEL_AUTO, 0u, stream);
}

pa_status pa_reshape_and_cache(const void* key, const void* value, void* key_cache,
                               void* value_cache, const int64_t* slot_mapping, int32_t num_tokens,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int32_t num_blocks, pa_dtype dtype, void* stream) {
  DT dt;
  if (!dtype_of(dtype, &dt)) return PA_ERR_UNSUPPORTED;
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks < 0)
    return PA_ERR_BAD_SHAPE;
  const long row_bytes = (long)head_dim * elem_bytes(dt);
  if (row_bytes % 16 != 0 || head_dim > 1024) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !key_cache || !value_cache || !slot_mapping) return PA_ERR_NULL_PTR;
  (void)hipGetLastError();
  return launch_status(pa::launch_reshape_and_cache(
      key, value, key_cache, value_cache, slot_mapping, num_tokens, (int)(row_bytes / 16),
      block_size, num_blocks, num_kv_heads, reinterpret_cast<hipStream_t>(stream)));
}

pa_status pa_copy_blocks(void* key_cache, void* value_cache, const int64_t* block_mapping,
                         int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t num_blocks, pa_dtype dtype, void* stream) {
  DT dt;
  if (!pool_dtype_of(dtype, &dt)) return PA_ERR_UNSUPPORTED;
  if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks < 0)
    return PA_ERR_BAD_SHAPE;
  const long block_bytes = (long)num_kv_heads * block_size * head_dim * elem_bytes(dt);
  if (block_bytes % 16 != 0) return PA_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PA_OK;
  if (!key_cache || !value_cache || !block_mapping) return PA_ERR_NULL_PTR;
  (void)hipGetLastError();
  return launch_status(pa::launch_block_copy(key_cache, value_cache, key_cache, value_cache,
                                             block_mapping, num_pairs, block_bytes / 16,
                                             num_blocks, num_blocks,
                                             reinterpret_cast<hipStream_t>(stream)));
}

pa_status pa_swap_blocks(const void* src_key_cache, const void* src_value_cache,
                         int32_t src_num_blocks, void* dst_key_cache, void* dst_value_cache,
                         int32_t dst_num_blocks, const int64_t* block_mapping, int32_t num_pairs,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         pa_dtype dtype, void* stream) {
  DT dt;
  if (!pool_dtype_of(dtype, &dt)) return PA_ERR_UNSUPPORTED;
  if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      src_num_blocks < 0 || dst_num_blocks < 0)
    return PA_ERR_BAD_SHAPE;
  const long block_bytes = (long)num_kv_heads * block_size * head_dim * elem_bytes(dt);
  if (block_bytes % 16 != 0) return PA_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PA_OK;
  if (!src_key_cache || !src_value_cache || !dst_key_cache || !dst_value_cache || !block_mapping)
    return PA_ERR_NULL_PTR;
  (void)hipGetLastError();
  return launch_status(pa::launch_block_copy(src_key_cache, src_value_cache, dst_key_cache,
                                             dst_value_cache, block_mapping, num_pairs,
                                             block_bytes / 16, src_num_blocks, dst_num_blocks,
                                             reinterpret_cast<hipStream_t>(stream)));
}

// Head dims of the prefill kernel: 64 and 128, and 80 (the 128-dim products on zero-padded rows).
static bool prefill_head_dim(int32_t d) { return d == 64 || d == 80 || d == 128; }

size_t pa_prefill_workspace_bytes(int32_t num_seqs, int32_t num_tokens, int32_t num_heads,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                  int32_t max_blocks_per_seq, int32_t max_query_len,
                                  int32_t kv_split) {
  if (check_shape(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                  0) != PA_OK || !prefill_head_dim(head_dim) || max_query_len < 0)
    return 0;
  PrefillPlan pl;
  if (prefill_plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                   max_query_len, num_tokens, kv_split, &pl) != PA_OK)
    return 0;
  return pl.ws_bytes;
}

// pa_prefill_ex and pa_prefill_fp8: kv8 selects E4M3 pools with scales k_scale and v_scale
static pa_status prefill_call(void* out, const void* query, const void* key_cache,
                              const void* value_cache, const int32_t* block_tables,
                              const int32_t* query_start_loc, const int32_t* context_lens,
                              int32_t num_seqs, int32_t num_tokens, int32_t num_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                              int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_query_len,
                              float scale, pa_dtype dtype, bool kv8, float k_scale, float v_scale,
                              int32_t kv_split, void* workspace, size_t workspace_bytes,
                              uint32_t flags, void* stream) {
  DT dt;
  if (!dtype_of(dtype, &dt)) return PA_ERR_UNSUPPORTED;
  pa_status st = check_shape(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                             max_blocks_per_seq, 0);
  if (st != PA_OK) return st;
  if (max_query_len < 0 || num_tokens < 0) return PA_ERR_BAD_SHAPE;
  if (dt == DT::F32 || !prefill_head_dim(head_dim)) return PA_ERR_UNSUPPORTED;
  if ((flags & ~PA_PREFILL_BF16_P) != 0) return PA_ERR_UNSUPPORTED;
  PrefillPlan pl;
  st = prefill_plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                    max_query_len, num_tokens, kv_split, &pl);
  if (st != PA_OK) return st;
  if (num_seqs == 0 || max_query_len == 0) return PA_OK;
  if (num_blocks <= 0) return PA_ERR_BAD_SHAPE;
  if (!out || !query || !key_cache || !value_cache || !block_tables || !query_start_loc ||
      !context_lens)
    return PA_ERR_NULL_PTR;
  if (!std::isfinite(scale)) return PA_ERR_BAD_SHAPE;
  if (kv8 && !(std::isfinite(k_scale) && k_scale > 0.0f && std::isfinite(v_scale) && v_scale > 0.0f))
    return PA_ERR_BAD_SHAPE;
  if (pl.ws_bytes > 0 && (!workspace || workspace_bytes < pl.ws_bytes)) return PA_ERR_WORKSPACE;
  const int G = num_heads / num_kv_heads;
  const long grid = (long)num_seqs * num_kv_heads * pl.row_tiles * pl.kv_splits;
  if (grid > 0x7FFFFFFFL || (long)max_query_len * G > 0x7FFFFFFFL) return PA_ERR_BAD_SHAPE;

  pa::PrefillParams p;
  p.out = out;
  p.q = query;
  p.kc = key_cache;
  p.vc = value_cache;
  p.block_tables = block_tables;
  p.query_start_loc = query_start_loc;
  p.context_lens = context_lens;
  p.num_seqs = num_seqs;
  p.num_heads = num_heads;
  p.num_kv_heads = num_kv_heads;
  p.group = G;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.num_blocks = num_blocks;
  p.max_query_len = max_query_len;
  p.row_tiles = (int)pl.row_tiles;
  // The kernel takes the row max on raw scores, which needs a positive multiplier: a negative
  // scale flips the query signs instead (exact), and 0 becomes the smallest normal float
  // (every score then rounds to a zero exponent, as scale 0 requires).
  // An E4M3 key pool's scale multiplies every score: folded in here (exact up to the one
  // rounding of the product).
  const float kmul = kv8 ? k_scale : 1.0f;
  p.scale_log2 = std::max(std::fabs(scale) * kmul * 1.4426950408889634f, 1.17549435e-38f);
  p.v_scale = kv8 ? v_scale : 1.0f;
  p.q_sign = std::signbit(scale) ? 0x80008000u : 0u;
  p.kv_splits = pl.kv_splits;
  p.split_tiles = pl.split_tiles;
  p.num_tokens = num_tokens;
  char* ws = reinterpret_cast<char*>(workspace);
  p.tok_len = pl.kv_splits > 1 ? reinterpret_cast<int32_t*>(ws) : nullptr;
  p.ws_ml = pl.kv_splits > 1 ? reinterpret_cast<float*>(ws + pl.tok_bytes) : nullptr;
  p.ws_o = pl.kv_splits > 1 ? reinterpret_cast<float*>(ws + pl.tok_bytes + pl.ml_bytes) : nullptr;
  const bool split_p = !(dt == DT::BF16 && (flags & PA_PREFILL_BF16_P));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  hipError_t e = pa::launch_prefill_mfma(dt, kv8, head_dim, block_size, split_p, p, (int)grid, s);
  if (e != hipSuccess || pl.kv_splits == 1) return launch_status(e);
  // combine the split partials: every query token is a "sequence" whose context is its
  // position + 1, partitioned by the split length
  pa::MergeParams m;
  m.out = out;
  m.context_lens = p.tok_len;
  m.ws_ml = p.ws_ml;
  m.ws_o = p.ws_o;
  m.num_seqs = num_tokens;
  m.num_heads = num_heads;
  m.max_blocks_per_seq = max_blocks_per_seq;
  m.block_size = block_size;
  m.partition = pl.split_tiles * 64;
  m.max_parts = pl.kv_splits;
  return launch_status(pa::launch_merge(dt, head_dim, m, s));
}

pa_status pa_prefill_ex(void* out, const void* query, const void* key_cache,
                        const void* value_cache, const int32_t* block_tables,
                        const int32_t* query_start_loc, const int32_t* context_lens,
                        int32_t num_seqs, int32_t num_tokens, int32_t num_heads,
                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                        int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_query_len,
                        float scale, pa_dtype dtype, int32_t kv_split, void* workspace,
                        size_t workspace_bytes, uint32_t flags, void* stream) {
  return prefill_call(out, query, key_cache, value_cache, block_tables, query_start_loc,
                      context_lens, num_seqs, num_tokens, num_heads, num_kv_heads, head_dim,
                      block_size, num_blocks, max_blocks_per_seq, max_query_len, scale, dtype,
                      false, 1.0f, 1.0f, kv_split, workspace, workspace_bytes, flags, stream);
}

pa_status pa_prefill_fp8(void* out, const void* query, const void* key_cache,
                         const void* value_cache, const int32_t* block_tables,
                         const int32_t* query_start_loc, const int32_t* context_lens,
                         int32_t num_seqs, int32_t num_tokens, int32_t num_heads,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_query_len,
                         float scale, pa_dtype dtype, float k_scale, float v_scale,
                         int32_t kv_split, void* workspace, size_t workspace_bytes,
                         uint32_t flags, void* stream) {
  return prefill_call(out, query, key_cache, value_cache, block_tables, query_start_loc,
                      context_lens, num_seqs, num_tokens, num_heads, num_kv_heads, head_dim,
                      block_size, num_blocks, max_blocks_per_seq, max_query_len, scale, dtype,
                      true, k_scale, v_scale, kv_split, workspace, workspace_bytes, flags, stream);
}

pa_status pa_prefill(void* out, const void* query, const void* key_cache, const void* value_cache,
                     const int32_t* block_tables, const int32_t* query_start_loc,
                     const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                     int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_query_len,
                     float scale, pa_dtype dtype, uint32_t flags, void* stream) {
  // one pass over every key (no split, no workspace): a split length past the table
  const long cap = (long)max_blocks_per_seq * block_size;
  const int32_t no_split = (int32_t)std::min<long>((cap + 63) / 64 * 64, 0x7FFFFFC0L);
  return pa_prefill_ex(out, query, key_cache, value_cache, block_tables, query_start_loc,
                       context_lens, num_seqs, 0, num_heads, num_kv_heads, head_dim, block_size,
                       num_blocks, max_blocks_per_seq, max_query_len, scale, dtype,
                       max_blocks_per_seq > 0 && block_size > 0 ? std::max<int32_t>(no_split, 64) : 64,
                       nullptr, 0, flags, stream);
}

pa_status pa_reshape_and_cache_fp8(const void* key, const void* value, void* key_cache,
                                   void* value_cache, const int64_t* slot_mapping,
                                   int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block_size, int32_t num_blocks, pa_dtype dtype,
                                   float k_scale, float v_scale, void* stream) {
  DT dt;
  if (!dtype_of(dtype, &dt) || dt == DT::F32) return PA_ERR_UNSUPPORTED;
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks < 0)
    return PA_ERR_BAD_SHAPE;
  if (head_dim % 8 != 0 || head_dim > 1024) return PA_ERR_UNSUPPORTED;
  if (!(k_scale > 0.0f) || !(v_scale > 0.0f) || !std::isfinite(k_scale) || !std::isfinite(v_scale))
    return PA_ERR_BAD_SHAPE;
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !key_cache || !value_cache || !slot_mapping) return PA_ERR_NULL_PTR;
  (void)hipGetLastError();
  return launch_status(pa::launch_reshape_and_cache_fp8(
      dt, key, value, key_cache, value_cache, slot_mapping, num_tokens, head_dim, block_size,
      num_blocks, num_kv_heads, 1.0f / k_scale, 1.0f / v_scale,
      reinterpret_cast<hipStream_t>(stream)));
}

pa_status pa_decode_fp8_partitions(void* out, const void* query, const void* key_cache,
                                   const void* value_cache, const int32_t* block_tables,
                                   const int32_t* context_lens, int32_t num_seqs,
                                   int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block_size, int32_t num_blocks,
                                   int32_t max_blocks_per_seq, float scale, pa_dtype dtype,
                                   float k_scale, float v_scale, int32_t partition_size,
                                   void* workspace, size_t workspace_bytes, uint32_t flags,
                                   void* stream) {
  DT dt;
  if (!dtype_of(dtype, &dt) || dt == DT::F32) return PA_ERR_UNSUPPORTED;
  pa_status st = check_shape(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                             max_blocks_per_seq, partition_size);
  if (st != PA_OK) return st;
  if ((flags & ~PA_DECODE_SHARED_BLOCKS) != 0) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PA_OK;
  if (num_blocks <= 0) return PA_ERR_BAD_SHAPE;
  if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens)
    return PA_ERR_NULL_PTR;
  if (!std::isfinite(scale) || !std::isfinite(k_scale) || !std::isfinite(v_scale))
    return PA_ERR_BAD_SHAPE;
  const Plan pl = make_plan(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                            max_blocks_per_seq, partition_size);
  if (pl.ws_bytes > 0 && (!workspace || workspace_bytes < pl.ws_bytes)) return PA_ERR_WORKSPACE;
  const int G = num_heads / num_kv_heads;
  // Grouped heads (a multiple of 4) run on the matrix cores, which read each K/V byte once per
  // KV head; otherwise the vector-ALU kernel, at most 2 heads per workgroup (16 fp32 outputs
  // per lane per head).
  const bool mfma = mfma_eligible(dt, head_dim, G, pl.partition);
  const int gt = mfma ? heads_per_wg(true, G, head_dim) : std::min(heads_per_wg(false, G, head_dim), 2);

  pa::DecodeParams p;
  p.out = out;
  p.q = query;
  p.kc = key_cache;
  p.vc = value_cache;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.ws_ml = pl.ws_bytes ? reinterpret_cast<float*>(workspace) : nullptr;
  p.ws_o = pl.ws_bytes ? reinterpret_cast<float*>((char*)workspace + pl.ws_ml_bytes) : nullptr;
  p.num_seqs = num_seqs;
  p.num_heads = num_heads;
  p.num_kv_heads = num_kv_heads;
  p.group = G;
  p.head_chunks = G / gt;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.num_blocks = num_blocks;
  p.partition = pl.partition;
  p.max_parts = pl.max_parts;
  p.scale_log2 = scale * k_scale * 1.4426950408889634f;
  p.v_scale = v_scale;
  const long units = (long)num_seqs * num_kv_heads * p.head_chunks;
  p.parts_per_wg = mfma ? mfma_parts_per_wg(pl.partition, pl.max_parts, units, gt, mfma_compute_dim(head_dim)) : 1;
  const long grid = mfma ? units * ((pl.max_parts + p.parts_per_wg - 1) / p.parts_per_wg)
                        : valu_grid(num_seqs, num_kv_heads, p.head_chunks, pl.max_parts);
  if (grid > 0x7FFFFFFFL) return PA_ERR_BAD_SHAPE;
  (void)hipGetLastError();
  // K/V read by several workgroups (a shared prefix, or several head chunks of one KV head)
  // use cache-allocating loads, so the later readers find them in L2
  const bool stream_kv = (flags & PA_DECODE_SHARED_BLOCKS) == 0 && p.head_chunks == 1;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return launch_status(mfma ? pa::launch_decode_mfma_fp8(dt, head_dim, block_size, gt, stream_kv, p,
                                                         (int)grid, s)
                            : pa::launch_decode_valu_fp8(dt, head_dim, block_size, gt, stream_kv, p,
                                                         (int)grid, s));
}

pa_status pa_decode_fp8(void* out, const void* query, const void* key_cache,
                        const void* value_cache, const int32_t* block_tables,
                        const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                        int32_t num_blocks, int32_t max_blocks_per_seq, float scale,
                        pa_dtype dtype, float k_scale, float v_scale, int32_t partition_size,
                        void* workspace, size_t workspace_bytes, uint32_t flags, void* stream) {
  pa_status st = pa_decode_fp8_partitions(out, query, key_cache, value_cache, block_tables,
                                          context_lens, num_seqs, num_heads, num_kv_heads,
                                          head_dim, block_size, num_blocks, max_blocks_per_seq,
                                          scale, dtype, k_scale, v_scale, partition_size,
                                          workspace, workspace_bytes, flags, stream);
  if (st != PA_OK) return st;
  return pa_decode_merge(out, context_lens, num_seqs, num_heads, num_kv_heads, head_dim,
                         block_size, max_blocks_per_seq, dtype, partition_size, workspace,
                         workspace_bytes, stream);
}


pa_status pa_append_slots(int32_t* block_tables, int32_t* context_lens, int32_t* ref_counts,
                          int32_t* free_stack, int32_t* free_top, int32_t num_seqs,
                          int32_t max_blocks_per_seq, int32_t block_size, int32_t num_blocks,
                          const int32_t* seq_ids, int32_t num_append, int64_t* slot_mapping,
                          int64_t* block_mapping, int32_t* num_pairs, int32_t* status,
                          void* stream) {
  pa::EngineState e;
  pa_status st = engine_of(block_tables, context_lens, ref_counts, free_stack, free_top, num_seqs,
                           max_blocks_per_seq, block_size, num_blocks, true, &e);
  if (st != PA_OK) return st;
  if (num_append < 0) return PA_ERR_BAD_SHAPE;
  if (!num_pairs || !status) return PA_ERR_NULL_PTR;
  if (num_append > 0 && (!seq_ids || !slot_mapping || !block_mapping)) return PA_ERR_NULL_PTR;
  (void)hipGetLastError();
  return launch_status(pa::launch_append_slots(e, seq_ids, num_append, slot_mapping,
                                               block_mapping, num_pairs, status,
                                               reinterpret_cast<hipStream_t>(stream)));
}

pa_status pa_fork_seqs(int32_t* block_tables, int32_t* context_lens, int32_t* ref_counts,
                       int32_t num_seqs, int32_t max_blocks_per_seq, int32_t block_size,
                       int32_t num_blocks, const int32_t* parent_child, int32_t num_forks,
                       void* stream) {
  pa::EngineState e;
  pa_status st = engine_of(block_tables, context_lens, ref_counts, nullptr, nullptr, num_seqs,
                           max_blocks_per_seq, block_size, num_blocks, false, &e);
  if (st != PA_OK) return st;
  if (num_forks < 0) return PA_ERR_BAD_SHAPE;
  if (num_forks == 0) return PA_OK;
  if (!parent_child) return PA_ERR_NULL_PTR;
  (void)hipGetLastError();
  return launch_status(pa::launch_fork(e, parent_child, num_forks,
                                       reinterpret_cast<hipStream_t>(stream)));
}

pa_status pa_free_seqs(int32_t* block_tables, int32_t* context_lens, int32_t* ref_counts,
                       int32_t* free_stack, int32_t* free_top, int32_t num_seqs,
                       int32_t max_blocks_per_seq, int32_t block_size, int32_t num_blocks,
                       const int32_t* seq_ids, int32_t num_free, void* stream) {
  pa::EngineState e;
  pa_status st = engine_of(block_tables, context_lens, ref_counts, free_stack, free_top, num_seqs,
                           max_blocks_per_seq, block_size, num_blocks, true, &e);
  if (st != PA_OK) return st;
  if (num_free < 0) return PA_ERR_BAD_SHAPE;
  if (num_free == 0) return PA_OK;
  if (!seq_ids) return PA_ERR_NULL_PTR;
  (void)hipGetLastError();
  return launch_status(pa::launch_free_seqs(e, seq_ids, num_free,
                                            reinterpret_cast<hipStream_t>(stream)));
}

pa_status pa_copy_blocks_counted(void* key_cache, void* value_cache, const int64_t* block_mapping,
                                 const int32_t* num_pairs, int32_t max_pairs,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                 int32_t num_blocks, pa_dtype dtype, void* stream) {
  DT dt;
  if (!pool_dtype_of(dtype, &dt)) return PA_ERR_UNSUPPORTED;
  if (max_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks < 0)
    return PA_ERR_BAD_SHAPE;
  const long block_bytes = (long)num_kv_heads * block_size * head_dim * elem_bytes(dt);
  if (block_bytes % 16 != 0) return PA_ERR_UNSUPPORTED;
  if (max_pairs == 0) return PA_OK;
  if (!key_cache || !value_cache || !block_mapping || !num_pairs) return PA_ERR_NULL_PTR;
  (void)hipGetLastError();
  return launch_status(pa::launch_block_copy(key_cache, value_cache, key_cache, value_cache,
                                             block_mapping, max_pairs, block_bytes / 16,
                                             num_blocks, num_blocks,
                                             reinterpret_cast<hipStream_t>(stream), num_pairs));
}

pa_status pa_read_tiles(const void* base, int64_t base_tiles, int32_t tile_bytes,
                        const int32_t* tile_ids, int32_t num_tiles, uint32_t* xor_out,
                        void* stream) {
  if (num_tiles < 0 || base_tiles <= 0) return PA_ERR_BAD_SHAPE;
  if (tile_bytes != 1024 && tile_bytes != 2048 && tile_bytes != 4096 && tile_bytes != 8192)
    return PA_ERR_UNSUPPORTED;
  if (!tile_ids && num_tiles > base_tiles) return PA_ERR_BAD_SHAPE;   // contiguous run past the buffer
  if (num_tiles == 0) return PA_OK;
  if (!base || !xor_out) return PA_ERR_NULL_PTR;
  (void)hipGetLastError();
  return launch_status(pa::launch_read_tiles(base, (long)base_tiles, tile_bytes, tile_ids, num_tiles,
                                             xor_out, reinterpret_cast<hipStream_t>(stream)));
}

pa_status pa_block_hashes(const int32_t* token_ids, const int32_t* num_tokens, int32_t num_seqs,
                          int32_t max_tokens, int32_t block_size, uint64_t* hashes,
                          void* stream) {
  if (num_seqs < 0 || max_tokens < 0 || block_size <= 0 || block_size > 4096)
    return PA_ERR_BAD_SHAPE;
  if (num_seqs == 0 || max_tokens < block_size) return PA_OK;
  if (!token_ids || !num_tokens || !hashes) return PA_ERR_NULL_PTR;
  (void)hipGetLastError();
  return launch_status(pa::launch_block_hashes(token_ids, num_tokens, num_seqs, max_tokens,
                                               block_size, hashes,
                                               reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
