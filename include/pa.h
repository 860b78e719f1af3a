/*
 * pa.h — C ABI of libpa.so for AMD MI355X (gfx950): paged attention (single-query decode and
 * chunked prefill) over a block-paged KV cache, the cache-writing and block-copy kernels
 * (16-bit and 8-bit pools, swaps to and from host memory) and a block engine on the device.
 *
 * The problem, as the pages state it: the K/V cache of every sequence lives in fixed-size
 * blocks of one physical pool; a per-sequence block table maps logical blocks, in order, to
 * non-contiguous physical blocks; the attention kernel reads K/V block by block through that
 * table (UltraLAB summary of Kwon et al., SOSP 2023 (xasun.com), sections 一 and 二;
 * "GPT-OSS显存管理技巧：PagedAttention机制解析" (yongjin360.com) §2.2; PyTorch-CUDA-v2.9
 * PagedAttention page (jsqmd.com), paged-memory section).  What is computed per query head is
 * scaled dot-product attention with a softmax ("PagedAttention技术：加速GPT推理的利器"
 * (yunthe.com) §1.1).
 *
 * Conventions for every entry point
 *   - All array arguments are DEVICE pointers owned by the caller; the library keeps no
 *     pointer after it returns and allocates no device memory.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL = the default
 *     stream) and the call returns without waiting.  The caller keeps every buffer alive
 *     until the stream has finished.  Calls on one stream run in order, so
 *     copy_blocks -> reshape_and_cache -> decode on one stream sees each write.
 *   - Every array is dense, row-major, with the shapes given below.
 *   - Problems that the host can see (null pointers, unsupported sizes, a short workspace)
 *     return an error code before anything is launched; nothing aborts and no C++ exception
 *     crosses this boundary.  Device-array contents are preconditions and are not checked
 *     on the host (that would need a synchronisation); the kernels still guard every index
 *     so that a bad one is skipped instead of read or written out of bounds.
 *   - `num_seqs`, `num_tokens` or `num_pairs` equal to 0 is a successful no-op.
 *   - The library keeps no state between calls; calls from several threads (on their own
 *     streams) are safe.
 *
 * Element types: `pa_dtype` selects the element type of q, out, key, value and both pools
 * (all of one call share it).  Sums accumulate in fp32 in every kernel.  The vector-ALU decode
 * kernels compute in fp32 throughout; the matrix-core kernels (grouped-query decode, prefill)
 * multiply the 16-bit q, K and V as stored.  The grouped-query decode kernel multiplies the
 * softmax probabilities as a 16-bit high part plus a 16-bit remainder (16 significant bits or
 * more); pa_prefill states its own options.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL_PTR = 1,     /* a required pointer is NULL */
  PA_ERR_BAD_SHAPE = 2,    /* a size is negative, zero where it must not be, or inconsistent */
  PA_ERR_UNSUPPORTED = 3,  /* a valid but unsupported combination (head_dim, block_size, dtype) */
  PA_ERR_WORKSPACE = 4,    /* the workspace is missing or smaller than required */
  PA_ERR_LAUNCH = 5        /* the HIP runtime reported an error when launching */
} pa_status;

/* Element types.  PA_FP8_E4M3 (OCP 8-bit E4M3, "FN" encoding: bias 7, largest finite 448, no
 * infinities, S.1111.111 = NaN) is a cache element type only: pools of the _fp8 entry points,
 * pa_copy_blocks and pa_swap_blocks. */
typedef enum { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2, PA_FP8_E4M3 = 3 } pa_dtype;

/* Kernel family for pa_decode_ex.  PA_KERNEL_AUTO is what pa_decode uses. */
typedef enum {
  PA_KERNEL_AUTO = 0,
  PA_KERNEL_VALU = 1,  /* vector-ALU kernel: any head grouping, every dtype */
  PA_KERNEL_MFMA = 2   /* matrix-core kernel for grouped-query attention (f16/bf16) */
} pa_kernel;

/*
 * Flags for pa_decode_ex / pa_decode_partitions (bitwise OR; 0 is what pa_decode uses).
 * PA_DECODE_SHARED_BLOCKS: some physical blocks are read by several sequences of this call
 * (a shared prompt prefix, parallel-sampling siblings; xasun.com summary §二, sharing item).
 * K/V are then fetched with cache-allocating loads so later readers of a shared block hit in
 * the L2; without the flag they are fetched as streaming (non-temporal) loads, which is faster
 * when every block is read once.  The results are identical either way.
 */
#define PA_DECODE_SHARED_BLOCKS 0x1u

/* Human-readable name of a status code (static storage, never NULL). */
const char* pa_status_string(pa_status s);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int32_t pa_version(void);

/*
 * Partition length, in tokens, that pa_decode uses for split-KV when the caller passes
 * partition_size = 0.  Depends only on host scalars.  Returns 0 for invalid arguments.
 */
int32_t pa_decode_auto_partition(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size,
                                 int32_t max_blocks_per_seq);

/*
 * Bytes of workspace pa_decode needs for this shape (0 when no split is needed).  The
 * workspace holds, per (sequence, query head, partition), the fp32 running max, the fp32
 * softmax denominator and the fp32 normalised partial output [head_dim]; the merge kernel
 * combines them by their log-sum-exp weights.  `partition_size` as for pa_decode.
 */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size,
                                 int32_t max_blocks_per_seq, int32_t partition_size);

/*
 * pa_decode — single-query paged decode attention.
 *
 * For every sequence s and query head h, with n = context_lens[s], G = num_heads /
 * num_kv_heads and KV head g = h / G (contiguous groups):
 *   K_t = key_cache[block_tables[s][t / block_size]][g][t % block_size][:]  (t < n), V alike
 *   z_t = scale * <query[s][h], K_t>
 *   out[s][h] = sum_t softmax(z)_t * V_t          (softmax evaluated stably, shifted by a
 *                                                   running maximum; fp32 accumulation)
 * and out[s][h] = 0 when n <= 0.  pa_decode runs the matrix-core kernel when dtype is
 * PA_F16/PA_BF16, head_dim is 64, 80, 128 or 256 (80: the 128-dim products with dims 80 .. 127
 * held as zeros, never loaded or stored) and G is a multiple of 4, and the vector-ALU kernel
 * otherwise (arithmetic of each: see the element-type note at the top).  Paging changes where K/V live, not the result (the
 * xasun.com summary, section 一, calls the scheme lossless).
 *
 *   out           [num_seqs][num_heads][head_dim]                   dtype   (written)
 *   query         [num_seqs][num_heads][head_dim]                   dtype
 *   key_cache     [num_blocks][num_kv_heads][block_size][head_dim]  dtype
 *   value_cache   same as key_cache
 *   block_tables  int32 [num_seqs][max_blocks_per_seq]; entries j < ceil(n/block_size) must
 *                 be in [0, num_blocks); later entries are never read
 *   context_lens  int32 [num_seqs]; tokens cached for the sequence, including the one being
 *                 decoded; must be <= max_blocks_per_seq * block_size (larger is clamped)
 *   scale         softmax scale (fp32), typically 1/sqrt(head_dim)
 *   partition_size  tokens per split-KV partition: 0 = library choice
 *                 (pa_decode_auto_partition), otherwise a positive multiple of block_size
 *                 and of 16;
 *                 a partition size covering the whole table means a single pass
 *   workspace     device buffer of at least pa_decode_workspace_bytes(...) bytes (may be
 *                 NULL when that is 0); contents on entry are ignored
 *
 * Supported: block_size in {8, 16, 32, 64, 128}; head_dim 64 or 128 for every 16/32-bit
 * pa_dtype, and also 80 or 256 for PA_F16 / PA_BF16; num_heads a multiple of num_kv_heads;
 * num_seqs * num_heads below 2^31 (otherwise PA_ERR_BAD_SHAPE).  Slots past a sequence's
 * context, unused blocks and unused table entries are never read as values, so they may hold
 * anything (NaN included).
 * Errors: PA_ERR_NULL_PTR, PA_ERR_BAD_SHAPE, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE,
 * PA_ERR_LAUNCH.
 */
pa_status pa_decode(void* out, const void* query, const void* key_cache, const void* value_cache,
                    const int32_t* block_tables, const int32_t* context_lens,
                    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                    float scale, pa_dtype dtype, int32_t partition_size,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_ex — pa_decode with an explicit kernel family and flags.  PA_KERNEL_MFMA
 * requires dtype f16/bf16, head_dim 64, 80, 128 or 256 and num_heads / num_kv_heads a multiple of 4
 * (PA_ERR_UNSUPPORTED otherwise); PA_KERNEL_VALU accepts every supported shape.  `flags` is
 * a combination of PA_DECODE_* bits (unknown bits: PA_ERR_UNSUPPORTED).  Same arguments,
 * results and errors as pa_decode otherwise.
 */
pa_status pa_decode_ex(void* out, const void* query, const void* key_cache,
                       const void* value_cache, const int32_t* block_tables,
                       const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                       int32_t num_blocks, int32_t max_blocks_per_seq, float scale,
                       pa_dtype dtype, int32_t partition_size, void* workspace,
                       size_t workspace_bytes, pa_kernel kernel, uint32_t flags, void* stream);

/*
 * The two launches of pa_decode, exposed so a caller (or a profiler harness) can bracket
 * each with its own events.  pa_decode == pa_decode_partitions followed by pa_decode_merge
 * on the same stream with the same arguments.  pa_decode_partitions writes `out` directly
 * for every (sequence, head) whose context fits one partition and fp32 partials to the
 * workspace for the others; pa_decode_merge combines those partials into `out` and leaves
 * the rest of `out` alone.
 */
pa_status pa_decode_partitions(void* out, const void* query, const void* key_cache,
                               const void* value_cache, const int32_t* block_tables,
                               const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int32_t num_blocks, int32_t max_blocks_per_seq, float scale,
                               pa_dtype dtype, int32_t partition_size, void* workspace,
                               size_t workspace_bytes, pa_kernel kernel, uint32_t flags,
                               void* stream);

pa_status pa_decode_merge(void* out, const int32_t* context_lens, int32_t num_seqs,
                          int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t block_size, int32_t max_blocks_per_seq, pa_dtype dtype,
                          int32_t partition_size, const void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * pa_decode_noalloc — pa_decode_ex for callers that cannot allocate device memory: code that a
 * HIP graph captures, tight serving loops, hosts that forbid allocation.  The split-KV
 * partials that pa_decode_ex keeps in the caller's workspace live instead in a fixed array of
 * PA_DECODE_NOALLOC_SCRATCH_BYTES bytes inside the library, one per GPU, held from the first
 * call on that GPU until the process ends.  Arguments, results and errors are pa_decode_ex's
 * without the workspace pair; a shape whose pa_decode_workspace_bytes exceeds the array
 * returns PA_ERR_WORKSPACE before anything is launched (use pa_decode_ex with a workspace).
 * The call allocates nothing and issues no memset.  Every call on one GPU uses that GPU's
 * array: calls that can run at the same time on one GPU (on different streams, or from
 * several threads) race on it and must be serialised by the caller; calls in order on one
 * stream are safe.  The first call on a GPU looks up the array's device address
 * (PA_ERR_LAUNCH if the runtime cannot).
 */
#define PA_DECODE_NOALLOC_SCRATCH_BYTES (32u << 20)
pa_status pa_decode_noalloc(void* out, const void* query, const void* key_cache,
                            const void* value_cache, const int32_t* block_tables,
                            const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                            int32_t num_blocks, int32_t max_blocks_per_seq, float scale,
                            pa_dtype dtype, int32_t partition_size, pa_kernel kernel,
                            uint32_t flags, void* stream);

/*
 * pa_reshape_and_cache — store each new token's K and V at its physical slot.
 *
 * Every decode step appends the new token's key/value to its sequence's cache (jsqmd.com
 * page, paged-memory section and serving-workflow list).  For token i with
 * slot = slot_mapping[i] >= 0:  block = slot / block_size, offset = slot % block_size and
 *   key_cache[block][h][offset][:] = key[i][h][:]   for every KV head h (value alike).
 * Bits are copied unchanged.  A negative slot is skipped (padding); a slot >= num_blocks *
 * block_size is skipped as out of range.  Slots must be distinct (otherwise which token wins
 * is unspecified).
 *
 *   key, value    [num_tokens][num_kv_heads][head_dim]  dtype
 *   key_cache, value_cache  [num_blocks][num_kv_heads][block_size][head_dim]  (updated in place)
 *   slot_mapping  int64 [num_tokens]
 * Supported: head_dim * sizeof(dtype) a multiple of 16 bytes, head_dim <= 1024; block_size >= 1.
 */
pa_status pa_reshape_and_cache(const void* key, const void* value, void* key_cache,
                               void* value_cache, const int64_t* slot_mapping, int32_t num_tokens,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int32_t num_blocks, pa_dtype dtype, void* stream);

/*
 * pa_copy_blocks — copy-on-write block copies.
 *
 * Blocks shared between sequences are reference-counted and copied before one of the
 * sharers writes (xasun.com summary, sections 一 and 二, sharing item).  For each pair
 * p, with (src, dst) = (block_mapping[2p], block_mapping[2p+1]), the whole of block src —
 * every KV head and every slot — is copied to block dst, in both pools.  Pairs with an id
 * outside [0, num_blocks) are skipped.  Destinations must be distinct and must not be a
 * source of another pair (true of copy-on-write, which copies into fresh blocks); under that
 * condition the result does not depend on the order of the pairs.
 *
 *   key_cache, value_cache  [num_blocks][num_kv_heads][block_size][head_dim]  (updated in place)
 *   block_mapping  int64 [num_pairs][2]
 * Supported: num_kv_heads * block_size * head_dim * sizeof(dtype) a multiple of 16 bytes; dtype
 * may be PA_FP8_E4M3 (1 byte).
 */
pa_status pa_copy_blocks(void* key_cache, void* value_cache, const int64_t* block_mapping,
                         int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t num_blocks, pa_dtype dtype, void* stream);

/*
 * pa_swap_blocks — whole-block copies between two different pools: the GPU pool and a pool in
 * pinned host memory, in either direction.
 *
 * The block engine keeps block pools on both the GPU and the CPU; a preempted sequence's blocks
 * can be swapped out to the CPU pool and back in when it resumes (xasun.com summary §二,
 * block-engine and scheduler items).  For each pair p, with (src, dst) = (block_mapping[2p],
 * block_mapping[2p+1]), block src of the source pools (every KV head, every slot) is copied to
 * block dst of the destination pools.  Pairs with src outside [0, src_num_blocks) or dst outside
 * [0, dst_num_blocks) are skipped.  Bits are copied unchanged; destinations must be distinct.
 *
 *   src_key_cache, src_value_cache  [src_num_blocks][num_kv_heads][block_size][head_dim]
 *   dst_key_cache, dst_value_cache  [dst_num_blocks][num_kv_heads][block_size][head_dim]
 *   block_mapping  int64 [num_pairs][2]
 * Every pointer must be usable by the GPU: device memory, or host memory allocated pinned
 * (hipHostMalloc, or a torch tensor created with pin_memory=True), which the kernel reads or
 * writes over the host link.  The pools are not synchronised with the host: the caller waits
 * on `stream` before reading a host pool.
 * Supported: num_kv_heads * block_size * head_dim * sizeof(dtype) a multiple of 16 bytes; dtype
 * may be PA_FP8_E4M3 (1 byte).
 */
pa_status pa_swap_blocks(const void* src_key_cache, const void* src_value_cache,
                         int32_t src_num_blocks, void* dst_key_cache, void* dst_value_cache,
                         int32_t dst_num_blocks, const int64_t* block_mapping, int32_t num_pairs,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         pa_dtype dtype, void* stream);

/*
 * pa_prefill — causal attention of a chunk of new tokens per sequence over the paged cache
 * (prefill, or one chunk of a chunked prefill).
 *
 * Prefill is the compute-heavy phase before decoding (xasun.com summary §三, compute-pattern
 * row), and a long prompt may be prefilled in chunks (the chunked-prefill switch in the vLLM
 * example on the jsqmd.com page).  Sequence s owns query rows
 * query_start_loc[s] .. query_start_loc[s+1]-1 (L_s rows, L_s <= max_query_len).  Its
 * n = context_lens[s] cached tokens already include the chunk's own K/V (call
 * pa_reshape_and_cache for the chunk first), so chunk token i sits at position n - L_s + i:
 *   out[row][h] = sum_{t <= n-L_s+i} softmax_t(scale * <query[row][h], K_s[t][h/G]>) V_s[t][h/G]
 * with K_s/V_s read through block_tables as in pa_decode and G = num_heads / num_kv_heads.
 *
 *   out, query     [T][num_heads][head_dim] dtype, T = query_start_loc[num_seqs]
 *   key_cache, value_cache  [num_blocks][num_kv_heads][block_size][head_dim] dtype
 *   block_tables   int32 [num_seqs][max_blocks_per_seq]
 *   query_start_loc  int32 [num_seqs + 1], non-decreasing, query_start_loc[0] = 0
 *   context_lens   int32 [num_seqs]
 * Rows of a sequence with L_s > n, or n > max_blocks_per_seq * block_size, are written as
 * zeros; rows past max_query_len of a longer chunk are not written.  Only the first
 * ceil(n / block_size) table entries and the first n slots are read.
 * Supported: dtype f16 or bf16, head_dim 64, 80 or 128 (80: the 128-dim products with dims
 * 80 .. 127 held as zeros, never loaded or stored), block_size 8, 16, 32, 64 or 128.  Arithmetic: 16-bit
 * operands on the matrix cores with fp32 accumulation; the softmax probabilities keep about
 * 16 significant bits for bf16 (two products) and 11 for f16, unless flags has
 * PA_PREFILL_BF16_P, which rounds bf16 probabilities to bfloat16 once (one product, faster,
 * about 8 bits).  No workspace; nothing is allocated.
 */
#define PA_PREFILL_BF16_P 0x1u
pa_status pa_prefill(void* out, const void* query, const void* key_cache, const void* value_cache,
                     const int32_t* block_tables, const int32_t* query_start_loc,
                     const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                     int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_query_len,
                     float scale, pa_dtype dtype, uint32_t flags, void* stream);


/*
 * pa_prefill_ex — pa_prefill with the keys of long contexts split over workgroups.  A grid of
 * (sequence, KV head, 128-row tile) workgroups that would not fill the GPU for long (small
 * batches over long cached prefixes) is also cut along the keys: split k covers key tiles
 * [k * kv_split, (k + 1) * kv_split) of every row; a row whose keys span several splits gets
 * one partial (max, denominator, normalised output) per split, combined by their log-sum-exp
 * weights in a second launch (the decode merge).  The result equals pa_prefill's up to
 * rounding order.
 *   num_tokens   T, the rows of query and out (= query_start_loc[num_seqs])
 *   kv_split     tokens per key split, a multiple of 64; 0 = library choice (split only
 *                grids below ~1024 workgroups, at least 512 tokens per split); a value
 *                covering the whole table means no split
 *   workspace    device buffer of at least pa_prefill_workspace_bytes(...) bytes (may be
 *                NULL when that is 0); contents on entry are ignored
 * Errors as pa_prefill, plus PA_ERR_WORKSPACE for a missing or short workspace and
 * PA_ERR_BAD_SHAPE for a kv_split that is negative or not a multiple of 64, or num_tokens
 * < 1 when the keys are split.
 */
size_t pa_prefill_workspace_bytes(int32_t num_seqs, int32_t num_tokens, int32_t num_heads,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                  int32_t max_blocks_per_seq, int32_t max_query_len,
                                  int32_t kv_split);
pa_status pa_prefill_ex(void* out, const void* query, const void* key_cache,
                        const void* value_cache, const int32_t* block_tables,
                        const int32_t* query_start_loc, const int32_t* context_lens,
                        int32_t num_seqs, int32_t num_tokens, int32_t num_heads,
                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                        int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_query_len,
                        float scale, pa_dtype dtype, int32_t kv_split, void* workspace,
                        size_t workspace_bytes, uint32_t flags, void* stream);
/*
 * 8-bit KV cache.  The cache element type is a serving choice (kv_cache_dtype in the vLLM
 * configuration on the yongjin360.com page, §3.2); an E4M3 cache halves the bytes decode
 * streams.  Each pool has one positive float scale: a stored code c stands for c * scale.
 *
 * pa_reshape_and_cache_fp8 — pa_reshape_and_cache into E4M3 pools: for token i with a slot in
 * the pool, every element x of key[i] is stored as E4M3(clamp(x * (1/k_scale), -448, 448)),
 * with 1/k_scale rounded to float once, the product in float, and nearest-even rounding to
 * E4M3 (value alike with v_scale).  Negative or out-of-pool slots are skipped.
 *   key, value  [num_tokens][num_kv_heads][head_dim]  dtype (PA_F16 or PA_BF16)
 *   key_cache, value_cache  uint8 [num_blocks][num_kv_heads][block_size][head_dim]
 * Supported: head_dim a multiple of 8, at most 1024.  Scales must be finite and > 0.
 */
pa_status pa_reshape_and_cache_fp8(const void* key, const void* value, void* key_cache,
                                   void* value_cache, const int64_t* slot_mapping,
                                   int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block_size, int32_t num_blocks, pa_dtype dtype,
                                   float k_scale, float v_scale, void* stream);

/*
 * pa_decode_fp8 — pa_decode over E4M3 pools: the result is decode attention over
 * K = code * k_scale and V = code * v_scale (exact values), with fp32 accumulation.  query and
 * out are dtype (PA_F16 or PA_BF16); pools are uint8 as above; partition_size, workspace
 * (pa_decode_workspace_bytes with the same sizes), flags and errors as pa_decode_ex.
 * pa_decode_fp8_partitions is its first launch (pa_decode_merge, with the same dtype, is the
 * second).  Supported: head_dim 64, 80, 128 or 256, block_size 8, 16, 32, 64 or 128.  When
 * head_dim is 64, 80, 128 or 256 and num_heads / num_kv_heads is a multiple of 4 (and partition_size
 * one of 16) the grouped heads run on the matrix cores, the codes converted exactly to dtype in
 * registers; otherwise on the vector ALUs.
 */
pa_status pa_decode_fp8(void* out, const void* query, const void* key_cache,
                        const void* value_cache, const int32_t* block_tables,
                        const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                        int32_t num_blocks, int32_t max_blocks_per_seq, float scale,
                        pa_dtype dtype, float k_scale, float v_scale, int32_t partition_size,
                        void* workspace, size_t workspace_bytes, uint32_t flags, void* stream);
pa_status pa_decode_fp8_partitions(void* out, const void* query, const void* key_cache,
                                   const void* value_cache, const int32_t* block_tables,
                                   const int32_t* context_lens, int32_t num_seqs,
                                   int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block_size, int32_t num_blocks,
                                   int32_t max_blocks_per_seq, float scale, pa_dtype dtype,
                                   float k_scale, float v_scale, int32_t partition_size,
                                   void* workspace, size_t workspace_bytes, uint32_t flags,
                                   void* stream);

/*
 * pa_prefill_fp8 — pa_prefill_ex over E4M3 pools: the result is prefill attention over
 * K = code * k_scale and V = code * v_scale (exact values).  query and out are dtype (PA_F16 or
 * PA_BF16); pools are uint8 as above.  The codes are widened exactly to dtype as each key/value
 * tile is staged, so the products, the probability precision (flags: PA_PREFILL_BF16_P) and the
 * key splits (kv_split, workspace: pa_prefill_workspace_bytes with the same sizes) are
 * pa_prefill_ex's; k_scale is folded into the score scale (one rounding of scale * k_scale) and
 * v_scale into the final normalisation.  Supported shapes as pa_prefill.  Errors as
 * pa_prefill_ex, plus PA_ERR_BAD_SHAPE for a scale that is not finite and > 0.
 */
pa_status pa_prefill_fp8(void* out, const void* query, const void* key_cache,
                         const void* value_cache, const int32_t* block_tables,
                         const int32_t* query_start_loc, const int32_t* context_lens,
                         int32_t num_seqs, int32_t num_tokens, int32_t num_heads,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_query_len,
                         float scale, pa_dtype dtype, float k_scale, float v_scale,
                         int32_t kv_split, void* workspace, size_t workspace_bytes,
                         uint32_t flags, void* stream);

/*
 * Block engine on the device.  The KV cache manager maps each sequence's logical blocks to
 * physical ones, allocates on demand and reclaims (xasun.com summary §二, block-engine item);
 * shared blocks carry reference counts and are copied before a sharer writes (same page,
 * sharing item).  These entry points keep that state in caller-owned device arrays so a
 * decode step's slots and copy pairs are produced on the GPU:
 *   block_tables  int32 [num_seqs][max_blocks_per_seq]
 *   context_lens  int32 [num_seqs]
 *   ref_counts    int32 [num_blocks]: how many table entries name each block
 *   free_stack    int32 [num_blocks]; free_top int32 [1]: free_stack[0 .. *free_top-1] are
 *                 the free blocks (the top entry is taken first)
 * Calls on one stream see each other's updates in order; calls that overlap on the same
 * state race.
 *
 * pa_append_slots — append one token to each sequence seq_ids[i] (distinct ids).  With n its
 * length: if n is a multiple of block_size, a free block is taken for the token; else if its
 * last block is shared (reference count > 1), a free block is taken, the pair (old, new) is
 * appended to block_mapping (int64 [num_append][2]; *num_pairs counts them), the old block
 * loses a reference and the table points at the new one; else the token goes into the last
 * block.  slot_mapping[i] (int64) = block * block_size + n % block_size and the length grows
 * by one.  The outcome equals some one-at-a-time order of the sequences (which free block a
 * sequence receives, and which sharer keeps a shared block, may differ between runs).  A
 * sequence that cannot append gets slot -1, keeps its state, and raises *status (int32,
 * device): 1 no free block, 2 table full, 3 a sequence or block id outside its array; 0 if
 * all appended.  *num_pairs and *status are always written, also for num_append = 0.
 */
pa_status pa_append_slots(int32_t* block_tables, int32_t* context_lens, int32_t* ref_counts,
                          int32_t* free_stack, int32_t* free_top, int32_t num_seqs,
                          int32_t max_blocks_per_seq, int32_t block_size, int32_t num_blocks,
                          const int32_t* seq_ids, int32_t num_append, int64_t* slot_mapping,
                          int64_t* block_mapping, int32_t* num_pairs, int32_t* status,
                          void* stream);

/*
 * pa_fork_seqs — for each (parent, child) row of parent_child (int32 [num_forks][2]), the
 * child gets the parent's table entries and length and every block of the parent gains one
 * reference (parallel sampling).  Children must be distinct, hold no blocks, and not be
 * parents in the same call.
 */
pa_status pa_fork_seqs(int32_t* block_tables, int32_t* context_lens, int32_t* ref_counts,
                       int32_t num_seqs, int32_t max_blocks_per_seq, int32_t block_size,
                       int32_t num_blocks, const int32_t* parent_child, int32_t num_forks,
                       void* stream);

/*
 * pa_free_seqs — drop each sequence seq_ids[i] (distinct): every block loses a reference,
 * blocks left with none are pushed on the free stack (in no particular order), the table
 * entries become -1 and the length 0.
 */
pa_status pa_free_seqs(int32_t* block_tables, int32_t* context_lens, int32_t* ref_counts,
                       int32_t* free_stack, int32_t* free_top, int32_t num_seqs,
                       int32_t max_blocks_per_seq, int32_t block_size, int32_t num_blocks,
                       const int32_t* seq_ids, int32_t num_free, void* stream);

/*
 * pa_copy_blocks_counted — pa_copy_blocks with the pair count read on the device
 * (*num_pairs, as pa_append_slots writes it); max_pairs bounds it and sizes the launch.
 * block_mapping must hold max_pairs readable rows (rows past *num_pairs are read, not used).
 */
pa_status pa_copy_blocks_counted(void* key_cache, void* value_cache, const int64_t* block_mapping,
                                 const int32_t* num_pairs, int32_t max_pairs,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                 int32_t num_blocks, pa_dtype dtype, void* stream);

/*
 * pa_block_hashes — prefix hashes of full blocks, so blocks of a common prompt prefix (a
 * fixed system prompt: yongjin360.com page §5.1, prefix caching) can be recognised:
 *   g_j = FNV-1a-64 of the block's block_size token ids (int32, little-endian bytes),
 *   h_j = FNV-1a-64 of the 16 bytes h_{j-1} || g_j (little-endian; h_{-1} = 0),
 * so h_j depends on exactly the tokens 0 .. (j+1)*block_size - 1.
 *   token_ids  int32 [num_seqs][max_tokens]; num_tokens int32 [num_seqs]
 *   hashes     uint64 [num_seqs][max_tokens / block_size] (written; 0 for blocks not full)
 */
pa_status pa_block_hashes(const int32_t* token_ids, const int32_t* num_tokens, int32_t num_seqs,
                          int32_t max_tokens, int32_t block_size, uint64_t* hashes,
                          void* stream);

/*
 * pa_read_tiles — read-only bandwidth probe (measurement, not part of the attention path).
 * Decode is bound by memory bandwidth (xasun.com summary §三, compute-pattern row), so its
 * achieved rate is compared with what a kernel that only reads can reach in the same access
 * pattern.  The buffer `base` holds base_tiles tiles of tile_bytes bytes each; tile t of the
 * call is tile tile_ids[t] of the buffer (tile_ids NULL: tile t itself, a contiguous run).
 * Every tile is read whole with the decode kernels' loads (16 bytes per lane, non-temporal)
 * and xor_out[t] (uint32, device, num_tiles entries, written) receives the XOR of its 32-bit
 * words; a tile id outside [0, base_tiles) is skipped and reports 0.
 * Supported: tile_bytes 1024, 2048, 4096 or 8192; with tile_ids NULL, num_tiles <= base_tiles.
 * Errors: PA_ERR_NULL_PTR, PA_ERR_BAD_SHAPE, PA_ERR_UNSUPPORTED, PA_ERR_LAUNCH.
 */
pa_status pa_read_tiles(const void* base, int64_t base_tiles, int32_t tile_bytes,
                        const int32_t* tile_ids, int32_t num_tiles, uint32_t* xor_out,
                        void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
