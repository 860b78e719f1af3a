// Block engine on the device: append one token per sequence with copy-on-write, fork, free,
// and prefix-block hashes, so a decode step's slots and copy pairs are produced where the
// tables live, with no host round trip.
//
// The KV cache manager maps logical to physical blocks, allocates on demand and reclaims
// (UltraLAB summary of Kwon et al. (xasun.com) §二, block-engine item); shared blocks carry
// reference counts and are copied before a sharer writes into them (same page, sharing item);
// full blocks of a common prompt prefix can be reused, which the per-block prefix hashes
// identify ("GPT-OSS显存管理技巧" (yongjin360.com) §5.1, prefix caching).
//
// Concurrency.  Appends of different sequences run in parallel threads of one workgroup and
// meet only in atomics: the free stack is popped with atomicSub on its top (the first `top`
// decrements succeed, later ones undo theirs, so a failed pop means the stack is empty for the
// rest of the call: nothing pushes during an append).  A sequence writing into a partly filled
// last block takes one reference off it with atomicSub.  If the count it saw was above 1 another
// holder remains, so it copies into a fresh block, or, with none left, puts its reference back
// and fails.  If it saw 1 it may be the last holder, but a sharer whose copy failed may still
// put its reference back: so it decides only after a barrier, once every copy of the batch has
// succeeded or failed.  A count still at 0 means every other sharer moved to a copy and it
// writes in place; otherwise a sharer stayed (the block is still shared) and, the stack being
// empty, it fails as well, as it would in any one-at-a-time order.  Batches of 1024 sequences
// run one after another.  Every outcome equals processing the sequences one at a time in some
// order; which popped block a sequence gets, and which sharer keeps a shared block, depend on
// that order.
#include "pa_common.h"

namespace pa {
namespace {

constexpr int kAppendThreads = 1024;

// Pops a free block id (-1 when none is left; an id outside the pool raises status 3).
__device__ __forceinline__ int pop_free(const EngineState& e, int32_t* status) {
  const int t = atomicSub(e.free_top, 1) - 1;
  if (t < 0) {                                       // empty: undo the decrement
    atomicAdd(e.free_top, 1);
    atomicMax(status, 1);
    return -1;
  }
  const int b = e.free_stack[t];
  if ((unsigned)b >= (unsigned)e.num_blocks) {
    atomicMax(status, 3);
    return -1;
  }
  return b;
}

// One workgroup: thread i appends to sequence seq_ids[i], then i + 1024, ... in batches
// separated by barriers (every thread runs every batch, so the barriers pair up).
__global__ __launch_bounds__(kAppendThreads) void append_slots_kernel(
    EngineState e, const int32_t* __restrict__ seq_ids, int n, int64_t* __restrict__ slots,
    int64_t* __restrict__ pairs, int32_t* __restrict__ num_pairs, int32_t* __restrict__ status) {
  if (threadIdx.x == 0) {
    *num_pairs = 0;
    *status = 0;
  }
  __syncthreads();
  const int bs = e.block_size;
  for (int batch = 0; batch < n; batch += blockDim.x) {
    const int i = batch + threadIdx.x;
    int64_t slot = -1;
    int s = -1, len = 0, off = 0;
    int last_block = -1;   // the partly filled last block this thread was last to let go of
    if (i < n) {
      s = seq_ids[i];
      if ((unsigned)s >= (unsigned)e.num_seqs) {       // not a sequence of these tables
        atomicMax(status, 3);
        s = -1;
      } else {
        len = e.context_lens[s];
        const int j = len / bs;
        off = len - j * bs;
        int32_t* row = e.tables + (size_t)s * e.max_blocks_per_seq;
        if (len < 0 || j >= e.max_blocks_per_seq) {    // the table is full
          atomicMax(status, 2);
        } else if (off == 0) {                         // the last block is full: a fresh one
          const int nb = pop_free(e, status);
          if (nb >= 0) {
            row[j] = nb;
            e.ref_counts[nb] = 1;
            slot = (int64_t)nb * bs;
          }
        } else if ((unsigned)row[j] >= (unsigned)e.num_blocks) {   // a broken table entry
          atomicMax(status, 3);
        } else {
          const int b = row[j];
          if (atomicSub(&e.ref_counts[b], 1) > 1) {    // another holder remains: copy on write
            const int nb = pop_free(e, status);
            if (nb < 0) {
              atomicAdd(&e.ref_counts[b], 1);          // no block left: keep the shared one
            } else {
              const int k = atomicAdd(num_pairs, 1);
              pairs[2 * k] = b;
              pairs[2 * k + 1] = nb;
              e.ref_counts[nb] = 1;
              row[j] = nb;
              slot = (int64_t)nb * bs + off;
            }
          } else {
            last_block = b;                            // decided after the barrier
          }
        }
      }
    }
    __syncthreads();   // every copy decision of this batch (and every put-back) is done
    if (last_block >= 0) {
      if (atomicAdd(&e.ref_counts[last_block], 0) == 0) {   // every other sharer moved off
        atomicAdd(&e.ref_counts[last_block], 1);
        slot = (int64_t)last_block * bs + off;
      } else {                                         // still shared and no block left
        atomicAdd(&e.ref_counts[last_block], 1);
        atomicMax(status, 1);
      }
    }
    if (i < n) {
      if (slot >= 0) e.context_lens[s] = len + 1;
      slots[i] = slot;
    }
    __syncthreads();   // the next batch sees this one's counts and lengths
  }
}

// One workgroup per (parent, child) pair.
__global__ __launch_bounds__(256) void fork_kernel(EngineState e,
                                                   const int32_t* __restrict__ parent_child) {
  const int parent = parent_child[2 * blockIdx.x], child = parent_child[2 * blockIdx.x + 1];
  if ((unsigned)parent >= (unsigned)e.num_seqs || (unsigned)child >= (unsigned)e.num_seqs) return;
  const int len = e.context_lens[parent];
  const int nb = min((len + e.block_size - 1) / e.block_size, e.max_blocks_per_seq);
  const int32_t* src = e.tables + (size_t)parent * e.max_blocks_per_seq;
  int32_t* dst = e.tables + (size_t)child * e.max_blocks_per_seq;
  for (int j = threadIdx.x; j < nb; j += blockDim.x) {
    const int b = src[j];
    dst[j] = b;
    if ((unsigned)b < (unsigned)e.num_blocks) atomicAdd(&e.ref_counts[b], 1);
  }
  if (threadIdx.x == 0) e.context_lens[child] = len;
}

// One workgroup per freed sequence.
__global__ __launch_bounds__(256) void free_kernel(EngineState e, const int32_t* __restrict__ seq_ids) {
  const int s = seq_ids[blockIdx.x];
  if ((unsigned)s >= (unsigned)e.num_seqs) return;
  const int len = e.context_lens[s];
  const int nb = min((len + e.block_size - 1) / e.block_size, e.max_blocks_per_seq);
  int32_t* row = e.tables + (size_t)s * e.max_blocks_per_seq;
  for (int j = threadIdx.x; j < nb; j += blockDim.x) {
    const int b = row[j];
    if ((unsigned)b < (unsigned)e.num_blocks && atomicSub(&e.ref_counts[b], 1) == 1) {
      const int t = atomicAdd(e.free_top, 1);
      if (t < e.num_blocks) e.free_stack[t] = b;
    }
    row[j] = -1;
  }
  __syncthreads();
  if (threadIdx.x == 0) e.context_lens[s] = 0;
}

// 64-bit FNV-1a over `nbytes` bytes of `words` (little-endian 32-bit words), from h.
__device__ __forceinline__ uint64_t fnv1a_words(uint64_t h, const uint32_t* words, int nwords) {
  constexpr uint64_t kPrime = 0x100000001B3ull;
  for (int w = 0; w < nwords; ++w) {
    const uint32_t v = words[w];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      h ^= (v >> (8 * k)) & 0xFFu;
      h *= kPrime;
    }
  }
  return h;
}

// One workgroup per sequence: 256 blocks' token hashes g_j in parallel, then one thread
// chains h_j = FNV(h_{j-1} || g_j) in order.
__global__ __launch_bounds__(256) void block_hashes_kernel(const int32_t* __restrict__ tokens,
                                                           const int32_t* __restrict__ num_tokens,
                                                           int max_tokens, int block_size,
                                                           uint64_t* __restrict__ hashes) {
  constexpr uint64_t kOffset = 0xCBF29CE484222325ull;
  __shared__ uint64_t s_g[256];
  const int s = blockIdx.x;
  const int max_blocks = max_tokens / block_size;
  const int full = min(num_tokens[s], max_tokens) / block_size;
  const uint32_t* tok = reinterpret_cast<const uint32_t*>(tokens) + (size_t)s * max_tokens;
  uint64_t* out = hashes + (size_t)s * max_blocks;
  uint64_t h = 0;
  for (int j0 = 0; j0 < full; j0 += 256) {
    const int j = j0 + threadIdx.x;
    if (j < full) s_g[threadIdx.x] = fnv1a_words(kOffset, tok + (size_t)j * block_size, block_size);
    __syncthreads();
    if (threadIdx.x == 0) {
      const int cnt = min(256, full - j0);
      for (int k = 0; k < cnt; ++k) {
        const uint32_t pair[4] = {(uint32_t)h, (uint32_t)(h >> 32), (uint32_t)s_g[k],
                                  (uint32_t)(s_g[k] >> 32)};
        h = fnv1a_words(kOffset, pair, 4);
        out[j0 + k] = h;
      }
    }
    __syncthreads();
  }
  for (int j = full + threadIdx.x; j < max_blocks; j += blockDim.x) out[j] = 0;
}

}  // namespace

hipError_t launch_append_slots(const EngineState& e, const int32_t* seq_ids, int n,
                               int64_t* slots, int64_t* pairs, int32_t* num_pairs,
                               int32_t* status, hipStream_t st) {
  hipLaunchKernelGGL(append_slots_kernel, dim3(1), dim3(kAppendThreads), 0, st, e, seq_ids, n,
                     slots, pairs, num_pairs, status);
  return hipGetLastError();
}

hipError_t launch_fork(const EngineState& e, const int32_t* parent_child, int n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fork_kernel, dim3(n), dim3(256), 0, st, e, parent_child);
  return hipGetLastError();
}

hipError_t launch_free_seqs(const EngineState& e, const int32_t* seq_ids, int n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(free_kernel, dim3(n), dim3(256), 0, st, e, seq_ids);
  return hipGetLastError();
}

hipError_t launch_block_hashes(const int32_t* tokens, const int32_t* num_tokens, int num_seqs,
                               int max_tokens, int block_size, uint64_t* hashes, hipStream_t st) {
  if (num_seqs <= 0) return hipSuccess;
  hipLaunchKernelGGL(block_hashes_kernel, dim3(num_seqs), dim3(256), 0, st, tokens, num_tokens,
                     max_tokens, block_size, hashes);
  return hipGetLastError();
}

}  // namespace pa
