// pa_decode_noalloc: pa_decode_ex for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, hosts that forbid allocation).  The split-KV partials
// that pa_decode_ex keeps in the caller's workspace live here in a fixed array, one per GPU,
// held until the process ends.
#include <mutex>

#include "pa_common.h"

#ifndef PA_DECODE_NOALLOC_SCRATCH_BYTES
#error "pa.h must define PA_DECODE_NOALLOC_SCRATCH_BYTES"
#endif

// In host code this name only stands for the symbol: passing it to a kernel would hand the
// kernel a host address.  scratch_address() looks up each device's own copy once, with that
// device current, and only that address is used.
static __device__ __align__(256) unsigned char scratch[PA_DECODE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first call on it).
pa_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PA_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return PA_ERR_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PA_OK;
}

}  // namespace

extern "C" pa_status pa_decode_noalloc(void* out, const void* query, const void* key_cache,
                                       const void* value_cache, const int32_t* block_tables,
                                       const int32_t* context_lens, int32_t num_seqs,
                                       int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                       int32_t block_size, int32_t num_blocks,
                                       int32_t max_blocks_per_seq, float scale, pa_dtype dtype,
                                       int32_t partition_size, pa_kernel kernel, uint32_t flags,
                                       void* stream) {
  if (num_seqs < 0) return PA_ERR_BAD_SHAPE;
  // pa_decode_workspace_bytes is 0 both for a single pass and for invalid shapes; pa_decode_ex
  // then reports the shape error itself
  const size_t need = pa_decode_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_dim,
                                                block_size, max_blocks_per_seq, partition_size);
  if (need > (size_t)PA_DECODE_NOALLOC_SCRATCH_BYTES) return PA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0 && num_seqs > 0) {
    const pa_status st = scratch_address(&ws);
    if (st != PA_OK) return st;
  }
  // Every partial the merge reads is written by the partition launch of the same call, so
  // whatever an earlier call left in the array is never read and nothing needs clearing.
  return pa_decode_ex(out, query, key_cache, value_cache, block_tables, context_lens, num_seqs,
                      num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                      max_blocks_per_seq, scale, dtype, partition_size, ws,
                      ws ? (size_t)PA_DECODE_NOALLOC_SCRATCH_BYTES : 0, kernel, flags, stream);
}
