// paged_attention_decode_noalloc: decode for callers that cannot allocate
// device memory (code under graph capture, tight serving loops, harnesses
// that forbid hipMalloc).  The work is paged_attention_decode's; its
// workspace (the split-K partials and the longest-first dispatch list) lives
// in `scratch`, a file-scope device array of kScratchBytes that each GPU the
// library runs on holds from the library's load until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is looked up once per device, with that device current,
// through hipGetSymbolAddress, and only that address is ever handed to a
// kernel.  Every call on one GPU shares that GPU's array, which keeps the
// last call's contents; nothing in it has to start at zero (a call writes
// every partial and list entry before it reads it), and calls that overlap
// on one GPU race on it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "internal.h"
#include "pagedattn.h"

namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;
constexpr int kMaxDevices = 64;

__device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_lookup_mutex;
std::atomic<void *> g_scratch_ptr[kMaxDevices];

// The device address of the current device's `scratch`, looked up on the
// first call on that device; nullptr if the runtime cannot give it.
void *scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_lookup_mutex);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (!p) {
    void *addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) return nullptr;
    p = addr;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" {

size_t paged_attention_noalloc_scratch_bytes(void) { return kScratchBytes; }

int32_t paged_attention_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                       const int32_t *block_tables, const int32_t *context_lens,
                                       float scale, float *out, int32_t num_seqs,
                                       int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                       int32_t max_blocks_per_seq, int32_t max_context_len,
                                       int32_t dtype, int32_t partition_size, void *stream) {
  const size_t need = paged_attention_workspace_size(num_seqs, num_q_heads, num_kv_heads,
                                                     head_dim, max_context_len, partition_size);
  if (need > kScratchBytes) return PA_ERR_SCRATCH;
  void *ws = nullptr;
  size_t ws_bytes = 0;
  if (need > 0) {
    ws = scratch_on_current_device();
    if (!ws) return PA_ERR_LAUNCH;
    ws_bytes = kScratchBytes;
  }
  return paged_attention_decode(q, k_cache, v_cache, block_tables, context_lens, scale, out,
                                num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                num_blocks, max_blocks_per_seq, max_context_len, dtype,
                                partition_size, ws, ws_bytes, stream);
}

}  // extern "C"
