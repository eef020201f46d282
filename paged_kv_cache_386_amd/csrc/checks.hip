// Index checking (a debug mode, off by default): before a call launches its
// kernels, one workgroup scans the indices those kernels will read -- context
// lengths, the used block-table entries, query offsets, slots, copy pairs --
// and records in a library-owned device word whether any is out of range;
// the host copies the word back after a stream synchronisation and the call
// returns PA_ERR_INDEX instead of launching.  Without the check the kernels
// clamp or skip such indices, so every access stays in bounds, but the
// numbers are unspecified.
//
// One workgroup writes the word with a plain store at its end, so no reset
// is needed between calls; calls that overlap on one device share the word
// and race.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <cstdlib>
#include <cstring>

#include "internal.h"
#include "pagedattn.h"

namespace pa {
namespace {

constexpr int kCheckThreads = 1024;

__device__ int32_t g_index_error;  // 1: the last check found a bad index

// -1: not decided yet (read PAGEDATTN_CHECK on first use), 0 off, 1 on
std::atomic<int> g_check_mode{-1};

__device__ __forceinline__ void publish(bool bad) {
  const int any = __syncthreads_or(bad ? 1 : 0);
  if (threadIdx.x == 0) g_index_error = any ? 1 : 0;
}

// Context lengths in [0, max_ctx]; entries 0 .. ceil(L/B)-1 of each row of
// the table in [0, nb) (L clamped to [0, max_ctx], which the host has
// checked against the row length).
__global__ __launch_bounds__(kCheckThreads) void check_tables_kernel(
    const int32_t *__restrict__ lens, const int32_t *__restrict__ tables, int S, int mb, int lgB,
    int nb, int max_ctx) {
  bool bad = false;
  for (int s = threadIdx.x; s < S; s += kCheckThreads) {
    const int L = lens[s];
    bad |= L < 0 || L > max_ctx;
  }
  const int64_t entries = (int64_t)S * mb;
  for (int64_t i = threadIdx.x; i < entries; i += kCheckThreads) {
    const int s = (int)(i / mb);
    const int j = (int)(i % mb);
    const int L = min(max(lens[s], 0), max_ctx);
    if (j < (L + (1 << lgB) - 1) >> lgB) {
      const int id = tables[i];
      bad |= id < 0 || id >= nb;
    }
  }
  publish(bad);
}

// query_start[0] == 0, non-decreasing, query_start[S] <= T, and each
// sequence's n rows at most its context and max_q.
__global__ __launch_bounds__(kCheckThreads) void check_queries_kernel(
    const int32_t *__restrict__ lens, const int32_t *__restrict__ query_start, int S, int T,
    int max_q) {
  bool bad = threadIdx.x == 0 && (query_start[0] != 0 || query_start[S] > T);
  for (int s = threadIdx.x; s < S; s += kCheckThreads) {
    const int n = query_start[s + 1] - query_start[s];
    bad |= n < 0 || n > max_q || n > lens[s];
  }
  publish(bad);
}

// Slots below num_slots (negative ones are padding).
__global__ __launch_bounds__(kCheckThreads) void check_slots_kernel(
    const int32_t *__restrict__ slots, int T, int64_t num_slots) {
  bool bad = false;
  for (int i = threadIdx.x; i < T; i += kCheckThreads) bad |= (int64_t)slots[i] >= num_slots;
  publish(bad);
}

// Both ids of every copy pair in [0, nb).
__global__ __launch_bounds__(kCheckThreads) void check_pairs_kernel(
    const int32_t *__restrict__ pairs, int num_pairs, int nb) {
  bool bad = false;
  for (int i = threadIdx.x; i < 2 * num_pairs; i += kCheckThreads) {
    const int id = pairs[i];
    bad |= id < 0 || id >= nb;
  }
  publish(bad);
}

// The verdict of the check just enqueued on `stream`.
int32_t read_verdict(hipStream_t stream) {
  if (hipGetLastError() != hipSuccess) return PA_ERR_LAUNCH;
  int32_t word = 0;
  if (hipMemcpyFromSymbolAsync(&word, HIP_SYMBOL(g_index_error), sizeof(word), 0,
                               hipMemcpyDeviceToHost, stream) != hipSuccess)
    return PA_ERR_LAUNCH;
  if (hipStreamSynchronize(stream) != hipSuccess) return PA_ERR_LAUNCH;
  return word ? PA_ERR_INDEX : PA_OK;
}

}  // namespace

bool index_check_on() {
  int mode = g_check_mode.load(std::memory_order_relaxed);
  if (mode < 0) {
    const char *env = std::getenv("PAGEDATTN_CHECK");
    const int fresh = (env && std::strcmp(env, "1") == 0) ? 1 : 0;
    int expected = -1;
    g_check_mode.compare_exchange_strong(expected, fresh);
    mode = g_check_mode.load(std::memory_order_relaxed);
  }
  return mode == 1;
}

void set_index_check(bool on) { g_check_mode.store(on ? 1 : 0, std::memory_order_relaxed); }

int32_t check_tables(const int32_t *lens, const int32_t *tables, int32_t num_seqs,
                     int32_t max_blocks_per_seq, int32_t log2_block_size, int32_t num_blocks,
                     int32_t max_context_len, hipStream_t stream) {
  hipLaunchKernelGGL(check_tables_kernel, dim3(1), dim3(kCheckThreads), 0, stream, lens, tables,
                     num_seqs, max_blocks_per_seq, log2_block_size, num_blocks, max_context_len);
  return read_verdict(stream);
}

int32_t check_queries(const int32_t *lens, const int32_t *query_start, int32_t num_seqs,
                      int32_t num_tokens, int32_t max_query_len, hipStream_t stream) {
  hipLaunchKernelGGL(check_queries_kernel, dim3(1), dim3(kCheckThreads), 0, stream, lens,
                     query_start, num_seqs, num_tokens, max_query_len);
  return read_verdict(stream);
}

int32_t check_slots(const int32_t *slots, int32_t num_tokens, int64_t num_slots,
                    hipStream_t stream) {
  hipLaunchKernelGGL(check_slots_kernel, dim3(1), dim3(kCheckThreads), 0, stream, slots,
                     num_tokens, num_slots);
  return read_verdict(stream);
}

int32_t check_pairs(const int32_t *pairs, int32_t num_pairs, int32_t num_blocks,
                    hipStream_t stream) {
  hipLaunchKernelGGL(check_pairs_kernel, dim3(1), dim3(kCheckThreads), 0, stream, pairs,
                     num_pairs, num_blocks);
  return read_verdict(stream);
}

}  // namespace pa

extern "C" {

void pagedattn_set_index_check(int32_t enable) { pa::set_index_check(enable != 0); }

int32_t pagedattn_index_check(void) { return pa::index_check_on() ? 1 : 0; }

}  // extern "C"
