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

// Prefix groups: each (first, count) with count in [1, max_members] inside
// [0, S), the groups in ascending order and disjoint; every shared length in
// [0, L]; a sequence outside every group shares nothing; and the rows of one
// group's members name the same blocks below the shorter of their two shared
// lengths (checked against the group's member with the longest shared
// length, which implies it for every pair).  Lengths are taken as the kernels
// take them: clamped, whole 16-token tiles.
__global__ __launch_bounds__(kCheckThreads) void check_prefix_kernel(
    const int32_t *__restrict__ lens, const int32_t *__restrict__ tables,
    const int32_t *__restrict__ groups, int num_groups, const int32_t *__restrict__ shared_lens,
    int S, int mb, int lgB, int max_ctx, int max_members) {
  bool bad = false;
  for (int i = threadIdx.x; i < num_groups; i += kCheckThreads) {
    const int first = groups[2 * i], count = groups[2 * i + 1];
    bad |= first < 0 || count < 1 || count > max_members || first >= S || count > S - first;
    if (i > 0) bad |= first < groups[2 * i - 2] + groups[2 * i - 1];
  }
  // each sequence: its group by binary search over the (ascending) firsts
  for (int s = threadIdx.x; s < S; s += kCheckThreads) {
    const int L = min(max(lens[s], 0), max_ctx);
    const int raw = shared_lens[s];
    bad |= raw < 0 || raw > L;
    const int sh = min(max(raw, 0), L) & ~15;
    int lo = 0, hi = num_groups - 1, gi = -1;
    while (lo <= hi) {
      const int mid = (lo + hi) / 2;
      if (groups[2 * mid] <= s) {
        gi = mid;
        lo = mid + 1;
      } else {
        hi = mid - 1;
      }
    }
    const bool member = gi >= 0 && s < groups[2 * gi] + groups[2 * gi + 1];
    if (!member) {
      bad |= sh > 0;
      continue;
    }
    const int f = groups[2 * gi];
    if (f < 0 || f >= S) continue;  // flagged above
    const int count = max(0, min(min(groups[2 * gi + 1], S - f), max_members));
    int top = f, top_sh = -1;
    for (int m = f; m < f + count; ++m) {
      const int Lm = min(max(lens[m], 0), max_ctx);
      const int shm = min(max(shared_lens[m], 0), Lm) & ~15;
      if (shm > top_sh) {
        top_sh = shm;
        top = m;
      }
    }
    const int nblk = (sh + (1 << lgB) - 1) >> lgB;
    for (int j = 0; j < nblk && j < mb; ++j)
      bad |= tables[(int64_t)s * mb + j] != tables[(int64_t)top * mb + j];
  }
  publish(bad);
}

// A dispatch list the caller planned: a permutation of the items 0 .. n-1
// (each exactly once; n at most 65536 items, the bitmap in LDS).
constexpr int kMaxListItems = 65536;
__global__ __launch_bounds__(kCheckThreads) void check_dispatch_kernel(
    const int32_t *__restrict__ dispatch, int n) {
  __shared__ uint32_t seen[kMaxListItems / 32];
  for (int i = threadIdx.x; i < kMaxListItems / 32; i += kCheckThreads) seen[i] = 0u;
  __syncthreads();
  bool bad = n > kMaxListItems;
  if (!bad) {
    for (int i = threadIdx.x; i < n; i += kCheckThreads) {
      const int c = dispatch[i];
      if (c < 0 || c >= n) {
        bad = true;
      } else {
        const uint32_t bit = 1u << (c & 31);
        bad |= (atomicOr(&seen[c >> 5], bit) & bit) != 0u;
      }
    }
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

int32_t check_prefix_groups(const int32_t *lens, const int32_t *tables, const int32_t *groups,
                            int32_t num_groups, const int32_t *shared_lens, int32_t num_seqs,
                            int32_t max_blocks_per_seq, int32_t log2_block_size,
                            int32_t max_context_len, int32_t max_members, hipStream_t stream) {
  hipLaunchKernelGGL(check_prefix_kernel, dim3(1), dim3(kCheckThreads), 0, stream, lens, tables,
                     groups, num_groups, shared_lens, num_seqs, max_blocks_per_seq,
                     log2_block_size, max_context_len, max_members);
  return read_verdict(stream);
}

int32_t check_dispatch(const int32_t *dispatch, int32_t num_items, hipStream_t stream) {
  hipLaunchKernelGGL(check_dispatch_kernel, dim3(1), dim3(kCheckThreads), 0, stream, dispatch,
                     num_items);
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
