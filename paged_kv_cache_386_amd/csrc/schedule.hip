// Longest-first dispatch order for the decode (and multi-query) work items.
//
// A decode launch has one workgroup per (sequence, KV head, partition), and
// the hardware starts workgroups in launch order.  With mixed context lengths
// (a lognormal batch, a continuous-batching step) the fixed order can leave a
// few long items running alone at the end while the rest of the chip idles.
// This kernel sorts the (sequence, partition) items by their token count,
// longest first, so that the last workgroups to start are the shortest ones
// (the classic longest-processing-time rule for list scheduling).  The decode
// kernels then read their item from the list; the KV heads of one item stay
// consecutive workgroups, as in the fixed order.
//
// Item c (c < num_seqs * P) is sequence c % num_seqs and partition
// P - 1 - c / num_seqs -- the fixed order's numbering.  Items are bucketed by
// token count (1024 size classes of 2^shift tokens, longest class first; an
// item past the sequence's last partition, which does no work, sorts last)
// with a counting sort in LDS.  Within a class the order is whatever the LDS
// atomics give: every item computes the same result wherever it runs, so the
// order changes timing only.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace pa {
namespace {

constexpr int kSchedThreads = 1024;
constexpr int kSizeClasses = 1024;  // + 1 for the empty items
static_assert(kSchedThreads == kSizeClasses, "the scan gives each thread one size class");

__global__ __launch_bounds__(kSchedThreads) void decode_schedule_kernel(
    const int32_t *__restrict__ context_lens, int32_t *__restrict__ order, int num_seqs, int P,
    int ps, int cap, int shift) {
  __shared__ int count[kSizeClasses + 1];
  __shared__ int wave_total[kSchedThreads / 64];
  const int tid = threadIdx.x;
  const int n = num_seqs * P;

  // the same clamps and partition bounds as the decode kernels
  auto size_class = [&](int c) -> int {
    const int s = c % num_seqs;
    const int p = (P - 1) - c / num_seqs;
    const int L = max(0, min(context_lens[s], cap));
    const int nparts = min((L + ps - 1) / ps, P);
    if (p >= max(nparts, 1)) return kSizeClasses;
    const int tokens = min(L, p * ps + ps) - p * ps;
    return (kSizeClasses - 1) - min(tokens >> shift, kSizeClasses - 1);
  };

  for (int i = tid; i <= kSizeClasses; i += kSchedThreads) count[i] = 0;
  __syncthreads();
  for (int c = tid; c < n; c += kSchedThreads) atomicAdd(&count[size_class(c)], 1);
  __syncthreads();

  // exclusive prefix sum over the size classes: within each wave by lane
  // shifts, then across the waves
  const int v = count[tid];
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if ((tid & 63) >= off) x += y;
  }
  if ((tid & 63) == 63) wave_total[tid >> 6] = x;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < (tid >> 6); ++w) base += wave_total[w];
  count[tid] = base + x - v;
  if (tid == kSizeClasses - 1) count[kSizeClasses] = base + x;
  __syncthreads();

  for (int c = tid; c < n; c += kSchedThreads) order[atomicAdd(&count[size_class(c)], 1)] = c;
}

}  // namespace

bool schedule_wanted(int64_t workgroups, int64_t num_seqs, int64_t P) {
  return workgroups > kScheduleMinWorkgroups && num_seqs * P < (int64_t(1) << 31);
}

hipError_t launch_schedule(const int32_t *context_lens, int32_t *order, int num_seqs, int P,
                           int ps, int cap, hipStream_t stream) {
  // one partition spans every clamped context: size the classes by the cap
  if (P <= 1) ps = cap;
  int shift = 0;
  while ((ps >> shift) >= kSizeClasses) ++shift;
  hipLaunchKernelGGL(decode_schedule_kernel, dim3(1), dim3(kSchedThreads), 0, stream,
                     context_lens, order, num_seqs, P, ps, cap, shift);
  return hipGetLastError();
}

}  // namespace pa
