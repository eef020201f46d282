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
// P - 1 - c / num_seqs -- the fixed order's numbering; an item past its
// sequence's last partition (or, with shared prefixes, wholly inside its
// shared length) is listed as ~c, so that its workgroups exit without
// reading the context length.  With shared prefixes, items num_seqs * P +
// ipg i + c are item c of prefix group i: in decode (ipg = 4) column set c,
// sized by the longest shared length among the members with columns in that
// set (empty when there are none); in a multi-query call, sized by the
// longest shared length of the group.  Items are bucketed by
// token count (512 size classes of 2^shift tokens, longest class first; an
// item past the sequence's last partition, which does no work, sorts last)
// with a counting sort in LDS that keeps, within a class, the fixed order
// between waves and rounds (and within a round, the order in which the LDS
// serves one atomic's lanes): sequences that share prefix blocks and have
// equal sizes then still run side by side and share those blocks' reads in
// L2 (measured: a fully stable order made the GQA prefix batch's decode kernel
// 3 us faster than one whose ties were in arbitrary order).  The order
// changes timing only: every item computes the same result wherever it runs.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace pa {
namespace {

constexpr int kSchedWaves = 16;
constexpr int kSchedThreads = 64 * kSchedWaves;
constexpr int kSizeClasses = 512;     // + 1 for the empty items
constexpr int kKeptClasses = 8192;    // item classes kept in LDS between passes

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Counting sort in three passes over the items, with wave w owning the
// contiguous range [w * chunk, (w + 1) * chunk), 64 items a round:
//  1. each wave counts its items per class (LDS atomics);
//  2. start[k][w] = items of classes before k (all waves) + items of class k
//     in waves before w;
//  3. each wave places its items round by round through its own starts, so
//     a class's items keep the order of the waves, and of the rounds within
//     a wave.
__global__ __launch_bounds__(kSchedThreads) void decode_schedule_kernel(
    const int32_t *__restrict__ context_lens, int32_t *__restrict__ order, int num_seqs, int P,
    int ps, int cap, int shift, const int32_t *__restrict__ groups,
    const int32_t *__restrict__ shared_lens, int num_groups, int G, int short_rule, int ipg) {
  // class-major, so one thread reads a class's 16 wave counts as 4 vectors
  __shared__ __attribute__((aligned(16))) int start[kSizeClasses + 1][kSchedWaves];
  __shared__ int wave_total[kSchedWaves];
  __shared__ uint16_t kept[kKeptClasses];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nseq_items = num_seqs * P;
  const int n = nseq_items + ipg * num_groups;
  const int chunk = ((n + kSchedWaves - 1) / kSchedWaves + 63) / 64 * 64;
  const int begin = min(n, wave * chunk), end = min(n, begin + chunk);

  // a sequence's shared length as the decode kernel takes it
  auto shared = [&](int s, int L) {
    return shared_lens ? min(max(shared_lens[s], 0), L) & ~15 : 0;
  };
  // the same clamps and partition bounds as the decode kernels
  auto size_class = [&](int c) -> int {
    int tokens;
    if (c >= nseq_items) {
      // a prefix item (group gi, column set cset): it walks the longest
      // shared length among the members with columns in its set (decode),
      // or among all the members (multi-query, G == 0)
      const int gi = (c - nseq_items) / ipg;
      const int cset = (c - nseq_items) - gi * ipg;
      const int first = min(max(groups[2 * gi], 0), num_seqs - 1);
      const int count =
          min(max(groups[2 * gi + 1], 0), min(num_seqs - first, G ? 64 / G : kMqPrefixMembers));
      const int m0 = G ? 16 * cset / G : 0;
      const int m1 = G ? min(count, (16 * cset + 15) / G + 1) : count;
      int longest = 0;
      bool extra = false;  // a short member's private tile
      for (int m = m0; m < m1; ++m) {
        const int L = max(0, min(context_lens[first + m], cap));
        const int sh = shared(first + m, L);
        longest = max(longest, sh);
        extra = extra || (short_rule && prefix_short(L, sh) && L > sh);
      }
      if (longest == 0) return kSizeClasses;
      tokens = longest + (extra ? 16 : 0);
    } else {
      const int s = c % num_seqs;
      const int p = (P - 1) - c / num_seqs;
      const int L = max(0, min(context_lens[s], cap));
      const int nparts = min((L + ps - 1) / ps, P);
      if (p >= max(nparts, 1)) return kSizeClasses;
      const int sh = shared(s, L);
      // a short member's prefix item reads its private tile too
      if (short_rule && prefix_short(L, sh)) return kSizeClasses;
      if (p < sh / ps) return kSizeClasses;  // wholly inside the shared prefix
      // (zero tokens still runs: it writes the empty partial the merge reads)
      tokens = max(0, min(L, p * ps + ps) - max(p * ps, sh));
    }
    return (kSizeClasses - 1) - min(tokens >> shift, kSizeClasses - 1);
  };

  for (int i = tid; i < (kSizeClasses + 1) * kSchedWaves / 4; i += kSchedThreads)
    reinterpret_cast<i32x4 *>(&start[0][0])[i] = i32x4{0, 0, 0, 0};
  __syncthreads();
  for (int c = begin + lane; c < end; c += 64) {
    const int k = size_class(c);
    if (c < kKeptClasses) kept[c] = (uint16_t)k;
    atomicAdd(&start[k][wave], 1);
  }
  __syncthreads();

  // thread k <= 512 owns class k: its total, an exclusive scan over the
  // classes (the empty class, thread 512, comes after every other), then the
  // per-wave starts
  i32x4 cnt[kSchedWaves / 4];
  int own = 0;
  if (tid <= kSizeClasses) {
    for (int v = 0; v < kSchedWaves / 4; ++v) {
      cnt[v] = reinterpret_cast<const i32x4 *>(&start[tid][0])[v];
      own += cnt[v][0] + cnt[v][1] + cnt[v][2] + cnt[v][3];
    }
    if (tid == kSizeClasses) own = 0;
  }
  int x = own;
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wave_total[wave] = x;
  __syncthreads();
  int run = x - own;
  for (int w = 0; w < wave; ++w) run += wave_total[w];
  if (tid <= kSizeClasses) {
    for (int v = 0; v < kSchedWaves / 4; ++v) {
      const i32x4 cv = cnt[v];
      const i32x4 st = {run, run + cv[0], run + cv[0] + cv[1], run + cv[0] + cv[1] + cv[2]};
      run += cv[0] + cv[1] + cv[2] + cv[3];
      reinterpret_cast<i32x4 *>(&start[tid][0])[v] = st;
    }
  }
  __syncthreads();

  // each wave places its items in order: its own start per class, so items
  // of one class keep the wave order; within a round, lanes that share a
  // class take their slots through one LDS atomic (lane order as the
  // hardware serves them)
  for (int c = begin + lane; c < end; c += 64) {
    const int k = c < kKeptClasses ? (int)kept[c] : size_class(c);
    // items with no tokens are listed as ~c (negative): their workgroups
    // exit on the list entry alone
    order[atomicAdd(&start[k][wave], 1)] = k == kSizeClasses ? ~c : c;
  }
}

}  // namespace

bool schedule_wanted(int64_t workgroups, int64_t num_seqs, int64_t P) {
  return workgroups > kScheduleMinWorkgroups && num_seqs * P < (int64_t(1) << 31);
}

hipError_t launch_schedule(const int32_t *context_lens, int32_t *order, int num_seqs, int P,
                           int ps, int cap, hipStream_t stream, const int32_t *groups,
                           const int32_t *shared_lens, int num_groups, int group,
                           bool short_rule, int ipg) {
  // one partition spans every clamped context: size the classes by the cap
  if (P <= 1) ps = cap;
  int shift = 0;
  while ((ps >> shift) >= kSizeClasses) ++shift;
  hipLaunchKernelGGL(decode_schedule_kernel, dim3(1), dim3(kSchedThreads), 0, stream,
                     context_lens, order, num_seqs, P, ps, cap, shift, groups, shared_lens,
                     num_groups, group, (int)short_rule, ipg);
  return hipGetLastError();
}

}  // namespace pa
