// Shared-prefix groups of a decode batch from its host block tables
// (declared in include/pagedattn_blocks.h).  Sequences that share a prompt
// prefix, or were forked from one parent, hold the same physical blocks at
// the same logical positions (section 5.2 of the chenxutan.com vLLM
// deep-dive, prefix caching; "关键设计二：Copy-on-Write" of the
// devpress.csdn.net/amd vLLM walkthrough); paged_attention_decode_prefix
// reads such blocks once per group.
#include <stdint.h>

#include <algorithm>

#include "pagedattn_blocks.h"

namespace {

// Leading block ids of row a equal to row b, among the first `limit`.
int32_t common_blocks(const int32_t *a, const int32_t *b, int32_t limit) {
  int32_t k = 0;
  while (k < limit && a[k] == b[k]) ++k;
  return k;
}

}  // namespace

extern "C" int32_t pa_prefix_groups(const int32_t *block_tables, const int32_t *context_lens,
                                    int32_t num_seqs, int32_t max_blocks_per_seq,
                                    int32_t block_size, int32_t max_members,
                                    int32_t min_shared_tokens, int32_t *groups,
                                    int32_t *shared_lens) {
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || block_size <= 0 || max_members < 1)
    return PA_ERR_SHAPE;
  if (num_seqs == 0) return 0;
  if (!block_tables || !context_lens || !groups || !shared_lens) return PA_ERR_NULL;
  const int64_t mb = max_blocks_per_seq;
  auto len = [&](int32_t s) {
    return std::min<int64_t>(std::max(context_lens[s], 0), mb * block_size);
  };
  auto blocks = [&](int32_t s) { return (int32_t)((len(s) + block_size - 1) / block_size); };
  auto row = [&](int32_t s) { return block_tables + s * mb; };
  int32_t ng = 0;
  int32_t i = 0;
  while (i < num_seqs) {
    const int32_t first = i;
    shared_lens[first] = 0;
    // the run: consecutive sequences whose first block is the first's
    int32_t count = 1;
    if (blocks(first) > 0)
      while (first + count < num_seqs && count < max_members && blocks(first + count) > 0 &&
             row(first + count)[0] == row(first)[0])
        ++count;
    if (count < 2) {
      ++i;
      continue;
    }
    // the reference row: the member with the most blocks (the earliest of
    // equals); every member's shared length is its agreement with that row
    int32_t ref = first;
    for (int32_t m = first + 1; m < first + count; ++m)
      if (blocks(m) > blocks(ref)) ref = m;
    int64_t longest = 0;  // longest shared length of a member other than ref
    for (int32_t m = first; m < first + count; ++m) {
      if (m == ref) continue;
      const int32_t k = common_blocks(row(m), row(ref), std::min(blocks(m), blocks(ref)));
      int64_t sh = std::min<int64_t>(len(m), (int64_t)k * block_size);
      if (sh < min_shared_tokens) sh = 0;
      shared_lens[m] = (int32_t)sh;
      longest = std::max(longest, sh);
    }
    shared_lens[ref] = (int32_t)std::min<int64_t>(len(ref), longest);
    if (longest > 0) {
      groups[2 * ng] = first;
      groups[2 * ng + 1] = count;
      ++ng;
    } else {
      for (int32_t m = first; m < first + count; ++m) shared_lens[m] = 0;
    }
    i += count;
  }
  return ng;
}
