// Host block manager of a paged KV cache (declared in include/pagedattn_blocks.h).
//
// The pool, the per-sequence block tables and append_slot follow the
// "关键设计一：分页管理" and "关键设计二：Copy-on-Write" sections of the
// devpress.csdn.net/amd vLLM walkthrough and sections 2.1 and 3.3 of the
// chenxutan.com vLLM deep-dive: the free list starts as 0 .. N-1 and hands out
// its last entry; a sequence takes a block when its next position opens one;
// a forked child shares its parent's blocks; appending into a shared last
// block first copies it to a fresh block.  Blocks are reference counted and go
// back to the free list when no table holds them any more.
#include <stdint.h>

#include <algorithm>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pagedattn_blocks.h"

struct pa_block_manager {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> free_list;  // the last entry is handed out next
  std::vector<int32_t> refs;       // per physical block
  struct Seq {
    std::vector<int32_t> table;
    int32_t len = 0;
    uint64_t mark = 0;  // the last prepare_decode call that listed it
  };
  std::unordered_map<int64_t, Seq> seqs;
  // prepare_decode's scratch, kept across calls: a call counter that marks
  // the sequences and simulated reference counts it has seen (a block's
  // simulated count is valid while its stamp equals the counter)
  uint64_t calls = 0;
  std::vector<uint64_t> sim_stamp;
  std::vector<int32_t> sim_refs;

  int32_t take() {
    const int32_t b = free_list.back();
    free_list.pop_back();
    refs[b] = 1;
    return b;
  }
  void drop(int32_t b) {
    if (--refs[b] == 0) free_list.push_back(b);
  }
  int32_t blocks_for(int64_t tokens) const {
    return (int32_t)((tokens + block_size - 1) / block_size);
  }
  // Blocks the next append of s takes from the free list (0 or 1) given
  // reference counts `ref` (the live ones, or a scratch copy while planning).
  template <typename RefOf>
  int32_t append_cost(const Seq &s, RefOf ref) const {
    if (s.len % block_size == 0) return 1;
    return ref(s.table.back()) > 1 ? 1 : 0;
  }
  // Performs the append (a free block is known to be there when needed).
  void append(Seq &s, int32_t *slot, int32_t *src, int32_t *dst) {
    *src = -1;
    *dst = -1;
    const int32_t off = s.len % block_size;
    if (off == 0) {
      s.table.push_back(take());
    } else if (refs[s.table.back()] > 1) {
      const int32_t old = s.table.back();
      const int32_t fresh = take();
      --refs[old];  // still held by the other sharers
      s.table.back() = fresh;
      *src = old;
      *dst = fresh;
    }
    *slot = s.table.back() * block_size + off;
    ++s.len;
  }
};

namespace {

bool valid_block_size(int32_t b) { return b >= 1 && b <= 1024 && (b & (b - 1)) == 0; }

}  // namespace

extern "C" {

pa_block_manager *pa_bm_create(int32_t num_blocks, int32_t block_size) {
  if (num_blocks <= 0 || !valid_block_size(block_size)) return nullptr;
  if ((int64_t)num_blocks * block_size >= (int64_t(1) << 31)) return nullptr;
  pa_block_manager *bm = new (std::nothrow) pa_block_manager();
  if (!bm) return nullptr;
  try {
    bm->num_blocks = num_blocks;
    bm->block_size = block_size;
    bm->free_list.resize(num_blocks);
    for (int32_t i = 0; i < num_blocks; ++i) bm->free_list[i] = i;
    bm->refs.assign(num_blocks, 0);
    bm->sim_stamp.assign(num_blocks, 0);
    bm->sim_refs.assign(num_blocks, 0);
  } catch (...) {
    delete bm;
    return nullptr;
  }
  return bm;
}

void pa_bm_destroy(pa_block_manager *bm) { delete bm; }

int32_t pa_bm_num_free_blocks(const pa_block_manager *bm) {
  if (!bm) return PA_ERR_NULL;
  return (int32_t)bm->free_list.size();
}

int32_t pa_bm_can_allocate(const pa_block_manager *bm, int32_t num_tokens) {
  if (!bm || num_tokens < 0) return 0;
  return bm->blocks_for(num_tokens) <= (int32_t)bm->free_list.size() ? 1 : 0;
}

int32_t pa_bm_add_sequence(pa_block_manager *bm, int64_t seq_id, int32_t num_tokens,
                           int32_t *slots) {
  if (!bm) return PA_ERR_NULL;
  if (num_tokens < 0) return PA_ERR_SHAPE;
  if (bm->seqs.count(seq_id)) return PA_ERR_SEQ_EXISTS;
  const int32_t need = bm->blocks_for(num_tokens);
  if (need > (int32_t)bm->free_list.size()) return PA_ERR_OOM;
  try {
    pa_block_manager::Seq s;
    s.table.reserve(need);
    for (int32_t j = 0; j < need; ++j) s.table.push_back(bm->take());
    s.len = num_tokens;
    if (slots)
      for (int32_t t = 0; t < num_tokens; ++t)
        slots[t] = s.table[t / bm->block_size] * bm->block_size + t % bm->block_size;
    bm->seqs.emplace(seq_id, std::move(s));
  } catch (...) {
    return PA_ERR_SHAPE;
  }
  return PA_OK;
}

int32_t pa_bm_fork(pa_block_manager *bm, int64_t parent, int64_t child) {
  if (!bm) return PA_ERR_NULL;
  auto it = bm->seqs.find(parent);
  if (it == bm->seqs.end()) return PA_ERR_NO_SEQ;
  if (bm->seqs.count(child)) return PA_ERR_SEQ_EXISTS;
  try {
    pa_block_manager::Seq c = it->second;
    for (int32_t b : c.table) ++bm->refs[b];
    bm->seqs.emplace(child, std::move(c));
  } catch (...) {
    return PA_ERR_SHAPE;
  }
  return PA_OK;
}

int32_t pa_bm_append_slot(pa_block_manager *bm, int64_t seq_id, int32_t *slot,
                          int32_t *copy_src, int32_t *copy_dst) {
  if (!bm || !slot || !copy_src || !copy_dst) return PA_ERR_NULL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_NO_SEQ;
  const int32_t cost = bm->append_cost(it->second, [&](int32_t b) { return bm->refs[b]; });
  if (cost > (int32_t)bm->free_list.size()) return PA_ERR_OOM;
  if ((int64_t)it->second.len + 1 > ((int64_t)1 << 30)) return PA_ERR_SHAPE;
  try {
    bm->append(it->second, slot, copy_src, copy_dst);
  } catch (...) {
    return PA_ERR_SHAPE;
  }
  return PA_OK;
}

int32_t pa_bm_free_sequence(pa_block_manager *bm, int64_t seq_id) {
  if (!bm) return PA_ERR_NULL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_NO_SEQ;
  for (int32_t b : it->second.table) bm->drop(b);
  bm->seqs.erase(it);
  return PA_OK;
}

int32_t pa_bm_context_len(const pa_block_manager *bm, int64_t seq_id) {
  if (!bm) return PA_ERR_NULL;
  auto it = bm->seqs.find(seq_id);
  return it == bm->seqs.end() ? PA_ERR_NO_SEQ : it->second.len;
}

int32_t pa_bm_block_table(const pa_block_manager *bm, int64_t seq_id, int32_t *table,
                          int32_t capacity) {
  if (!bm) return PA_ERR_NULL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_NO_SEQ;
  const std::vector<int32_t> &t = it->second.table;
  if (table)
    for (int32_t j = 0; j < capacity && j < (int32_t)t.size(); ++j) table[j] = t[j];
  return (int32_t)t.size();
}

int32_t pa_bm_prepare_decode(pa_block_manager *bm, const int64_t *seq_ids, int32_t n,
                             int32_t max_blocks, int32_t pad_block, int32_t *slot_mapping,
                             int32_t *copy_pairs, int32_t *num_pairs, int32_t *block_tables,
                             int32_t *context_lens) {
  if (!bm) return PA_ERR_NULL;
  if (n < 0 || max_blocks < 0) return PA_ERR_SHAPE;
  if (n == 0) {
    if (num_pairs) *num_pairs = 0;
    return PA_OK;
  }
  if (!seq_ids || !slot_mapping || !copy_pairs || !num_pairs || !block_tables || !context_lens)
    return PA_ERR_NULL;
  try {
    // plan: look every id up once, refuse repeats (marked by this call's
    // number), and count the blocks the appends take in this order, with
    // reference counts simulated on stamped scratch
    std::vector<pa_block_manager::Seq *> seqs(n);
    const uint64_t call = ++bm->calls;
    int64_t need = 0;
    auto ref = [&](int32_t b) {
      return bm->sim_stamp[b] == call ? bm->sim_refs[b] : bm->refs[b];
    };
    for (int32_t i = 0; i < n; ++i) {
      auto it = bm->seqs.find(seq_ids[i]);
      if (it == bm->seqs.end()) return PA_ERR_NO_SEQ;
      pa_block_manager::Seq &s = it->second;
      if (s.mark == call) return PA_ERR_SEQ_EXISTS;
      s.mark = call;
      seqs[i] = &s;
      if (bm->blocks_for((int64_t)s.len + 1) > max_blocks) return PA_ERR_SHAPE;
      const int32_t c = bm->append_cost(s, ref);
      if (c && s.len % bm->block_size != 0) {
        const int32_t b = s.table.back();
        bm->sim_refs[b] = ref(b) - 1;
        bm->sim_stamp[b] = call;
      }
      need += c;
    }
    if (need > (int64_t)bm->free_list.size()) return PA_ERR_OOM;
    int32_t pairs = 0;
    for (int32_t i = 0; i < n; ++i) {
      int32_t src, dst;
      bm->append(*seqs[i], &slot_mapping[i], &src, &dst);
      if (src >= 0) {
        copy_pairs[2 * pairs] = src;
        copy_pairs[2 * pairs + 1] = dst;
        ++pairs;
      }
    }
    *num_pairs = pairs;
    for (int32_t i = 0; i < n; ++i) {
      const pa_block_manager::Seq &s = *seqs[i];
      int32_t *row = block_tables + (int64_t)i * max_blocks;
      const int32_t nb = (int32_t)s.table.size();
      std::copy(s.table.begin(), s.table.end(), row);
      std::fill(row + nb, row + max_blocks, pad_block);
      context_lens[i] = s.len;
    }
  } catch (...) {
    return PA_ERR_SHAPE;
  }
  return PA_OK;
}

int32_t pa_bm_stats(const pa_block_manager *bm, pa_block_stats *out) {
  if (!bm || !out) return PA_ERR_NULL;
  try {
    // a slot is stored once however many tables hold its block: per block,
    // the fullest use any sequence makes of it
    std::vector<int32_t> fill(bm->num_blocks, 0);
    int64_t logical = 0;
    for (const auto &kv : bm->seqs) {
      const pa_block_manager::Seq &s = kv.second;
      logical += s.len;
      for (size_t j = 0; j < s.table.size(); ++j) {
        const int64_t used = std::min<int64_t>(bm->block_size, s.len - (int64_t)j * bm->block_size);
        fill[s.table[j]] = std::max<int32_t>(fill[s.table[j]], (int32_t)std::max<int64_t>(used, 0));
      }
    }
    int64_t stored = 0;
    int32_t used_blocks = 0, shared = 0;
    for (int32_t b = 0; b < bm->num_blocks; ++b) {
      if (bm->refs[b] > 0) {
        ++used_blocks;
        stored += fill[b];
      }
      if (bm->refs[b] > 1) ++shared;
    }
    out->num_blocks = bm->num_blocks;
    out->free_blocks = (int32_t)bm->free_list.size();
    out->shared_blocks = shared;
    out->num_sequences = (int32_t)bm->seqs.size();
    out->tokens_logical = logical;
    out->tokens_stored = stored;
    out->slots_allocated = (int64_t)used_blocks * bm->block_size;
    out->utilisation =
        out->slots_allocated > 0 ? (double)stored / (double)out->slots_allocated : 1.0;
  } catch (...) {
    return PA_ERR_SHAPE;
  }
  return PA_OK;
}

}  // extern "C"
