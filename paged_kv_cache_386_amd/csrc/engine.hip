// Continuously batched decode engine (declared in include/pagedattn_engine.h):
// a first-come-first-served scheduler over the block manager, turning each
// step into one host-to-device copy of index arrays and the device calls of
// pagedattn.h on one stream.
//
// Follows [P1] "vLLM 深度拆解..." section 2.2 (the batch is re-formed every
// decode step; finished requests free their blocks at once) and the
// devpress.csdn.net/amd walkthrough, "关键设计三：Continuous Batching" (admit
// while blocks can be allocated, one token per running request per step,
// free the finished) and "关键设计二：Copy-on-Write" (parallel samples fork).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <chrono>
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "internal.h"
#include "pagedattn.h"
#include "pagedattn_blocks.h"
#include "pagedattn_engine.h"

namespace {

constexpr int32_t kMaxSamples = 256;
constexpr int32_t kSampleBits = 8;
constexpr int64_t kMaxRequestId = int64_t(1) << 54;

// A unit of admission: a fresh request (all its samples) or one preempted
// sample waiting to be recomputed.
struct Waiting {
  int64_t request;
  int32_t rows;        // tokens to write at admission (prompt, or all held)
  int32_t remaining;   // decode steps left
  int32_t samples;     // sequences admitted together
  int32_t first;       // sample index of the first sequence
};

struct Running {
  int64_t seq;
  int64_t request;
  int64_t group;       // admission counter: preemption takes the newest group
  int32_t remaining;
  int32_t sample;
};

int64_t seq_id_of(int64_t request, int32_t sample) {
  return (request << kSampleBits) | sample;
}

int32_t cdiv(int64_t a, int64_t b) { return (int32_t)((a + b - 1) / b); }

}  // namespace

struct pa_engine {
  pa_engine_config cfg{};
  pa_block_manager *bm = nullptr;
  void *k_cache = nullptr, *v_cache = nullptr;
  int32_t max_blocks = 0;     // block-table row length
  int32_t watermark = 0;      // blocks admission leaves free
  std::deque<Waiting> waiting;
  std::vector<Running> running;
  std::unordered_map<int64_t, int32_t> live_requests;  // request -> samples not finished
  int64_t next_group = 0;

  // index arrays, int32: [slots maxb][lens maxb][pairs 2 maxb][groups 2 maxb]
  // [shared lengths maxb][dispatch list cap][prompt slots R][tables maxb*MB]
  size_t off_lens = 0, off_pairs = 0, off_groups = 0, off_shared = 0, off_dispatch = 0;
  size_t off_prompt = 0, off_tables = 0, words = 0;
  int32_t dispatch_cap = 0;
  bool q8 = false;  // an 8-bit pool (FP8 E4M3 or INT8)
  int32_t *staging[2] = {nullptr, nullptr};  // pinned host (device mode) or heap
  // double buffering: step t uses staging[t % 2] and dev_index[t % 2]; the
  // index copy runs on the engine's own copy stream, so that it overlaps the
  // previous step's kernels, and the caller's stream waits for it
  hipEvent_t copied[2] = {nullptr, nullptr};    // copy stream: staging -> device done
  hipEvent_t consumed[2] = {nullptr, nullptr};  // caller's stream: the step's kernels done
  bool pending[2] = {false, false};
  bool used[2] = {false, false};
  int32_t *dev_index[2] = {nullptr, nullptr};
  hipStream_t copy_stream = nullptr;
  void *workspace = nullptr;
  size_t workspace_bytes = 0;
  int parity = 0;

  // host reports of the last step
  std::vector<int64_t> batch_ids, admitted_ids, preempted_ids, finished_ids;
  std::vector<int32_t> admitted_rows;
};

namespace {

void release(pa_engine *e) {
  if (!e) return;
  // device work of earlier steps may still read the index buffers
  if (e->cfg.device) (void)hipDeviceSynchronize();
  for (int b = 0; b < 2; ++b) {
    if (e->copied[b]) (void)hipEventDestroy(e->copied[b]);
    if (e->consumed[b]) (void)hipEventDestroy(e->consumed[b]);
    if (e->dev_index[b]) (void)hipFree(e->dev_index[b]);
    if (e->staging[b]) {
      if (e->cfg.device)
        (void)hipHostFree(e->staging[b]);
      else
        delete[] e->staging[b];
    }
  }
  if (e->copy_stream) (void)hipStreamDestroy(e->copy_stream);
  if (e->workspace) (void)hipFree(e->workspace);
  if (e->bm) pa_bm_destroy(e->bm);
  delete e;
}

// Blocks a request of `rows` tokens and `samples` samples takes at admission
// plus its first step: the prompt's blocks, then per sample either a new
// block (the prompt ends on a block boundary) or, for all but one sample, a
// copy of the shared partly filled last block.
int64_t admission_cost(int32_t rows, int32_t samples, int32_t B) {
  return cdiv(rows, B) + (rows % B == 0 ? samples : samples - 1);
}

// Blocks a request needs over its whole life if it ran alone.
int64_t lifetime_cost(int32_t rows, int32_t new_tokens, int32_t samples, int32_t B) {
  const int64_t shared = rows / B;
  return shared + (int64_t)samples * (cdiv((int64_t)rows + new_tokens, B) - shared);
}

// Frees every running sequence of the newest admission group and queues each
// as a one-sample request at the front of the waiting queue (in sample order).
void preempt_newest(pa_engine *e) {
  const int64_t g = e->running.back().group;
  std::vector<Running> taken;
  while (!e->running.empty() && e->running.back().group == g) {
    taken.push_back(e->running.back());
    e->running.pop_back();
  }
  // taken is newest-last reversed: push to the front so that the first
  // sample ends up first
  for (const Running &r : taken) {
    const int32_t held = pa_bm_context_len(e->bm, r.seq);
    pa_bm_free_sequence(e->bm, r.seq);
    e->waiting.push_front(Waiting{r.request, held, r.remaining, 1, r.sample});
    e->preempted_ids.push_back(r.seq);
  }
}

}  // namespace

extern "C" {

int32_t pa_engine_create(const pa_engine_config *cfg, void *k_cache, void *v_cache,
                         pa_engine **out) {
  if (!cfg || !out) return PA_ERR_NULL;
  *out = nullptr;
  const pa_engine_config c = *cfg;
  const bool q8 = c.dtype == PA_FP8_E4M3 || c.dtype == PA_INT8;
  if (c.dtype != PA_F32 && c.dtype != PA_BF16 && !q8) return PA_ERR_DTYPE;
  if (c.num_blocks <= 0 || c.block_size <= 0 || c.block_size > 1024 ||
      (c.block_size & (c.block_size - 1)) || c.num_q_heads <= 0 || c.num_kv_heads <= 0 ||
      c.num_q_heads % c.num_kv_heads || c.max_batch <= 0 || c.max_batch > 65536 ||
      c.max_context_len <= 0 || c.max_prompt_rows < c.max_context_len ||
      (int64_t)c.num_blocks * c.block_size >= (int64_t(1) << 31) ||
      (c.device != 0 && c.device != 1) || (c.host_plan != 0 && c.host_plan != 1))
    return PA_ERR_SHAPE;
  if (q8) {
    if (!pa::decode_q8_supported(c.head_dim, c.num_q_heads / c.num_kv_heads))
      return PA_ERR_UNSUPPORTED;
    if (!(c.k_scale > 0.f && c.k_scale < __builtin_huge_valf()) ||
        !(c.v_scale > 0.f && c.v_scale < __builtin_huge_valf()))
      return PA_ERR_SHAPE;
  } else if (!pa::decode_supported(c.dtype, c.head_dim, c.num_q_heads / c.num_kv_heads)) {
    return PA_ERR_UNSUPPORTED;
  }
  if (paged_attention_num_partitions(1, c.num_kv_heads, c.max_context_len, c.partition_size) < 0)
    return PA_ERR_SHAPE;
  if (c.device && (!k_cache || !v_cache)) return PA_ERR_NULL;

  pa_engine *e = new (std::nothrow) pa_engine();
  if (!e) return PA_ERR_OOM;
  e->cfg = c;
  e->q8 = q8;
  e->k_cache = k_cache;
  e->v_cache = v_cache;
  e->max_blocks = cdiv(c.max_context_len, c.block_size);
  e->watermark = c.num_blocks / 100;
  e->bm = pa_bm_create(c.num_blocks, c.block_size);
  if (!e->bm) {
    release(e);
    return PA_ERR_OOM;
  }
  const size_t mb = (size_t)c.max_batch;
  // the longest dispatch list of any step: batch * partitions (largest for
  // the longest context) plus four entries per prefix group
  int64_t cap = 0;
  if (c.host_plan)
    for (int32_t n = 1; n <= c.max_batch; ++n)
      cap = std::max<int64_t>(
          cap, (int64_t)n * paged_attention_num_partitions(n, c.num_kv_heads, c.max_context_len,
                                                           c.partition_size) +
                   4 * (int64_t)n);
  if (cap >= (int64_t(1) << 31)) {
    release(e);
    return PA_ERR_SHAPE;
  }
  e->dispatch_cap = (int32_t)cap;
  e->off_lens = mb;
  e->off_pairs = 2 * mb;
  e->off_groups = 4 * mb;
  e->off_shared = 6 * mb;
  e->off_dispatch = 7 * mb;
  e->off_prompt = e->off_dispatch + (size_t)cap;
  e->off_tables = e->off_prompt + (size_t)c.max_prompt_rows;
  e->words = e->off_tables + mb * (size_t)e->max_blocks;
  const size_t bytes = e->words * sizeof(int32_t);
  try {
    e->batch_ids.reserve(mb);
    e->finished_ids.reserve(mb);
    e->preempted_ids.reserve(mb);
    e->admitted_ids.reserve(mb);
    e->admitted_rows.reserve(mb);
  } catch (...) {
    release(e);
    return PA_ERR_OOM;
  }
  for (int b = 0; b < 2; ++b) {
    if (c.device) {
      if (hipHostMalloc((void **)&e->staging[b], bytes, hipHostMallocDefault) != hipSuccess) {
        e->staging[b] = nullptr;
        release(e);
        return PA_ERR_OOM;
      }
      if (hipEventCreateWithFlags(&e->copied[b], hipEventDisableTiming) != hipSuccess) {
        e->copied[b] = nullptr;
        release(e);
        return PA_ERR_LAUNCH;
      }
      if (hipEventCreateWithFlags(&e->consumed[b], hipEventDisableTiming) != hipSuccess) {
        e->consumed[b] = nullptr;
        release(e);
        return PA_ERR_LAUNCH;
      }
      if (hipMalloc((void **)&e->dev_index[b], bytes) != hipSuccess) {
        e->dev_index[b] = nullptr;
        release(e);
        return PA_ERR_OOM;
      }
    } else {
      e->staging[b] = new (std::nothrow) int32_t[e->words];
      if (!e->staging[b]) {
        release(e);
        return PA_ERR_OOM;
      }
    }
  }
  if (c.device) {
    // default priority; non-blocking so that it never waits on the legacy
    // default stream implicitly (every dependency is an explicit event)
    if (hipStreamCreateWithFlags(&e->copy_stream, hipStreamNonBlocking) != hipSuccess) {
      e->copy_stream = nullptr;
      release(e);
      return PA_ERR_LAUNCH;
    }
    // the split-K workspace of the largest step: for a fixed batch the
    // partition count grows with the longest context, so the longest one
    // allowed bounds every step
    size_t ws = 0;
    for (int32_t s = 1; s <= c.max_batch; ++s)
      ws = std::max(ws, c.host_plan ? paged_attention_prefix_workspace_size(
                                          s, c.num_q_heads, c.num_kv_heads, c.head_dim,
                                          c.max_context_len, c.partition_size, s, c.dtype)
                                    : paged_attention_workspace_size(
                                          s, c.num_q_heads, c.num_kv_heads, c.head_dim,
                                          c.max_context_len, c.partition_size));
    if (ws) {
      if (hipMalloc(&e->workspace, ws) != hipSuccess) {
        e->workspace = nullptr;
        release(e);
        return PA_ERR_OOM;
      }
      e->workspace_bytes = ws;
    }
  }
  *out = e;
  return PA_OK;
}

void pa_engine_destroy(pa_engine *e) { release(e); }

int32_t pa_engine_submit(pa_engine *e, int64_t request_id, int32_t prompt_len,
                         int32_t max_new_tokens, int32_t num_samples) {
  if (!e) return PA_ERR_NULL;
  const pa_engine_config &c = e->cfg;
  if (request_id < 0 || request_id >= kMaxRequestId) return PA_ERR_SEQ_EXISTS;
  if (prompt_len < 1 || prompt_len > c.max_prompt_rows || max_new_tokens < 1 ||
      (int64_t)prompt_len + max_new_tokens > c.max_context_len || num_samples < 1 ||
      num_samples > std::min(c.max_batch, kMaxSamples))
    return PA_ERR_SHAPE;
  // a request must be able to run alone, or the queue could stall behind it
  // (its lifetime need also bounds its admission cost)
  if (lifetime_cost(prompt_len, max_new_tokens, num_samples, c.block_size) >
      c.num_blocks - e->watermark)
    return PA_ERR_SHAPE;
  if (e->live_requests.count(request_id)) return PA_ERR_SEQ_EXISTS;
  try {
    e->live_requests.emplace(request_id, num_samples);
    e->waiting.push_back(Waiting{request_id, prompt_len, max_new_tokens, num_samples, 0});
  } catch (...) {
    e->live_requests.erase(request_id);
    return PA_ERR_OOM;
  }
  return PA_OK;
}

int32_t pa_engine_num_waiting(const pa_engine *e) {
  return e ? (int32_t)e->waiting.size() : PA_ERR_NULL;
}

int32_t pa_engine_num_running(const pa_engine *e) {
  return e ? (int32_t)e->running.size() : PA_ERR_NULL;
}

const pa_block_manager *pa_engine_blocks(const pa_engine *e) { return e ? e->bm : nullptr; }

int32_t pa_engine_step(pa_engine *e, const void *q, const void *k_new, const void *v_new,
                       const void *prompt_k, const void *prompt_v, float scale, float *out,
                       void *stream, pa_step_info *info) {
  if (!e || !info) return PA_ERR_NULL;
  using clock = std::chrono::steady_clock;
  const auto t_start = clock::now();
  const pa_engine_config &c = e->cfg;
  if (c.device && (!q || !k_new || !v_new || !prompt_k || !prompt_v || !out)) return PA_ERR_NULL;
  hipStream_t st = (hipStream_t)stream;
  const int32_t B = c.block_size, MB = e->max_blocks;

  // the staging buffer of this step was last copied from two steps ago
  const int buf = e->parity;
  double wait_us = 0.0;
  if (e->pending[buf]) {
    const auto t0 = clock::now();
    if (hipEventSynchronize(e->copied[buf]) != hipSuccess) return PA_ERR_LAUNCH;
    wait_us = std::chrono::duration<double, std::micro>(clock::now() - t0).count();
    e->pending[buf] = false;
  }
  int32_t *hs = e->staging[buf];
  int32_t *slots = hs, *lens = hs + e->off_lens, *pairs = hs + e->off_pairs;
  int32_t *prompt_slots = hs + e->off_prompt, *tables = hs + e->off_tables;
  int32_t *groups = hs + e->off_groups, *shared = hs + e->off_shared;
  int32_t *dispatch = hs + e->off_dispatch;

  e->batch_ids.clear();
  e->admitted_ids.clear();
  e->admitted_rows.clear();
  e->preempted_ids.clear();
  e->finished_ids.clear();

  try {
    // 1. one new slot for every running sequence, preempting the newest
    //    admission group while the pool cannot cover the step
    int32_t nr = 0, np = 0;
    std::vector<int64_t> ids;
    for (;;) {
      ids.clear();
      for (const Running &r : e->running) ids.push_back(r.seq);
      nr = (int32_t)ids.size();
      if (nr == 0) break;
      const int32_t rc = pa_bm_prepare_decode(e->bm, ids.data(), nr, MB, 0, slots, pairs, &np,
                                              tables, lens);
      if (rc == PA_OK) break;
      if (rc != PA_ERR_OOM) return rc;
      preempt_newest(e);
    }
    e->batch_ids.assign(ids.begin(), ids.end());

    // 2. admission, oldest first, unless this step had to preempt
    int32_t rows_used = 0;
    std::vector<int64_t> new_ids;
    if (e->preempted_ids.empty()) {
      int64_t free_blocks = pa_bm_num_free_blocks(e->bm);
      while (!e->waiting.empty()) {
        const Waiting w = e->waiting.front();
        const int64_t cost = admission_cost(w.rows, w.samples, B);
        if (nr + (int32_t)new_ids.size() + w.samples > c.max_batch) break;
        if (rows_used + w.rows > c.max_prompt_rows) break;
        if (cost > free_blocks - e->watermark) break;
        const int64_t s0 = seq_id_of(w.request, w.first);
        int32_t rc = pa_bm_add_sequence(e->bm, s0, w.rows, prompt_slots + rows_used);
        if (rc != PA_OK) return rc;
        for (int32_t s = 1; s < w.samples; ++s) {
          rc = pa_bm_fork(e->bm, s0, seq_id_of(w.request, w.first + s));
          if (rc != PA_OK) return rc;
        }
        const int64_t group = e->next_group++;
        for (int32_t s = 0; s < w.samples; ++s) {
          const int64_t sid = seq_id_of(w.request, w.first + s);
          new_ids.push_back(sid);
          e->running.push_back(Running{sid, w.request, group, w.remaining, w.first + s});
        }
        e->admitted_ids.push_back(s0);
        e->admitted_rows.push_back(w.rows);
        rows_used += w.rows;
        free_blocks -= cost;
        e->waiting.pop_front();
      }
    }
    // admitted_ids lists the sequences whose prompt rows were written; their
    // forks appear only in batch_ids

    // 3. the new sequences' first slots (covered by the admission cost)
    const int32_t na = (int32_t)new_ids.size();
    if (na) {
      int32_t np2 = 0;
      const int32_t rc = pa_bm_prepare_decode(e->bm, new_ids.data(), na, MB, 0, slots + nr,
                                              pairs + 2 * np, &np2, tables + (size_t)nr * MB,
                                              lens + nr);
      if (rc != PA_OK) return rc;
      np += np2;
      e->batch_ids.insert(e->batch_ids.end(), new_ids.begin(), new_ids.end());
    }
    const int32_t n = nr + na;

    int32_t max_ctx = 0;
    int64_t ctx_tokens = 0;
    for (int32_t i = 0; i < n; ++i) {
      max_ctx = std::max(max_ctx, lens[i]);
      ctx_tokens += lens[i];
    }

    // 3. the decode call planned on the host: shared-prefix groups (forked
    //    samples hold their prompt's blocks) and the longest-first list
    int32_t ng = 0, nd = 0;
    int64_t unique_tokens = ctx_tokens;
    if (n > 0) {
      ng = pa_prefix_groups(tables, lens, n, MB, B, 64 / (c.num_q_heads / c.num_kv_heads), 16,
                            groups, shared);
      if (ng < 0) return ng;
      // a group's members read the shared slots [0, longest shared length) once
      for (int32_t g = 0; g < ng; ++g) {
        int64_t sum = 0, longest = 0;
        for (int32_t m = groups[2 * g]; m < groups[2 * g] + groups[2 * g + 1]; ++m) {
          sum += shared[m];
          longest = std::max<int64_t>(longest, shared[m]);
        }
        unique_tokens -= sum - longest;
      }
      if (!c.host_plan) ng = 0;  // counted only
    }
    if (c.host_plan && n > 0) {
      nd = paged_attention_decode_plan(lens, groups, ng, shared, n, c.num_q_heads,
                                       c.num_kv_heads, c.head_dim, B, MB, max_ctx, c.dtype,
                                       c.partition_size, dispatch, e->dispatch_cap);
      if (nd < 0) return nd;
    }

    // 4. the device work: one copy of the index arrays, then prompt writes,
    //    copy-on-write copies, new-token writes and decode, in stream order
    //    (an 8-bit pool: quantising writes of bfloat16 rows, 8-bit decode)
    if (c.device && n > 0) {
      const size_t words = e->off_tables + (size_t)n * MB;
      int32_t *dix = e->dev_index[buf];
      // the copy may overwrite dix only once the kernels of two steps ago,
      // which read it, are done
      if ((e->used[buf] && hipStreamWaitEvent(e->copy_stream, e->consumed[buf], 0) != hipSuccess) ||
          hipMemcpyAsync(dix, hs, words * sizeof(int32_t), hipMemcpyHostToDevice,
                         e->copy_stream) != hipSuccess ||
          hipEventRecord(e->copied[buf], e->copy_stream) != hipSuccess ||
          hipStreamWaitEvent(st, e->copied[buf], 0) != hipSuccess)
        return PA_ERR_LAUNCH;
      e->pending[buf] = true;
      const int32_t *d_slots = dix, *d_lens = dix + e->off_lens;
      const int32_t *d_pairs = dix + e->off_pairs;
      const int32_t *d_prompt = dix + e->off_prompt;
      const int32_t *d_tables = dix + e->off_tables;
      const int32_t *d_groups = dix + e->off_groups, *d_shared = dix + e->off_shared;
      const int32_t *d_dispatch = dix + e->off_dispatch;
      auto write = [&](const void *k, const void *v, const int32_t *sl, int32_t rows) {
        if (c.dtype == PA_FP8_E4M3)
          return kv_cache_write_fp8(k, v, sl, rows, e->k_cache, e->v_cache, c.num_blocks, B,
                                    c.num_kv_heads, c.head_dim, PA_BF16, c.k_scale, c.v_scale,
                                    stream);
        if (c.dtype == PA_INT8)
          return kv_cache_write_int8(k, v, sl, rows, e->k_cache, e->v_cache, c.num_blocks, B,
                                     c.num_kv_heads, c.head_dim, PA_BF16, c.k_scale, c.v_scale,
                                     stream);
        return kv_cache_write(k, v, sl, rows, e->k_cache, e->v_cache, c.num_blocks, B,
                              c.num_kv_heads, c.head_dim, c.dtype, stream);
      };
      int32_t rc;
      if (rows_used) {
        rc = write(prompt_k, prompt_v, d_prompt, rows_used);
        if (rc != PA_OK) return rc;
      }
      // the step's copies and its new tokens in one launch (after the prompt
      // rows, which a copy may read)
      rc = kv_cache_append(np ? d_pairs : nullptr, np, k_new, v_new, d_slots, n, e->k_cache,
                           e->v_cache, c.num_blocks, B, c.num_kv_heads, c.head_dim,
                           e->q8 ? PA_BF16 : c.dtype, c.dtype, c.k_scale, c.v_scale,
                           np ? pairs : nullptr, stream);
      if (rc != PA_OK) return rc;
      if (c.host_plan) {
        rc = paged_attention_decode_prefix(
            q, e->k_cache, e->v_cache, d_tables, d_lens, ng ? d_groups : nullptr, ng,
            ng ? d_shared : nullptr, d_dispatch, scale, c.k_scale, c.v_scale, out, n,
            c.num_q_heads, c.num_kv_heads, c.head_dim, B, c.num_blocks, MB, max_ctx, c.dtype,
            c.partition_size, e->workspace, e->workspace_bytes, stream);
      } else if (e->q8) {
        auto dec = c.dtype == PA_FP8_E4M3 ? paged_attention_decode_fp8
                                          : paged_attention_decode_int8;
        rc = dec(q, e->k_cache, e->v_cache, d_tables, d_lens, scale, c.k_scale, c.v_scale, out,
                 n, c.num_q_heads, c.num_kv_heads, c.head_dim, B, c.num_blocks, MB, max_ctx,
                 c.partition_size, e->workspace, e->workspace_bytes, stream);
      } else {
        rc = paged_attention_decode(q, e->k_cache, e->v_cache, d_tables, d_lens, scale, out, n,
                                    c.num_q_heads, c.num_kv_heads, c.head_dim, B, c.num_blocks,
                                    MB, max_ctx, c.dtype, c.partition_size, e->workspace,
                                    e->workspace_bytes, stream);
      }
      if (rc != PA_OK) return rc;
      if (hipEventRecord(e->consumed[buf], st) != hipSuccess) return PA_ERR_LAUNCH;
      e->used[buf] = true;
      e->parity ^= 1;
    }

    // 5. one token done for every sequence; free the finished
    size_t keep = 0;
    for (size_t i = 0; i < e->running.size(); ++i) {
      Running r = e->running[i];
      if (--r.remaining == 0) {
        pa_bm_free_sequence(e->bm, r.seq);
        e->finished_ids.push_back(r.seq);
        // a request leaves once all its samples have finished
        auto it = e->live_requests.find(r.request);
        if (it != e->live_requests.end() && --it->second == 0) e->live_requests.erase(it);
      } else {
        e->running[keep++] = r;
      }
    }
    e->running.resize(keep);

    info->batch = n;
    info->admitted = (int32_t)e->admitted_ids.size();
    info->prompt_rows = rows_used;
    info->preempted = (int32_t)e->preempted_ids.size();
    info->finished = (int32_t)e->finished_ids.size();
    info->num_copies = np;
    info->max_context_len = max_ctx;
    info->free_blocks = pa_bm_num_free_blocks(e->bm);
    info->context_tokens = ctx_tokens;
    info->batch_seq_ids = e->batch_ids.data();
    info->context_lens = lens;
    info->slot_mapping = slots;
    info->block_tables = tables;
    info->copy_pairs = pairs;
    info->admitted_seq_ids = e->admitted_ids.data();
    info->admitted_rows = e->admitted_rows.data();
    info->prompt_slots = prompt_slots;
    info->preempted_seq_ids = e->preempted_ids.data();
    info->finished_seq_ids = e->finished_ids.data();
    info->max_blocks_per_seq = MB;
    info->num_groups = ng;
    info->unique_tokens = unique_tokens;
    info->prefix_groups = groups;
    info->shared_lens = shared;
    info->dispatch_len = nd;
    info->dispatch = dispatch;
    info->wait_us = (float)wait_us;
    info->host_us =
        (float)std::chrono::duration<double, std::micro>(clock::now() - t_start).count();
  } catch (...) {
    return PA_ERR_OOM;
  }
  return PA_OK;
}

}  // extern "C"
