/*
 * libpagedattn engine -- a continuously batched decode loop on one GPU: a
 * first-come-first-served scheduler over submitted requests, the block
 * manager of pagedattn_blocks.h, and the device calls of pagedattn.h, driven
 * one step at a time.
 *
 * Sources (web pages, cited by title and section):
 *  [P1] "vLLM 深度拆解：当大模型推理学会「分页注意力」..." (chenxutan.com/d/4834.html),
 *       section 2.2 (continuous batching: the batch is re-formed at every
 *       decode step; a request that finishes frees its blocks at once and a
 *       waiting one takes its place) and section 3.3 (BlockSpaceManager:
 *       append_slot per new token, free when a request ends).
 *  [P2] "vLLM为何成为大模型推理的事实标准？技术拆解来了", section
 *       "连续批处理：让 GPU 几乎 never idle" (requests join and leave the
 *       running batch per step).
 *  [P3] the vLLM PagedAttention walkthrough at
 *       devpress.csdn.net/amd/6a31086710ee7a33f27dd05a.html, section
 *       "关键设计三：Continuous Batching" (admit waiting requests in order while
 *       the block manager can allocate, generate one token for every running
 *       request, free the finished; the schedule also reports preempted
 *       requests) and "关键设计二：Copy-on-Write" (parallel samples of one
 *       request fork its sequence and share its blocks).
 *
 * Readings where the pages are loose: admission is first come first served
 * and stops at the first request that does not fit; "can allocate" counts
 * the request's first step and keeps a watermark free; preemption (the pages
 * name it, without a policy) takes the newest admission group and recomputes
 * it later.
 *
 * What a step does (pa_engine_step), in order:
 *  1. planning: every running sequence gets the slot of one new token
 *     (pa_bm_prepare_decode).  If the pool cannot cover the step, the newest
 *     admission group is preempted -- its sequences are freed and each goes
 *     back to the front of the waiting queue as a request of one sample whose
 *     prompt is everything it held (to be recomputed) -- and planning is
 *     retried;
 *  2. admission (only when step 1 preempted nothing): waiting requests,
 *     oldest first, join while the batch has room for all their samples, the
 *     step's prompt-row budget holds their prompts, and the free blocks, less
 *     a watermark of num_blocks / 100, cover their prompts and their first
 *     appends; admission stops at the first request that does not fit.  An
 *     admitted request's first sample is a new sequence holding its prompt,
 *     the others are forks of it; they get their first slots after the
 *     running sequences (batch rows nr .. n-1);
 *  3. with host_plan (pa_engine_config), the decode call is planned on the
 *     host from the step's tables and lengths: the shared-prefix groups
 *     (pa_prefix_groups: forked samples share their prompt's blocks) and the
 *     longest-first dispatch list (paged_attention_decode_plan);
 *  4. one host-to-device copy of the step's index arrays, then on `stream`:
 *     kv_cache_write of the admitted prompts, one kv_cache_append of the
 *     copy-on-write pairs and the new tokens (the quantising writes for an
 *     8-bit pool) and decode over the whole batch
 *     (paged_attention_decode_prefix with the step's groups and list when
 *     host_plan is set, else paged_attention_decode; the FP8 / INT8 forms
 *     for an 8-bit pool);
 *  5. every sequence that has now produced its max_new_tokens tokens is freed.
 *
 * The token data are the caller's: a step reads the prompt rows of the
 * admitted sequences from prompt_k/prompt_v (packed in admission order), and
 * row i of q, k_new and v_new for batch row i; decode writes out row i.  The
 * step's info (below) says which sequence each row belongs to.  Token rows
 * and q are in the pool's dtype, or bfloat16 for an 8-bit pool (FP8 E4M3 or
 * INT8, one scale per cache: [P3] architecture figure, FP8/INT8 in the
 * kernel layer), whose writes quantise them.
 *
 * Sequence ids: sample s of request r is (r << 8) | s.  A preempted sample
 * keeps its id when it is re-admitted.
 *
 * Unlike the calls of pagedattn.h, an engine owns memory and a stream: two
 * pinned host staging buffers and two device index buffers (steps alternate
 * between them), a split-K workspace, and a copy stream (default priority)
 * on which a step's index copy runs while the previous step's kernels still
 * run on the caller's stream, which then waits for it through an event.
 * Everything is allocated once by pa_engine_create; nothing per step.  The pool
 * (k_cache, v_cache) stays the caller's.  Calls on one engine must not
 * overlap, and every step of an engine must use the same stream (or streams
 * the caller orders): a step's device work reads index buffers the next step
 * overwrites.
 *
 * With device == 0 (pa_engine_config), the engine only plans: nothing is
 * allocated on or copied to the GPU and no kernel is launched; the step's
 * index arrays are still produced in host memory (for tests and dry runs).
 */
#ifndef PAGEDATTN_ENGINE_H
#define PAGEDATTN_ENGINE_H

#include <stdint.h>

#include "pagedattn.h"
#include "pagedattn_blocks.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_engine pa_engine;

typedef struct pa_engine_config {
  int32_t num_blocks;         /* pool size in blocks */
  int32_t block_size;         /* tokens per block (power of two, <= 1024) */
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;           /* 64 or 128 */
  int32_t dtype;              /* pa_dtype of the pool and of every token row */
  int32_t max_batch;          /* most sequences in one step (<= 65536) */
  int32_t max_context_len;    /* longest sequence, prompt plus generated */
  int32_t max_prompt_rows;    /* prompt rows one step may write (>= max_context_len:
                                 a preempted sequence is re-admitted whole) */
  int32_t partition_size;     /* decode partition policy, as in pagedattn.h */
  int32_t device;             /* 1 = run on the current HIP device, 0 = plan only */
  float k_scale, v_scale;     /* 8-bit pools (dtype PA_FP8_E4M3 or PA_INT8): a stored
                                 code c means value(c) * scale; finite and > 0 */
  int32_t host_plan;          /* 1 = find shared prefixes and plan the dispatch list on
                                 the host every step (step 3); 0 = plain decode */
} pa_engine_config;

/* Per-step report.  The arrays are the engine's host memory, valid until the
 * next pa_engine_step on the same engine. */
typedef struct pa_step_info {
  int32_t batch;               /* sequences decoded: rows 0 .. batch-1 */
  int32_t admitted;            /* sequences admitted (prompts written) */
  int32_t prompt_rows;         /* rows of prompt_k / prompt_v consumed */
  int32_t preempted;           /* sequences preempted back to the queue */
  int32_t finished;            /* sequences finished and freed after the step */
  int32_t num_copies;          /* copy-on-write pairs */
  int32_t max_context_len;     /* longest context attended */
  int32_t free_blocks;         /* after the step's frees */
  int64_t context_tokens;      /* attended tokens, summed over the batch */
  const int64_t *batch_seq_ids;     /* [batch] sequence of each row */
  const int32_t *context_lens;      /* [batch] lengths attended */
  const int32_t *slot_mapping;      /* [batch] slot of each new token */
  const int32_t *block_tables;      /* [batch][max_blocks_per_seq] */
  const int32_t *copy_pairs;        /* [num_copies][2] */
  const int64_t *admitted_seq_ids;  /* [admitted], in prompt-row order */
  const int32_t *admitted_rows;     /* [admitted] prompt rows of each */
  const int32_t *prompt_slots;      /* [prompt_rows] slot of each prompt row */
  const int64_t *preempted_seq_ids; /* [preempted] */
  const int64_t *finished_seq_ids;  /* [finished] */
  int32_t max_blocks_per_seq;       /* row length of block_tables */
  int32_t num_groups;               /* shared-prefix groups of the step (host_plan) */
  const int32_t *prefix_groups;     /* [num_groups][2] (first batch row, members) */
  const int32_t *shared_lens;       /* [batch] positions read through the group */
  int32_t dispatch_len;             /* entries of the dispatch list (host_plan) */
  const int32_t *dispatch;          /* [dispatch_len] */
  int64_t unique_tokens;            /* attended tokens with each shared prefix slot once
                                       (context_tokens less, per group, the members' shared
                                       lengths beyond the longest; the groups are found
                                       even without host_plan) */
  float host_us;                    /* host time of the call, microseconds */
  float wait_us;                    /* of it, waiting for a staging buffer to free up
                                       (the device still reading it two steps back) */
} pa_step_info;

/* Creates an engine over the caller's pool (device pointers laid out as in
 * pagedattn.h; ignored when cfg->device is 0).  *out receives the engine.
 * dtype PA_FP8_E4M3 or PA_INT8 needs head_dim 64 or 128 (the 8-bit decode)
 * and valid scales; other dtypes ignore the scales.
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_DTYPE, PA_ERR_UNSUPPORTED, PA_ERR_OOM
 * (host or device allocation failed), PA_ERR_LAUNCH. */
int32_t pa_engine_create(const pa_engine_config *cfg, void *k_cache, void *v_cache,
                         pa_engine **out);

/* Waits for the device to finish the engine's work, then frees what the
 * engine owns. */
void pa_engine_destroy(pa_engine *e);

/* Queues a request: a prompt of prompt_len tokens (1 .. max_prompt_rows),
 * max_new_tokens >= 1 steps of decode, num_samples parallel samples
 * (1 .. min(max_batch, 256)).  prompt_len + max_new_tokens must not exceed
 * max_context_len, and the request must fit the pool alone for its whole
 * life (its prompt's full blocks shared, every sample's other blocks its own)
 * with the admission watermark (num_blocks / 100 blocks) kept free, so that
 * the oldest request can always run.  Errors: PA_ERR_NULL, PA_ERR_SHAPE,
 * PA_ERR_SEQ_EXISTS (request_id in use, or outside [0, 2^54)). */
int32_t pa_engine_submit(pa_engine *e, int64_t request_id, int32_t prompt_len,
                         int32_t max_new_tokens, int32_t num_samples);

/* One step (see above).  Device pointers (ignored when planning only):
 *   q          [max_batch][num_q_heads][head_dim], dtype (bfloat16 for an 8-bit pool)
 *   k_new,
 *   v_new      [max_batch][num_kv_heads][head_dim], the same
 *   prompt_k,
 *   prompt_v   [max_prompt_rows][num_kv_heads][head_dim], the same
 *   out        float32 [max_batch][num_q_heads][head_dim]
 * An empty step (nothing running or admitted) enqueues nothing.  A step
 * that preempts admits nothing.
 * Errors: PA_ERR_NULL, PA_ERR_OOM (host allocation failed), PA_ERR_LAUNCH
 * and the errors of the device calls; after an error the engine's state is
 * unspecified and it should be destroyed. */
int32_t pa_engine_step(pa_engine *e, const void *q, const void *k_new, const void *v_new,
                       const void *prompt_k, const void *prompt_v, float scale, float *out,
                       void *stream, pa_step_info *info);

/* Requests waiting (including preempted samples) and sequences running. */
int32_t pa_engine_num_waiting(const pa_engine *e);
int32_t pa_engine_num_running(const pa_engine *e);

/* The engine's block manager (owned by the engine), for stats, lengths and
 * tables.  Changing it from outside voids the engine's bookkeeping. */
const pa_block_manager *pa_engine_blocks(const pa_engine *e);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_ENGINE_H */
