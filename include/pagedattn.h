/*
 * libpagedattn -- PagedAttention decode and its KV-cache edits for AMD Instinct
 * MI355X (gfx950), behind a plain C ABI.
 *
 * Sources (web pages, cited by title and section):
 *  [P1] "vLLM 深度拆解：当大模型推理学会「分页注意力」——PagedAttention、连续批处理与
 *       V1 引擎如何重写 GPU 推理服务的心智模型" (chenxutan.com/d/4834.html)
 *  [P2] "vLLM为何成为大模型推理的事实标准？技术拆解来了"
 *       (devpress.csdn.net/awstech/6a9264832b83d06f0ec8e065.html)
 *  [P3] the vLLM PagedAttention walkthrough at
 *       devpress.csdn.net/amd/6a31086710ee7a33f27dd05a.html
 *
 * Conventions for every entry point:
 *  - Pointers marked "device" point to GPU memory on the current HIP device;
 *    the caller owns every buffer.  The library never allocates, frees or keeps
 *    a pointer after the call returns.  Its only mutable global state is the
 *    index-check mode (a process-wide flag) and, per device, the one word the
 *    index check writes its verdict into (see "Index checking" below: calls
 *    that overlap on one device with checking on race on that word), and the
 *    static scratch array of paged_attention_decode_noalloc (calls of that
 *    entry point that overlap on one device race on it); otherwise calls
 *    share nothing and may run concurrently on any streams.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *    asynchronously on it; nothing is synchronised.
 *  - Arguments are validated on the host before anything is enqueued.  A
 *    negative pa_status is returned on bad arguments (nothing is enqueued) or
 *    when the launch itself fails.  Nothing aborts, prints or throws.
 *  - Index contents on the device (block ids, slots, context lengths) are not
 *    validated on the host.  The kernels clamp or skip out-of-range values so
 *    that they never read or write outside the buffers described by the sizes
 *    passed in; the numbers produced for such inputs are unspecified.
 *
 * KV pool layout (one layer): k_cache and v_cache are each
 *   [num_blocks][num_kv_heads][block_size][head_dim], head_dim contiguous
 * (the order of the cache in [P3] section "核心代码拆解"): one token's row for
 * one KV head is head_dim contiguous elements, and a KV head's rows of one
 * block are block_size*head_dim contiguous elements.  The slot of logical
 * position t of a sequence whose block table row is `tbl` is
 * tbl[t / block_size] * block_size + t % block_size ([P1] section 2.1 block
 * table; [P1] section 3.3 append into the current block until it is full);
 * its row for KV head h is at element
 * ((slot / block_size * num_kv_heads + h) * block_size + slot % block_size)
 * * head_dim.
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL = -1,        /* a required pointer is NULL */
  PA_ERR_SHAPE = -2,       /* inconsistent or out-of-range sizes */
  PA_ERR_DTYPE = -3,       /* unknown dtype code */
  PA_ERR_UNSUPPORTED = -4, /* valid but not compiled in (head_dim, group size) */
  PA_ERR_WORKSPACE = -5,   /* split-K workspace missing or too small */
  PA_ERR_ALIAS = -6,       /* copy pairs overlap (checked only when requested) */
  PA_ERR_LAUNCH = -7,      /* the HIP runtime refused the launch */
  PA_ERR_OOM = -8,         /* block manager: no free block left */
  PA_ERR_NO_SEQ = -9,      /* block manager: unknown sequence id */
  PA_ERR_SEQ_EXISTS = -10, /* block manager: sequence id already in use */
  PA_ERR_INDEX = -11,      /* a device index is out of range (only with index checking on) */
  PA_ERR_SCRATCH = -12     /* the call needs more than the library's static scratch holds */
} pa_status;

typedef enum pa_dtype {
  PA_F32 = 0,      /* IEEE binary32 */
  PA_BF16 = 1,     /* bfloat16 (the high half of a binary32), stored as 16-bit words */
  PA_FP8_E4M3 = 2, /* pools only: OCP 8-bit float E4M3 (bias 7, no infinities, max 448),
                      one code per byte, meaning code value * the cache's scale */
  PA_INT8 = 3      /* pools only: signed byte codes in [-127, 127], meaning code * the
                      cache's scale */
} pa_dtype;

/*
 * paged_attention_decode -- one decode step of attention over a paged KV pool.
 *
 * For every sequence s and query head h, with G = num_q_heads / num_kv_heads,
 * g = h / G and L = context_lens[s]:
 *   K_t, V_t = rows of KV head g at the slots of positions t = 0 .. L-1
 *   x_t      = scale * dot(q[s][h], K_t)
 *   out[s][h] = sum_t exp(x_t - max x) V_t / sum_t exp(x_t - max x)
 * ([P3] section "核心代码拆解": translate each logical block through the block
 * table, read K, take the scaled dot with q, then softmax and the weighted sum
 * of V; [P1] section 2.1 block table; [P1] section 2.3 decode reads the whole
 * KV cache per generated token).  L = 0 gives zeros.  Arithmetic is fp32 with
 * an online (running-maximum) softmax; bf16 inputs are read exactly.  Where
 * the products run on the matrix cores (bf16 with G = 4 or 8), q.K is exact
 * products with fp32 accumulation, and the probabilities enter p.V as a pair
 * of bfloat16 values hi + lo (about 16 significant bits) with fp32
 * accumulation; the vector-ALU path (fp32, and bf16 with G = 1 or 2) keeps
 * every step in fp32.
 *
 *   q              device, [num_seqs][num_q_heads][head_dim], dtype
 *   k_cache,
 *   v_cache        device, the pool described above, dtype
 *   block_tables   device int32 [num_seqs][max_blocks_per_seq]; entries past
 *                  ceil(L/block_size) never address the pool and may hold any
 *                  value.  As a cache hint, the kernels also read the entries of
 *                  the neighbouring rows s-1 and s+1 at the block indices row s
 *                  uses (a block a neighbour holds at the same logical position
 *                  is read with ordinary, cached loads, every other block with
 *                  streaming ones); those reads stay inside the
 *                  [num_seqs][max_blocks_per_seq] array, and their values only
 *                  steer caching
 *   context_lens   device int32 [num_seqs]; must not exceed max_context_len
 *   scale          softmax scale applied to the dot product (e.g. 1/sqrt(d))
 *   out            device float32 [num_seqs][num_q_heads][head_dim]; written
 *                  for every (s, h); must not alias an input
 *   max_context_len host upper bound of context_lens (sizes the launch);
 *                  must be <= max_blocks_per_seq * block_size
 *   dtype          element type of q, k_cache and v_cache
 *   partition_size split-K partition in tokens: 0 = automatic (4096-token
 *                  partitions for contexts above 4096 when there are at least
 *                  256 (sequence, KV head) pairs; with fewer, floor(512 /
 *                  pairs) equal partitions per context, at least 512
 *                  tokens), negative = never split, positive = that many
 *                  tokens (a multiple of 16).  With
 *                  more than one partition, the sequences whose context
 *                  spans several partitions leave per-partition (max, sum,
 *                  output) partials in the workspace and a second kernel
 *                  merges them in ascending partition order; the others are
 *                  written directly.
 *   workspace      device scratch of workspace_bytes bytes, at least
 *                  paged_attention_workspace_size(...) for the same arguments;
 *                  may be NULL when that size is 0.  Its contents on entry do
 *                  not matter; it must not be used by other work in flight.
 *                  It holds the split partials, then (for launches of more
 *                  than 1024 workgroups, one per sequence, KV head and
 *                  partition) a dispatch list: a first small kernel sorts
 *                  the work longest first, so that short items, not long
 *                  ones, finish the launch.  A workspace too small for the
 *                  list but large enough for the partials still gives the
 *                  same results, in a fixed order (slower on mixed lengths).
 *
 * Supported: head_dim 64 or 128; G in {1, 2, 4, 8}; block_size a power of two
 * in [1, 1024]; num_blocks * block_size < 2^31.
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_DTYPE, PA_ERR_UNSUPPORTED,
 * PA_ERR_WORKSPACE, PA_ERR_LAUNCH; PA_ERR_INDEX with index checking on.
 */
int32_t paged_attention_decode(const void *q, const void *k_cache, const void *v_cache,
                               const int32_t *block_tables, const int32_t *context_lens,
                               float scale, float *out,
                               int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size, int32_t num_blocks,
                               int32_t max_blocks_per_seq, int32_t max_context_len,
                               int32_t dtype, int32_t partition_size,
                               void *workspace, size_t workspace_bytes, void *stream);

/*
 * paged_attention_decode_prefix -- paged_attention_decode for a batch whose
 * sequences share prefixes, reading each shared block once per group instead
 * of once per sequence ([P1] section 5.2 prefix caching: requests with a
 * common prompt prefix keep its blocks once and reuse them; [P3]
 * "关键设计二：Copy-on-Write": forked sequences share their parent's
 * blocks).  The result is that of paged_attention_decode (or of its FP8 /
 * INT8 forms) on the same tables: the groups only change which reads are
 * shared.
 *
 *   prefix_groups  device int32 [num_groups][2]: (first sequence, members)
 *                  of each group, a run of consecutive sequences; groups in
 *                  ascending order and disjoint; members in [1, 64 / G]
 *   num_groups     host, 0 .. num_seqs (0: plain decode)
 *   shared_lens    device int32 [num_seqs]: sequence s reads positions
 *                  [0, shared_lens[s]) through its group (in [0, L]; 0 for a
 *                  sequence in no group).  The rows of two members of one
 *                  group must name the same blocks below the shorter of
 *                  their two shared lengths.  Lengths are used rounded down
 *                  to whole 16-token tiles.
 *   dispatch       device int32 list of the launch's work items in the order
 *                  to run them, as paged_attention_decode_plan writes it for
 *                  the same arguments (planned on the host, where the lengths
 *                  are known, instead of sorted on the device), or NULL to
 *                  sort on the device as paged_attention_decode does.  The
 *                  order changes timing only; the list must hold every item
 *                  of the launch exactly once (entries that are not an item
 *                  of it are skipped and their outputs go unwritten)
 *   kv_dtype       the pool's element type: PA_F32 or PA_BF16 (q the same),
 *                  PA_FP8_E4M3 or PA_INT8 (q bfloat16; k_scale and v_scale as
 *                  in paged_attention_decode_fp8; ignored otherwise)
 *   workspace      at least paged_attention_prefix_workspace_size(...) bytes
 * Every other argument is paged_attention_decode's.  With groups, the work
 * items of each (group, KV head) attend the group's shared positions for
 * all of its (member, query head) pairs, 16 pairs per item, on the matrix
 * cores, and each sequence's own items attend only the rest of its context;
 * a merge kernel then combines every member's prefix and private partials in
 * ascending position order.
 * Where this is not compiled (fp32 pools, head_dim 64) or num_groups is 0,
 * the call is plain decode and the groups are ignored.
 * Supported and errors: as paged_attention_decode (and its FP8 / INT8
 * forms); PA_ERR_SHAPE for num_groups outside [0, num_seqs], PA_ERR_NULL for
 * missing groups or shared lengths.  Groups and shared lengths that break the
 * rules above give unspecified numbers, every access staying in bounds; with
 * index checking on they give PA_ERR_INDEX.
 */
int32_t paged_attention_decode_prefix(const void *q, const void *k_cache, const void *v_cache,
                                      const int32_t *block_tables, const int32_t *context_lens,
                                      const int32_t *prefix_groups, int32_t num_groups,
                                      const int32_t *shared_lens, const int32_t *dispatch,
                                      float scale, float k_scale, float v_scale, float *out,
                                      int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                      int32_t max_blocks_per_seq, int32_t max_context_len,
                                      int32_t kv_dtype, int32_t partition_size, void *workspace,
                                      size_t workspace_bytes, void *stream);

/*
 * paged_attention_decode_plan -- the dispatch list of
 * paged_attention_decode_prefix for these arguments, computed on the host:
 * every work item of the launch (the (sequence, partition) items, then four
 * 16-column items per prefix group when the prefix path runs), longest first
 * by tokens to attend, equal sizes in item order, items with no work last.
 * A launch starts workgroups in list order, so the long items no longer
 * finish last (the longest-processing-time rule of list scheduling).
 *
 *   context_lens, prefix_groups, shared_lens   host copies of the device
 *                  arrays the call will get (groups and shared lengths may
 *                  be NULL when num_groups is 0)
 *   dispatch       host int32 out, capacity entries
 * Every other argument is paged_attention_decode_prefix's.  Returns the
 * number of entries written (num_seqs * P + 4 * groups on the prefix path),
 * or PA_ERR_NULL, PA_ERR_SHAPE (including capacity too small), PA_ERR_DTYPE.
 */
int32_t paged_attention_decode_plan(const int32_t *context_lens, const int32_t *prefix_groups,
                                    int32_t num_groups, const int32_t *shared_lens,
                                    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t block_size,
                                    int32_t max_blocks_per_seq, int32_t max_context_len,
                                    int32_t kv_dtype, int32_t partition_size, int32_t *dispatch,
                                    int32_t capacity);

/* Workspace bytes of paged_attention_decode_prefix: with the prefix path,
 * 4 * num_seqs * num_q_heads * (P + 1) * (head_dim + 2) for the partials plus
 * 4 * (num_seqs * P + 4 * num_groups) for the dispatch list when the launch
 * has more than 1024 workgroups; otherwise paged_attention_workspace_size's.
 * 0 for arguments the call rejects. */
size_t paged_attention_prefix_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                             int32_t num_kv_heads, int32_t head_dim,
                                             int32_t max_context_len, int32_t partition_size,
                                             int32_t num_groups, int32_t kv_dtype);

/*
 * paged_attention_decode_noalloc -- paged_attention_decode without a
 * workspace argument, for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  It allocates nothing and calls no allocating routine; the
 * split-K partials and the dispatch list go to a static device array of the
 * library, paged_attention_noalloc_scratch_bytes() bytes (32 MiB) on each GPU
 * it runs on, held from the library's load until the process ends.  Its
 * device address is looked up on the first call on each device, so that
 * call must find the device current.
 *
 * Arguments, results (bit for bit those of paged_attention_decode with a
 * workspace of paged_attention_workspace_size bytes), support and errors are
 * those of paged_attention_decode, plus PA_ERR_SCRATCH (nothing enqueued)
 * when paged_attention_workspace_size for these arguments exceeds the static
 * size.  Every call on one GPU uses that GPU's one array: calls that overlap
 * on one GPU (other streams, other threads) race on it and must be ordered
 * by the caller.  Nothing in it needs to start at zero: a call writes every
 * byte of it that it reads.
 */
int32_t paged_attention_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                       const int32_t *block_tables, const int32_t *context_lens,
                                       float scale, float *out, int32_t num_seqs,
                                       int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                       int32_t max_blocks_per_seq, int32_t max_context_len,
                                       int32_t dtype, int32_t partition_size, void *stream);

/* Bytes of the static scratch paged_attention_decode_noalloc uses per GPU. */
size_t paged_attention_noalloc_scratch_bytes(void);

/*
 * paged_attention_decode_fp8 -- paged_attention_decode over an FP8 (E4M3)
 * pool ([P3] architecture figure: FP8/INT8 quantisation in the kernel layer;
 * [P1] section 5.3: FP8 trades a little precision for memory and bandwidth).
 *
 * k_cache and v_cache hold one E4M3 code per element in the layout above; an
 * element's value is e4m3(code) * k_scale (K) or * v_scale (V), so the
 * result is that of paged_attention_decode on the dequantised pool.  q is
 * bfloat16.  K and V codes are widened exactly to bfloat16 (an E4M3 value
 * has at most 4 significant bits).  At head_dim 128 both products run on the
 * bfloat16 matrix cores with fp32 accumulation, and the probabilities enter
 * p.V as a pair of bfloat16 values hi + lo (about 16 significant bits); at
 * head_dim 64 the vector kernel forms q.k with paired bfloat16 dot products
 * and p.V with fp32 fused multiply-adds.  k_scale joins the softmax scale
 * and v_scale multiplies the output.  Every other argument, the workspace
 * (same size as paged_attention_decode's) and the partition policy are those
 * of paged_attention_decode.
 * Supported: head_dim 64 or 128, G in {1, 2, 4, 8}; k_scale and v_scale
 * finite and > 0.
 * Errors: as paged_attention_decode.
 */
int32_t paged_attention_decode_fp8(const void *q, const void *k_cache, const void *v_cache,
                                   const int32_t *block_tables, const int32_t *context_lens,
                                   float scale, float k_scale, float v_scale, float *out,
                                   int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                   int32_t max_blocks_per_seq, int32_t max_context_len,
                                   int32_t partition_size, void *workspace,
                                   size_t workspace_bytes, void *stream);

/*
 * paged_attention_decode_int8 -- paged_attention_decode_fp8 over an INT8
 * pool ([P3] architecture figure: FP8/INT8 quantisation): an element's value
 * is code * k_scale (K) or * v_scale (V), the code a signed byte.  Codes are
 * widened exactly to bfloat16 (at most 7 significant bits) for both products,
 * with the probabilities entering p.V as a bfloat16 pair at head_dim 128, as
 * for FP8.
 * Arguments, support and errors are those of paged_attention_decode_fp8.
 */
int32_t paged_attention_decode_int8(const void *q, const void *k_cache, const void *v_cache,
                                    const int32_t *block_tables, const int32_t *context_lens,
                                    float scale, float k_scale, float v_scale, float *out,
                                    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                    int32_t max_blocks_per_seq, int32_t max_context_len,
                                    int32_t partition_size, void *workspace,
                                    size_t workspace_bytes, void *stream);

/*
 * Bytes of workspace paged_attention_decode (and its FP8 / INT8 forms) needs
 * for these arguments: 4 * num_seqs * num_q_heads * P * (head_dim + 2) for
 * the partials when the call splits into P > 1 partitions, plus 4 * num_seqs
 * * P for the dispatch list when num_seqs * num_kv_heads * P > 1024; 0 when
 * neither applies.  Returns 0 for arguments decode would reject.
 */
size_t paged_attention_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim,
                                      int32_t max_context_len, int32_t partition_size);

/*
 * The number of split-K partitions decode will use for these arguments
 * (1 = no split), or a negative pa_status for a partition_size decode rejects.
 */
int32_t paged_attention_num_partitions(int32_t num_seqs, int32_t num_kv_heads,
                                       int32_t max_context_len, int32_t partition_size);

/*
 * The number of tokens per split-K partition decode will use for these
 * arguments: the partition length when it splits, else max_context_len; or a
 * negative pa_status for a partition_size decode rejects.
 */
int32_t paged_attention_partition_tokens(int32_t num_seqs, int32_t num_kv_heads,
                                         int32_t max_context_len, int32_t partition_size);

/*
 * paged_attention_multi_query -- causal attention of several query tokens per
 * sequence over the paged pool: a slice of a long prompt (chunked prefill) or
 * tokens to verify (speculative decoding) ([P1] sections 2.3, 4.3, 5.1, 5.4).
 *
 * Sequence s owns query rows query_start[s] .. query_start[s+1]-1; with n of
 * them and L = context_lens[s], they are the sequence's last n cached
 * positions (their K/V must already be in the pool, e.g. by kv_cache_write).
 * Row query_start[s] + i sits at position p = L - n + i, and for each query
 * head h (KV head g = h / G):
 *   out[row][h] = sum_{t <= p} exp(x_t - max) V_t / sum_{t <= p} exp(x_t - max),
 *   x_t = scale * dot(q[row][h], K_t)
 * with K_t, V_t read through block_tables[s] as in paged_attention_decode.
 *
 *   q              device, [num_tokens][num_q_heads][head_dim], dtype
 *   query_start    device int32 [num_seqs + 1], non-decreasing, starting at 0
 *   context_lens,
 *   block_tables   as in paged_attention_decode
 *   out            device float32 [num_tokens][num_q_heads][head_dim]; rows
 *                  that belong to no sequence are not written
 *   max_query_len  host: at least every sequence's n (rows past it are not
 *                  computed)
 *   max_context_len host: at least every context_lens[s]; sets the number of
 *                  partitions
 *   partition_size split-K partition in tokens: 0 = automatic (chunks of at
 *                  most 64 query rows per KV head are split like decode,
 *                  rounded up to whole 64-token tiles; longer chunks are not
 *                  split), negative = never, positive = that many tokens (a
 *                  multiple of 64).  With more than one partition, the
 *                  sequences whose context spans several partitions leave
 *                  partials in the workspace and a second kernel merges them
 *                  in ascending order; the others are written directly.
 *   workspace      device scratch of workspace_bytes bytes, at least
 *                  paged_attention_multi_query_workspace_size(...); may be
 *                  NULL when that is 0.  As for decode, it holds the partials
 *                  and then, for launches of more than 1024 workgroups, the
 *                  longest-first dispatch list; with room for the partials
 *                  only, the results are the same, in a fixed order.
 * Chunks longer than their context, or reaching past num_tokens, are cut to
 * fit; the numbers are then unspecified but every access stays in bounds.
 * The products run on bfloat16 matrix instructions with fp32 accumulation;
 * probabilities enter them as a pair of bfloat16 values (about 16
 * significant bits).
 * Supported: dtype PA_BF16; head_dim 64 or 128; any G; block_size a power of
 * two in [1, 1024].
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_DTYPE, PA_ERR_UNSUPPORTED,
 * PA_ERR_WORKSPACE, PA_ERR_LAUNCH; PA_ERR_INDEX with index checking on.
 */
int32_t paged_attention_multi_query(const void *q, const void *k_cache, const void *v_cache,
                                    const int32_t *block_tables, const int32_t *context_lens,
                                    const int32_t *query_start, float scale, float *out,
                                    int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                    int32_t num_blocks, int32_t max_blocks_per_seq,
                                    int32_t max_query_len, int32_t max_context_len,
                                    int32_t dtype, int32_t partition_size, void *workspace,
                                    size_t workspace_bytes, void *stream);

/* Partitions paged_attention_multi_query will use for these arguments (1 = no
 * split), or a negative pa_status for a partition_size it rejects. */
int32_t paged_attention_multi_query_partitions(int32_t num_seqs, int32_t num_q_heads,
                                               int32_t num_kv_heads, int32_t max_query_len,
                                               int32_t max_context_len, int32_t partition_size);

/* Workspace bytes paged_attention_multi_query needs: 4 * num_tokens *
 * num_q_heads * P * (head_dim + 2) for the partials when it splits into P > 1
 * partitions, plus 4 * num_seqs * P for the dispatch list when the launch has
 * more than 1024 workgroups; 0 when neither applies. */
size_t paged_attention_multi_query_workspace_size(int32_t num_seqs, int32_t num_tokens,
                                                  int32_t num_q_heads, int32_t num_kv_heads,
                                                  int32_t head_dim, int32_t max_query_len,
                                                  int32_t max_context_len,
                                                  int32_t partition_size);

/*
 * paged_attention_multi_query_fp8 -- paged_attention_multi_query over an FP8
 * (E4M3) pool, as paged_attention_decode_fp8 reads it: a stored code c means
 * e4m3(c) * k_scale (K) or * v_scale (V), widened exactly to bfloat16 for the
 * products ([P1] sections 5.3 and 5.4: FP8 KV cache, speculative decoding).
 * Arguments as in paged_attention_multi_query, with q in bfloat16 and
 * k_cache, v_cache one code per byte; k_scale, v_scale finite and > 0.
 * Chunks of at most 64 (token, head) rows per KV head at head_dim 128
 * (verification-sized) run on the decode kernel's walk; longer chunks
 * (chunked prefill) and head_dim 64 on the row-tile kernel, which loads the
 * codes and widens them exactly to bfloat16 as it stages each tile in LDS.
 * Supported: head_dim 64 or 128; any G; block_size a power of two in
 * [1, 1024].
 * Errors: as paged_attention_multi_query.
 */
int32_t paged_attention_multi_query_fp8(const void *q, const void *k_cache, const void *v_cache,
                                        const int32_t *block_tables, const int32_t *context_lens,
                                        const int32_t *query_start, float scale, float k_scale,
                                        float v_scale, float *out, int32_t num_seqs,
                                        int32_t num_tokens, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                        int32_t num_blocks, int32_t max_blocks_per_seq,
                                        int32_t max_query_len, int32_t max_context_len,
                                        int32_t partition_size, void *workspace,
                                        size_t workspace_bytes, void *stream);

/*
 * paged_attention_multi_query_int8 -- the same over an INT8 pool (a stored
 * signed code c means c * k_scale or c * v_scale, as in
 * paged_attention_decode_int8).  Supported and errors as
 * paged_attention_multi_query_fp8.
 */
int32_t paged_attention_multi_query_int8(const void *q, const void *k_cache, const void *v_cache,
                                         const int32_t *block_tables, const int32_t *context_lens,
                                         const int32_t *query_start, float scale, float k_scale,
                                         float v_scale, float *out, int32_t num_seqs,
                                         int32_t num_tokens, int32_t num_q_heads,
                                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                         int32_t num_blocks, int32_t max_blocks_per_seq,
                                         int32_t max_query_len, int32_t max_context_len,
                                         int32_t partition_size, void *workspace,
                                         size_t workspace_bytes, void *stream);

/*
 * paged_attention_multi_query_prefix -- paged_attention_multi_query (or its
 * FP8 / INT8 form, by kv_dtype) for a batch whose sequences share prefixes,
 * reading each shared block once per group instead of once per sequence
 * ([P1] section 5.2 prefix caching, section 5.4 speculative decoding: the
 * draft tokens of sequences that share a prompt are verified against the
 * same prefix blocks; [P3] "关键设计二：Copy-on-Write").  The result is that
 * of the plain call on the same tables: the groups only change which reads
 * are shared.
 *
 *   prefix_groups,
 *   num_groups,
 *   shared_lens    as in paged_attention_decode_prefix, with at most 16
 *                  members per group (pa_prefix_groups with max_members 16)
 *   dispatch       device int32 list of the launch's work items in the order
 *                  to run them, as paged_attention_multi_query_plan writes
 *                  it for the same arguments (planned on the host instead of
 *                  sorted on the device each call), or NULL to sort on the
 *                  device when the launch is large enough.  The order changes
 *                  timing only; the list must hold every item of the launch
 *                  exactly once (entries that are not an item of it are
 *                  skipped and their outputs go unwritten)
 *   kv_dtype       PA_BF16, PA_FP8_E4M3 or PA_INT8 (q bfloat16; k_scale and
 *                  v_scale as in paged_attention_multi_query_fp8, ignored for
 *                  PA_BF16); prefix items over bf16 pools only (over 8-bit
 *                  pools the shared walk measured slower: the call is the
 *                  plain FP8 / INT8 one)
 *   workspace      at least paged_attention_multi_query_prefix_workspace_size
 *                  (...) bytes
 * Every other argument is paged_attention_multi_query's.  The prefix path
 * serves bf16 pools with at most 8 (token, head) rows per sequence and KV
 * head (max_query_len * G <= 8) at head_dim 128: items per (group, KV head)
 * attend the group's shared positions for 16 of the members' (token, head)
 * rows each, every row up to its own position and below its member's shared
 * length, and each sequence's own items attend only the rest of its context;
 * the merge then combines every row's prefix and private partials in
 * ascending position order.  With more rows per member an item covers too
 * few members for the shared walk to pay (each item walks the whole prefix):
 * there, as with num_groups 0, the call is the plain one and the groups are
 * ignored (a dispatch list still applies).
 * Supported and errors: as paged_attention_multi_query (and its FP8 / INT8
 * forms); PA_ERR_SHAPE for num_groups outside [0, num_seqs], PA_ERR_NULL for
 * missing groups or shared lengths.  Groups and shared lengths that break the
 * rules give unspecified numbers, every access staying in bounds; with index
 * checking on they give PA_ERR_INDEX.
 */
int32_t paged_attention_multi_query_prefix(
    const void *q, const void *k_cache, const void *v_cache, const int32_t *block_tables,
    const int32_t *context_lens, const int32_t *query_start, const int32_t *prefix_groups,
    int32_t num_groups, const int32_t *shared_lens, const int32_t *dispatch, float scale,
    float k_scale, float v_scale, float *out, int32_t num_seqs, int32_t num_tokens,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_query_len,
    int32_t max_context_len, int32_t kv_dtype, int32_t partition_size, void *workspace,
    size_t workspace_bytes, void *stream);

/*
 * paged_attention_multi_query_plan -- the dispatch list of
 * paged_attention_multi_query_prefix for these arguments, computed on the
 * host: every work item of the launch (the (sequence, partition) items, then
 * the groups' prefix items when the prefix path runs), longest first by
 * tokens to attend (a sequence item its private positions in its partition,
 * a prefix item its group's longest shared length), equal sizes in item
 * order, items with no work last -- the order the device sort gives, with
 * exact token counts instead of size classes.
 *
 *   context_lens, prefix_groups, shared_lens   host copies of the device
 *                  arrays the call will get (groups and shared lengths may
 *                  be NULL when num_groups is 0)
 *   dispatch       host int32 out, capacity entries
 * Every other argument is paged_attention_multi_query_prefix's.  Returns the
 * number of entries written, or PA_ERR_NULL, PA_ERR_SHAPE (including
 * capacity too small), PA_ERR_DTYPE.
 */
int32_t paged_attention_multi_query_plan(const int32_t *context_lens,
                                         const int32_t *prefix_groups, int32_t num_groups,
                                         const int32_t *shared_lens, int32_t num_seqs,
                                         int32_t num_q_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t block_size,
                                         int32_t max_blocks_per_seq, int32_t max_query_len,
                                         int32_t max_context_len, int32_t kv_dtype,
                                         int32_t partition_size, int32_t *dispatch,
                                         int32_t capacity);

/* Workspace bytes paged_attention_multi_query_prefix needs: with the prefix
 * path, 4 * num_tokens * num_q_heads * (P + 1) * (head_dim + 2) for the
 * partials (the last slot of each row the prefix's), plus the dispatch list
 * (4 bytes per item: the num_seqs * P sequence items and the groups' items)
 * for launches of more than 1024 workgroups; otherwise
 * paged_attention_multi_query_workspace_size. */
size_t paged_attention_multi_query_prefix_workspace_size(
    int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t max_query_len, int32_t max_context_len, int32_t partition_size,
    int32_t num_groups, int32_t kv_dtype);

/*
 * kv_cache_write -- store each new token's K and V rows in the pool.
 *
 * For i in [0, num_tokens) with slot = slot_mapping[i] >= 0: copies
 * k[i] and v[i] (num_kv_heads rows of head_dim elements each) to block
 * slot / block_size, offset slot % block_size of every KV head of k_cache and
 * v_cache, bit for bit ([P1] section 3.1: the generated token's K/V is written back to the
 * cache; section 3.3 append_slot).  Negative slots are skipped (padding);
 * slots >= num_blocks*block_size are skipped too.  Two tokens must not share a
 * slot (the winner would be unspecified).
 *
 *   k, v           device, [num_tokens][num_kv_heads][head_dim], dtype
 *   slot_mapping   device int32 [num_tokens]
 *   k_cache,
 *   v_cache        device pool (layout above), modified in place
 * dtype may also be PA_FP8_E4M3 or PA_INT8 (codes copied as bytes).  A head row
 * (head_dim elements) must be a multiple of 16 bytes.
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_DTYPE, PA_ERR_LAUNCH; PA_ERR_INDEX
 * with index checking on.
 */
int32_t kv_cache_write(const void *k, const void *v, const int32_t *slot_mapping,
                       int32_t num_tokens, void *k_cache, void *v_cache,
                       int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                       int32_t head_dim, int32_t dtype, void *stream);

/*
 * kv_cache_write_fp8 -- kv_cache_write into an FP8 (E4M3) pool: each element
 * x of k (v) is stored as the code of y = x / k_scale (x / v_scale), the
 * division done in fp32 (correctly rounded), y clamped to [-448, 448] and
 * rounded to the nearest E4M3 value, ties to the even mantissa; NaN is
 * stored as NaN.
 *
 *   k, v           device, [num_tokens][num_kv_heads][head_dim], src_dtype
 *                  (PA_F32 or PA_BF16)
 *   slot_mapping   device int32 [num_tokens] (negative or out-of-pool slots
 *                  are skipped; two tokens must not share a slot)
 *   k_cache,
 *   v_cache        device FP8 pool (layout above), modified in place
 * head_dim must be a multiple of 16; scales finite and > 0; k and v aligned
 * to four elements (16 bytes for PA_F32, 8 for PA_BF16; PA_ERR_SHAPE
 * otherwise).
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_DTYPE, PA_ERR_LAUNCH; PA_ERR_INDEX
 * with index checking on.
 */
int32_t kv_cache_write_fp8(const void *k, const void *v, const int32_t *slot_mapping,
                           int32_t num_tokens, void *k_cache, void *v_cache, int32_t num_blocks,
                           int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                           int32_t src_dtype, float k_scale, float v_scale, void *stream);

/*
 * kv_cache_write_int8 -- kv_cache_write into an INT8 pool: each element x of
 * k (v) is stored as round(x / k_scale) (x / v_scale), the division done in
 * fp32 (correctly rounded), rounded to the nearest integer with ties to
 * even and clamped to [-127, 127]; NaN is stored as 0.  Arguments and errors
 * are those of kv_cache_write_fp8.
 */
int32_t kv_cache_write_int8(const void *k, const void *v, const int32_t *slot_mapping,
                            int32_t num_tokens, void *k_cache, void *v_cache, int32_t num_blocks,
                            int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                            int32_t src_dtype, float k_scale, float v_scale, void *stream);

/*
 * copy_blocks -- copy-on-write block copies.
 *
 * For each pair i, copies physical block src = pairs[2i] onto dst = pairs[2i+1]
 * in both k_cache and v_cache (block_size*num_kv_heads*head_dim elements each),
 * bit for bit ([P3] section "关键设计二：Copy-on-Write": a shared last block is
 * copied into a new block before the forked sequence appends to it).
 * Semantics are those of applying the pairs in list order; the pairs run
 * concurrently, so every dst must be distinct and no dst may also be a src
 * (checked on the host, reading the pairs from host memory, only when
 * host_pairs is non-NULL: PA_ERR_ALIAS).  Pairs with an id outside
 * [0, num_blocks) or src == dst are skipped.
 *
 *   src_dst_pairs  device int32 [num_pairs][2]
 *   host_pairs     optional host copy of the same pairs for the alias check
 * dtype is that of the pool (8-bit kinds included); a head row must be a
 * multiple of 16 bytes.
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_DTYPE, PA_ERR_ALIAS, PA_ERR_LAUNCH;
 * PA_ERR_INDEX with index checking on.
 */
int32_t copy_blocks(const int32_t *src_dst_pairs, int32_t num_pairs, void *k_cache,
                    void *v_cache, int32_t num_blocks, int32_t block_size,
                    int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                    const int32_t *host_pairs, void *stream);

/*
 * kv_cache_append -- a step's cache edits in one launch: copy_blocks of the
 * pairs, then the write of the new tokens (kv_cache_write, or
 * kv_cache_write_fp8 / _int8 for a quantising write), with exactly the
 * pools those two calls in that order leave ([P3] section "关键设计二：
 * Copy-on-Write": a forked sequence's shared last block is copied before it
 * appends; [P1] sections 3.1 and 3.3: the new token's K/V goes into its
 * slot).  Both run concurrently: a copy skips the positions that new tokens
 * write in its source or destination block, and the workgroup of a token
 * that writes into a copy's source block copies that position's old rows
 * first (unless a token also writes that position of the destination).
 *
 *   src_dst_pairs  device int32 [num_pairs][2] (may be NULL when num_pairs is 0)
 *   k, v           device, [num_tokens][num_kv_heads][head_dim], src_dtype
 *   slot_mapping   device int32 [num_tokens]
 *   k_cache,
 *   v_cache        device pool of kv_dtype (layout above), modified in place
 *   src_dtype      kv_dtype (rows stored bit for bit), or PA_F32 / PA_BF16
 *                  with an 8-bit kv_dtype (quantised with k_scale, v_scale as
 *                  in kv_cache_write_fp8 / _int8; the scales are ignored
 *                  otherwise)
 *   host_pairs     optional host copy of the pairs for the overlap check
 * The preconditions are those of the two calls: every dst distinct and never
 * a src (PA_ERR_ALIAS when host_pairs is given), no two tokens on one slot;
 * pairs and slots outside the pool are skipped.  k and v aligned to 16 bytes
 * (stored rows) or to four elements (quantised rows), else PA_ERR_SHAPE.
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_DTYPE, PA_ERR_ALIAS,
 * PA_ERR_LAUNCH; PA_ERR_INDEX with index checking on.
 */
int32_t kv_cache_append(const int32_t *src_dst_pairs, int32_t num_pairs, const void *k,
                        const void *v, const int32_t *slot_mapping, int32_t num_tokens,
                        void *k_cache, void *v_cache, int32_t num_blocks, int32_t block_size,
                        int32_t num_kv_heads, int32_t head_dim, int32_t src_dtype,
                        int32_t kv_dtype, float k_scale, float v_scale,
                        const int32_t *host_pairs, void *stream);

/*
 * Index checking -- a debug mode, off by default.  It is on when the
 * environment variable PAGEDATTN_CHECK is "1" at the library's first call
 * that consults it, or after pagedattn_set_index_check(1) (0 turns it off).
 * While it is on, before launching anything:
 *   paged_attention_decode (_fp8, _int8) and paged_attention_multi_query
 *     check every context length in [0, max_context_len] and, for each
 *     sequence, block_tables entries 0 .. ceil(L/block_size)-1 in
 *     [0, num_blocks);
 *   paged_attention_multi_query also checks query_start[0] == 0,
 *     query_start non-decreasing, query_start[num_seqs] <= num_tokens and
 *     every chunk at most its context length and max_query_len;
 *   kv_cache_write (_fp8, _int8) checks every slot < num_blocks*block_size
 *     (negative slots are padding);
 *   copy_blocks checks both ids of every pair in [0, num_blocks);
 *   kv_cache_append makes both of those checks;
 *   paged_attention_decode_prefix also checks the groups and shared lengths
 *     (the rules stated there) and that a given dispatch list holds every
 *     item exactly once (lists of at most 65536 items);
 *   paged_attention_multi_query_prefix makes the multi-query checks and
 *     checks the groups and shared lengths (at most 16 members).
 * A check runs one small kernel on the call's stream, synchronises that
 * stream and reads back one device word the library owns (one per device;
 * calls that overlap on one device race on it); on a bad index the call
 * returns PA_ERR_INDEX and launches nothing.  Not for graph capture.  With
 * checking off, the kernels clamp block ids into the pool and skip slots and
 * pairs outside it, so every access stays in bounds and the results for such
 * inputs are unspecified ([P1] section 2.1: every logical block maps through
 * the table to a physical block of the pool).
 */
void pagedattn_set_index_check(int32_t enable);
/* 1 while index checking is on, else 0. */
int32_t pagedattn_index_check(void);

/* A static English description of a pa_status value. */
const char *pagedattn_status_string(int32_t status);

/* Library version string, e.g. "libpagedattn 0.1 gfx950". */
const char *pagedattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
