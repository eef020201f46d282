// Internal launch interface between the C ABI layer (api.hip) and the kernel
// translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

struct DecodeArgs {
  const void *q;
  const void *k_cache;
  const void *v_cache;
  const int32_t *block_tables;
  const int32_t *context_lens;
  float *out;
  float *ws_o;   // [S][Hq][P][D] normalised partition outputs (P > 1 only)
  float *ws_ml;  // [S][Hq][P][2] partition (max, sum) in the log2 domain (P > 1 only)
  float scale;
  int32_t num_seqs, num_q_heads, num_kv_heads, head_dim;
  int32_t log2_block_size, num_blocks, max_blocks_per_seq;
  int32_t partition_size;  // tokens per partition (>= every context when P == 1)
  int32_t num_partitions;  // P
  int32_t dtype;           // of q and, unless kv_dtype says otherwise, of the pool: 0 = f32, 1 = bf16
  int32_t kv_dtype = -1;   // 2 = FP8 E4M3, 3 = INT8 pool (bf16 q, matrix-core kernel only);
                           // -1 = dtype
  float k_scale = 1.f;     // 8-bit pools: stored code c means value(c) * scale
  float v_scale = 1.f;
  int32_t *order = nullptr;  // [S * P (+ 4 * num_groups)] dispatch order of the (sequence,
                             // partition) items and the prefix items, written by
                             // launch_schedule; nullptr = fixed order
  bool order_ready = false;  // order was planned by the caller: no sort kernel
  // shared prefixes (matrix-core kernel only): num_groups > 0 adds four items
  // (16-column sets) per group and KV head that read the group's shared tiles
  // once; the partials then have num_partitions + 1 slots per row, the last
  // one the prefix's
  const int32_t *groups = nullptr;       // [num_groups][2] (first sequence, members)
  const int32_t *shared_lens = nullptr;  // [num_seqs] positions read through the group
  int32_t num_groups = 0;
};

// Over 8-bit pools, a member of a prefix group whose private positions
// [sh, L) fit in one 16-token tile ("short"): the group's prefix item reads
// that tile too and writes the member's rows to out, so the member has no
// sequence items and no merge (measured on the GQA prefix batch: FP8
// 90.7 -> 87.1 us per call; over bf16 pools the longer prefix items cost
// more than they save, 167.5 -> 168.5 us, so bf16 keeps separate items).
// sh is the shared length as the kernels take it (clamped to [0, L],
// rounded down to 16 tokens).
__host__ __device__ inline bool prefix_short(int L, int sh) { return sh > 0 && L - sh <= 16; }
__host__ __device__ inline bool short_members(int kv_dtype) { return kv_dtype == 2 || kv_dtype == 3; }

// Launches with more workgroups than this run their longest items first (a
// smaller grid is resident at once, so its order does not matter).
constexpr int64_t kScheduleMinWorkgroups = 1024;
bool schedule_wanted(int64_t workgroups, int64_t num_seqs, int64_t P);
// Writes order[0 .. S*P-1] (schedule.hip): the (sequence, partition) items
// c (sequence c % S, partition P - 1 - c / S), longest first, those past a
// sequence's last partition last and as ~c (negative); ps = tokens
// per partition, cap = the most tokens a sequence may have.  launch_decode
// and launch_multi_query call it when their args carry an order buffer.
// With groups: ipg items per group follow the sequence items; a decode
// prefix item (group = G) is sized by the members with columns in its set,
// a multi-query one (group = 0) by every member.
hipError_t launch_schedule(const int32_t *context_lens, int32_t *order, int num_seqs, int P,
                           int ps, int cap, hipStream_t stream,
                           const int32_t *groups = nullptr, const int32_t *shared_lens = nullptr,
                           int num_groups = 0, int group = 1, bool short_rule = false,
                           int ipg = 4);

// Enqueues decode (and the partition merge when P > 1).  Returns hipSuccess or
// the launch error; hipErrorNotSupported when no kernel is compiled for the
// (dtype, head_dim, group) combination.
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);
bool decode_supported(int32_t dtype, int32_t head_dim, int32_t group);

// The matrix-core decode (decode_mfma.hip): bfloat16, head_dim 128, G in {4, 8}.
bool decode_mfma_supported(int32_t dtype, int32_t head_dim, int32_t group);
// 8-bit (FP8 / INT8) pools with bfloat16 queries: head_dim 128, G in {1, 2, 4, 8}.
bool decode_q8_supported(int32_t head_dim, int32_t group);
// Shared-prefix items (bfloat16 or 8-bit pools, bfloat16 q): head_dim 128,
// G in {1, 2, 4, 8}; at most 64 / G members per group.
bool decode_prefix_supported(int32_t head_dim, int32_t group);
hipError_t launch_decode_mfma(const DecodeArgs &a, hipStream_t stream);

// Merge of the per-partition partials into `out` (P > 1 only).
hipError_t launch_partition_merge(const DecodeArgs &a, hipStream_t stream);

struct MultiQueryArgs {
  const void *q;             // [num_tokens][Hq][D]
  const void *k_cache;
  const void *v_cache;
  const int32_t *block_tables;
  const int32_t *context_lens;
  const int32_t *query_start;  // [num_seqs + 1]
  float *out;                // [num_tokens][Hq][D]
  float scale;
  int32_t num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim;
  int32_t log2_block_size, num_blocks, max_blocks_per_seq, max_query_len;
  int32_t dtype;
  int32_t partition_size;  // tokens per partition (a multiple of 64) when P > 1
  int32_t num_partitions;  // P
  float *ws_o;             // [num_tokens][Hq][P][D] (P > 1 only)
  float *ws_ml;            // [num_tokens][Hq][P][2]
  int32_t *order = nullptr;  // [S * P] longest-first (sequence, partition) list, or nullptr
  bool order_ready = false;  // order was planned by the caller: no sort kernel
  int32_t kv_dtype = -1;     // 2 = FP8 E4M3, 3 = INT8 pool (decode walk only); -1 = dtype
  float k_scale = 1.f;       // 8-bit pools: stored code c means value(c) * scale
  float v_scale = 1.f;
  // shared prefixes (decode walk only): groups [num_groups][2] (first
  // sequence, members), shared_lens [num_seqs]; the partials then hold one
  // more slot per row (P + 1, the prefix partial last)
  const int32_t *groups = nullptr;
  const int32_t *shared_lens = nullptr;
  int32_t num_groups = 0;
};

// Most members of a shared-prefix group in a multi-query call.
constexpr int kMqPrefixMembers = 16;
// A multi-query call takes prefix items only with at most this many (token,
// head) rows per sequence and KV head, so that one 16-column item covers at
// least two members (measured on the speculative-verification structure,
// G = 4: 1 and 2 tokens per sequence gain 17% and 7%, 3 break even, 5 lose
// 10%: each item walks the whole prefix, and L2 already serves most of the
// members' repeated reads).  Items of two column sets (32 rows, one pass per
// two members at 5 tokens) lost too: 3, 4, 5 and 8 tokens 7-29% slower.
constexpr int64_t kMqPrefixRows = 8;
// Prefix items per group of such a call: each covers 16 (member, token,
// head) rows.
inline int64_t mq_prefix_items_per_group(int64_t max_query_len, int64_t gh) {
  return (kMqPrefixMembers * max_query_len * gh + 15) / 16;
}

// Workgroups of a multi-query launch (either kernel), for the schedule
// decision and the workspace size.
int64_t multi_query_workgroups(int64_t num_seqs, int64_t num_q_heads, int64_t num_kv_heads,
                               int64_t head_dim, int64_t max_query_len, int64_t P);

// Multi-query launches with at most this many (token, head) rows per KV head
// take the decode walk (decode_mfma.hip) when it supports them.
constexpr int64_t kMqFewRows = 64;

// Multi-query attention on the decode kernel (decode_mfma.hip) when every KV
// head has at most 64 (token, head) rows, in sets of 16: bfloat16, head_dim
// 128.  Writes
// out, or the partition partials that the multi-query merge combines.
bool multi_query_few_rows_supported(const struct MultiQueryArgs &a);
// Workgroups per (sequence, KV head, partition) of that path for csets sets
// of 16 rows (a wave carries two sets when there are at least two).
int64_t multi_query_few_rows_groups(int64_t csets);
hipError_t launch_multi_query_few_rows(const struct MultiQueryArgs &a, hipStream_t stream);

// Causal multi-query attention (multi_query.hip): bfloat16, head_dim 64 or 128.
bool multi_query_supported(int32_t dtype, int32_t head_dim);
hipError_t launch_multi_query(const MultiQueryArgs &a, hipStream_t stream);

hipError_t launch_kv_cache_write(const void *k, const void *v, const int32_t *slot_mapping,
                                 int32_t num_tokens, void *k_cache, void *v_cache,
                                 int64_t num_slots, int32_t log2_block_size, int32_t num_kv_heads,
                                 int64_t head_row_bytes, hipStream_t stream);

// Quantising write into an 8-bit pool: kv_dtype 2 = FP8 E4M3, 3 = INT8.
hipError_t launch_kv_cache_write_q8(const void *k, const void *v, const int32_t *slot_mapping,
                                    int32_t num_tokens, void *k_cache, void *v_cache,
                                    int64_t num_slots, int32_t log2_block_size,
                                    int32_t num_kv_heads, int32_t head_dim, int32_t src_dtype,
                                    int32_t kv_dtype, float k_scale, float v_scale,
                                    hipStream_t stream);

// Index checking (checks.hip): on when PAGEDATTN_CHECK=1 at first use or
// after pagedattn_set_index_check(1).  Each check enqueues one workgroup on
// `stream`, synchronises it and returns PA_OK, PA_ERR_INDEX or PA_ERR_LAUNCH.
bool index_check_on();
void set_index_check(bool on);
int32_t check_tables(const int32_t *lens, const int32_t *tables, int32_t num_seqs,
                     int32_t max_blocks_per_seq, int32_t log2_block_size, int32_t num_blocks,
                     int32_t max_context_len, hipStream_t stream);
int32_t check_queries(const int32_t *lens, const int32_t *query_start, int32_t num_seqs,
                      int32_t num_tokens, int32_t max_query_len, hipStream_t stream);
int32_t check_prefix_groups(const int32_t *lens, const int32_t *tables, const int32_t *groups,
                            int32_t num_groups, const int32_t *shared_lens, int32_t num_seqs,
                            int32_t max_blocks_per_seq, int32_t log2_block_size,
                            int32_t max_context_len, int32_t max_members, hipStream_t stream);
int32_t check_dispatch(const int32_t *dispatch, int32_t num_items, hipStream_t stream);
int32_t check_slots(const int32_t *slots, int32_t num_tokens, int64_t num_slots,
                    hipStream_t stream);
int32_t check_pairs(const int32_t *pairs, int32_t num_pairs, int32_t num_blocks,
                    hipStream_t stream);

hipError_t launch_copy_blocks(const int32_t *pairs, int32_t num_pairs, void *k_cache,
                              void *v_cache, int32_t num_blocks, int64_t block_bytes,
                              hipStream_t stream);

// copy_blocks then the write, in one launch (cache_ops.hip): stored bytes
// when kv_dtype == src_dtype, else a quantising write into an 8-bit pool.
hipError_t launch_kv_cache_append(const int32_t *pairs, int32_t num_pairs, const void *k,
                                  const void *v, const int32_t *slot_mapping, int32_t num_tokens,
                                  void *k_cache, void *v_cache, int32_t num_blocks,
                                  int32_t log2_block_size, int32_t num_kv_heads,
                                  int64_t head_row_bytes, int32_t src_dtype, int32_t kv_dtype,
                                  float k_scale, float v_scale, hipStream_t stream);

}  // namespace pa
