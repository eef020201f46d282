// The C ABI of libpagedattn: argument validation, the split-K partition
// policy, workspace sizing, status strings and the kernel launches.  All
// entry points are declared (and their contracts described) in
// include/pagedattn.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <new>
#include <vector>

#include "internal.h"
#include "pagedattn.h"

namespace {

constexpr int32_t kChunkTokens = 16;
constexpr int32_t kAutoPartition = 4096;
constexpr int64_t kCUs = 256;                // MI355X compute units
constexpr int64_t kTargetWorkgroups = 512;  // about two per CU
constexpr int64_t kMinAutoPartition = 512;
constexpr int64_t kMaxTokensPerSeq = int64_t(1) << 30;

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

int log2_exact(int64_t x) {
  int n = 0;
  while ((int64_t(1) << n) < x) ++n;
  return n;
}

int64_t elem_bytes(int32_t dtype) { return dtype == PA_F32 ? 4 : dtype == PA_BF16 ? 2 : 1; }

bool is_q8(int32_t dtype) { return dtype == PA_FP8_E4M3 || dtype == PA_INT8; }

bool known_dtype(int32_t dtype) { return dtype == PA_F32 || dtype == PA_BF16; }

// pools may also hold FP8 codes (moved as raw bytes by the edits)
bool known_pool_dtype(int32_t dtype) { return known_dtype(dtype) || is_q8(dtype); }

// head rows must be whole 16-byte vectors for the edit kernels
bool head_row_ok(int32_t head_dim, int32_t dtype) {
  return head_dim > 0 && ((int64_t)head_dim * elem_bytes(dtype)) % 16 == 0;
}

bool valid_scale(float x) { return x > 0.f && x < __builtin_huge_valf(); }

// Partition policy.  Returns the number of partitions (>= 1) and the partition
// size through *ps, or a negative pa_status.
//   partition_size < 0: never split;
//   partition_size > 0: that many tokens, a multiple of the 16-token chunk;
//   partition_size == 0: automatic.  With at least one (sequence, KV head)
//     pair per CU, contexts longer than 4096 tokens are split into 4096-token
//     partitions: shorter ones balance long and short sequences better over
//     the 256 CUs, but every workgroup pays a fixed start-up latency (context
//     length, table, first tile) and every split sequence a merge.  With the
//     longest-first dispatch order, 4096 was the fastest size measured on the
//     GQA prefix-sharing batch (lognormal lengths, median 1024, cap 8192;
//     172 us against 178 us at 2048 with shared prefixes, 201 against 204
//     without), on its FP8 form (96.6 against 101-102 us), on the
//     Llama-7B-shaped batch (373.6 against 378.5 us) and on speculative
//     verification; the fork step was unchanged.  With fewer pairs (a few long
//     sequences), each pair's context is cut into floor(512 / pairs) equal
//     partitions (a multiple of 16 tokens, at least 512), about two
//     workgroups per CU: on 8 sequences of 32768 tokens with 8 KV heads,
//     4096-token partitions (512 workgroups) were faster than 2048, 2736
//     (768 workgroups) or 8192 (256 workgroups).
int32_t resolve_partitions(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len,
                           int32_t partition_size, int32_t *ps) {
  if (max_context_len < 0) return PA_ERR_SHAPE;
  int32_t want = partition_size;
  if (want == 0) {
    int64_t size = kAutoPartition;
    const int64_t pairs = (int64_t)num_seqs * num_kv_heads;
    if (pairs > 0 && pairs < kCUs) {
      const int64_t parts = kTargetWorkgroups / pairs;
      size = ((max_context_len + parts - 1) / parts + kChunkTokens - 1) / kChunkTokens * kChunkTokens;
      if (size < kMinAutoPartition) size = kMinAutoPartition;
    }
    want = max_context_len > size ? (int32_t)size : -1;
  }
  if (want > 0 && want % kChunkTokens != 0) return PA_ERR_SHAPE;
  if (want < 0 || max_context_len <= want) {
    *ps = want > 0 ? want : kChunkTokens;
    return 1;
  }
  *ps = want;
  return (int32_t)(((int64_t)max_context_len + want - 1) / want);
}

// Multi-query partitions: the row tiles of one (sequence, KV head) already
// give the chip work when chunks are long, so only chunks of at most 64 query
// rows per KV head are split, by the decode policy rounded up to whole
// 64-token tiles; an explicit size must be a multiple of 64.
int32_t resolve_mq_partitions(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t max_query_len, int32_t max_context_len,
                              int32_t partition_size, int32_t *ps) {
  if (max_context_len < 0 || max_query_len < 0 || num_kv_heads <= 0) return PA_ERR_SHAPE;
  const int64_t rows = (int64_t)max_query_len * (num_q_heads / num_kv_heads);
  int32_t want = partition_size;
  if (want == 0) {
    want = -1;
    if (rows <= 64) {
      int32_t dps = 0;
      const int32_t dp = resolve_partitions(num_seqs, num_kv_heads, max_context_len, 0, &dps);
      if (dp > 1) want = (dps + 63) / 64 * 64;
    }
  }
  if (want > 0 && want % 64 != 0) return PA_ERR_SHAPE;
  if (want < 0 || max_context_len <= want) {
    *ps = 1 << 30;
    return 1;
  }
  *ps = want;
  return (int32_t)(((int64_t)max_context_len + want - 1) / want);
}

// A decode call's workspace: the split-K partials ([S][Hq][P][D] outputs, then
// [S][Hq][P][2] (max, sum); P > 1 only), followed by the longest-first
// dispatch list (int32 [S * P]) when the launch is large enough to use one.
// With num_groups > 0 (shared prefixes), every row has P + 1 partial slots
// (the last one the prefix's) and the list also holds the groups' items.
struct DecodeWorkspace {
  size_t partials, order;
};
DecodeWorkspace decode_workspace(int64_t num_seqs, int64_t num_q_heads, int64_t num_kv_heads,
                                 int64_t head_dim, int64_t P, int64_t num_groups = 0) {
  DecodeWorkspace w;
  const int64_t slots = P + (num_groups > 0 ? 1 : 0);
  w.partials =
      slots > 1 ? (size_t)(num_seqs * num_q_heads * slots * (head_dim + 2)) * sizeof(float) : 0;
  const int64_t items = num_seqs * P + 4 * num_groups;
  w.order = pa::schedule_wanted(items * num_kv_heads, items, 1)
                ? (size_t)items * sizeof(int32_t)
                : 0;
  return w;
}

// A multi-query call's workspace: the split partials ([T][Hq][P][D], then
// [T][Hq][P][2]; P > 1 only), then the longest-first list (int32 [S * P])
// when the launch is large enough to use one.
struct MultiQueryWorkspace {
  size_t partials, order;
};
// With num_groups > 0 (shared prefixes, decode walk only) every row has P + 1
// partial slots (the last one the prefix's) and the list also holds the
// groups' prefix items.
MultiQueryWorkspace multi_query_workspace(int64_t num_seqs, int64_t num_tokens,
                                          int64_t num_q_heads, int64_t num_kv_heads,
                                          int64_t head_dim, int64_t max_query_len, int64_t P,
                                          int64_t num_groups = 0) {
  MultiQueryWorkspace w;
  const int64_t slots = P + (num_groups > 0 ? 1 : 0);
  w.partials = slots > 1
                   ? (size_t)(num_tokens * num_q_heads * slots * (head_dim + 2)) * sizeof(float)
                   : 0;
  const int64_t ipg =
      num_groups > 0 ? pa::mq_prefix_items_per_group(max_query_len, num_q_heads / num_kv_heads)
                     : 0;
  const int64_t items = num_seqs * P + ipg * num_groups;
  const int64_t wgs = pa::multi_query_workgroups(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                 max_query_len, P) +
                      ipg * num_groups * num_kv_heads;
  w.order = pa::schedule_wanted(wgs, items, 1) ? (size_t)items * sizeof(int32_t) : 0;
  return w;
}

// Whether a multi-query call with shared prefixes takes the prefix path
// (the decode walk over a bf16 pool, head_dim 128, at most kMqPrefixRows
// (token, head) rows per sequence and KV head; else it is the plain
// multi-query call).  Over 8-bit pools the prefix items measured slower
// even at 2 tokens per sequence (FP8 100.9 -> 106.1 us, INT8 112.1 -> 116.0
// on the speculative-verification structure): half the bytes per position
// leave less for the shared walk to save.
bool mq_prefix_path(int32_t kv_dtype, int32_t head_dim, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t max_query_len, int32_t num_groups) {
  return num_groups > 0 && kv_dtype == PA_BF16 && head_dim == 128 && num_kv_heads > 0 &&
         num_q_heads % num_kv_heads == 0 && max_query_len > 0 &&
         (int64_t)max_query_len * (num_q_heads / num_kv_heads) <= pa::kMqPrefixRows;
}

}  // namespace

extern "C" {

int32_t paged_attention_multi_query_partitions(int32_t num_seqs, int32_t num_q_heads,
                                               int32_t num_kv_heads, int32_t max_query_len,
                                               int32_t max_context_len, int32_t partition_size) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads)
    return PA_ERR_SHAPE;
  int32_t ps = 0;
  return resolve_mq_partitions(num_seqs, num_q_heads, num_kv_heads, max_query_len,
                               max_context_len, partition_size, &ps);
}

size_t paged_attention_multi_query_workspace_size(int32_t num_seqs, int32_t num_tokens,
                                                  int32_t num_q_heads, int32_t num_kv_heads,
                                                  int32_t head_dim, int32_t max_query_len,
                                                  int32_t max_context_len,
                                                  int32_t partition_size) {
  if (num_tokens < 0 || head_dim <= 0) return 0;
  const int32_t P = paged_attention_multi_query_partitions(
      num_seqs, num_q_heads, num_kv_heads, max_query_len, max_context_len, partition_size);
  if (P < 1) return 0;
  const MultiQueryWorkspace w = multi_query_workspace(num_seqs, num_tokens, num_q_heads,
                                                      num_kv_heads, head_dim, max_query_len, P);
  return w.partials + w.order;
}

const char *pagedattn_status_string(int32_t status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "a required pointer is NULL";
    case PA_ERR_SHAPE: return "inconsistent or out-of-range sizes";
    case PA_ERR_DTYPE: return "unknown dtype";
    case PA_ERR_UNSUPPORTED: return "head_dim or query-group size not compiled in";
    case PA_ERR_WORKSPACE: return "split-K workspace missing or too small";
    case PA_ERR_ALIAS: return "copy pairs overlap (a dst repeats or is also a src)";
    case PA_ERR_INDEX: return "an index read on the device is out of range (index checking)";
    case PA_ERR_LAUNCH: return "the HIP runtime refused the kernel launch";
    case PA_ERR_OOM: return "no free KV block left";
    case PA_ERR_NO_SEQ: return "unknown sequence id";
    case PA_ERR_SEQ_EXISTS: return "sequence id already in use";
    case PA_ERR_SCRATCH:
      return "the call needs more workspace than the library's static scratch holds";
    default: return "unknown status";
  }
}

const char *pagedattn_version(void) { return "libpagedattn 0.1 gfx950"; }

int32_t paged_attention_num_partitions(int32_t num_seqs, int32_t num_kv_heads,
                                       int32_t max_context_len, int32_t partition_size) {
  int32_t ps = 0;
  return resolve_partitions(num_seqs, num_kv_heads, max_context_len, partition_size, &ps);
}

int32_t paged_attention_partition_tokens(int32_t num_seqs, int32_t num_kv_heads,
                                         int32_t max_context_len, int32_t partition_size) {
  int32_t ps = 0;
  const int32_t P =
      resolve_partitions(num_seqs, num_kv_heads, max_context_len, partition_size, &ps);
  if (P < 0) return P;
  return P > 1 ? ps : max_context_len;
}

size_t paged_attention_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim,
                                      int32_t max_context_len, int32_t partition_size) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0) return 0;
  int32_t ps = 0;
  const int32_t P = resolve_partitions(num_seqs, num_kv_heads, max_context_len, partition_size, &ps);
  if (P < 1) return 0;
  const DecodeWorkspace w = decode_workspace(num_seqs, num_q_heads, num_kv_heads, head_dim, P);
  return w.partials + w.order;
}

}  // extern "C"

namespace {

// Decode over a pool of kv_dtype (dtype for a bf16/fp32 pool, PA_FP8_E4M3
// with bf16 queries); the checks and launch shared by both entry points.
int32_t decode_impl(const void *q, const void *k_cache, const void *v_cache,
                    const int32_t *block_tables, const int32_t *context_lens, float scale,
                    float *out, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                    int32_t head_dim, int32_t block_size, int32_t num_blocks,
                    int32_t max_blocks_per_seq, int32_t max_context_len, int32_t dtype,
                    int32_t kv_dtype, float k_scale, float v_scale, int32_t partition_size,
                    void *workspace, size_t workspace_bytes, void *stream,
                    const int32_t *groups = nullptr, int32_t num_groups = 0,
                    const int32_t *shared_lens = nullptr, const int32_t *dispatch = nullptr) {
  if (!known_dtype(dtype)) return PA_ERR_DTYPE;
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      num_blocks <= 0 || max_blocks_per_seq <= 0 || max_context_len < 0)
    return PA_ERR_SHAPE;
  if (!is_pow2(block_size) || block_size > 1024) return PA_ERR_SHAPE;
  if (num_q_heads % num_kv_heads != 0) return PA_ERR_SHAPE;
  if ((int64_t)num_blocks * block_size >= (int64_t(1) << 31)) return PA_ERR_SHAPE;
  // byte offsets inside one block are 32-bit in the kernels
  if ((int64_t)block_size * num_kv_heads * head_dim * elem_bytes(kv_dtype) >= (int64_t(1) << 31))
    return PA_ERR_SHAPE;
  if ((int64_t)max_blocks_per_seq * block_size > kMaxTokensPerSeq) return PA_ERR_SHAPE;
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size) return PA_ERR_SHAPE;
  if (is_q8(kv_dtype)) {
    if (dtype != PA_BF16 || !pa::decode_q8_supported(head_dim, num_q_heads / num_kv_heads))
      return PA_ERR_UNSUPPORTED;
    if (!valid_scale(k_scale) || !valid_scale(v_scale)) return PA_ERR_SHAPE;
  } else if (!pa::decode_supported(dtype, head_dim, num_q_heads / num_kv_heads)) {
    return PA_ERR_UNSUPPORTED;
  }
  if (num_groups < 0 || num_groups > num_seqs) return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out) return PA_ERR_NULL;
  if (num_groups > 0 && (!groups || !shared_lens)) return PA_ERR_NULL;

  int32_t ps = 0;
  const int32_t P = resolve_partitions(num_seqs, num_kv_heads, max_context_len, partition_size, &ps);
  if (P < 0) return P;
  if (((int64_t)num_seqs * P + 4 * (int64_t)num_groups) * num_kv_heads >= (int64_t(1) << 32))
    return PA_ERR_SHAPE;
  if ((int64_t)num_seqs * num_q_heads >= (int64_t(1) << 31)) return PA_ERR_SHAPE;

  pa::DecodeArgs a;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.out = out;
  a.ws_o = nullptr;
  a.ws_ml = nullptr;
  a.scale = scale;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.log2_block_size = log2_exact(block_size);
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_partitions = P;
  a.dtype = dtype;
  a.kv_dtype = kv_dtype;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.groups = groups;
  a.shared_lens = shared_lens;
  a.num_groups = num_groups;
  const int64_t slots = P + (num_groups > 0 ? 1 : 0);
  const DecodeWorkspace w =
      decode_workspace(num_seqs, num_q_heads, num_kv_heads, head_dim, P, num_groups);
  if (slots > 1) {
    if (!workspace || workspace_bytes < w.partials) return PA_ERR_WORKSPACE;
    a.ws_o = static_cast<float *>(workspace);
    a.ws_ml = a.ws_o + (size_t)num_seqs * num_q_heads * slots * head_dim;
  }
  if (P > 1) {
    a.partition_size = ps;
  } else {
    // one partition covers any context the kernel will accept after clamping
    a.partition_size = (int32_t)((int64_t)max_blocks_per_seq * block_size);
  }
  // a list the caller planned; else, with room for it, the longest-first
  // list sorted on the device; else the fixed order
  if (dispatch) {
    a.order = const_cast<int32_t *>(dispatch);
    a.order_ready = true;
  } else if (w.order > 0 && workspace && workspace_bytes >= w.partials + w.order) {
    a.order = reinterpret_cast<int32_t *>(static_cast<uint8_t *>(workspace) + w.partials);
  }
  if (pa::index_check_on()) {
    int32_t st = pa::check_tables(context_lens, block_tables, num_seqs, max_blocks_per_seq,
                                  a.log2_block_size, num_blocks, max_context_len,
                                  static_cast<hipStream_t>(stream));
    if (st == PA_OK && num_groups > 0)
      st = pa::check_prefix_groups(context_lens, block_tables, groups, num_groups, shared_lens,
                                   num_seqs, max_blocks_per_seq, a.log2_block_size,
                                   max_context_len, 64 / (num_q_heads / num_kv_heads),
                                   static_cast<hipStream_t>(stream));
    if (st == PA_OK && dispatch)
      st = pa::check_dispatch(dispatch, (int32_t)((int64_t)num_seqs * P + 4 * (int64_t)num_groups),
                              static_cast<hipStream_t>(stream));
    if (st != PA_OK) return st;
  }
  const hipError_t e = pa::launch_decode(a, static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported) return PA_ERR_UNSUPPORTED;
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int32_t paged_attention_decode(const void *q, const void *k_cache, const void *v_cache,
                               const int32_t *block_tables, const int32_t *context_lens,
                               float scale, float *out, int32_t num_seqs, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int32_t num_blocks, int32_t max_blocks_per_seq,
                               int32_t max_context_len, int32_t dtype, int32_t partition_size,
                               void *workspace, size_t workspace_bytes, void *stream) {
  return decode_impl(q, k_cache, v_cache, block_tables, context_lens, scale, out, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, max_context_len, dtype, dtype, 1.f, 1.f, partition_size,
                     workspace, workspace_bytes, stream);
}

int32_t paged_attention_decode_fp8(const void *q, const void *k_cache, const void *v_cache,
                                   const int32_t *block_tables, const int32_t *context_lens,
                                   float scale, float k_scale, float v_scale, float *out,
                                   int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                   int32_t max_blocks_per_seq, int32_t max_context_len,
                                   int32_t partition_size, void *workspace,
                                   size_t workspace_bytes, void *stream) {
  return decode_impl(q, k_cache, v_cache, block_tables, context_lens, scale, out, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, max_context_len, PA_BF16, PA_FP8_E4M3, k_scale, v_scale,
                     partition_size, workspace, workspace_bytes, stream);
}

int32_t paged_attention_decode_int8(const void *q, const void *k_cache, const void *v_cache,
                                    const int32_t *block_tables, const int32_t *context_lens,
                                    float scale, float k_scale, float v_scale, float *out,
                                    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                    int32_t max_blocks_per_seq, int32_t max_context_len,
                                    int32_t partition_size, void *workspace,
                                    size_t workspace_bytes, void *stream) {
  return decode_impl(q, k_cache, v_cache, block_tables, context_lens, scale, out, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, max_context_len, PA_BF16, PA_INT8, k_scale, v_scale,
                     partition_size, workspace, workspace_bytes, stream);
}

// Whether a shared-prefix call takes the prefix path (else it is plain decode).
static bool prefix_path(int32_t kv_dtype, int32_t head_dim, int32_t num_q_heads,
                        int32_t num_kv_heads, int32_t num_groups) {
  return num_groups > 0 && kv_dtype != PA_F32 && num_kv_heads > 0 &&
         num_q_heads % num_kv_heads == 0 &&
         pa::decode_prefix_supported(head_dim, num_q_heads / num_kv_heads);
}

size_t paged_attention_prefix_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                             int32_t num_kv_heads, int32_t head_dim,
                                             int32_t max_context_len, int32_t partition_size,
                                             int32_t num_groups, int32_t kv_dtype) {
  if (!prefix_path(kv_dtype, head_dim, num_q_heads, num_kv_heads, num_groups))
    return paged_attention_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                          max_context_len, partition_size);
  if (num_seqs < 0 || num_groups > num_seqs) return 0;
  int32_t ps = 0;
  const int32_t P = resolve_partitions(num_seqs, num_kv_heads, max_context_len, partition_size, &ps);
  if (P < 1) return 0;
  const DecodeWorkspace w =
      decode_workspace(num_seqs, num_q_heads, num_kv_heads, head_dim, P, num_groups);
  return w.partials + w.order;
}

int32_t paged_attention_decode_prefix(const void *q, const void *k_cache, const void *v_cache,
                                      const int32_t *block_tables, const int32_t *context_lens,
                                      const int32_t *prefix_groups, int32_t num_groups,
                                      const int32_t *shared_lens, const int32_t *dispatch,
                                      float scale, float k_scale, float v_scale, float *out,
                                      int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                      int32_t max_blocks_per_seq, int32_t max_context_len,
                                      int32_t kv_dtype, int32_t partition_size, void *workspace,
                                      size_t workspace_bytes, void *stream) {
  if (!known_pool_dtype(kv_dtype)) return PA_ERR_DTYPE;
  if (num_groups < 0) return PA_ERR_SHAPE;
  const int32_t q_dtype = is_q8(kv_dtype) ? PA_BF16 : kv_dtype;
  const bool pfx = prefix_path(kv_dtype, head_dim, num_q_heads, num_kv_heads, num_groups);
  return decode_impl(q, k_cache, v_cache, block_tables, context_lens, scale, out, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_blocks_per_seq, max_context_len, q_dtype, kv_dtype,
                     is_q8(kv_dtype) ? k_scale : 1.f, is_q8(kv_dtype) ? v_scale : 1.f,
                     partition_size, workspace, workspace_bytes, stream,
                     pfx ? prefix_groups : nullptr, pfx ? num_groups : 0,
                     pfx ? shared_lens : nullptr, dispatch);
}

}  // extern "C"

namespace {

// The dispatch list of n items, longest first by tokens_of(c) (the tokens an
// item attends, -1 when it does no work): sort keys hold (tokens + 1) in the
// high word, complemented so that larger counts come first, and the item
// number in the low word, so equal counts keep item order and items with no
// work sort last.
template <typename F>
void plan_longest_first(int64_t n, F tokens_of, int32_t *dispatch) {
  std::vector<uint64_t> keys((size_t)n);
  for (int64_t c = 0; c < n; ++c)
    keys[(size_t)c] =
        ((uint64_t)(0xFFFFFFFFu - (uint32_t)(tokens_of(c) + 1)) << 32) | (uint32_t)c;
  std::sort(keys.begin(), keys.end());
  for (int64_t i = 0; i < n; ++i) dispatch[i] = (int32_t)(keys[(size_t)i] & 0xFFFFFFFFu);
}

}  // namespace

extern "C" {

int32_t paged_attention_decode_plan(const int32_t *context_lens, const int32_t *prefix_groups,
                                    int32_t num_groups, const int32_t *shared_lens,
                                    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t block_size,
                                    int32_t max_blocks_per_seq, int32_t max_context_len,
                                    int32_t kv_dtype, int32_t partition_size, int32_t *dispatch,
                                    int32_t capacity) {
  if (!known_pool_dtype(kv_dtype)) return PA_ERR_DTYPE;
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      max_blocks_per_seq <= 0 || max_context_len < 0 || num_groups < 0 ||
      num_groups > num_seqs || num_q_heads % num_kv_heads != 0)
    return PA_ERR_SHAPE;
  if (!is_pow2(block_size) || block_size > 1024) return PA_ERR_SHAPE;
  if ((int64_t)max_blocks_per_seq * block_size > kMaxTokensPerSeq) return PA_ERR_SHAPE;
  if (num_seqs == 0) return 0;
  const bool pfx = prefix_path(kv_dtype, head_dim, num_q_heads, num_kv_heads, num_groups);
  const int32_t ng = pfx ? num_groups : 0;
  if (!context_lens || !dispatch || (ng > 0 && (!prefix_groups || !shared_lens)))
    return PA_ERR_NULL;
  int32_t ps = 0;
  const int32_t P = resolve_partitions(num_seqs, num_kv_heads, max_context_len, partition_size, &ps);
  if (P < 0) return P;
  const int64_t cap = (int64_t)max_blocks_per_seq * block_size;
  if (P <= 1) ps = (int32_t)cap;  // as decode: one partition spans any clamped context
  const int64_t n = (int64_t)num_seqs * P + 4 * (int64_t)ng;
  if (n >= (int64_t(1) << 31) || capacity < n) return PA_ERR_SHAPE;
  const int32_t G = num_q_heads / num_kv_heads;
  const bool short_rule = ng > 0 && pa::short_members(kv_dtype);
  // the decode kernels' clamps and item bounds: tokens of item c, -1 when it
  // does no work
  auto L_of = [&](int32_t s) {
    return (int32_t)std::min<int64_t>(std::max(context_lens[s], 0), cap);
  };
  auto shared_of = [&](int32_t s, int32_t L) {
    return ng > 0 ? (std::min(std::max(shared_lens[s], 0), L) & ~15) : 0;
  };
  // longest first; equal sizes keep item order (members of a prefix group and
  // the column sets of one group stay side by side); items with no work last
  plan_longest_first(n, [&](int64_t c) -> int64_t {
    int64_t tokens;
    if (c < (int64_t)num_seqs * P) {
      const int32_t s = (int32_t)(c % num_seqs);
      const int32_t p = (P - 1) - (int32_t)(c / num_seqs);
      const int32_t L = L_of(s);
      const int32_t nparts = std::min((int32_t)(((int64_t)L + ps - 1) / ps), P);
      const int32_t sh = shared_of(s, L);
      // (a short member's prefix item reads its private tile too)
      if (p >= std::max(nparts, 1) || (sh > 0 && p < sh / ps) ||
          (short_rule && pa::prefix_short(L, sh))) {
        tokens = -1;
      } else {
        tokens = std::max<int64_t>(
            0, std::min<int64_t>(L, (int64_t)p * ps + ps) - std::max<int64_t>((int64_t)p * ps, sh));
      }
    } else {
      const int64_t gi = (c - (int64_t)num_seqs * P) >> 2;
      const int32_t cset = (int32_t)((c - (int64_t)num_seqs * P) & 3);
      const int32_t first = std::min(std::max(prefix_groups[2 * gi], 0), num_seqs - 1);
      const int32_t count =
          std::min(std::max(prefix_groups[2 * gi + 1], 0), std::min(num_seqs - first, 64 / G));
      tokens = -1;
      bool extra = false;  // a short member's private tile
      for (int32_t m = 16 * cset / G; m < std::min(count, (16 * cset + 15) / G + 1); ++m) {
        const int32_t L = L_of(first + m);
        const int32_t sh = shared_of(first + m, L);
        if (sh > 0) tokens = std::max<int64_t>(tokens, sh);
        extra = extra || (short_rule && pa::prefix_short(L, sh) && L > sh);
      }
      if (tokens > 0 && extra) tokens += 16;
    }
    return tokens;
  }, dispatch);
  return (int32_t)n;
}

int32_t paged_attention_multi_query_plan(const int32_t *context_lens,
                                         const int32_t *prefix_groups, int32_t num_groups,
                                         const int32_t *shared_lens, int32_t num_seqs,
                                         int32_t num_q_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t block_size,
                                         int32_t max_blocks_per_seq, int32_t max_query_len,
                                         int32_t max_context_len, int32_t kv_dtype,
                                         int32_t partition_size, int32_t *dispatch,
                                         int32_t capacity) {
  if (!known_pool_dtype(kv_dtype)) return PA_ERR_DTYPE;
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      max_blocks_per_seq <= 0 || max_query_len < 0 || max_context_len < 0 || num_groups < 0 ||
      num_groups > num_seqs || num_q_heads % num_kv_heads != 0)
    return PA_ERR_SHAPE;
  if (!is_pow2(block_size) || block_size > 1024) return PA_ERR_SHAPE;
  if ((int64_t)max_blocks_per_seq * block_size > kMaxTokensPerSeq) return PA_ERR_SHAPE;
  if (num_seqs == 0) return 0;
  const bool pfx = mq_prefix_path(kv_dtype, head_dim, num_q_heads, num_kv_heads, max_query_len,
                                  num_groups);
  const int32_t ng = pfx ? num_groups : 0;
  if (!context_lens || !dispatch || (ng > 0 && (!prefix_groups || !shared_lens)))
    return PA_ERR_NULL;
  int32_t ps = 0;
  const int32_t P = resolve_mq_partitions(num_seqs, num_q_heads, num_kv_heads, max_query_len,
                                          max_context_len, partition_size, &ps);
  if (P < 0) return P;
  const int64_t cap = (int64_t)max_blocks_per_seq * block_size;
  if (P <= 1) ps = (int32_t)cap;  // one partition spans any clamped context
  const int64_t ipg =
      ng > 0 ? pa::mq_prefix_items_per_group(max_query_len, num_q_heads / num_kv_heads) : 0;
  const int64_t n = (int64_t)num_seqs * P + ipg * ng;
  if (n >= (int64_t(1) << 31) || capacity < n) return PA_ERR_SHAPE;
  // the multi-query kernels' clamps and item bounds, as the device sort takes
  // them: a sequence item by its private positions in its partition, a
  // prefix item by its group's longest shared length
  auto L_of = [&](int32_t s) {
    return (int32_t)std::min<int64_t>(std::max(context_lens[s], 0), cap);
  };
  auto shared_of = [&](int32_t s, int32_t L) {
    return ng > 0 ? (std::min(std::max(shared_lens[s], 0), L) & ~15) : 0;
  };
  plan_longest_first(n, [&](int64_t c) -> int64_t {
    if (c < (int64_t)num_seqs * P) {
      const int32_t s = (int32_t)(c % num_seqs);
      const int32_t p = (P - 1) - (int32_t)(c / num_seqs);
      const int32_t L = L_of(s);
      const int32_t nparts = std::min((int32_t)(((int64_t)L + ps - 1) / ps), P);
      const int32_t sh = shared_of(s, L);
      if (p >= std::max(nparts, 1) || (sh > 0 && p < sh / ps)) return -1;
      return std::max<int64_t>(
          0, std::min<int64_t>(L, (int64_t)p * ps + ps) - std::max<int64_t>((int64_t)p * ps, sh));
    }
    const int64_t gi = (c - (int64_t)num_seqs * P) / ipg;
    const int32_t first = std::min(std::max(prefix_groups[2 * gi], 0), num_seqs - 1);
    const int32_t count = std::min(std::max(prefix_groups[2 * gi + 1], 0),
                                   std::min(num_seqs - first, pa::kMqPrefixMembers));
    int64_t longest = 0;
    for (int32_t m = 0; m < count; ++m)
      longest = std::max<int64_t>(longest, shared_of(first + m, L_of(first + m)));
    return longest > 0 ? longest : -1;
  }, dispatch);
  return (int32_t)n;
}

}  // extern "C"

namespace {

int32_t write_q8(const void *k, const void *v, const int32_t *slot_mapping, int32_t num_tokens,
                 void *k_cache, void *v_cache, int32_t num_blocks, int32_t block_size,
                 int32_t num_kv_heads, int32_t head_dim, int32_t src_dtype, int32_t kv_dtype,
                 float k_scale, float v_scale, void *stream) {
  if (!known_dtype(src_dtype)) return PA_ERR_DTYPE;
  if (num_tokens < 0 || num_blocks <= 0 || num_kv_heads <= 0 || !head_row_ok(head_dim, kv_dtype))
    return PA_ERR_SHAPE;
  if (!is_pow2(block_size) || block_size > 1024) return PA_ERR_SHAPE;
  if ((int64_t)num_blocks * block_size >= (int64_t(1) << 31)) return PA_ERR_SHAPE;
  if (!valid_scale(k_scale) || !valid_scale(v_scale)) return PA_ERR_SHAPE;
  if ((int64_t)num_kv_heads * head_dim / 4 > (int64_t)128 * 65535) return PA_ERR_SHAPE;
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache) return PA_ERR_NULL;
  // the rows are read four elements per load
  const uintptr_t quad = 4 * (uintptr_t)(src_dtype == PA_F32 ? 4 : 2);
  if (((uintptr_t)k | (uintptr_t)v) % quad != 0) return PA_ERR_SHAPE;
  if (pa::index_check_on()) {
    const int32_t st = pa::check_slots(slot_mapping, num_tokens, (int64_t)num_blocks * block_size,
                                       static_cast<hipStream_t>(stream));
    if (st != PA_OK) return st;
  }
  const hipError_t e = pa::launch_kv_cache_write_q8(
      k, v, slot_mapping, num_tokens, k_cache, v_cache, (int64_t)num_blocks * block_size,
      log2_exact(block_size), num_kv_heads, head_dim, src_dtype, kv_dtype, k_scale, v_scale,
      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int32_t kv_cache_write_fp8(const void *k, const void *v, const int32_t *slot_mapping,
                           int32_t num_tokens, void *k_cache, void *v_cache, int32_t num_blocks,
                           int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                           int32_t src_dtype, float k_scale, float v_scale, void *stream) {
  return write_q8(k, v, slot_mapping, num_tokens, k_cache, v_cache, num_blocks, block_size,
                  num_kv_heads, head_dim, src_dtype, PA_FP8_E4M3, k_scale, v_scale, stream);
}

int32_t kv_cache_write_int8(const void *k, const void *v, const int32_t *slot_mapping,
                            int32_t num_tokens, void *k_cache, void *v_cache, int32_t num_blocks,
                            int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                            int32_t src_dtype, float k_scale, float v_scale, void *stream) {
  return write_q8(k, v, slot_mapping, num_tokens, k_cache, v_cache, num_blocks, block_size,
                  num_kv_heads, head_dim, src_dtype, PA_INT8, k_scale, v_scale, stream);
}

}  // extern "C"

namespace {

// Multi-query attention over a pool of kv_dtype (dtype for a bf16 pool,
// PA_FP8_E4M3 or PA_INT8 with bf16 queries); the checks and launch shared by
// the entry points.
int32_t multi_query_impl(const void *q, const void *k_cache, const void *v_cache,
                         const int32_t *block_tables, const int32_t *context_lens,
                         const int32_t *query_start, float scale, float *out, int32_t num_seqs,
                         int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, int32_t num_blocks,
                         int32_t max_blocks_per_seq, int32_t max_query_len,
                         int32_t max_context_len, int32_t dtype, int32_t kv_dtype, float k_scale,
                         float v_scale, int32_t partition_size, void *workspace,
                         size_t workspace_bytes, void *stream, const int32_t *groups = nullptr,
                         int32_t num_groups = 0, const int32_t *shared_lens = nullptr,
                         const int32_t *dispatch = nullptr) {
  if (!known_dtype(dtype)) return PA_ERR_DTYPE;
  if (num_groups < 0 || num_groups > std::max(num_seqs, 0)) return PA_ERR_SHAPE;
  if (num_seqs < 0 || num_tokens < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      head_dim <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0 || max_query_len < 0 ||
      max_context_len < 0)
    return PA_ERR_SHAPE;
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size) return PA_ERR_SHAPE;
  if (!is_pow2(block_size) || block_size > 1024) return PA_ERR_SHAPE;
  if (num_q_heads % num_kv_heads != 0) return PA_ERR_SHAPE;
  if ((int64_t)num_blocks * block_size * num_kv_heads * head_dim >= (int64_t(1) << 40))
    return PA_ERR_SHAPE;
  if ((int64_t)max_blocks_per_seq * block_size > kMaxTokensPerSeq) return PA_ERR_SHAPE;
  if (!pa::multi_query_supported(dtype, head_dim)) return PA_ERR_UNSUPPORTED;
  if (is_q8(kv_dtype)) {
    // bf16 queries; both kernels (the decode walk for at most 64 (token,
    // head) rows per KV head at head_dim 128, the row-tile kernel otherwise)
    if (dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
    if (!valid_scale(k_scale) || !valid_scale(v_scale)) return PA_ERR_SHAPE;
  }
  const int64_t G = num_q_heads / num_kv_heads;
  const int64_t rows = (int64_t)max_query_len * G;
  const int64_t tiles = (rows + 63) / 64;
  int32_t ps = 0;
  const int32_t P = resolve_mq_partitions(num_seqs, num_q_heads, num_kv_heads, max_query_len,
                                          max_context_len, partition_size, &ps);
  if (P < 0) return P;
  if ((int64_t)num_seqs * num_kv_heads * tiles * P + 8 >= (int64_t(1) << 31)) return PA_ERR_SHAPE;
  if ((int64_t)num_tokens * num_q_heads * head_dim >= (int64_t(1) << 40)) return PA_ERR_SHAPE;
  if ((int64_t)num_tokens * num_q_heads >= (int64_t(1) << 31)) return PA_ERR_SHAPE;
  // the merge has one workgroup per (sequence, chunk token, head)
  if (P > 1 && (int64_t)num_seqs * max_query_len * num_q_heads >= (int64_t(1) << 31))
    return PA_ERR_SHAPE;
  if (num_seqs == 0 || num_tokens == 0 || max_query_len == 0) return PA_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start || !out)
    return PA_ERR_NULL;
  if (num_groups > 0 && (!groups || !shared_lens)) return PA_ERR_NULL;
  // the launch's items (the prefix items after the sequence items), times
  // the KV heads, index the grid in 32 bits
  if (num_groups > 0 &&
      ((int64_t)num_seqs * P + pa::mq_prefix_items_per_group(max_query_len, G) * num_groups) *
                  num_kv_heads + 8 >= (int64_t(1) << 31))
    return PA_ERR_SHAPE;
  float *ws_o = nullptr, *ws_ml = nullptr;
  const MultiQueryWorkspace w =
      multi_query_workspace(num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim,
                            max_query_len, P, num_groups);
  const int64_t slots = P + (num_groups > 0 ? 1 : 0);
  if (slots > 1) {
    if (!workspace || workspace_bytes < w.partials) return PA_ERR_WORKSPACE;
    ws_o = static_cast<float *>(workspace);
    ws_ml = ws_o + (size_t)num_tokens * num_q_heads * slots * head_dim;
  }
  pa::MultiQueryArgs a;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start = query_start;
  a.out = out;
  a.scale = scale;
  a.num_seqs = num_seqs;
  a.num_tokens = num_tokens;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.log2_block_size = log2_exact(block_size);
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_query_len = max_query_len;
  a.dtype = dtype;
  a.kv_dtype = kv_dtype;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.partition_size = ps;
  a.num_partitions = P;
  a.ws_o = ws_o;
  a.ws_ml = ws_ml;
  a.groups = groups;
  a.shared_lens = shared_lens;
  a.num_groups = num_groups;
  // a list the caller planned; else, with room for it, the longest-first
  // list sorted on the device; else the fixed order
  if (dispatch) {
    a.order = const_cast<int32_t *>(dispatch);
    a.order_ready = true;
  } else if (w.order > 0 && workspace && workspace_bytes >= w.partials + w.order) {
    a.order = reinterpret_cast<int32_t *>(static_cast<uint8_t *>(workspace) + w.partials);
  }
  if (pa::index_check_on()) {
    const hipStream_t st_stream = static_cast<hipStream_t>(stream);
    int32_t st = pa::check_tables(context_lens, block_tables, num_seqs, max_blocks_per_seq,
                                  a.log2_block_size, num_blocks, max_context_len, st_stream);
    if (st == PA_OK)
      st = pa::check_queries(context_lens, query_start, num_seqs, num_tokens, max_query_len,
                             st_stream);
    if (st == PA_OK && num_groups > 0)
      st = pa::check_prefix_groups(context_lens, block_tables, groups, num_groups, shared_lens,
                                   num_seqs, max_blocks_per_seq, a.log2_block_size,
                                   max_context_len, pa::kMqPrefixMembers, st_stream);
    if (st == PA_OK && dispatch)
      st = pa::check_dispatch(
          dispatch,
          (int32_t)((int64_t)num_seqs * P +
                    (num_groups > 0 ? pa::mq_prefix_items_per_group(max_query_len, G) : 0) *
                        num_groups),
          st_stream);
    if (st != PA_OK) return st;
  }
  const hipError_t e = pa::launch_multi_query(a, static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported) return PA_ERR_UNSUPPORTED;
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // namespace

namespace {

// The copy_blocks precondition on host copies of the pairs: every dst
// distinct and never a src, so the pairs commute and may run concurrently.
// Ids outside the pool (and src == dst) are skipped by the kernels and
// ignored here.  PA_OK, PA_ERR_ALIAS, or PA_ERR_SHAPE when the host is out
// of memory.
int32_t pairs_alias_status(const int32_t *host_pairs, int32_t num_pairs, int32_t num_blocks) {
  bool *is_dst = new (std::nothrow) bool[(size_t)num_blocks]();
  bool *is_src = new (std::nothrow) bool[(size_t)num_blocks]();
  int32_t status = PA_OK;
  if (!is_dst || !is_src) {
    status = PA_ERR_SHAPE;
  } else {
    for (int32_t i = 0; i < num_pairs && status == PA_OK; ++i) {
      const int32_t s = host_pairs[2 * i], d = host_pairs[2 * i + 1];
      if (s >= 0 && s < num_blocks && d >= 0 && d < num_blocks && s != d) {
        if (is_dst[d]) status = PA_ERR_ALIAS;
        is_dst[d] = true;
        is_src[s] = true;
      }
    }
    for (int32_t b = 0; b < num_blocks && status == PA_OK; ++b)
      if (is_dst[b] && is_src[b]) status = PA_ERR_ALIAS;
  }
  delete[] is_dst;
  delete[] is_src;
  return status;
}

}  // namespace

extern "C" {

int32_t paged_attention_multi_query(const void *q, const void *k_cache, const void *v_cache,
                                    const int32_t *block_tables, const int32_t *context_lens,
                                    const int32_t *query_start, float scale, float *out,
                                    int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                    int32_t num_blocks, int32_t max_blocks_per_seq,
                                    int32_t max_query_len, int32_t max_context_len,
                                    int32_t dtype, int32_t partition_size, void *workspace,
                                    size_t workspace_bytes, void *stream) {
  return multi_query_impl(q, k_cache, v_cache, block_tables, context_lens, query_start, scale,
                          out, num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim,
                          block_size, num_blocks, max_blocks_per_seq, max_query_len,
                          max_context_len, dtype, dtype, 1.f, 1.f, partition_size, workspace,
                          workspace_bytes, stream);
}

int32_t paged_attention_multi_query_fp8(const void *q, const void *k_cache, const void *v_cache,
                                        const int32_t *block_tables, const int32_t *context_lens,
                                        const int32_t *query_start, float scale, float k_scale,
                                        float v_scale, float *out, int32_t num_seqs,
                                        int32_t num_tokens, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                        int32_t num_blocks, int32_t max_blocks_per_seq,
                                        int32_t max_query_len, int32_t max_context_len,
                                        int32_t partition_size, void *workspace,
                                        size_t workspace_bytes, void *stream) {
  return multi_query_impl(q, k_cache, v_cache, block_tables, context_lens, query_start, scale,
                          out, num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim,
                          block_size, num_blocks, max_blocks_per_seq, max_query_len,
                          max_context_len, PA_BF16, PA_FP8_E4M3, k_scale, v_scale,
                          partition_size, workspace, workspace_bytes, stream);
}

int32_t paged_attention_multi_query_int8(const void *q, const void *k_cache, const void *v_cache,
                                         const int32_t *block_tables, const int32_t *context_lens,
                                         const int32_t *query_start, float scale, float k_scale,
                                         float v_scale, float *out, int32_t num_seqs,
                                         int32_t num_tokens, int32_t num_q_heads,
                                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                         int32_t num_blocks, int32_t max_blocks_per_seq,
                                         int32_t max_query_len, int32_t max_context_len,
                                         int32_t partition_size, void *workspace,
                                         size_t workspace_bytes, void *stream) {
  return multi_query_impl(q, k_cache, v_cache, block_tables, context_lens, query_start, scale,
                          out, num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim,
                          block_size, num_blocks, max_blocks_per_seq, max_query_len,
                          max_context_len, PA_BF16, PA_INT8, k_scale, v_scale,
                          partition_size, workspace, workspace_bytes, stream);
}

int32_t paged_attention_multi_query_prefix(
    const void *q, const void *k_cache, const void *v_cache, const int32_t *block_tables,
    const int32_t *context_lens, const int32_t *query_start, const int32_t *prefix_groups,
    int32_t num_groups, const int32_t *shared_lens, const int32_t *dispatch, float scale,
    float k_scale, float v_scale, float *out, int32_t num_seqs, int32_t num_tokens,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_query_len,
    int32_t max_context_len, int32_t kv_dtype, int32_t partition_size, void *workspace,
    size_t workspace_bytes, void *stream) {
  if (!known_pool_dtype(kv_dtype)) return PA_ERR_DTYPE;
  if (num_groups < 0) return PA_ERR_SHAPE;
  const bool pfx = mq_prefix_path(kv_dtype, head_dim, num_q_heads, num_kv_heads, max_query_len,
                                  num_groups);
  const bool q8 = is_q8(kv_dtype);
  return multi_query_impl(q, k_cache, v_cache, block_tables, context_lens, query_start, scale,
                          out, num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim,
                          block_size, num_blocks, max_blocks_per_seq, max_query_len,
                          max_context_len, q8 ? PA_BF16 : kv_dtype, kv_dtype,
                          q8 ? k_scale : 1.f, q8 ? v_scale : 1.f, partition_size, workspace,
                          workspace_bytes, stream, pfx ? prefix_groups : nullptr,
                          pfx ? num_groups : 0, pfx ? shared_lens : nullptr, dispatch);
}

size_t paged_attention_multi_query_prefix_workspace_size(
    int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t max_query_len, int32_t max_context_len, int32_t partition_size,
    int32_t num_groups, int32_t kv_dtype) {
  if (!mq_prefix_path(kv_dtype, head_dim, num_q_heads, num_kv_heads, max_query_len, num_groups))
    return paged_attention_multi_query_workspace_size(num_seqs, num_tokens, num_q_heads,
                                                      num_kv_heads, head_dim, max_query_len,
                                                      max_context_len, partition_size);
  if (num_tokens < 0 || num_seqs < 0 || num_groups > num_seqs) return 0;
  const int32_t P = paged_attention_multi_query_partitions(
      num_seqs, num_q_heads, num_kv_heads, max_query_len, max_context_len, partition_size);
  if (P < 1) return 0;
  const MultiQueryWorkspace w = multi_query_workspace(
      num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim, max_query_len, P, num_groups);
  return w.partials + w.order;
}

int32_t kv_cache_write(const void *k, const void *v, const int32_t *slot_mapping,
                       int32_t num_tokens, void *k_cache, void *v_cache, int32_t num_blocks,
                       int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                       int32_t dtype, void *stream) {
  if (!known_pool_dtype(dtype)) return PA_ERR_DTYPE;
  if (num_tokens < 0 || num_blocks <= 0 || num_kv_heads <= 0 || !head_row_ok(head_dim, dtype))
    return PA_ERR_SHAPE;
  if (!is_pow2(block_size) || block_size > 1024) return PA_ERR_SHAPE;
  if ((int64_t)num_blocks * block_size >= (int64_t(1) << 31)) return PA_ERR_SHAPE;
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache) return PA_ERR_NULL;
  const int64_t head_row_bytes = (int64_t)head_dim * elem_bytes(dtype);
  const int64_t row_bytes = (int64_t)num_kv_heads * head_row_bytes;
  // the grid covers a token's rows in stripes of 128 vectors
  if (row_bytes / 16 > (int64_t)128 * 65535) return PA_ERR_SHAPE;
  if (pa::index_check_on()) {
    const int32_t st = pa::check_slots(slot_mapping, num_tokens, (int64_t)num_blocks * block_size,
                                       static_cast<hipStream_t>(stream));
    if (st != PA_OK) return st;
  }
  const hipError_t e = pa::launch_kv_cache_write(
      k, v, slot_mapping, num_tokens, k_cache, v_cache, (int64_t)num_blocks * block_size,
      log2_exact(block_size), num_kv_heads, head_row_bytes, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

int32_t copy_blocks(const int32_t *src_dst_pairs, int32_t num_pairs, void *k_cache,
                    void *v_cache, int32_t num_blocks, int32_t block_size,
                    int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                    const int32_t *host_pairs, void *stream) {
  if (!known_pool_dtype(dtype)) return PA_ERR_DTYPE;
  if (num_pairs < 0 || num_blocks <= 0 || num_kv_heads <= 0 || !head_row_ok(head_dim, dtype))
    return PA_ERR_SHAPE;
  if (!is_pow2(block_size) || block_size > 1024) return PA_ERR_SHAPE;
  if ((int64_t)num_blocks * block_size >= (int64_t(1) << 31)) return PA_ERR_SHAPE;
  if (num_pairs == 0) return PA_OK;
  if (!src_dst_pairs || !k_cache || !v_cache) return PA_ERR_NULL;
  if (host_pairs) {
    const int32_t status = pairs_alias_status(host_pairs, num_pairs, num_blocks);
    if (status != PA_OK) return status;
  }
  if (pa::index_check_on()) {
    const int32_t st =
        pa::check_pairs(src_dst_pairs, num_pairs, num_blocks, static_cast<hipStream_t>(stream));
    if (st != PA_OK) return st;
  }
  const int64_t block_bytes = (int64_t)block_size * num_kv_heads * head_dim * elem_bytes(dtype);
  const hipError_t e = pa::launch_copy_blocks(src_dst_pairs, num_pairs, k_cache, v_cache,
                                              num_blocks, block_bytes,
                                              static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

int32_t kv_cache_append(const int32_t *src_dst_pairs, int32_t num_pairs, const void *k,
                        const void *v, const int32_t *slot_mapping, int32_t num_tokens,
                        void *k_cache, void *v_cache, int32_t num_blocks, int32_t block_size,
                        int32_t num_kv_heads, int32_t head_dim, int32_t src_dtype,
                        int32_t kv_dtype, float k_scale, float v_scale,
                        const int32_t *host_pairs, void *stream) {
  if (!known_pool_dtype(kv_dtype) || !known_pool_dtype(src_dtype)) return PA_ERR_DTYPE;
  const bool quantise = kv_dtype != src_dtype;
  // a quantising write takes fp32 or bfloat16 rows into an 8-bit pool
  if (quantise && ((kv_dtype != PA_FP8_E4M3 && kv_dtype != PA_INT8) ||
                   (src_dtype != PA_F32 && src_dtype != PA_BF16)))
    return PA_ERR_DTYPE;
  if (num_pairs < 0 || num_tokens < 0 || num_blocks <= 0 || num_kv_heads <= 0 ||
      !head_row_ok(head_dim, kv_dtype))
    return PA_ERR_SHAPE;
  if (!is_pow2(block_size) || block_size > 1024) return PA_ERR_SHAPE;
  if ((int64_t)num_blocks * block_size >= (int64_t(1) << 31)) return PA_ERR_SHAPE;
  if (quantise && !valid_scale(k_scale)) return PA_ERR_SHAPE;
  if (quantise && !valid_scale(v_scale)) return PA_ERR_SHAPE;
  const int64_t head_row_bytes = (int64_t)head_dim * elem_bytes(kv_dtype);
  const int64_t block_bytes = head_row_bytes * num_kv_heads * block_size;
  const int64_t per = 256 * 4 * 16;  // bytes a copy workgroup moves
  if ((int64_t)num_pairs * 2 * ((block_bytes + per - 1) / per) + num_tokens >=
      (int64_t(1) << 31))
    return PA_ERR_SHAPE;
  if (num_pairs == 0 && num_tokens == 0) return PA_OK;
  if (!k_cache || !v_cache || (num_pairs > 0 && !src_dst_pairs) ||
      (num_tokens > 0 && (!k || !v || !slot_mapping)))
    return PA_ERR_NULL;
  // source rows are read 16 bytes (stored bytes) or four elements
  // (quantised) per load
  const uintptr_t align = quantise ? 4 * (uintptr_t)elem_bytes(src_dtype) : 16;
  if (num_tokens > 0 && ((uintptr_t)k | (uintptr_t)v) % align != 0) return PA_ERR_SHAPE;
  if (host_pairs && num_pairs > 0) {
    const int32_t status = pairs_alias_status(host_pairs, num_pairs, num_blocks);
    if (status != PA_OK) return status;
  }
  if (pa::index_check_on()) {
    if (num_pairs > 0) {
      const int32_t st = pa::check_pairs(src_dst_pairs, num_pairs, num_blocks,
                                         static_cast<hipStream_t>(stream));
      if (st != PA_OK) return st;
    }
    if (num_tokens > 0) {
      const int32_t st = pa::check_slots(slot_mapping, num_tokens,
                                         (int64_t)num_blocks * block_size,
                                         static_cast<hipStream_t>(stream));
      if (st != PA_OK) return st;
    }
  }
  const hipError_t e = pa::launch_kv_cache_append(
      src_dst_pairs, num_pairs, k, v, slot_mapping, num_tokens, k_cache, v_cache, num_blocks,
      log2_exact(block_size), num_kv_heads, head_row_bytes, src_dtype, kv_dtype, k_scale,
      v_scale, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // extern "C"
