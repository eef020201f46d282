// KV-cache edits of a decode step, for gfx950:
//
//  * kv_cache_write: each new token's K and V rows (one head_dim row per KV
//    head; in the pool [blocks][kv_heads][block_size][head_dim] each goes to
//    its head's slab of the slot's block) are stored at its slot ("3.1" and "3.3" sections of the chenxutan.com vLLM
//    deep-dive: the generated token's K/V goes back into the cache, appended
//    into the sequence's current block);
//  * kv_cache_write_fp8 / _int8: the same store into an FP8 (E4M3) or INT8
//    pool, each element divided by its cache's fp32 scale and rounded to the
//    nearest E4M3 value or integer (the FP8/INT8 quantisation named in the
//    kernel layer of the devpress.csdn.net/amd walkthrough's architecture
//    figure; the formats and the per-cache scale are this library's choice,
//    as the pages give none);
//  * copy_blocks: whole physical blocks copied onto others, the copy-on-write
//    step taken before a forked sequence appends to a shared block
//    ("关键设计二：Copy-on-Write" section of the devpress.csdn.net/amd vLLM
//    walkthrough);
//  * kv_cache_append: a step's copies and its new tokens' writes in one
//    launch, with the result of copy_blocks followed by the write.
//
// Both move raw bits with 16-byte vector loads and stores (NaN payloads and
// signed zeros survive), and both skip indices outside the pool so a bad index
// can never touch memory outside it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace pa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWriteThreads = 128;
constexpr int kCopyThreads = 256;
constexpr int kCopyVecsPerThread = 4;

// grid.x = token, grid.y = stripe of the token's rows (hkv heads of head_vecs
// 16-byte vectors each, contiguous in the source).  Vector j belongs to head
// j / head_vecs and lands in that head's slab of the slot's block.  The row is
// loaded before the slot is read, so the two loads overlap.
__global__ __launch_bounds__(kWriteThreads) void kv_cache_write_kernel(
    const u32x4 *__restrict__ k, const u32x4 *__restrict__ v,
    const int32_t *__restrict__ slot_mapping, u32x4 *__restrict__ kc, u32x4 *__restrict__ vc,
    int64_t num_slots, int lgB, int hkv, int head_vecs) {
  const int64_t i = blockIdx.x;
  const int row_vecs = hkv * head_vecs;
  const int j = blockIdx.y * kWriteThreads + threadIdx.x;
  if (j >= row_vecs) return;
  const u32x4 kx = k[i * row_vecs + j];
  const u32x4 vx = v[i * row_vecs + j];
  const int32_t slot = slot_mapping[i];
  if (slot < 0 || slot >= num_slots) return;
  const int h = j / head_vecs;
  const int jj = j - h * head_vecs;
  const int64_t blk = slot >> lgB;
  const int off = slot & ((1 << lgB) - 1);
  const int64_t dst = (((blk * hkv + h) << lgB) + off) * head_vecs + jj;
  kc[dst] = kx;
  vc[dst] = vx;
}

// E4M3 code of y: saturate to +-448, nearest value, ties to the even
// mantissa; NaN gives the NaN code.  (OCP 8-bit floating point, E4M3: bias
// 7, subnormals m/8 * 2^-6, the all-ones code is NaN, no infinities.)
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7Fu;  // NaN
  if (a >= 0x43E00000u) return sign | 0x7Eu;  // 448 and above: saturate
  if (a >= 0x3C800000u) {                     // 2^-6 and above: normal
    const uint32_t keep = (a >> 20) & 7u;
    const uint32_t rem = a & 0xFFFFFu;
    uint32_t code = (((a >> 23) - 120u) << 3) | keep;
    if (rem > 0x80000u || (rem == 0x80000u && (keep & 1u))) ++code;  // may carry
    return sign | code;
  }
  // below 2^-6: multiples of 2^-9 (codes 0..8), rounded half to even
  return sign | (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.f);
}

// INT8 code of y: nearest integer, ties to even, clamped to [-127, 127];
// NaN gives 0.
__device__ __forceinline__ uint32_t int8_encode(float y) {
  if (y != y) return 0u;
  const float r = fminf(fmaxf(__builtin_rintf(y), -127.f), 127.f);
  return (uint32_t)(uint8_t)(int8_t)(int32_t)r;
}

template <int Q8>
__device__ __forceinline__ uint32_t encode8(float y) {
  if constexpr (Q8 == 1)
    return e4m3_encode(y);
  else
    return int8_encode(y);
}

template <typename T>
__device__ __forceinline__ float widen(T x);
template <>
__device__ __forceinline__ float widen<float>(float x) {
  return x;
}
template <>
__device__ __forceinline__ float widen<uint16_t>(uint16_t x) {
  return __uint_as_float((uint32_t)x << 16);
}

template <typename T>
struct Quad;  // four source elements, one vector load
template <>
struct Quad<float> {
  typedef float type __attribute__((ext_vector_type(4)));
};
template <>
struct Quad<uint16_t> {
  typedef uint16_t type __attribute__((ext_vector_type(4)));
};

// grid.x = token, grid.y = stripe of the token's 4-element words (hkv heads
// of head_words words each).  Word j of head h = j / head_words: its four
// elements are each divided by the cache's scale and encoded, and the four
// codes are stored as one 32-bit word in that head's slab of the slot's
// block.  Four elements per lane keep each lane's divide-and-encode chain
// short; the row is loaded before the slot is read.
template <typename T, int Q8>
__global__ __launch_bounds__(kWriteThreads) void kv_cache_write_q8_kernel(
    const typename Quad<T>::type *__restrict__ k, const typename Quad<T>::type *__restrict__ v,
    const int32_t *__restrict__ slot_mapping, uint32_t *__restrict__ kc,
    uint32_t *__restrict__ vc, float k_scale, float v_scale, int64_t num_slots, int lgB, int hkv,
    int head_words) {
  const int64_t i = blockIdx.x;
  const int row_words = hkv * head_words;
  const int j = blockIdx.y * kWriteThreads + threadIdx.x;
  if (j >= row_words) return;
  const typename Quad<T>::type kx = k[i * row_words + j];
  const typename Quad<T>::type vx = v[i * row_words + j];
  const int32_t slot = slot_mapping[i];
  if (slot < 0 || slot >= num_slots) return;
  const int h = j / head_words;
  const int jj = j - h * head_words;
  const int64_t blk = slot >> lgB;
  const int off = slot & ((1 << lgB) - 1);
  const int64_t dst = (((blk * hkv + h) << lgB) + off) * head_words + jj;
  uint32_t kw = 0, vw = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    kw |= encode8<Q8>(widen<T>(kx[b]) / k_scale) << (8 * b);
    vw |= encode8<Q8>(widen<T>(vx[b]) / v_scale) << (8 * b);
  }
  kc[dst] = kw;
  vc[dst] = vw;
}

// grid.x = pair, grid.y = stripe of kCopyThreads*kCopyVecsPerThread vectors of
// the block, grid.z = 0 for K, 1 for V.
__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(
    const int32_t *__restrict__ pairs, u32x4 *__restrict__ kc, u32x4 *__restrict__ vc,
    int32_t num_blocks, int64_t block_vecs) {
  const int32_t src = pairs[2 * blockIdx.x];
  const int32_t dst = pairs[2 * blockIdx.x + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks || src == dst) return;
  u32x4 *cache = blockIdx.z == 0 ? kc : vc;
  const u32x4 *s = cache + (int64_t)src * block_vecs;
  u32x4 *d = cache + (int64_t)dst * block_vecs;
  const int64_t base = (int64_t)blockIdx.y * kCopyThreads * kCopyVecsPerThread + threadIdx.x;
  u32x4 tmp[kCopyVecsPerThread];
#pragma unroll
  for (int u = 0; u < kCopyVecsPerThread; ++u) {
    const int64_t j = base + (int64_t)u * kCopyThreads;
    if (j < block_vecs) tmp[u] = s[j];
  }
#pragma unroll
  for (int u = 0; u < kCopyVecsPerThread; ++u) {
    const int64_t j = base + (int64_t)u * kCopyThreads;
    if (j < block_vecs) d[j] = tmp[u];
  }
}

// Both halves of a step's cache edits in one grid: workgroups [0, copy_wgs)
// copy stripes of the pairs' blocks (grid role of copy_blocks_kernel: pair,
// stripe, K or V), the rest write one new token each (its whole K and V
// rows).  The outcome is that of every copy followed by every write:
//  * a position of a copy's destination that a token writes is left to the
//    token (the copy skips it);
//  * a position of a copy's source that a token writes is copied by that
//    token's workgroup, which reads the old row before it writes the new one
//    (the copy skips it too), unless a token also writes that position of
//    the destination;
//  * every other position is copied by the copy workgroups and written by
//    no token.
// The skipped positions are found by scanning the slots (copy workgroups)
// and the pairs (token workgroups); pairs with an id outside the pool or
// src == dst are skipped here as in copy_blocks.  KIND 0 stores the source
// rows' bytes (16-byte vectors), KIND 1 / 2 quantise T rows to FP8 / INT8
// codes (four elements per 32-bit word, as kv_cache_write_q8_kernel).
constexpr int kAppendThreads = 256;
constexpr int kAppendVecsPerThread = 4;
constexpr int kMaxSkipWords = 32;  // a skip bit per position of a block (B <= 1024)

template <int KIND, typename T>
__global__ __launch_bounds__(kAppendThreads) void kv_cache_append_kernel(
    const int32_t *__restrict__ pairs, int num_pairs, int copy_wgs, int cstripes,
    const void *__restrict__ k, const void *__restrict__ v,
    const int32_t *__restrict__ slot_mapping, int num_tokens, u32x4 *__restrict__ kc,
    u32x4 *__restrict__ vc, int32_t num_blocks, int lgB, int hkv, int hv, float k_scale,
    float v_scale) {
  const int tid = threadIdx.x;
  const int B = 1 << lgB;
  const int64_t num_slots = (int64_t)num_blocks << lgB;
  const int bid = blockIdx.x;
  if (bid < copy_wgs) {
    __shared__ uint32_t skip[kMaxSkipWords];
    const int i = bid / (2 * cstripes);
    const int rem = bid - i * 2 * cstripes;
    const int z = rem / cstripes, y = rem - z * cstripes;
    const int32_t src = pairs[2 * i], dst = pairs[2 * i + 1];
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks || src == dst) return;
    if (tid < kMaxSkipWords) skip[tid] = 0u;
    __syncthreads();
    for (int t = tid; t < num_tokens; t += kAppendThreads) {
      const int32_t slot = slot_mapping[t];
      if (slot < 0 || slot >= num_slots) continue;
      const int32_t b = slot >> lgB;
      if (b == src || b == dst) {
        const int q = slot & (B - 1);
        atomicOr(&skip[q >> 5], 1u << (q & 31));
      }
    }
    __syncthreads();
    // the block: hkv << lgB rows of hv vectors, position q = row % B
    const int64_t block_vecs = ((int64_t)hkv << lgB) * hv;
    u32x4 *cache = z == 0 ? kc : vc;
    const u32x4 *sp = cache + (int64_t)src * block_vecs;
    u32x4 *dp = cache + (int64_t)dst * block_vecs;
    const int64_t base = (int64_t)y * kAppendThreads * kAppendVecsPerThread + tid;
    u32x4 tmp[kAppendVecsPerThread];
    bool keep[kAppendVecsPerThread];
#pragma unroll
    for (int u = 0; u < kAppendVecsPerThread; ++u) {
      const int64_t j = base + (int64_t)u * kAppendThreads;
      keep[u] = false;
      if (j < block_vecs) {
        const int q = (int)((j / hv) & (B - 1));
        keep[u] = !((skip[q >> 5] >> (q & 31)) & 1u);
      }
      if (keep[u]) tmp[u] = sp[j];
    }
#pragma unroll
    for (int u = 0; u < kAppendVecsPerThread; ++u)
      if (keep[u]) dp[base + (int64_t)u * kAppendThreads] = tmp[u];
    return;
  }

  const int t = bid - copy_wgs;
  const int32_t slot = slot_mapping[t];
  if (slot < 0 || slot >= num_slots) return;
  const int32_t blk = slot >> lgB;
  const int q = slot & (B - 1);
  const int lane = tid & 63;
  const int row_vecs = hkv * hv;  // 16-byte vectors of one position's rows
  // a position's row of head h in block b, in 16-byte vectors
  auto row_at = [&](int64_t b, int h) { return (((b * hkv + h) << lgB) + q) * hv; };

  // 1. pairs whose source is this token's block: copy the old rows of
  // position q to their destination first (each wave scans every pair, so
  // the waves meet the same matches in the same order)
  bool copied = false;
  for (int p0 = 0; p0 < num_pairs; p0 += 64) {
    const int p = p0 + lane;
    int32_t src = -1, dst = -1;
    if (p < num_pairs) {
      src = pairs[2 * p];
      dst = pairs[2 * p + 1];
    }
    const bool match = p < num_pairs && src == blk && dst >= 0 && dst < num_blocks && dst != src;
    uint64_t m = __builtin_amdgcn_ballot_w64(match);
    while (m) {
      const int l = (int)__builtin_ctzll(m);
      m &= m - 1;
      const int32_t d = __builtin_amdgcn_readlane(dst, l);
      // a token that writes position q of the destination wins over the copy
      const int64_t dslot = ((int64_t)d << lgB) + q;
      bool taken = false;
      for (int t0 = 0; t0 < num_tokens && !taken; t0 += 64) {
        const int tt = t0 + lane;
        taken = __builtin_amdgcn_ballot_w64(tt < num_tokens && slot_mapping[tt] == dslot) != 0;
      }
      if (taken) continue;
      copied = true;
      for (int j = tid; j < row_vecs; j += kAppendThreads) {
        const int h = j / hv, jj = j - h * hv;
        kc[row_at(d, h) + jj] = kc[row_at(blk, h) + jj];
        vc[row_at(d, h) + jj] = vc[row_at(blk, h) + jj];
      }
    }
  }
  // every old row is read before any thread overwrites it
  if (copied) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();

  // 2. the token's rows
  if constexpr (KIND == 0) {
    const u32x4 *ks = static_cast<const u32x4 *>(k) + (int64_t)t * row_vecs;
    const u32x4 *vs = static_cast<const u32x4 *>(v) + (int64_t)t * row_vecs;
    for (int j = tid; j < row_vecs; j += kAppendThreads) {
      const int h = j / hv, jj = j - h * hv;
      const u32x4 kx = ks[j], vx = vs[j];
      kc[row_at(blk, h) + jj] = kx;
      vc[row_at(blk, h) + jj] = vx;
    }
  } else {
    typedef typename Quad<T>::type Q;
    const int hw = 4 * hv;  // 32-bit code words per head row
    const Q *ks = static_cast<const Q *>(k) + (int64_t)t * hkv * hw;
    const Q *vs = static_cast<const Q *>(v) + (int64_t)t * hkv * hw;
    uint32_t *kw32 = reinterpret_cast<uint32_t *>(kc);
    uint32_t *vw32 = reinterpret_cast<uint32_t *>(vc);
    for (int j = tid; j < hkv * hw; j += kAppendThreads) {
      const int h = j / hw, jj = j - h * hw;
      const Q kx = ks[j], vx = vs[j];
      uint32_t kw = 0, vw = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        kw |= encode8<KIND>(widen<T>(kx[b]) / k_scale) << (8 * b);
        vw |= encode8<KIND>(widen<T>(vx[b]) / v_scale) << (8 * b);
      }
      kw32[4 * row_at(blk, h) + jj] = kw;
      vw32[4 * row_at(blk, h) + jj] = vw;
    }
  }
}

}  // namespace

hipError_t launch_kv_cache_write(const void *k, const void *v, const int32_t *slot_mapping,
                                 int32_t num_tokens, void *k_cache, void *v_cache,
                                 int64_t num_slots, int32_t log2_block_size, int32_t num_kv_heads,
                                 int64_t head_row_bytes, hipStream_t stream) {
  if (num_tokens <= 0) return hipSuccess;
  const int64_t head_vecs = head_row_bytes / 16;
  const int64_t row_vecs = head_vecs * num_kv_heads;
  const int64_t stripes = (row_vecs + kWriteThreads - 1) / kWriteThreads;
  hipLaunchKernelGGL(kv_cache_write_kernel, dim3((uint32_t)num_tokens, (uint32_t)stripes),
                     dim3(kWriteThreads), 0, stream, static_cast<const u32x4 *>(k),
                     static_cast<const u32x4 *>(v), slot_mapping, static_cast<u32x4 *>(k_cache),
                     static_cast<u32x4 *>(v_cache), num_slots, (int)log2_block_size,
                     (int)num_kv_heads, (int)head_vecs);
  return hipGetLastError();
}

namespace {

template <typename T, int Q8>
void launch_q8(const void *k, const void *v, const int32_t *slot_mapping, int32_t num_tokens,
               void *k_cache, void *v_cache, int64_t num_slots, int32_t log2_block_size,
               int32_t num_kv_heads, int head_words, float k_scale, float v_scale,
               hipStream_t stream) {
  typedef typename Quad<T>::type Q;
  const int64_t row_words = (int64_t)head_words * num_kv_heads;
  const int64_t stripes = (row_words + kWriteThreads - 1) / kWriteThreads;
  hipLaunchKernelGGL((kv_cache_write_q8_kernel<T, Q8>),
                     dim3((uint32_t)num_tokens, (uint32_t)stripes), dim3(kWriteThreads), 0,
                     stream, static_cast<const Q *>(k), static_cast<const Q *>(v), slot_mapping,
                     static_cast<uint32_t *>(k_cache), static_cast<uint32_t *>(v_cache), k_scale,
                     v_scale, num_slots, (int)log2_block_size, (int)num_kv_heads, head_words);
}

}  // namespace

hipError_t launch_kv_cache_write_q8(const void *k, const void *v, const int32_t *slot_mapping,
                                    int32_t num_tokens, void *k_cache, void *v_cache,
                                    int64_t num_slots, int32_t log2_block_size,
                                    int32_t num_kv_heads, int32_t head_dim, int32_t src_dtype,
                                    int32_t kv_dtype, float k_scale, float v_scale,
                                    hipStream_t stream) {
  if (num_tokens <= 0) return hipSuccess;
  const int hv = head_dim / 4;  // 4-element words per head row
  if (src_dtype == 0) {
    if (kv_dtype == 2)
      launch_q8<float, 1>(k, v, slot_mapping, num_tokens, k_cache, v_cache, num_slots,
                          log2_block_size, num_kv_heads, hv, k_scale, v_scale, stream);
    else
      launch_q8<float, 2>(k, v, slot_mapping, num_tokens, k_cache, v_cache, num_slots,
                          log2_block_size, num_kv_heads, hv, k_scale, v_scale, stream);
  } else {
    if (kv_dtype == 2)
      launch_q8<uint16_t, 1>(k, v, slot_mapping, num_tokens, k_cache, v_cache, num_slots,
                             log2_block_size, num_kv_heads, hv, k_scale, v_scale, stream);
    else
      launch_q8<uint16_t, 2>(k, v, slot_mapping, num_tokens, k_cache, v_cache, num_slots,
                             log2_block_size, num_kv_heads, hv, k_scale, v_scale, stream);
  }
  return hipGetLastError();
}

hipError_t launch_copy_blocks(const int32_t *pairs, int32_t num_pairs, void *k_cache,
                              void *v_cache, int32_t num_blocks, int64_t block_bytes,
                              hipStream_t stream) {
  if (num_pairs <= 0) return hipSuccess;
  const int64_t block_vecs = block_bytes / 16;
  const int64_t per = (int64_t)kCopyThreads * kCopyVecsPerThread;
  const int64_t stripes = (block_vecs + per - 1) / per;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((uint32_t)num_pairs, (uint32_t)stripes, 2),
                     dim3(kCopyThreads), 0, stream, pairs, static_cast<u32x4 *>(k_cache),
                     static_cast<u32x4 *>(v_cache), num_blocks, block_vecs);
  return hipGetLastError();
}

hipError_t launch_kv_cache_append(const int32_t *pairs, int32_t num_pairs, const void *k,
                                  const void *v, const int32_t *slot_mapping, int32_t num_tokens,
                                  void *k_cache, void *v_cache, int32_t num_blocks,
                                  int32_t log2_block_size, int32_t num_kv_heads,
                                  int64_t head_row_bytes, int32_t src_dtype, int32_t kv_dtype,
                                  float k_scale, float v_scale, hipStream_t stream) {
  const int hv = (int)(head_row_bytes / 16);
  const int64_t block_vecs = ((int64_t)num_kv_heads << log2_block_size) * hv;
  const int64_t per = (int64_t)kAppendThreads * kAppendVecsPerThread;
  const int cstripes = (int)((block_vecs + per - 1) / per);
  const int copy_wgs = num_pairs * 2 * cstripes;
  const int64_t grid = (int64_t)copy_wgs + num_tokens;
  if (grid <= 0) return hipSuccess;
  u32x4 *kc = static_cast<u32x4 *>(k_cache), *vc = static_cast<u32x4 *>(v_cache);
#define PA_APPEND(KIND, T)                                                                    \
  hipLaunchKernelGGL((kv_cache_append_kernel<KIND, T>), dim3((uint32_t)grid),                 \
                     dim3(kAppendThreads), 0, stream, pairs, num_pairs, copy_wgs, cstripes, k, \
                     v, slot_mapping, num_tokens, kc, vc, num_blocks, (int)log2_block_size,    \
                     (int)num_kv_heads, hv, k_scale, v_scale)
  if (kv_dtype == src_dtype)
    PA_APPEND(0, uint16_t);
  else if (kv_dtype == 2 && src_dtype == 0)
    PA_APPEND(1, float);
  else if (kv_dtype == 2)
    PA_APPEND(1, uint16_t);
  else if (src_dtype == 0)
    PA_APPEND(2, float);
  else
    PA_APPEND(2, uint16_t);
#undef PA_APPEND
  return hipGetLastError();
}

}  // namespace pa
