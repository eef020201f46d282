// PagedAttention decode on the matrix cores of gfx950, for head_dim 128 and
// a GQA group of 4 or 8 query heads per KV head, over bfloat16, FP8 (E4M3)
// or INT8 pools; also causal multi-query attention for chunks of at most 64
// (token, head) rows per KV head.
//
// The operation is the one of decode.hip (the "核心代码拆解" section of the
// devpress.csdn.net/amd vLLM walkthrough: table lookup per logical block, scaled
// q.k, softmax, weighted sum of V).  With G >= 4 query heads sharing a KV head,
// every K/V row meets G queries, and on the vector ALU those G multiply-adds per
// element are what bounds the kernel; here both products run on MFMA:
//
//  * q.K: v_mfma_f32_16x16x32_bf16.  A = 16 K rows of a 16-token tile (lane
//    n = lane%16 loads token n; lane group g = lane/16 holds its share of the
//    elements, see Tile), B = the query rows over the 16 columns (column n
//    holds query n % G, or row n of a multi-query chunk).  Products of
//    bfloat16 values are exact and accumulate in fp32; 8-bit codes are
//    widened exactly to bfloat16 first.  The result gives lane (g, n) the
//    scores of column n with tokens 4g .. 4g+3 of the tile.
//  * p.V: the same instruction over pairs of tiles, O^T += V^T P^T (see
//    MfmaDecode::pv_pair): the probabilities enter as a bfloat16 pair hi + lo
//    (about 16 significant bits), V^T comes from the wave's LDS slice through
//    gfx950's transposing LDS reads, and every accumulator of a lane belongs
//    to its own column, so the online softmax needs two cross-lane max steps
//    per tile and nothing else.
//  * A running maximum is raised only when a tile's maximum exceeds it by
//    more than 8 (log2 units), so accumulators are rarely rescaled;
//    probabilities stay below 2^8 and the result is the same ratio of sums.
//
// Work split, tiles, partitions and the merge of partition partials are those
// of decode.hip: one workgroup of 4 waves per (sequence, KV head, partition),
// 16-token tiles round-robin over the waves, double-buffered in registers.
// Accumulation order depends only on logical token positions, so results are
// bitwise reproducible and invariant under a relabelling of physical blocks.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <climits>
#include <type_traits>

#include "internal.h"

namespace pa {
namespace {

constexpr int kD = 128;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 16;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kSlack = 8.f;  // allowed growth of scores over the running max (log2)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float neg_inf() { return -__builtin_huge_valf(); }

// Buffer descriptor over `bytes` bytes from `base` (raw buffer, no stride):
// loads at offsets past the end return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           0x00020000);
}
// Cache policies of a buffer load: normal, or non-temporal (streamed once).
constexpr int kCacheNormal = 0;
constexpr int kCacheStream = 2;
template <int POLICY>
__device__ __forceinline__ u32x4 buffer_load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, POLICY));
}


typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// bfloat16 bits of a (low half) and b (high half), rounded to nearest even:
// one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t bf16x2_bits(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// K rows are fetched 16 bytes per lane: for bfloat16, lane group g takes
// elements 32s + 8g .. +7 of k-step s (s = 0..3); for FP8 a 16-byte load
// holds two k-steps, so lane group g takes elements 16(4i + g) .. +15 in load
// i (i = 0, 1), giving k-step 2i + u its elements 16(4i + g) + 8u .. +7.  The
// dot product sums over all 128 elements either way; q's operand is loaded
// with the same assignment.  Each load instruction then covers 64
// contiguous bytes of every token row it touches.
template <bool FP8>
struct Tile {
  u32x4 k[FP8 ? 2 : 4];  // token n of the tile (see above)
  // V, 16 bytes per lane and load (see v_token / v_elem): bfloat16, token
  // 4g + j of the tile, elements 8n .. 8n+7 (j = 0..3); 8-bit codes, token
  // 8j + lane / 8, elements 16 (lane % 8) .. +15 (j = 0, 1)
  u32x4 v[FP8 ? 2 : 4];
};

// First element of lane group g's part of K load i (see Tile).
template <bool FP8>
__device__ __forceinline__ int k_load_elem(int g, int i) {
  return FP8 ? 16 * (4 * i + g) : 32 * i + 8 * g;
}
// First element of lane group g's part of k-step s.
template <bool FP8>
__device__ __forceinline__ int k_step_elem(int g, int s) {
  return FP8 ? 16 * (4 * (s >> 1) + g) + 8 * (s & 1) : 32 * s + 8 * g;
}

// Four signed 8-bit codes (one dword) to fp32 (exact).
__device__ __forceinline__ void i8x4_to_f32(uint32_t w, float (&f)[4]) {
#pragma unroll
  for (int b = 0; b < 4; ++b) f[b] = (float)((int32_t)(w << (24 - 8 * b)) >> 24);
}

// Eight 8-bit codes to the bfloat16 MFMA operand, exactly (an E4M3 value has
// at most 4 significant bits and an INT8 code at most 7).  E4M3: gfx950's
// scaled conversion with scale 1 turns the two codes of one 16-bit half into
// two bfloat16, the low byte into the low half (OCP E4M3, as the hardware's
// other FP8 conversions).  INT8: widened to fp32, whose high halves are the
// bfloat16 values, paired with one byte permute.
template <int Q8>
__device__ __forceinline__ bf16x8 codes8_to_bf16(u32x2 w) {
  u32x4 r;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if constexpr (Q8 == 1) {
      r[2 * h] = __builtin_bit_cast(uint32_t,
                                    __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[h], 1.f, false));
      r[2 * h + 1] = __builtin_bit_cast(
          uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[h], 1.f, true));
    } else {
      float f[4];
      i8x4_to_f32(w[h], f);
      // (f0 >> 16) | (f1 & 0xffff0000): bytes 2, 3 of f0, then bytes 2, 3 of f1
      r[2 * h] = __builtin_amdgcn_perm(__float_as_uint(f[1]), __float_as_uint(f[0]), 0x07060302u);
      r[2 * h + 1] =
          __builtin_amdgcn_perm(__float_as_uint(f[3]), __float_as_uint(f[2]), 0x07060302u);
    }
  }
  return __builtin_bit_cast(bf16x8, r);
}

// Q8: the pool's element kind -- 0 bfloat16, 1 FP8 (E4M3), 2 INT8 (signed
// codes); the two 8-bit kinds share every load and differ only in widening.
template <int G, bool SMALLB, int Q8>
struct MfmaDecode {
  static constexpr bool FP8 = Q8 != 0;  // one byte per element
  using KV = typename std::conditional<FP8, uint8_t, uint16_t>::type;
  using TileT = Tile<FP8>;
  static constexpr int kElem = FP8 ? 1 : 2;  // bytes per element
  static constexpr int kKLoads = FP8 ? 2 : 4;
  static constexpr int kVLoads = FP8 ? 2 : 4;
  // tile token and first element of lane (g, n)'s V chunk j
  static __device__ __forceinline__ int v_token(int j, int g, int n) {
    return FP8 ? 8 * j + 2 * g + n / 8 : 4 * g + j;
  }
  static __device__ __forceinline__ int v_elem(int g, int n) { return FP8 ? 16 * (n % 8) : 8 * n; }
  // LDS row of tile token t in slot `slot` of the pair (see below)
  static __device__ __forceinline__ int v_row(int slot, int t) {
    return 8 * (t / 4) + 4 * slot + t % 4;
  }
  // the A operand of k-step s
  static __device__ __forceinline__ bf16x8 k_operand(const TileT &T, int s) {
    if constexpr (FP8) {
      const u32x4 &w = T.k[s >> 1];
      return codes8_to_bf16<Q8>((s & 1) ? u32x2{w[2], w[3]} : u32x2{w[0], w[1]});
    } else {
      return __builtin_bit_cast(bf16x8, T.k[s]);
    }
  }

  // Issue the loads of the tile starting at token cs.  Rows of tokens at or
  // past t1 are not read (their registers are zero) when MASK is set.
  template <bool MASK>
  static __device__ __forceinline__ void load(TileT &T, const KV *__restrict__ kc,
                                              const KV *__restrict__ vc,
                                              const int32_t *__restrict__ tbl, int ent,
                                              bool stream_v, int cs, int t1,
                                              int lgB, int nb, int g, int n, int row_elems,
                                              int head_off, int64_t block_elems) {
    const int bm1 = (1 << lgB) - 1;
    if constexpr (!SMALLB) {
      // a 16-aligned tile lies inside one block, whose id the caller read
      // ahead of time (ent); its rows are read through buffer descriptors
      // spanning the block (reads past it return zeros)
      const uint32_t pid = min((uint32_t)ent, (uint32_t)(nb - 1));
      const uint32_t bbytes = (uint32_t)(block_elems * kElem);
      const auto rk = block_rsrc(kc + (int64_t)pid * block_elems, bbytes);
      const auto rv = block_rsrc(vc + (int64_t)pid * block_elems, bbytes);
      const int o = cs & bm1;
      const uint32_t krow = (uint32_t)(((o + n) * row_elems + head_off) * kElem);
      const bool okk = !MASK || cs + n < t1;
      // bfloat16 K rows follow the V hint; 8-bit K rows always use ordinary
      // loads (streaming them lost 9-10% on the FP8 pools, where each load
      // instruction covers half of a row's 128 bytes)
      if (!FP8 && stream_v) {
#pragma unroll
        for (int i = 0; i < kKLoads; ++i)
          T.k[i] = okk ? buffer_load<kCacheStream>(rk, krow + k_load_elem<FP8>(g, i) * kElem)
                       : u32x4{0, 0, 0, 0};
      } else {
#pragma unroll
        for (int i = 0; i < kKLoads; ++i)
          T.k[i] = okk ? buffer_load<kCacheNormal>(rk, krow + k_load_elem<FP8>(g, i) * kElem)
                       : u32x4{0, 0, 0, 0};
      }
      uint32_t voff[kVLoads];
      bool ok[kVLoads];
#pragma unroll
      for (int j = 0; j < kVLoads; ++j) {
        const int t = v_token(j, g, n);
        voff[j] = (uint32_t)(((o + t) * row_elems + head_off + v_elem(g, n)) * kElem);
        ok[j] = !MASK || cs + t < t1;
      }
      if (stream_v) {
#pragma unroll
        for (int j = 0; j < kVLoads; ++j)
          T.v[j] = ok[j] ? buffer_load<kCacheStream>(rv, voff[j]) : u32x4{0, 0, 0, 0};
      } else {
#pragma unroll
        for (int j = 0; j < kVLoads; ++j)
          T.v[j] = ok[j] ? buffer_load<kCacheNormal>(rv, voff[j]) : u32x4{0, 0, 0, 0};
      }
    } else {
      // blocks shorter than a tile: each token row looks up its own block
      const int tk = cs + n;
      if (!MASK || tk < t1) {
        const uint32_t pid = min((uint32_t)tbl[tk >> lgB], (uint32_t)(nb - 1));
        const KV *krow = kc + (int64_t)pid * block_elems + head_off + (tk & bm1) * row_elems;
#pragma unroll
        for (int i = 0; i < kKLoads; ++i)
          T.k[i] = *reinterpret_cast<const u32x4 *>(krow + k_load_elem<FP8>(g, i));
      } else {
#pragma unroll
        for (int i = 0; i < kKLoads; ++i) T.k[i] = u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int j = 0; j < kVLoads; ++j) {
        const int tv = cs + v_token(j, g, n);
        if (!MASK || tv < t1) {
          const uint32_t pid = min((uint32_t)tbl[tv >> lgB], (uint32_t)(nb - 1));
          T.v[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(
              vc + (int64_t)pid * block_elems + head_off + (tv & bm1) * row_elems +
              v_elem(g, n)));
        } else {
          T.v[j] = u32x4{0, 0, 0, 0};
        }
      }
    }
    // keep these loads ahead of the computation that follows them
    __builtin_amdgcn_sched_barrier(0);
  }

  // p.V runs on v_mfma_f32_16x16x32_bf16 over pairs of tiles (32 tokens per
  // k-step): O^T += V^T P^T.  B = the probabilities as the q.K product left
  // them (lane (g, n): column n, tokens 4g .. 4g+3 of each tile of the pair),
  // as a bfloat16 pair hi + lo (about 16 significant bits); A = the same
  // tokens of V for 16 head_dim elements.  V rows are staged in the wave's
  // LDS slice, 32 rows in the order row(slot, t) = 8 (t / 4) + 4 slot + t % 4
  // (slot = tile of the pair), so that the transposing LDS reads of gfx950
  // deliver V^T directly: for bfloat16 two ds_read_b64_tr_b16 (rows
  // 8g .. 8g+3 and 8g+4 .. 8g+7, lane n receiving element 16 b + n of each),
  // for 8-bit codes one ds_read_b64_tr_b8 (rows 8g .. 8g+7), widened exactly
  // to bfloat16.  The result leaves lane (g, n) with column n, elements
  // 16 b + 4 g + i: all of a lane's accumulators belong to its own column.
  static constexpr int kVRow = kD + 16;  // LDS row (elements); padded against bank conflicts
  static constexpr int kSliceBytes = 32 * kVRow * kElem;

  static __device__ __forceinline__ void stage_v(const TileT &T, KV *slice, int slot, int g,
                                                 int n) {
#pragma unroll
    for (int j = 0; j < kVLoads; ++j)
      *reinterpret_cast<u32x4 *>(slice + v_row(slot, v_token(j, g, n)) * kVRow + v_elem(g, n)) =
          T.v[j];
  }
  static __device__ __forceinline__ void zero_v(KV *slice, int slot, int g, int n) {
#pragma unroll
    for (int j = 0; j < kVLoads; ++j)
      *reinterpret_cast<u32x4 *>(slice + v_row(slot, v_token(j, g, n)) * kVRow + v_elem(g, n)) =
          u32x4{0, 0, 0, 0};
  }
  static __device__ __forceinline__ bf16x8 v_operand(const KV *slice, int b, int g, int n) {
    typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    if constexpr (FP8) {
      const KV *pa = slice + (8 * g + n / 2) * kVRow + 16 * b + 8 * (n % 2);
      const i32x2 w = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2 *)(pa));
      return codes8_to_bf16<Q8>(__builtin_bit_cast(u32x2, w));
    } else {
      const KV *pa = slice + (8 * g + n / 4) * kVRow + 16 * b + 4 * (n % 4);
      const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                     (lds_i16x4 *)(pa)));
      const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                     (lds_i16x4 *)(pa + 4 * kVRow)));
      return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
    }
  }

  // acc[c][b] += V^T P^T for the staged pair, for each of the NC column sets
  // c; p0: the first tile's probabilities, p1: the second's (zeros when the
  // pair is incomplete).  The V^T operands are read once for all sets.
  template <int NC>
  static __device__ __forceinline__ void pv_pair(const KV *slice, const float (&p0)[NC][4],
                                                 const float (&p1)[NC][4], f32x4 (&acc)[NC][8],
                                                 int g, int n) {
    bf16x8 phi[NC], plo[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const float a = h < 2 ? p0[c][2 * h] : p1[c][2 * h - 4];
        const float b = h < 2 ? p0[c][2 * h + 1] : p1[c][2 * h - 3];
        hw[h] = bf16x2_bits(a, b);
        lw[h] = bf16x2_bits(a - __uint_as_float(hw[h] << 16),
                            b - __uint_as_float(hw[h] & 0xFFFF0000u));
      }
      phi[c] = __builtin_bit_cast(bf16x8, u32x4{hw[0], hw[1], hw[2], hw[3]});
      plo[c] = __builtin_bit_cast(bf16x8, u32x4{lw[0], lw[1], lw[2], lw[3]});
    }
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bf16x8 a = v_operand(slice, b, g, n);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        acc[c][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, phi[c], acc[c][b], 0, 0, 0);
        acc[c][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, plo[c], acc[c][b], 0, 0, 0);
      }
    }
  }

  // Fold one tile into the running state of NC column sets: q.K (the K
  // operand read once for all sets), the online softmax (m: this lane's
  // column's running maximum in log2 units, shared by the four lane groups;
  // lsum: the lane's own tokens), the V rows staged into slot `slot` of the
  // pair; with the pair complete, p.V.  p0 keeps the first tile's
  // probabilities until then (and is rescaled with the accumulators).
  // cpos: this lane's column's last attended position (multi-query: a
  // causal mask per column; decode passes INT_MAX).
  template <bool MASK, int NC>
  static __device__ __forceinline__ void compute(const TileT &T, const bf16x8 (&qb)[NC][4],
                                                 f32x4 (&acc)[NC][8], float (&m)[NC],
                                                 float (&lsum)[NC], float (&p0)[NC][4],
                                                 int &slot, KV *slice, int cs, int t1, int g,
                                                 int n, float sl2, const int (&cpos)[NC]) {
    f32x4 sc[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) sc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bf16x8 a = k_operand(T, s);
#pragma unroll
      for (int c = 0; c < NC; ++c)
        sc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[c][s], sc[c], 0, 0, 0);
    }
    float p[NC][4];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float x[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = cs + 4 * g + j;
        x[j] = ((!MASK || t < t1) && t <= cpos[c]) ? sc[c][j] * sl2 : neg_inf();
      }
      float cm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      cm = fmaxf(cm, __shfl_xor(cm, 16));
      cm = fmaxf(cm, __shfl_xor(cm, 32));
      if (cm > m[c] + kSlack) {  // false while both are -inf
        const float alpha = __builtin_amdgcn_exp2f(m[c] - cm);  // 0 when m was -inf
        lsum[c] *= alpha;
#pragma unroll
        for (int b = 0; b < 8; ++b) acc[c][b] *= alpha;
#pragma unroll
        for (int j = 0; j < 4; ++j) p0[c][j] *= alpha;
        m[c] = cm;
      }
      const float mu = (m[c] == neg_inf()) ? 0.f : m[c];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        p[c][j] = __builtin_amdgcn_exp2f(x[j] - mu);
        lsum[c] += p[c][j];
      }
    }
    stage_v(T, slice, slot, g, n);
    if (slot == 0) {
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) p0[c][j] = p[c][j];
      slot = 1;
    } else {
      pv_pair<NC>(slice, p0, p, acc, g, n);
      slot = 0;
    }
  }

  // Completes a half-filled pair with a zero tile.
  template <int NC>
  static __device__ __forceinline__ void flush(const float (&p0)[NC][4], int slot, KV *slice,
                                               f32x4 (&acc)[NC][8], int g, int n) {
    if (slot == 1) {
      zero_v(slice, 1, g, n);
      float z[NC][4];
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) z[c][j] = 0.f;
      pv_pair<NC>(slice, p0, z, acc, g, n);
    }
  }
};

// Multi-query mode (MQ, G = 16 columns): the same walk for a few query tokens
// per sequence (at most 64 (token, head) rows per KV head, in sets of 16),
// column n of set c being row R = 16 c + n of the chunk: token R / gh and
// head R % gh of the KV head's gh query heads.  The chunk is the sequence's
// last nq positions and row R attends positions up to L - nq + R / gh (the
// causal mask of multi_query.hip).  Each wave carries NC column sets, which
// share every K/V load, the V staging and the V^T operand reads.
//
// Shared-prefix mode (PFX, decode only): besides the (sequence, partition)
// items, the launch has items for prefix groups -- a group is a run of
// `count` consecutive sequences from `first` whose table rows name the same
// blocks below their shared lengths shared_lens[s].  Item (group, column set
// c, KV head) reads the group's shared tiles once for 16 (member, query head)
// pairs: column n is R = 16 c + n (member R / G, head R % G; at most 64 / G
// members, so at most four sets), walked like a sequence item (tiles
// round-robin over the four waves) through the table row of the set's
// member with the longest shared length; column R attends positions below
// its member's shared length.  A sequence's own items then cover only
// [shared length, L), and every member's prefix partial and private
// partials meet in the merge kernel.  Shared lengths are used rounded down
// to whole 16-token tiles, so a private walk still starts on a tile
// boundary.
template <int G, bool SMALLB, int Q8, bool MQ, int NC = 1, bool PFX = false>
__global__ __launch_bounds__(kThreads, NC == 1 ? 3 : 2) void paged_decode_mfma_kernel(
    const uint16_t *__restrict__ q,
    const typename MfmaDecode<G, SMALLB, Q8>::KV *__restrict__ kc,
    const typename MfmaDecode<G, SMALLB, Q8>::KV *__restrict__ vc,
    const int32_t *__restrict__ block_tables, const int32_t *__restrict__ context_lens,
    float *__restrict__ out, float *__restrict__ ws_o, float *__restrict__ ws_ml, float sl2,
    float v_scale, int num_seqs, int hkv, int lgB, int nb, int mb, int ps, int P,
    const int32_t *__restrict__ query_start, int num_tokens, int gh, int max_q, int csets,
    const int32_t *__restrict__ order, const int32_t *__restrict__ groups,
    const int32_t *__restrict__ shared_lens, int slots, int ipg, int ngroups) {
  using K = MfmaDecode<G, SMALLB, Q8>;
  using TileT = typename K::TileT;
  constexpr bool FP8 = K::FP8;

  int id = blockIdx.x;
  // multi-query with more than 16 * NC rows per KV head: workgroup group cg
  // takes column sets NC cg .. NC cg + NC - 1.  The groups of one item are 8
  // workgroups apart, so they run on the same XCD (workgroup b runs on XCD
  // b % 8) and the later groups' K/V reads hit its L2.
  int cgroup = 0;
  if constexpr (MQ) {
    const int cgroups = (csets + NC - 1) / NC;
    const int t = id / 8;
    cgroup = t % cgroups;
    id = (t / cgroups) * 8 + id % 8;
    if (id >= (num_seqs * P + (PFX ? ipg * ngroups : 0)) * hkv) return;
  }
  // work item: KV head fastest, then (sequence, partition) from the
  // longest-first list or the fixed order (as in decode.hip); with PFX, the
  // prefix-group items follow the num_seqs * P sequence items
  const int kvh = id % hkv;
  const int item = order ? order[id / hkv] : id / hkv;
  // listed as empty (past the sequence's end), or not an item of this launch
  // (a list the caller planned is trusted only this far)
  const int nitems = MQ ? num_seqs * P + (PFX ? ipg * ngroups : 0) : (int)(gridDim.x / hkv);
  if (item < 0 || item >= nitems) return;
  const int hq = hkv * (MQ ? gh : G);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int n = lane & 15;

  // the walk: tiles cstart(j) = t0 + (wave + 4 j) * 16 of [t0, t1) through
  // table row tbl
  bool pitem = false;
  int s = 0, p = 0, L = 0, nparts = 1, t0 = 0, t1 = 0, sh = 0;
  int qs = 0, nq = 0, ncols[NC];
  const int32_t *tbl;
  // prefix item: its column set, this lane's column (member, head) and its
  // sequence
  int pset = 0, pfirst = 0, pmember = 0, pseq = 0;
  bool pcol = false;
  // a multi-query prefix item: each column's output row (token * hq + head)
  // and the last position it attends, or -1
  int mrow[NC], mcpos[NC];
  __shared__ int sm_prow[(MQ && PFX) ? NC : 1][16];
#pragma unroll
  for (int c = 0; c < NC; ++c) ncols[c] = G;
  if constexpr (PFX) pitem = item >= num_seqs * P;
  if (MQ && pitem) {
    // Item gi * ipg + ci of group gi covers the group's rows 16 (NC ci + c)
    // + n: the members' (token, head) rows in member order, token-major
    // within a member.  A column attends the prefix positions below its
    // member's shared length, up to its own token's position.
    if (cgroup > 0) return;  // the item's sets are all in column group 0
    const int pi = item - num_seqs * P;
    const int gi = pi / ipg, ci = pi - gi * ipg;
    pfirst = min(max(groups[2 * gi], 0), num_seqs - 1);
    const int count = min(max(groups[2 * gi + 1], 0), min(num_seqs - pfirst, kMqPrefixMembers));
    int colsh[NC], colseq[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      mrow[c] = -1;
      mcpos[c] = -1;
      colsh[c] = 0;
      colseq[c] = pfirst;
    }
    int off = 0;
    for (int mm = 0; mm < count; ++mm) {
      const int sm = pfirst + mm;
      const int Lm = max(0, min(context_lens[sm], mb << lgB));
      const int qsm = max(0, min(query_start[sm], num_tokens));
      const int nqm =
          max(0, min(min(query_start[sm + 1] - qsm, Lm), min(max_q, num_tokens - qsm)));
      const int shm = min(max(shared_lens[sm], 0), Lm) & ~(kTile - 1);
      const int rows_m = nqm * gh;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int R = 16 * (NC * ci + c) + n;
        if (R >= off && R < off + rows_m) {
          const int r = R - off;
          mrow[c] = (qsm + r / gh) * hq + kvh * gh + r % gh;
          mcpos[c] = min(shm - 1, Lm - nqm + r / gh);
          colsh[c] = shm;
          colseq[c] = sm;
        }
      }
      off += rows_m;
    }
    int shx = 0, seqx = pfirst;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      ncols[c] = min(max(off - 16 * (NC * ci + c), 0), 16);
      if (mrow[c] >= 0 && colsh[c] > shx) {
        shx = colsh[c];
        seqx = colseq[c];
      }
    }
    if (wave == 0 && g == 0) {
#pragma unroll
      for (int c = 0; c < NC; ++c) sm_prow[c][n] = mrow[c];
    }
    int wmax = shx;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) wmax = max(wmax, __shfl_xor(wmax, o));
    t1 = __builtin_amdgcn_readfirstlane(wmax);
    if (t1 <= 0) return;  // the same in every wave: the workgroup leaves whole
    const uint64_t longest = __builtin_amdgcn_ballot_w64(shx == wmax);
    const int walk_seq = __builtin_amdgcn_readlane(seqx, (int)__builtin_ctzll(longest));
    tbl = block_tables + (int64_t)walk_seq * mb;
  } else if (pitem) {
    // (decode: NC == 1)
    const int pi = item - num_seqs * P;
    const int gi = pi >> 2;
    pset = pi & 3;
    pfirst = min(max(groups[2 * gi], 0), num_seqs - 1);
    const int count = min(max(groups[2 * gi + 1], 0), min(num_seqs - pfirst, 64 / G));
    const int R = 16 * pset + n;
    pmember = R / G;
    pcol = pmember < count;
    pseq = pfirst + min(pmember, max(count - 1, 0));
    ncols[0] = min(max(count * G - 16 * pset, 0), 16);
    int shm = 0;
    if (pcol) {
      const int Lm = max(0, min(context_lens[pseq], mb << lgB));
      shm = min(max(shared_lens[pseq], 0), Lm) & ~(kTile - 1);
    }
    sh = shm;
    // the walk covers the longest shared length among the set's columns
    // (every wave has the same columns; lanes of one column hold the same
    // value), through the table row of the member that has it: members'
    // rows name the same blocks below their shared lengths, so that row
    // serves every column
    int wmax = shm;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) wmax = max(wmax, __shfl_xor(wmax, off));
    t1 = __builtin_amdgcn_readfirstlane(wmax);
    if (t1 <= 0) return;  // the same in every wave: the workgroup leaves whole
    const uint64_t longest = __builtin_amdgcn_ballot_w64(pcol && shm == wmax);
    const int walk_seq = __builtin_amdgcn_readlane(pseq, (int)__builtin_ctzll(longest));
    tbl = block_tables + (int64_t)walk_seq * mb;
  } else {
    s = item % num_seqs;
    p = (P - 1) - item / num_seqs;
    L = context_lens[s];
    L = max(0, min(L, mb << lgB));
    if constexpr (MQ) {
      qs = max(0, min(query_start[s], num_tokens));
      nq = max(0, min(min(query_start[s + 1] - qs, L), min(max_q, num_tokens - qs)));
#pragma unroll
      for (int c = 0; c < NC; ++c) ncols[c] = min(nq * gh - G * (NC * cgroup + c), G);
      if (ncols[0] <= 0) return;
    }
    nparts = min((L + ps - 1) / ps, P);
    if (p >= max(nparts, 1)) return;
    t0 = p * ps;
    t1 = min(L, t0 + ps);
    if constexpr (PFX) {
      // positions below the shared length come from the group's prefix item
      sh = min(max(shared_lens[s], 0), L) & ~(kTile - 1);
      if (Q8 != 0 && !MQ && prefix_short(L, sh)) return;  // the prefix item reads it all
      if (p < sh / ps) return;  // the whole partition is shared: no partial
      t0 = max(t0, sh);
    }
    tbl = block_tables + (int64_t)s * mb;
  }

  // B operand of q.K for each column set: column n is query head n % G of
  // this KV head (decode), or row 16 c + n of the chunk (multi-query; columns
  // past the chunk are zero and fully masked), or (member, head) of the
  // group (prefix item)
  bf16x8 qb[NC][4];
  int cpos[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    cpos[c] = INT_MAX;
    if constexpr (MQ) {
      const int R = G * (NC * cgroup + c) + n;  // this column's row of the chunk
      cpos[c] = pitem ? mcpos[c] : n < ncols[c] ? L - nq + R / gh : -1;
      const int64_t qr = pitem ? mrow[c] : n < ncols[c] ? (int64_t)(qs + R / gh) * hq + kvh * gh + R % gh : -1;
#pragma unroll
      for (int k = 0; k < 4; ++k) qb[c][k] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
      if (qr >= 0) {
        const uint16_t *qrow = q + qr * kD;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          qb[c][k] = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const u32x4 *>(qrow + k_step_elem<FP8>(g, k)));
      }
    } else {
      const int qseq = pitem ? pseq : s;
      const int qhead = pitem ? (16 * pset + n) % G : n % G;
      const uint16_t *qrow = q + ((int64_t)qseq * hq + kvh * G + qhead) * kD;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        qb[c][k] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4 *>(qrow + k_step_elem<FP8>(g, k)));
      if (pitem) cpos[c] = pcol ? sh - 1 : -1;
    }
  }

  f32x4 acc[NC][8];
  float m[NC], lsum[NC];
  float p0[NC][4];  // the pending first tile of a pair
#pragma unroll
  for (int c = 0; c < NC; ++c) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[c][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    m[c] = neg_inf();
    lsum[c] = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) p0[c][j] = 0.f;
  }
  int slot = 0;
  // the wave's LDS slice: V rows of the pair in the loop, then its results
  constexpr int kCols = PFX ? 16 : G;  // result columns a wave may hold
  constexpr int kSlice =
      K::kSliceBytes > kCols * kD * 4 ? K::kSliceBytes : kCols * kD * 4;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kWaves][kSlice];
  typename K::KV *slice = reinterpret_cast<typename K::KV *>(smem[wave]);

  // pool layout [blocks][kv_heads][block_size][head_dim]: consecutive tokens of
  // one KV head are kD elements apart, a head's slab of a block is kD << lgB
  const int row_elems = kD;
  const int head_off = kvh * (kD << lgB);
  const int64_t block_elems = ((int64_t)hkv * kD) << lgB;

  // full tiles round-robin over the waves (this wave's j-th tile is tile
  // wave + 4j), two-stage register pipeline, the last one or two peeled; the
  // final partial tile goes to the wave it falls to, with masked loads
  const int nfull = max(t1 - t0, 0) / kTile;
  const int nw = nfull > wave ? (nfull - wave + kWaves - 1) / kWaves : 0;
  auto cstart = [&](int j) { return t0 + (wave + kWaves * j) * kTile; };

  // Block ids of this wave's tiles, read 64 tiles at a time into a register
  // (lane i: tile 64c + i) one chunk ahead of use, so no table read sits
  // between a tile's loads and the previous tile's.  With them, a cache hint
  // per tile: a block that the previous or next sequence holds at the same
  // logical position (a shared prefix, forked siblings) is likely to be read
  // again soon, so its rows are read normally; every other block's V rows
  // (and K rows, in bfloat16 pools) are streamed with non-temporal loads.
  // (The hint only steers caching; entries past a neighbour's length may
  // match by chance, which is harmless.)  A prefix item's tiles are read by
  // the group's other column sets too and always use ordinary loads.
  int ent_cur = 0, ent_next = 0;
  uint64_t nt_cur = 0, nt_next = 0;
  auto chunk_entries = [&](int c, uint64_t &ntmask) {
    const int cs = cstart(64 * c + lane);
    int e = 0;
    bool stream = false;
    if (!SMALLB && cs < t1) {
      const int jb = cs >> lgB;
      e = tbl[jb];
      if (!pitem) {
        const bool prev_same = s > 0 && tbl[jb - mb] == e;
        const bool next_same = s + 1 < num_seqs && tbl[jb + mb] == e;
        stream = !prev_same && !next_same;
      }
    }
    ntmask = __builtin_amdgcn_ballot_w64(stream);
    return e;
  };
  ent_cur = chunk_entries(0, nt_cur);
  ent_next = chunk_entries(1, nt_next);
  // the j-th tile's block id; stream_v receives its hint
  auto entry = [&](int j, bool &stream_v) {
    if constexpr (SMALLB) {
      stream_v = !pitem;
      return 0;
    }
    if (j > 0 && (j & 63) == 0) {
      ent_cur = ent_next;
      nt_cur = nt_next;
      ent_next = chunk_entries((j >> 6) + 1, nt_next);
    }
    stream_v = (nt_cur >> (j & 63)) & 1;
    return __builtin_amdgcn_readlane(ent_cur, j & 63);
  };
  if constexpr (Q8 != 0 && !MQ && G <= 4) {
    // 8-bit pools: a tile is half the bytes of a bfloat16 one, so two tiles
    // stay in flight while one is computed (three register buffers, which
    // the 8-bit tiles can afford without losing a wave per SIMD).  Measured
    // against two buffers: FP8 G=1 203.8 -> 196.3 us, G=4 116.0 -> 114.5 and
    // 193.1 -> 189.7 us, INT8 G=4 126.7 -> 122.9 us; G=8 (long contexts)
    // 87.3 -> 88.4 us, so it keeps two.
    TileT A, Bt, C;
    bool sv = true;
    int ent = 0;
    auto load_full = [&](TileT &T, int jj) {
      ent = entry(jj, sv);
      K::template load<false>(T, kc, vc, tbl, ent, sv, cstart(jj), t1, lgB, nb, g, n, row_elems,
                              head_off, block_elems);
    };
    auto compute_full = [&](const TileT &T, int jj) {
      K::template compute<false, NC>(T, qb, acc, m, lsum, p0, slot, slice, cstart(jj), t1, g, n,
                                     sl2, cpos);
    };
    if (nw > 0) load_full(A, 0);
    if (nw > 1) load_full(Bt, 1);
    int j = 0;
    for (; j + 3 <= nw; j += 3) {
      load_full(C, j + 2);
      compute_full(A, j);
      if (j + 3 < nw) load_full(A, j + 3);
      compute_full(Bt, j + 1);
      if (j + 4 < nw) load_full(Bt, j + 4);
      compute_full(C, j + 2);
    }
    // A holds tile j and Bt tile j + 1 where they exist
    if (j < nw) compute_full(A, j);
    if (j + 1 < nw) compute_full(Bt, j + 1);
    if (t0 + nfull * kTile < t1 && nfull % kWaves == wave) {
      const int cs = t0 + nfull * kTile;
      ent = entry(nw, sv);
      K::template load<true>(A, kc, vc, tbl, ent, sv, cs, t1, lgB, nb, g, n, row_elems,
                             head_off, block_elems);
      K::template compute<true, NC>(A, qb, acc, m, lsum, p0, slot, slice, cs, t1, g, n, sl2,
                                     cpos);
    }
  } else {
    TileT A, Bt;
    bool sv = true;
    int ent = 0;
    if (nw > 0) {
      ent = entry(0, sv);
      K::template load<false>(A, kc, vc, tbl, ent, sv, cstart(0), t1, lgB, nb, g, n, row_elems,
                              head_off, block_elems);
      int j = 0;
      for (; j + 2 < nw; j += 2) {
        ent = entry(j + 1, sv);
        K::template load<false>(Bt, kc, vc, tbl, ent, sv, cstart(j + 1), t1, lgB, nb, g, n,
                                row_elems, head_off, block_elems);
        K::template compute<false, NC>(A, qb, acc, m, lsum, p0, slot, slice, cstart(j), t1, g,
                                       n, sl2, cpos);
        ent = entry(j + 2, sv);
        K::template load<false>(A, kc, vc, tbl, ent, sv, cstart(j + 2), t1, lgB, nb, g, n,
                                row_elems, head_off, block_elems);
        K::template compute<false, NC>(Bt, qb, acc, m, lsum, p0, slot, slice, cstart(j + 1),
                                       t1, g, n, sl2, cpos);
      }
      if (j + 2 == nw) {
        ent = entry(j + 1, sv);
        K::template load<false>(Bt, kc, vc, tbl, ent, sv, cstart(j + 1), t1, lgB, nb, g, n,
                                row_elems, head_off, block_elems);
        K::template compute<false, NC>(A, qb, acc, m, lsum, p0, slot, slice, cstart(j), t1, g,
                                       n, sl2, cpos);
        K::template compute<false, NC>(Bt, qb, acc, m, lsum, p0, slot, slice, cstart(j + 1),
                                       t1, g, n, sl2, cpos);
      } else {
        K::template compute<false, NC>(A, qb, acc, m, lsum, p0, slot, slice, cstart(j), t1, g,
                                       n, sl2, cpos);
      }
    }
    if (t0 + nfull * kTile < t1 && nfull % kWaves == wave) {
      const int cs = t0 + nfull * kTile;
      ent = entry(nw, sv);
      K::template load<true>(A, kc, vc, tbl, ent, sv, cs, t1, lgB, nb, g, n, row_elems,
                             head_off, block_elems);
      K::template compute<true, NC>(A, qb, acc, m, lsum, p0, slot, slice, cs, t1, g, n, sl2,
                                     cpos);
    }
  }

  if constexpr (PFX && Q8 != 0 && !MQ) {
    // A prefix item also reads the private tile [sh, L) of each short member
    // of its set (one tile each, the set's members dealt round-robin to the
    // waves), with every other member's columns masked, so that those
    // members' rows are complete here.
    if (pitem) {
      const int gi = (item - num_seqs * P) >> 2;
      const int count = min(max(groups[2 * gi + 1], 0), min(num_seqs - pfirst, 64 / G));
      const int mset = 16 / G;  // members per column set
      for (int mm = wave; mm < mset; mm += kWaves) {
        const int mem = (16 * pset) / G + mm;
        if (mem >= count) break;
        const int seq = pfirst + mem;
        const int Lm = max(0, min(context_lens[seq], mb << lgB));
        const int shm = min(max(shared_lens[seq], 0), Lm) & ~(kTile - 1);
        if (!prefix_short(Lm, shm) || Lm == shm) continue;
        const int32_t *tbm = block_tables + (int64_t)seq * mb;
        const int ent = SMALLB ? 0 : tbm[shm >> lgB];
        int cpos_m[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) cpos_m[c] = (pcol && pmember == mem) ? Lm - 1 : -1;
        TileT A;
        K::template load<true>(A, kc, vc, tbm, ent, true, shm, Lm, lgB, nb, g, n, row_elems,
                               head_off, block_elems);
        K::template compute<true, NC>(A, qb, acc, m, lsum, p0, slot, slice, shm, Lm, g, n, sl2,
                                       cpos_m);
      }
    }
  }

  K::template flush<NC>(p0, slot, slice, acc, g, n);

  // This wave's results per column, one column set at a time: the maximum m
  // is already the column's; the sum combines the four lane groups; the
  // accumulators (lane (g, n): column n, elements 16 b + 4 g + i) go to the
  // wave's LDS slice, which its own loop no longer uses.  A sequence item's
  // columns past G repeat earlier ones (decode); a prefix item's 16 columns
  // are all its own.
  __shared__ float sm_m[kWaves][kCols];
  __shared__ float sm_l[kWaves][kCols];
  float *wacc = reinterpret_cast<float *>(smem[wave]);  // [kCols][kD]
  const int wcols = pitem ? 16 : G;  // distinct columns of this item
  // a sequence with one partition and no shared prefix goes straight to out
  // (its merge skips it)
  const bool final_out = !pitem && nparts <= 1 && sh == 0;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (ncols[c] <= 0) break;  // the group's later sets are empty too
    if (c > 0) __syncthreads();  // every wave has read the previous set's slices
    float lcol = lsum[c];
    lcol += __shfl_xor(lcol, 16);
    lcol += __shfl_xor(lcol, 32);
    if (n < wcols) {
#pragma unroll
      for (int b = 0; b < 8; ++b)
        *reinterpret_cast<f32x4 *>(wacc + n * kD + 16 * b + 4 * g) = acc[c][b];
      if (g == 0) {
        sm_m[wave][n] = m[c];
        sm_l[wave][n] = lcol;
      }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < wcols * kD; i += kThreads) {
      const int h = i / kD;
      const int d = i % kD;
      float M = sm_m[0][h];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm_m[w][h]);
      float ls = 0.f, o = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float mw = sm_m[w][h];
        const float f = (mw == neg_inf()) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
        ls = fmaf(sm_l[w][h], f, ls);
        o = fmaf(reinterpret_cast<const float *>(smem[w])[h * kD + d], f, o);
      }
      int64_t row;
      int slot_of = p;
      bool to_out = final_out;
      if constexpr (MQ) {
        if (h >= ncols[c]) continue;
        if (pitem) {
          // the row's prefix partial is its last slot
          row = sm_prow[c][h];
          if (row < 0) continue;
          slot_of = slots - 1;
        } else {
          const int R = G * (NC * cgroup + c) + h;
          row = (int64_t)(qs + R / gh) * hq + kvh * gh + R % gh;
        }
      } else {
        if (pitem) {
          // (member, head) of the group; its prefix partial is the row's
          // last slot
          if (h >= ncols[0]) continue;
          const int R = 16 * pset + h;
          const int seq = pfirst + R / G;
          row = (int64_t)seq * hq + kvh * G + R % G;
          slot_of = slots - 1;
          // a short member's row is complete: straight to out
          const int Lm = max(0, min(context_lens[seq], mb << lgB));
          to_out = Q8 != 0 &&
                   prefix_short(Lm, min(max(shared_lens[seq], 0), Lm) & ~(kTile - 1));
        } else {
          row = (int64_t)s * hq + kvh * G + h;
        }
      }
      if (to_out) {
        out[row * kD + d] = ls > 0.f ? v_scale * (o / ls) : 0.f;
      } else {
        const int64_t at = row * slots + slot_of;
        ws_o[at * kD + d] = ls > 0.f ? v_scale * (o / ls) : 0.f;
        if (d == 0) {
          ws_ml[at * 2 + 0] = M;
          ws_ml[at * 2 + 1] = ls;
        }
      }
    }
  }
}

template <int G, bool SMALLB, int Q8>
hipError_t launch_typed(const DecodeArgs &a, hipStream_t stream) {
  using KV = typename MfmaDecode<G, SMALLB, Q8>::KV;
  constexpr bool FP8 = Q8 != 0;  // scaled 8-bit codes
  const bool pfx = a.num_groups > 0;
  // with groups, four column-set items per group follow the sequence items
  const int64_t grid =
      ((int64_t)a.num_seqs * a.num_partitions + (pfx ? 4 * (int64_t)a.num_groups : 0)) *
      a.num_kv_heads;
  if (grid <= 0) return hipSuccess;
  // the K scale multiplies every score, so it joins the softmax scale
  const float sl2 = a.scale * (FP8 ? a.k_scale : 1.f) * kLog2e;
  auto kernel = pfx ? paged_decode_mfma_kernel<G, SMALLB, Q8, false, 1, true>
                    : paged_decode_mfma_kernel<G, SMALLB, Q8, false, 1, false>;
  hipLaunchKernelGGL(kernel, dim3((uint32_t)grid), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t *>(a.q), static_cast<const KV *>(a.k_cache),
                     static_cast<const KV *>(a.v_cache), a.block_tables, a.context_lens, a.out,
                     a.ws_o, a.ws_ml, sl2, FP8 ? a.v_scale : 1.f, a.num_seqs, a.num_kv_heads,
                     a.log2_block_size, a.num_blocks, a.max_blocks_per_seq, a.partition_size,
                     a.num_partitions, nullptr, 0, 0, 0, 1, a.order, a.groups, a.shared_lens,
                     a.num_partitions + (pfx ? 1 : 0), 4, a.num_groups);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || (a.num_partitions <= 1 && !pfx)) return e;
  return launch_partition_merge(a, stream);
}

template <int G, int Q8>
hipError_t launch_b(const DecodeArgs &a, hipStream_t stream) {
  if (a.log2_block_size >= 4) return launch_typed<G, false, Q8>(a, stream);
  return launch_typed<G, true, Q8>(a, stream);
}

template <bool SMALLB, int Q8>
hipError_t launch_mq(const MultiQueryArgs &a, hipStream_t stream) {
  using KV = typename MfmaDecode<16, SMALLB, Q8>::KV;
  constexpr bool FP8 = Q8 != 0;
  const int gh = a.num_q_heads / a.num_kv_heads;
  const bool pfx = a.num_groups > 0;
  // with groups, ipg prefix items per group follow the sequence items
  const int ipg = pfx ? (int)mq_prefix_items_per_group(a.max_query_len, gh) : 0;
  const int64_t items =
      ((int64_t)a.num_seqs * a.num_partitions + (int64_t)ipg * a.num_groups) * a.num_kv_heads;
  if (items <= 0) return hipSuccess;
  const int csets = (int)(((int64_t)a.max_query_len * gh + 15) / 16);
  // two column sets per wave from 17 rows up (one pass over K/V for 32
  // columns), one otherwise
  const int64_t grid = (items + 7) / 8 * 8 * multi_query_few_rows_groups(csets);
  // (prefix items come over bf16 pools with at most 8 rows per KV head: one
  // column set)
  if (pfx && (csets > 1 || Q8 != 0)) return hipErrorNotSupported;
  auto kernel = csets >= 2 ? paged_decode_mfma_kernel<16, SMALLB, Q8, true, 2, false>
                           : paged_decode_mfma_kernel<16, SMALLB, Q8, true, 1, false>;
  if constexpr (Q8 == 0) {
    if (pfx) kernel = paged_decode_mfma_kernel<16, SMALLB, 0, true, 1, true>;
  }
  // as in decode: the K scale joins the softmax scale, the V scale the output
  const float sl2 = a.scale * (FP8 ? a.k_scale : 1.f) * kLog2e;
  hipLaunchKernelGGL(kernel, dim3((uint32_t)grid), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t *>(a.q), static_cast<const KV *>(a.k_cache),
                     static_cast<const KV *>(a.v_cache), a.block_tables, a.context_lens, a.out,
                     a.ws_o, a.ws_ml, sl2, FP8 ? a.v_scale : 1.f, a.num_seqs, a.num_kv_heads,
                     a.log2_block_size, a.num_blocks, a.max_blocks_per_seq, a.partition_size,
                     a.num_partitions, a.query_start, a.num_tokens, gh, a.max_query_len, csets,
                     a.order, pfx ? a.groups : nullptr, pfx ? a.shared_lens : nullptr,
                     a.num_partitions + (pfx ? 1 : 0), ipg, pfx ? a.num_groups : 0);
  return hipGetLastError();
}

}  // namespace

int64_t multi_query_few_rows_groups(int64_t csets) {
  return csets >= 2 ? (csets + 1) / 2 : 1;
}

bool multi_query_few_rows_supported(const MultiQueryArgs &a) {
  return a.dtype == 1 && a.head_dim == kD &&
         (int64_t)a.max_query_len * (a.num_q_heads / a.num_kv_heads) <= kMqFewRows;
}

hipError_t launch_multi_query_few_rows(const MultiQueryArgs &a, hipStream_t stream) {
  if (a.kv_dtype == 2) {  // FP8 E4M3 pool
    if (a.log2_block_size >= 4) return launch_mq<false, 1>(a, stream);
    return launch_mq<true, 1>(a, stream);
  }
  if (a.kv_dtype == 3) {  // INT8 pool
    if (a.log2_block_size >= 4) return launch_mq<false, 2>(a, stream);
    return launch_mq<true, 2>(a, stream);
  }
  if (a.log2_block_size >= 4) return launch_mq<false, 0>(a, stream);
  return launch_mq<true, 0>(a, stream);
}

bool decode_mfma_supported(int32_t dtype, int32_t head_dim, int32_t group) {
  // bfloat16 pools with G < 4 stay on the vector kernel (decode.hip), measured
  // faster there (Llama-7B-shaped layer, G = 1: 382 vs 387 us); 8-bit pools
  // run only here, for every G
  return dtype == 1 && head_dim == kD && (group == 4 || group == 8);
}

bool decode_prefix_supported(int32_t head_dim, int32_t group) {
  return head_dim == kD && (group == 1 || group == 2 || group == 4 || group == 8);
}

bool decode_q8_supported(int32_t head_dim, int32_t group) {
  // head_dim 64 runs on the vector kernel (decode.hip)
  return (head_dim == kD || head_dim == 64) &&
         (group == 1 || group == 2 || group == 4 || group == 8);
}

template <int G>
hipError_t launch_kind(const DecodeArgs &a, hipStream_t stream) {
  switch (a.kv_dtype) {
    case 2: return launch_b<G, 1>(a, stream);  // FP8 E4M3
    case 3: return launch_b<G, 2>(a, stream);  // INT8
    default: return launch_b<G, 0>(a, stream);
  }
}

hipError_t launch_decode_mfma(const DecodeArgs &a, hipStream_t stream) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_kind<1>(a, stream);
    case 2: return launch_kind<2>(a, stream);
    case 4: return launch_kind<4>(a, stream);
    case 8: return launch_kind<8>(a, stream);
    default: return hipErrorNotSupported;
  }
}

}  // namespace pa
