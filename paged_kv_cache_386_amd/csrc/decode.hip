// PagedAttention decode for gfx950 (MI355X), with an optional split-K
// partitioning of long contexts and a separate merge kernel.
//
// What is computed: for each sequence and query head, the scaled dot of q with
// every K row of the sequence's context (found through the block table), a
// softmax, and the weighted sum of the V rows ("核心代码拆解" section of the
// devpress.csdn.net/amd vLLM walkthrough; block tables in section 2.1 of the
// chenxutan.com vLLM deep-dive).  That page's kernel gives one CUDA block per
// (sequence, head) and walks a [blocks][heads][block_size][head_size] cache one
// token at a time; it is prior art only.  Here:
//
//  * one workgroup of 4 wave64s per (sequence, KV head, partition); the G query
//    heads of a GQA group share every K/V read;
//  * the pool is [blocks][kv_heads][block_size][head_dim]: a KV head's rows
//    of one block are contiguous, a row of LPR lanes reads one whole row with
//    16-byte loads and a wave reads 64/LPR consecutive rows per load
//    instruction;
//  * each wave takes 16-token chunks round-robin and double-buffers them in
//    registers (the next chunk's loads are in flight while the current one is
//    computed); a 16-aligned chunk never straddles a block when
//    block_size >= 16, so its block id is one scalar load;
//  * q.k for bf16 uses v_dot2_f32_bf16 on packed pairs (exact products, fp32
//    accumulation); the row's partial dots are summed with DPP lane moves;
//  * every row of lanes keeps its own fp32 running max / sum / accumulator
//    (online softmax, base 2 with log2(e) folded into the scale), so the hot
//    loop has no cross-row traffic; rows, then waves (through LDS), are merged
//    once at the end;
//  * with more than one partition, each workgroup writes its partition's
//    (max, sum, normalised output) and a second kernel merges them in
//    ascending partition order.
//
// Accumulation order is fixed by logical token position, never by physical
// block id, so results are bitwise reproducible and bitwise invariant under a
// relabelling of physical blocks.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "internal.h"

namespace pa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kChunk = 16;  // tokens per wave iteration

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

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

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

// Sixteen 8-bit codes (one 16-byte vector, code i in byte i) to sixteen
// bfloat16 values, exactly (an E4M3 value has at most 4 significant bits, an
// INT8 code at most 7): pair word j holds elements 2 j (low half) and 2 j + 1.
// FP8 (Q8 = 1) through gfx950's scaled conversion at scale 1, two codes per
// instruction; INT8 (Q8 = 2) widened to fp32, whose high halves are the
// bfloat16 values, paired with one byte permute.
template <int Q8>
__device__ __forceinline__ void codes16_to_bf16(u32x4 w, uint32_t (&b)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (Q8 == 1) {
      b[2 * i] = __builtin_bit_cast(uint32_t,
                                    __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.f, false));
      b[2 * i + 1] = __builtin_bit_cast(uint32_t,
                                        __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.f, true));
    } else {
      float f[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) f[j] = (float)((int32_t)(w[i] << (24 - 8 * j)) >> 24);
      b[2 * i] = __builtin_amdgcn_perm(__float_as_uint(f[1]), __float_as_uint(f[0]), 0x07060302u);
      b[2 * i + 1] =
          __builtin_amdgcn_perm(__float_as_uint(f[3]), __float_as_uint(f[2]), 0x07060302u);
    }
  }
}

// DPP lane moves inside a row of 16 lanes.
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror: lane ^ 7 within 8
constexpr int kDppMirror = 0x140;      // row_mirror: lane ^ 15 within 16

template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// Sum over the LPR consecutive lanes of a row; every lane of the row gets the
// total.  Each step adds the value of a partner lane whose index differs in one
// more bit group, so after log2(LPR) steps all LPR lanes are covered.
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
  static_assert(LPR == 4 || LPR == 8 || LPR == 16, "rows are 4, 8 or 16 lanes");
  x += dpp_move<kDppQuadXor1>(x);
  x += dpp_move<kDppQuadXor2>(x);
  if constexpr (LPR >= 8) x += dpp_move<kDppHalfMirror>(x);
  if constexpr (LPR >= 16) x += dpp_move<kDppMirror>(x);
  return x;
}

template <typename T, int D, int G>
struct Shape {
  static constexpr int EPV = 16 / (int)sizeof(T);            // elements per 16-byte vector
  static constexpr int VPR = D / EPV;                        // vectors per KV row
  static constexpr int LPR_WANT = G >= 8 ? 16 : 8;
  static constexpr int LPR = LPR_WANT < VPR ? LPR_WANT : VPR;  // lanes per row
  static constexpr int VPL = VPR / LPR;                      // vectors per lane
  static constexpr int ROWS = 64 / LPR;                      // rows per wave load
  static constexpr int TPL = kChunk / ROWS;                  // tokens per lane per chunk
  static constexpr int DPL = VPL * EPV;                      // head dims per lane
  static_assert(VPR % LPR == 0, "row must split evenly over lanes");
  static_assert(TPL >= 1 && kChunk % ROWS == 0, "chunk must cover whole rows");
};

// Q8: the pool's element kind -- 0 the type T itself (fp32 or bfloat16), 1
// FP8 (E4M3) or 2 INT8 codes (T = uint8_t, 16 per vector), each vector
// widened to bfloat16 pairs when it is computed; q is then bfloat16, held as
// QW = 2 vectors per code vector.
template <typename T, int D, int G, bool SMALLB, int Q8 = 0>
struct Decode {
  using S = Shape<T, D, G>;
  static constexpr int TPL = S::TPL, VPL = S::VPL, LPR = S::LPR, ROWS = S::ROWS,
                       EPV = S::EPV, DPL = S::DPL;
  static constexpr int QW = Q8 ? 2 : 1;

  struct Regs {
    u32x4 k[TPL][VPL];
    u32x4 v[TPL][VPL];
  };

  // Issue the loads of one chunk's K and V rows for this lane.  Tokens at or
  // past t1 are not read (their registers are zeroed) when MASK is set.
  // lane_off: this lane's element offset inside a block
  // ((kvh * block_size + r) * D + c * EPV); row_elems = D (token stride of
  // one KV head); block_elems =
  // block_size * hkv * D; mb = the table row length; has_prev / has_next:
  // whether the sequence has a neighbour row in the table.
  template <bool MASK>
  static __device__ __forceinline__ void load(Regs &R, const T *__restrict__ kc,
                                              const T *__restrict__ vc,
                                              const int32_t *__restrict__ tbl, int cs, int t1,
                                              int lgB, int nb, int r, uint32_t lane_off,
                                              int row_elems, int64_t block_elems, int mb,
                                              bool has_prev, bool has_next) {
    const int bm1 = (1 << lgB) - 1;
    if constexpr (!SMALLB) {
      // the whole 16-token chunk lies in one block: one (scalar) table read,
      // then buffer loads through descriptors spanning the block.  Cache
      // hint: a block the previous or next sequence also holds at this
      // logical position (a shared prefix, forked siblings) is read normally;
      // any other block is streamed with non-temporal loads.
      const int jb = cs >> lgB;
      const int e = tbl[jb];
      const bool reused = (has_prev && tbl[jb - mb] == e) || (has_next && tbl[jb + mb] == e);
      const uint32_t pid = min((uint32_t)e, (uint32_t)(nb - 1));
      const uint32_t bbytes = (uint32_t)(block_elems * (int64_t)sizeof(T));
      const auto rk = block_rsrc(kc + (int64_t)pid * block_elems, bbytes);
      const auto rv = block_rsrc(vc + (int64_t)pid * block_elems, bbytes);
      const uint32_t base = (uint32_t)((cs & bm1) * row_elems) + lane_off;
      uint32_t off[TPL];
      bool ok[TPL];
#pragma unroll
      for (int k = 0; k < TPL; ++k) {
        off[k] = (base + (uint32_t)(ROWS * k * row_elems)) * (uint32_t)sizeof(T);
        ok[k] = !MASK || cs + r + ROWS * k < t1;
      }
      if (reused) {
#pragma unroll
        for (int k = 0; k < TPL; ++k)
#pragma unroll
          for (int v = 0; v < VPL; ++v) {
            const uint32_t o = off[k] + 16 * LPR * v;
            R.k[k][v] = ok[k] ? buffer_load<kCacheNormal>(rk, o) : u32x4{0, 0, 0, 0};
            R.v[k][v] = ok[k] ? buffer_load<kCacheNormal>(rv, o) : u32x4{0, 0, 0, 0};
          }
      } else {
#pragma unroll
        for (int k = 0; k < TPL; ++k)
#pragma unroll
          for (int v = 0; v < VPL; ++v) {
            const uint32_t o = off[k] + 16 * LPR * v;
            R.k[k][v] = ok[k] ? buffer_load<kCacheStream>(rk, o) : u32x4{0, 0, 0, 0};
            R.v[k][v] = ok[k] ? buffer_load<kCacheStream>(rv, o) : u32x4{0, 0, 0, 0};
          }
      }
    } else {
      // blocks shorter than a chunk: every token row looks up its own block
#pragma unroll
      for (int k = 0; k < TPL; ++k) {
        const int t = cs + r + ROWS * k;
        const bool ok = !MASK || t < t1;
        if (ok) {
          const uint32_t pid = min((uint32_t)tbl[t >> lgB], (uint32_t)(nb - 1));
          // lane_off already holds r's row; remove it and add this token's offset
          const int64_t kb = (int64_t)pid * block_elems + (int64_t)((t & bm1) - r) * row_elems;
          const u32x4 *kp = reinterpret_cast<const u32x4 *>(kc + kb + lane_off);
          const u32x4 *vp = reinterpret_cast<const u32x4 *>(vc + kb + lane_off);
#pragma unroll
          for (int v = 0; v < VPL; ++v) {
            R.k[k][v] = __builtin_nontemporal_load(kp + LPR * v);
            R.v[k][v] = __builtin_nontemporal_load(vp + LPR * v);
          }
        } else {
#pragma unroll
          for (int v = 0; v < VPL; ++v) {
            R.k[k][v] = u32x4{0, 0, 0, 0};
            R.v[k][v] = u32x4{0, 0, 0, 0};
          }
        }
      }
    }
    // keep these loads ahead of the computation that follows them
    __builtin_amdgcn_sched_barrier(0);
  }

  // Fold one chunk into this row's running (max, sum, accumulator).
  template <bool MASK>
  static __device__ __forceinline__ void compute(const Regs &R, const u32x4 (&qv)[G][VPL * QW],
                                                 float (&acc)[G][DPL], float (&m)[G],
                                                 float (&l)[G], int cs, int t1, int r,
                                                 float sl2) {
    // 8-bit codes: each K vector as 8 bfloat16 pairs, shared by the G heads
    uint32_t kb[TPL][VPL][Q8 ? 8 : 1];
    if constexpr (Q8 != 0) {
#pragma unroll
      for (int k = 0; k < TPL; ++k)
#pragma unroll
        for (int v = 0; v < VPL; ++v) codes16_to_bf16<Q8>(R.k[k][v], kb[k][v]);
    }
    float x[TPL][G];
#pragma unroll
    for (int k = 0; k < TPL; ++k) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float d = 0.f;
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
          if constexpr (Q8 != 0) {
#pragma unroll
            for (int j = 0; j < 8; ++j) d = dot2_bf16(qv[h][2 * v + j / 4][j % 4], kb[k][v][j], d);
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              if constexpr (sizeof(T) == 2)
                d = dot2_bf16(qv[h][v][i], R.k[k][v][i], d);
              else
                d = fmaf(__uint_as_float(qv[h][v][i]), __uint_as_float(R.k[k][v][i]), d);
            }
          }
        }
        d = row_sum<LPR>(d);
        x[k][h] = (!MASK || cs + r + ROWS * k < t1) ? d * sl2 : neg_inf();
      }
    }
    float p[TPL][G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float cm = x[0][h];
#pragma unroll
      for (int k = 1; k < TPL; ++k) cm = fmaxf(cm, x[k][h]);
      if (cm > m[h]) {
        const float a = __builtin_amdgcn_exp2f(m[h] - cm);  // 0 when m was -inf
        l[h] *= a;
#pragma unroll
        for (int j = 0; j < DPL; ++j) acc[h][j] *= a;
        m[h] = cm;
      }
      const float mu = (m[h] == neg_inf()) ? 0.f : m[h];
#pragma unroll
      for (int k = 0; k < TPL; ++k) {
        p[k][h] = __builtin_amdgcn_exp2f(x[k][h] - mu);
        l[h] += p[k][h];
      }
    }
#pragma unroll
    for (int k = 0; k < TPL; ++k) {
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        if constexpr (Q8 != 0) {
          uint32_t vb[8];
          codes16_to_bf16<Q8>(R.v[k][v], vb);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float lo = bf16_lo(vb[j]), hi = bf16_hi(vb[j]);
#pragma unroll
            for (int h = 0; h < G; ++h) {
              acc[h][v * EPV + 2 * j] = fmaf(p[k][h], lo, acc[h][v * EPV + 2 * j]);
              acc[h][v * EPV + 2 * j + 1] = fmaf(p[k][h], hi, acc[h][v * EPV + 2 * j + 1]);
            }
          }
          continue;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t w = R.v[k][v][i];
          if constexpr (sizeof(T) == 2) {
            const float lo = bf16_lo(w), hi = bf16_hi(w);
#pragma unroll
            for (int h = 0; h < G; ++h) {
              acc[h][v * EPV + 2 * i] = fmaf(p[k][h], lo, acc[h][v * EPV + 2 * i]);
              acc[h][v * EPV + 2 * i + 1] = fmaf(p[k][h], hi, acc[h][v * EPV + 2 * i + 1]);
            }
          } else {
            const float f = __uint_as_float(w);
#pragma unroll
            for (int h = 0; h < G; ++h) acc[h][v * EPV + i] = fmaf(p[k][h], f, acc[h][v * EPV + i]);
          }
        }
      }
    }
  }
};

// (8-bit pools: q is bfloat16, the K scale is part of sl2 and the V scale
// multiplies the normalised output)
template <typename T, int D, int G, bool SMALLB, int Q8 = 0>
__global__ __launch_bounds__(kThreads) void paged_decode_kernel(
    const typename std::conditional<Q8 != 0, uint16_t, T>::type *__restrict__ q,
    const T *__restrict__ kc, const T *__restrict__ vc,
    const int32_t *__restrict__ block_tables, const int32_t *__restrict__ context_lens,
    float *__restrict__ out, float *__restrict__ ws_o, float *__restrict__ ws_ml, float sl2,
    float v_scale, int num_seqs, int hkv, int lgB, int nb, int mb, int ps, int P,
    const int32_t *__restrict__ order) {
  using K = Decode<T, D, G, SMALLB, Q8>;
  constexpr int TPL = K::TPL, VPL = K::VPL, LPR = K::LPR, EPV = K::EPV, DPL = K::DPL;
  constexpr int QW = K::QW;
  (void)TPL;

  // Work item: KV head fastest, then item = (sequence, partition), from
  // the longest-first list when there is one, else the fixed order --
  // sequence, then partition from the last down (long sequences' later
  // partitions start first).  With the hardware's round-robin placement of
  // consecutive workgroups over the 8 XCDs, items that share a KV head (and
  // so a prefix block's head slice) land on the same XCD whenever
  // num_kv_heads is a multiple of 8.
  const int kvh = blockIdx.x % hkv;
  const int item = order ? order[blockIdx.x / hkv] : (int)(blockIdx.x / hkv);
  // listed as empty (past the sequence's end), or not an item of this launch
  if (item < 0 || item >= num_seqs * P) return;
  const int s = item % num_seqs;
  const int p = (P - 1) - item / num_seqs;
  const int hq = hkv * G;

  int L = context_lens[s];
  L = max(0, min(L, mb << lgB));
  const int nparts = min((L + ps - 1) / ps, P);
  if (p >= max(nparts, 1)) return;
  const int t0 = p * ps;
  const int t1 = min(L, t0 + ps);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane / LPR;
  const int c = lane % LPR;
  const int32_t *tbl = block_tables + (int64_t)s * mb;
  const bool has_prev = s > 0, has_next = s + 1 < num_seqs;

  // this lane's elements of q: the EPV elements of each of its VPL vectors
  // (QW 16-byte vectors of q per vector of the pool)
  u32x4 qv[G][VPL * QW];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const u32x4 *qp =
        reinterpret_cast<const u32x4 *>(q + ((int64_t)s * hq + kvh * G + h) * D) + QW * c;
#pragma unroll
    for (int v = 0; v < VPL; ++v)
#pragma unroll
      for (int w = 0; w < QW; ++w) qv[h][QW * v + w] = qp[QW * LPR * v + w];
  }

  float acc[G][DPL];
  float m[G], l[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = neg_inf();
    l[h] = 0.f;
#pragma unroll
    for (int j = 0; j < DPL; ++j) acc[h][j] = 0.f;
  }

  const uint32_t lane_off = (uint32_t)(((kvh << lgB) + r) * D + c * EPV);
  const int row_elems = D;
  const int64_t block_elems = ((int64_t)hkv * D) << lgB;

  // Full 16-token chunks go round-robin over the waves (this wave's j-th chunk
  // is chunk wave + 4j) through a two-stage register pipeline: the loads of
  // the next chunk are issued before the current chunk is computed.  The
  // steady-state loop issues its loads unconditionally, so the compiler's
  // wait counts only ever cover the chunk being computed; the last one or two
  // chunks are peeled.  The final, partial chunk is done afterwards by the wave
  // it falls to, with masked loads.
  const int nfull = (t1 - t0) / kChunk;
  const int nw = nfull > wave ? (nfull - wave + kWaves - 1) / kWaves : 0;
  {
    typename K::Regs A, Bq;
    auto cstart = [&](int j) { return t0 + (wave + kWaves * j) * kChunk; };
    if (nw > 0) {
      K::template load<false>(A, kc, vc, tbl, cstart(0), t1, lgB, nb, r, lane_off, row_elems,
                              block_elems, mb, has_prev, has_next);
      int j = 0;
      for (; j + 2 < nw; j += 2) {
        K::template load<false>(Bq, kc, vc, tbl, cstart(j + 1), t1, lgB, nb, r, lane_off,
                                row_elems, block_elems, mb, has_prev, has_next);
        K::template compute<false>(A, qv, acc, m, l, cstart(j), t1, r, sl2);
        K::template load<false>(A, kc, vc, tbl, cstart(j + 2), t1, lgB, nb, r, lane_off,
                                row_elems, block_elems, mb, has_prev, has_next);
        K::template compute<false>(Bq, qv, acc, m, l, cstart(j + 1), t1, r, sl2);
      }
      if (j + 2 == nw) {
        K::template load<false>(Bq, kc, vc, tbl, cstart(j + 1), t1, lgB, nb, r, lane_off,
                                row_elems, block_elems, mb, has_prev, has_next);
        K::template compute<false>(A, qv, acc, m, l, cstart(j), t1, r, sl2);
        K::template compute<false>(Bq, qv, acc, m, l, cstart(j + 1), t1, r, sl2);
      } else {
        K::template compute<false>(A, qv, acc, m, l, cstart(j), t1, r, sl2);
      }
    }
    if (t0 + nfull * kChunk < t1 && nfull % kWaves == wave) {
      const int cs = t0 + nfull * kChunk;
      K::template load<true>(A, kc, vc, tbl, cs, t1, lgB, nb, r, lane_off, row_elems,
                             block_elems, mb, has_prev, has_next);
      K::template compute<true>(A, qv, acc, m, l, cs, t1, r, sl2);
    }
  }

  // Merge the rows of this wave: common max, rescale, sum over rows.
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float M = m[h];
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
    const float f = (m[h] == neg_inf()) ? 0.f : __builtin_amdgcn_exp2f(m[h] - M);
    float lh = l[h] * f;
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) lh += __shfl_xor(lh, off);
    l[h] = lh;
    m[h] = M;
#pragma unroll
    for (int j = 0; j < DPL; ++j) {
      float a = acc[h][j] * f;
#pragma unroll
      for (int off = LPR; off < 64; off <<= 1) a += __shfl_xor(a, off);
      acc[h][j] = a;
    }
  }

  // Merge the waves through LDS.
  __shared__ float sm_acc[kWaves][G][D];
  __shared__ float sm_m[kWaves][G];
  __shared__ float sm_l[kWaves][G];
  if (lane < LPR) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int v = 0; v < VPL; ++v)
#pragma unroll
        for (int e = 0; e < EPV; ++e) sm_acc[wave][h][(c + LPR * v) * EPV + e] = acc[h][v * EPV + e];
      if (lane == 0) {
        sm_m[wave][h] = m[h];
        sm_l[wave][h] = l[h];
      }
    }
  }
  __syncthreads();
  const bool final_out = nparts <= 1;
  for (int i = threadIdx.x; i < G * D; i += kThreads) {
    const int h = i / D;
    const int d = i % D;
    float M = sm_m[0][h];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm_m[w][h]);
    float lsum = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = sm_m[w][h];
      const float f = (mw == neg_inf()) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      lsum = fmaf(sm_l[w][h], f, lsum);
      o = fmaf(sm_acc[w][h][d], f, o);
    }
    const int64_t row = (int64_t)s * hq + kvh * G + h;
    if (final_out) {
      out[row * D + d] = lsum > 0.f ? (Q8 ? v_scale * (o / lsum) : o / lsum) : 0.f;
    } else {
      ws_o[(row * P + p) * D + d] = Q8 ? v_scale * (o / lsum) : o / lsum;
      if (d == 0) {
        ws_ml[(row * P + p) * 2 + 0] = M;
        ws_ml[(row * P + p) * 2 + 1] = lsum;
      }
    }
  }
}

// Merge of the partition partials of one (sequence, query head) per wave
// (four rows per workgroup, D / 64 elements per lane): weights
// l_p * 2^(m_p - max m), summed in ascending position order.  A row has
// `slots` partial slots: partitions 0 .. P-1, and with shared prefixes
// (shared_lens non-null) a last slot holding the prefix, positions
// [0, shared length), which comes first; partitions that lie wholly inside
// the shared length were not computed and are skipped.  The shared length is
// taken as the decode kernel takes it (clamped to the context, whole 16-token
// tiles).
constexpr int kMergeRows = 4;
// Partials of a row the merge loads in one batch (max, sum and rows): the
// prefix's and two partitions cover the GQA prefix batch (merge 5.95 -> 5.28
// us per call).
constexpr int kMergeAhead = 3;
template <int D>
__global__ __launch_bounds__(64 * kMergeRows) void paged_decode_merge_kernel(
    const int32_t *__restrict__ context_lens, const float *__restrict__ ws_o,
    const float *__restrict__ ws_ml, float *__restrict__ out, int rows, int hq, int cap, int ps,
    int P, const int32_t *__restrict__ shared_lens, int slots, int short_rule) {
  constexpr int EPL = D / 64;  // elements per lane
  const int row = blockIdx.x * kMergeRows + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const int s = row / hq;
  int L = context_lens[s];
  L = max(0, min(L, cap));  // the same clamp as the decode kernel
  const int n = min((L + ps - 1) / ps, P);
  const int sh = shared_lens ? min(max(shared_lens[s], 0), L) & ~15 : 0;
  // written by the decode kernel directly: one partition and no shared
  // prefix, or a short member of a prefix group (its prefix item wrote it)
  if ((n <= 1 && sh == 0) || (short_rule && prefix_short(L, sh))) return;
  const int first = sh > 0 ? sh / ps : 0;  // first partition with private positions
  const float *ml = ws_ml + (int64_t)row * slots * 2;
  const float *o = ws_o + (int64_t)row * slots * D + lane * EPL;
  const int pre = slots - 1;  // the prefix slot (used when sh > 0)
  // the partials in merge order: the prefix's, then the private partitions
  // ascending; the first kMergeAhead are loaded (max, sum and rows) in one
  // batch, so their rows do not wait on the maximum
  const int cnt = (sh > 0 ? 1 : 0) + max(n - first, 0);
  auto slot_at = [&](int k) { return sh > 0 ? (k == 0 ? pre : first + k - 1) : first + k; };
  float am[kMergeAhead], al[kMergeAhead], ao[kMergeAhead][EPL];
#pragma unroll
  for (int k = 0; k < kMergeAhead; ++k) {
    am[k] = -__builtin_huge_valf();
    al[k] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) ao[k][e] = 0.f;
    if (k < cnt) {
      const int j = slot_at(k);
      am[k] = ml[2 * j];
      al[k] = ml[2 * j + 1];
#pragma unroll
      for (int e = 0; e < EPL; ++e) ao[k][e] = o[(int64_t)j * D + e];
    }
  }
  float M = -__builtin_huge_valf();
#pragma unroll
  for (int k = 0; k < kMergeAhead; ++k) M = fmaxf(M, am[k]);
  for (int k = kMergeAhead; k < cnt; ++k) M = fmaxf(M, ml[2 * slot_at(k)]);
  float num[EPL], den = 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) num[e] = 0.f;
  auto add = [&](float mj, float lj, const float *oj) {
    const float w = mj == -__builtin_huge_valf() ? 0.f : lj * __builtin_amdgcn_exp2f(mj - M);
#pragma unroll
    for (int e = 0; e < EPL; ++e) num[e] = fmaf(w, oj[e], num[e]);
    den += w;
  };
#pragma unroll
  for (int k = 0; k < kMergeAhead; ++k)
    if (k < cnt) add(am[k], al[k], ao[k]);
  for (int k = kMergeAhead; k < cnt; ++k) {
    const int j = slot_at(k);
    float oj[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) oj[e] = o[(int64_t)j * D + e];
    add(ml[2 * j], ml[2 * j + 1], oj);
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e)
    out[(int64_t)row * D + lane * EPL + e] = den > 0.f ? num[e] / den : 0.f;
}

template <typename T, int D, int G, bool SMALLB, int Q8>
hipError_t launch_typed(const DecodeArgs &a, hipStream_t stream) {
  using QT = typename std::conditional<Q8 != 0, uint16_t, T>::type;
  const int64_t grid = (int64_t)a.num_seqs * a.num_kv_heads * a.num_partitions;
  if (grid <= 0) return hipSuccess;
  // 8-bit pools: the K scale joins the softmax scale
  const float sl2 = a.scale * (Q8 ? a.k_scale : 1.f) * kLog2e;
  hipLaunchKernelGGL((paged_decode_kernel<T, D, G, SMALLB, Q8>), dim3((uint32_t)grid),
                     dim3(kThreads), 0, stream, static_cast<const QT *>(a.q),
                     static_cast<const T *>(a.k_cache), static_cast<const T *>(a.v_cache),
                     a.block_tables, a.context_lens, a.out, a.ws_o, a.ws_ml, sl2,
                     Q8 ? a.v_scale : 1.f, a.num_seqs, a.num_kv_heads, a.log2_block_size,
                     a.num_blocks, a.max_blocks_per_seq, a.partition_size, a.num_partitions,
                     a.order);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.num_partitions <= 1) return e;
  return launch_partition_merge(a, stream);
}

template <typename T, int D, int G, int Q8>
hipError_t launch_b(const DecodeArgs &a, hipStream_t stream) {
  if (a.log2_block_size >= 4) return launch_typed<T, D, G, false, Q8>(a, stream);
  return launch_typed<T, D, G, true, Q8>(a, stream);
}

template <typename T, int D, int Q8 = 0>
hipError_t launch_g(const DecodeArgs &a, hipStream_t stream) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_b<T, D, 1, Q8>(a, stream);
    case 2: return launch_b<T, D, 2, Q8>(a, stream);
    case 4: return launch_b<T, D, 4, Q8>(a, stream);
    case 8: return launch_b<T, D, 8, Q8>(a, stream);
    default: return hipErrorNotSupported;
  }
}

template <typename T>
hipError_t launch_d(const DecodeArgs &a, hipStream_t stream) {
  switch (a.head_dim) {
    case 64: return launch_g<T, 64>(a, stream);
    case 128: return launch_g<T, 128>(a, stream);
    default: return hipErrorNotSupported;
  }
}

}  // namespace

bool decode_supported(int32_t dtype, int32_t head_dim, int32_t group) {
  if (dtype != 0 && dtype != 1) return false;
  if (head_dim != 64 && head_dim != 128) return false;
  return group == 1 || group == 2 || group == 4 || group == 8;
}

hipError_t launch_partition_merge(const DecodeArgs &a, hipStream_t stream) {
  const uint32_t rows = (uint32_t)((int64_t)a.num_seqs * a.num_q_heads);
  const int cap = a.max_blocks_per_seq << a.log2_block_size;
  const bool pfx = a.num_groups > 0;
  const int32_t *sh = pfx ? a.shared_lens : nullptr;
  const int slots = a.num_partitions + (pfx ? 1 : 0);
  const uint32_t grid = (rows + kMergeRows - 1) / kMergeRows;
  switch (a.head_dim) {
    case 64:
      hipLaunchKernelGGL((paged_decode_merge_kernel<64>), dim3(grid), dim3(64 * kMergeRows), 0,
                         stream, a.context_lens, a.ws_o, a.ws_ml, a.out, (int)rows,
                         a.num_q_heads, cap, a.partition_size, a.num_partitions, sh, slots,
                         (int)short_members(a.kv_dtype));
      break;
    case 128:
      hipLaunchKernelGGL((paged_decode_merge_kernel<128>), dim3(grid), dim3(64 * kMergeRows), 0,
                         stream, a.context_lens, a.ws_o, a.ws_ml, a.out, (int)rows,
                         a.num_q_heads, cap, a.partition_size, a.num_partitions, sh, slots,
                         (int)short_members(a.kv_dtype));
      break;
    default: return hipErrorNotSupported;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream) {
  const int G = a.num_q_heads / a.num_kv_heads;
  const bool pfx = a.num_groups > 0;
  if (a.order && !a.order_ready) {
    const hipError_t e = launch_schedule(
        a.context_lens, a.order, a.num_seqs, a.num_partitions, a.partition_size,
        a.max_blocks_per_seq << a.log2_block_size, stream, pfx ? a.groups : nullptr,
        pfx ? a.shared_lens : nullptr, pfx ? a.num_groups : 0, G,
        pfx && short_members(a.kv_dtype));
    if (e != hipSuccess) return e;
  }
  const bool q8 = a.kv_dtype == 2 || a.kv_dtype == 3;
  // 8-bit pools at head_dim 64 (no shared-prefix items there): the vector
  // kernel, widening each vector of codes as it computes it
  if (q8 && a.head_dim == 64 && !pfx) {
    if (a.kv_dtype == 2) return launch_g<uint8_t, 64, 1>(a, stream);
    return launch_g<uint8_t, 64, 2>(a, stream);
  }
  if (q8 ||  // other 8-bit pools: the matrix-core kernel
      pfx ||  // so are shared-prefix items
      decode_mfma_supported(a.dtype, a.head_dim, G))
    return launch_decode_mfma(a, stream);
  if (a.dtype == 0) return launch_d<float>(a, stream);
  if (a.dtype == 1) return launch_d<uint16_t>(a, stream);
  return hipErrorNotSupported;
}

}  // namespace pa
