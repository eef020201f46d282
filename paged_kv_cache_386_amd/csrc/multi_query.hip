// Causal multi-query paged attention on the matrix cores of gfx950: several
// query tokens per sequence (a chunk of a long prompt, or tokens to verify),
// the chunk being the sequence's last cached positions, each token attending
// every cached position up to its own ("vLLM 深度拆解..." at chenxutan.com,
// sections 2.3, 4.3, 5.1 and 5.4; the attention itself is the one of the
// "核心代码拆解" section of the devpress.csdn.net/amd walkthrough).
//
// Here the query side is a real dense tile: the chunk's tokens times the G
// query heads of a KV head.  One workgroup (4 waves) takes 64 * RS query rows
// of one (sequence, KV head) -- rows ordered token-major, row R being token
// R / G, head R % G -- and walks the sequence's K/V in 64-token tiles through
// the block table, up to the last position its rows attend.  Each tile is
// staged in LDS once and shared by the 4 waves, each of which owns 16 * RS
// rows (RS row sets of 16):
//
//  * S^T = K Q^T on v_mfma_f32_16x16x32_bf16: A = 16 K rows from LDS (lane n
//    = lane%16 reads token n, elements 32s + 8g .. +7 with g = lane/16),
//    B = the 16 query rows of a row set, kept in registers (column n = query
//    row n).  Lane (g, n) receives the scores of query row n with tokens
//    4g .. 4g+3 of each 16-token block.
//  * O^T += V^T P^T on the same instruction: B = the probabilities as they
//    sit after the first product (a 32-token k-step takes lane (g, n)'s
//    tokens 4g .. 4g+3 of two 16-token blocks, the k order being any
//    permutation shared by A and B), A = the same tokens of V for 16 head_dim
//    elements, read from the row-major V tile with gfx950's transposing LDS
//    reads (ds_read_b64_tr_b16).  So all of a
//    lane's accumulators belong to its own query row, whose running maximum
//    and sum the lane holds: the online softmax needs no shuffles beyond the
//    two that combine a row's four lane groups per tile.
//  * The probabilities (fp32) enter the product as a bfloat16 pair hi + lo
//    (hi = p rounded, lo = the rest rounded), two MFMAs sharing one A
//    operand: the pair carries p to about 2^-16 relative, so the bfloat16
//    matrix cores give fp32-grade weights.
//  * The causal mask is applied to scores (token t > the row's position
//    gets -inf) only in tiles that reach past the workgroup's first row.
//  * Software pipeline: K runs one tile ahead of V, so each wave issues the
//    q.K products of tile t + 1 while its vector unit forms tile t's
//    probabilities, and the tiles arrive by gfx950's direct global -> LDS
//    loads (no staging registers), a full iteration ahead of their use.
//
// Workgroups are mapped to the 8 XCDs so that all row tiles of one
// (sequence, KV head), which read the same K/V, run on one XCD and share its
// L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <climits>
#include <type_traits>

#include "internal.h"

namespace pa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTk = 64;          // tokens per tile
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
constexpr int kXcds = 8;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kSlack = 8.f;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float neg_inf() { return -__builtin_huge_valf(); }

// Maximum of x over the lanes n, n + 16, n + 32 and n + 48 (the four lane
// groups of column n), with gfx950's lane-swap instructions: after
// v_permlane16_swap on two copies of x, lane l of the pair holds x of lanes
// l and l ^ 16; after v_permlane32_swap, x of lanes l and l ^ 32.
__device__ __forceinline__ float group_max4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// bfloat16 bits of a (low half) and b (high half), rounded to nearest even:
// one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t bf16x2_bits(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// Four signed 8-bit codes (one dword) to fp32 (exact).
__device__ __forceinline__ void i8x4_to_f32(uint32_t w, float (&f)[4]) {
#pragma unroll
  for (int b = 0; b < 4; ++b) f[b] = (float)((int32_t)(w << (24 - 8 * b)) >> 24);
}

// Eight 8-bit codes to eight bfloat16 values, exactly (an E4M3 value has at
// most 4 significant bits, an INT8 code at most 7): FP8 through gfx950's
// scaled conversion at scale 1 (two codes of a 16-bit half per instruction,
// the low byte into the low half; OCP E4M3), INT8 widened to fp32, whose
// high halves are the bfloat16 values, paired with one byte permute.
template <int Q8>
__device__ __forceinline__ u32x4 widen8(u32x2 w) {
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
      r[2 * h] = __builtin_amdgcn_perm(__float_as_uint(f[1]), __float_as_uint(f[0]), 0x07060302u);
      r[2 * h + 1] =
          __builtin_amdgcn_perm(__float_as_uint(f[3]), __float_as_uint(f[2]), 0x07060302u);
    }
  }
  return r;
}

// Q8: the pool's element kind -- 0 bfloat16, 1 FP8 (E4M3), 2 INT8.  An 8-bit
// tile is loaded as codes (8 bytes per chunk) and widened exactly to
// bfloat16 when it is stored to LDS, so the products are those of the
// bfloat16 pool.
template <int D, int RS, int Q8>
__global__ __launch_bounds__(kThreads, 2) void paged_multi_query_kernel(
    const uint16_t *__restrict__ q, const void *__restrict__ kc_raw,
    const void *__restrict__ vc_raw, const int32_t *__restrict__ block_tables,
    const int32_t *__restrict__ context_lens, const int32_t *__restrict__ query_start,
    float *__restrict__ out, float *__restrict__ ws_o, float *__restrict__ ws_ml, float sl2,
    float v_scale, int num_tokens, int hkv, int G, int lgB, int nb, int mb, int max_q,
    int row_tiles, int units, int ps, int P, const int32_t *__restrict__ order) {
  using KV = typename std::conditional<Q8 == 0, uint16_t, uint8_t>::type;
  const KV *__restrict__ kc = static_cast<const KV *>(kc_raw);
  const KV *__restrict__ vc = static_cast<const KV *>(vc_raw);
  constexpr int kRows = 64 * RS;  // query rows per workgroup
  constexpr int kSteps = D / 32;              // k-steps of q.K
  constexpr int kDb = D / 16;                 // 16-element blocks of the output

  // XCD-aware order.  A unit r is a KV head (r % hkv) of a (sequence,
  // partition) item (r / hkv: from the longest-first list when there is one,
  // else sequence r / hkv % S, partition from the last down); its row tiles
  // read the same K/V.  Units are dealt round-robin to the XCDs (workgroup b
  // runs on XCD b % 8), so each XCD gets every eighth unit of the list, and
  // each XCD runs its units' row tiles back to back, sharing their reads in
  // its L2.
  const int j = blockIdx.x / kXcds;
  const int r = (j / row_tiles) * kXcds + blockIdx.x % kXcds;
  const int rt = j % row_tiles;
  if (r >= units) return;
  const int kvh = r % hkv;
  const int num_seqs = units / (hkv * P);
  const int item = order ? order[r / hkv] : r / hkv;
  // listed as empty (past the sequence's end), or not an item of this launch
  // (a list the caller planned is trusted only this far)
  if (item < 0 || item >= units / hkv) return;
  const int s = item % num_seqs;
  const int part = (P - 1) - item / num_seqs;
  const int hq = hkv * G;

  int L = context_lens[s];
  L = max(0, min(L, mb << lgB));
  const int qs = max(0, min(query_start[s], num_tokens));
  int n = query_start[s + 1] - qs;
  n = max(0, min(min(n, L), min(max_q, num_tokens - qs)));
  const int rows = n * G;
  const int row0 = rt * kRows;
  if (row0 >= rows) return;
  const int row_end = min(row0 + kRows, rows);
  // positions attended by the workgroup: [0, pos_last]; tiles wholly below
  // pos_first need no mask
  const int pos_first = L - n + row0 / G;
  const int pos_last = L - n + (row_end - 1) / G;
  // this partition's tiles: [k_begin, k_end) (ps is a multiple of the tile)
  const int k_begin = part * ps;
  if (k_begin > pos_last) return;
  const int k_end = min(k_begin + ps, pos_last + 1);
  const int ntiles = (k_end - k_begin + kTk - 1) / kTk;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g4 = lane >> 4;
  const int c16 = lane & 15;
  const int32_t *tbl = block_tables + (int64_t)s * mb;
  const int bm1 = (1 << lgB) - 1;
  const int64_t head_off = (int64_t)kvh * (D << lgB);
  const int64_t block_elems = ((int64_t)hkv * D) << lgB;

  // this lane's query rows (one per row set), their positions and the B
  // operand of q.K; sl2 becomes |sl2| once q carries the scale's sign
  int pos[RS];
  bf16x8 qb[RS][kSteps];
#pragma unroll
  for (int r = 0; r < RS; ++r) {
    const int R = row0 + (wave * RS + r) * 16 + c16;
    const bool active = R < rows;
    const int tok = R / G;
    pos[r] = active ? L - n + tok : -1;
#pragma unroll
    for (int k = 0; k < kSteps; ++k) qb[r][k] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
    if (active) {
      const uint16_t *qrow = q + ((int64_t)(qs + tok) * hq + kvh * G + R % G) * D + 8 * g4;
      // a negative scale moves onto q (exact sign flips), so sl2 >= 0 below
      const uint32_t flip = sl2 < 0.f ? 0x80008000u : 0u;
#pragma unroll
      for (int k = 0; k < kSteps; ++k)
        qb[r][k] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4 *>(qrow + 32 * k) ^ u32x4{flip, flip, flip, flip});
    }
  }
  sl2 = fmaxf(__builtin_fabsf(sl2), 1.17549435e-38f);
  // kSlack in raw score units, kept finite so that the first tile with a
  // finite maximum always sets m (-inf + slack stays -inf)
  const float slack = fminf(kSlack / sl2, 3.40282347e38f);

  // K and V tiles in LDS as unpadded rows of 2 D bytes whose 16-byte chunks
  // are permuted per row (chunk c of row t stored at c ^ swz(t)), so that
  // the 16-row reads of K and the transposing reads of V (4 rows x 32 bytes
  // per 16 lanes) meet every bank once.  A tile is filled in 1 KB groups:
  // group j of wave w is bytes [1024 (4 j + w), +1024), lane l writing its
  // 16 bytes at 16 l -- the layout of gfx950's direct global -> LDS loads,
  // which bfloat16 pools use (8-bit codes arrive the same way and are
  // widened in LDS, see below).  K runs one tile ahead of V (the scores of
  // tile t + 1 are computed while tile t's probabilities are formed); in
  // iteration t the waves read K(t + 1) and V(t) while K(t + 2) and V(t + 1)
  // arrive in the other two buffers.
  constexpr int kCpr = D / 8;            // 16-byte chunks per row
  constexpr int kRpb = 16 / kCpr;        // rows per 256 bytes (all 64 banks)
  constexpr int kRpg = 512 / D;          // rows per 1 KB group
  constexpr int kGroups = D / 32;        // 1 KB groups per wave and tile
  // (four separate arrays, each named statically in the loop below: the
  // compiler then knows that reading one buffer never waits for the direct
  // loads into another)
  __shared__ __attribute__((aligned(1024))) uint16_t sk0[kTk * D];
  __shared__ __attribute__((aligned(1024))) uint16_t sk1[kTk * D];
  __shared__ __attribute__((aligned(1024))) uint16_t sv0[kTk * D];
  __shared__ __attribute__((aligned(1024))) uint16_t sv1[kTk * D];
  // Byte addresses of each token's K and V rows (this KV head) for three
  // consecutive tiles (tile j in slot j % 3), written by the 64 threads that
  // read the block table, one tile ahead of the loads that use them: the
  // table read and the row reads never wait on each other, and a lane's
  // load address is one add.
  __shared__ __attribute__((aligned(16))) uint64_t sadr[3][kTk][2];
  auto swz_k = [](int t) { return (t / kRpb) & (kCpr - 1); };
  auto swz_v = [](int t) { return 2 * ((t / kRpb) & (kCpr / 2 - 1)); };

  auto table_entry = [&](int k0) -> uint32_t {  // token k0 + threadIdx.x (< 64 threads)
    const int tok = k0 + (int)threadIdx.x;
    return tok <= pos_last ? min((uint32_t)tbl[tok >> lgB], (uint32_t)(nb - 1)) : 0u;
  };

  constexpr int kEs = Q8 ? 1 : 2;  // bytes per element
  const uint64_t kbase = (uint64_t)kc + (uint64_t)head_off * kEs;
  const uint64_t vbase = (uint64_t)vc + (uint64_t)head_off * kEs;
  const uint64_t block_bytes = (uint64_t)block_elems * kEs;
  auto put_addrs = [&](int slot, int k0, uint32_t id) {  // threads < 64
    const int tok = k0 + (int)threadIdx.x;
    const uint64_t off = (uint64_t)id * block_bytes + (uint64_t)((tok & bm1) * D * kEs);
    *reinterpret_cast<u64x2 *>(&sadr[slot][threadIdx.x][0]) = u64x2{kbase + off, vbase + off};
  };

  // This lane's share of a tile: in group j, row t0 + kRpg kWaves j, stored
  // chunk lane % kCpr, which holds the row's chunk (lane % kCpr) ^ swz(row)
  // -- the same chunk in every group.  Tokens past pos_last have table entry
  // 0, so every address is a row of the pool.
  const int grow = lane / kCpr;
  const int t0 = kRpg * wave + grow;
  const uint32_t ck = 16 * ((lane % kCpr) ^ swz_k(t0));  // byte offset in the row
  const uint32_t cv = 16 * ((lane % kCpr) ^ swz_v(t0));
  auto row_addr = [&](int slot, int j, bool is_v) -> uint64_t {
    return sadr[slot][t0 + kRpg * kWaves * j][is_v] + (is_v ? cv : ck);
  };
  auto lds_group = [&](uint16_t *buf, int j) { return buf + 512 * (kWaves * j + wave); };
  // bfloat16: the loads write LDS themselves
  auto dma_rows = [&](uint16_t *buf, int slot, bool is_v) {
#pragma unroll
    for (int j = 0; j < kGroups; ++j)
      __builtin_amdgcn_global_load_lds(
          (const void *)row_addr(slot, j, is_v),
          (__attribute__((address_space(3))) void *)lds_group(buf, j), 16, 0, 0);
  };
  // through registers: a bfloat16 V tile holding tokens past pos_last, whose
  // rows there are zeroed (p = 0 there, and 0 * NaN would not vanish; K rows
  // there only meet masked scores)
  auto fetch_v_tail = [&](uint16_t *buf, int k0, int slot) {
    u32x4 R[kGroups];
#pragma unroll
    for (int j = 0; j < kGroups; ++j) {
      const u32x4 x =
          *reinterpret_cast<const __attribute__((address_space(1))) u32x4 *>(row_addr(slot, j, true));
      R[j] = k0 + t0 + kRpg * kWaves * j <= pos_last ? x : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < kGroups; ++j)
      *reinterpret_cast<u32x4 *>(lds_group(buf, j) + 8 * lane) = R[j];
  };

  // 8-bit pools.  A tile's codes are loaded directly in 1 KB groups too:
  // group g = 4 j + wave holds rows kQRows g .. +kQRows-1 (16 codes per
  // lane) and lands in the first half of the 2 KB those rows take as
  // bfloat16.  The wave that loaded a group widens it there: it reads the
  // codes, then writes the rows over the same 2 KB, which no other wave
  // touches, so the rewrite needs no barrier of its own (LDS serves a
  // wave's instructions in order, and the writes wait on the read's data).
  constexpr int kQGroups = D / 64;  // code groups per wave and tile
  constexpr int kQRows = 1024 / D;  // rows per code group
  constexpr int kQcpr = D / 16;     // 16-code chunks per row
  auto dma_codes = [&](uint16_t *buf, int slot, bool is_v) {
#pragma unroll
    for (int j = 0; j < kQGroups; ++j) {
      const int g = kWaves * j + wave;
      const int t = kQRows * g + lane / kQcpr;
      __builtin_amdgcn_global_load_lds(
          (const void *)(sadr[slot][t][is_v] + 16 * (lane % kQcpr)),
          (__attribute__((address_space(3))) void *)(buf + 1024 * g), 16, 0, 0);
    }
  };
  auto expand_codes = [&](uint16_t *buf, int k0, bool is_v) {
    // this wave's direct loads of the codes must have landed.  Placed by
    // hand: the compiler's own wait is missing on the path where the K
    // tile's expansion before this one is skipped, and codes that land after
    // the rewrite would leave raw bytes among the bfloat16 rows.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
#pragma unroll
    for (int j = 0; j < kQGroups; ++j) {
      const int g = kWaves * j + wave;
      const int t = kQRows * g + lane / kQcpr;
      const u32x4 codes = *reinterpret_cast<const u32x4 *>(buf + 1024 * g + 8 * lane);
      u32x4 lo = widen8<Q8>(u32x2{codes[0], codes[1]});
      u32x4 hi = widen8<Q8>(u32x2{codes[2], codes[3]});
      if (is_v && k0 + t > pos_last) lo = hi = u32x4{0, 0, 0, 0};
      const int c = 2 * (lane % kQcpr);
      const int sw = is_v ? swz_v(t) : swz_k(t);
      *reinterpret_cast<u32x4 *>(buf + t * D + 8 * (c ^ sw)) = lo;
      *reinterpret_cast<u32x4 *>(buf + t * D + 8 * ((c + 1) ^ sw)) = hi;
    }
  };

  // S^T of one tile into sc, less the running maximum: the first product of
  // each chain starts from seed[r] = (-m, -m, -m, -m) of the lane's row (0
  // while m is -inf), so the scores come out relative to m and the softmax
  // needs no subtraction per score.  k-step outermost, so that the 4 * RS
  // accumulator chains interleave and no product waits on the one before it.
  // Row 16 tb + c16 keeps swz_k(c16) for every tb.
  const int sk_lane = c16 * D;
  const int swk = swz_k(c16);
  f32x4 seed[RS];
  auto scores = [&](f32x4 (&sc)[RS][4], const uint16_t *sk) {
#pragma unroll
    for (int k = 0; k < kSteps; ++k) {
      const uint16_t *kp = sk + sk_lane + 8 * ((4 * k + g4) ^ swk);
      bf16x8 a[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
        a[tb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(kp + 16 * tb * D));
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int r = 0; r < RS; ++r)
          sc[r][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[tb], qb[r][k],
                                                              k ? sc[r][tb] : seed[r], 0, 0, 0);
    }
  };
  // V rows 32 kk + 16 h + 4 g4 + c16 / 4 keep swz_v(4 g4 + c16 / 4)
  const int sv_lane = (4 * g4 + c16 / 4) * D + 4 * (c16 & 1);
  const int swv = swz_v(4 * g4 + c16 / 4);

  f32x4 acc[RS][kDb];
#pragma unroll
  for (int r = 0; r < RS; ++r)
#pragma unroll
    for (int b = 0; b < kDb; ++b) acc[r][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[RS], lsum[RS];
#pragma unroll
  for (int r = 0; r < RS; ++r) {
    m[r] = neg_inf();
    lsum[r] = 0.f;
    seed[r] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // bfloat16 V tile at k0 into buf: directly, or through registers when it
  // runs past pos_last (at most the last tile)
  auto fetch_v = [&](uint16_t *buf, int k0, int slot) {
    if (k0 + kTk - 1 <= pos_last)
      dma_rows(buf, slot, true);
    else
      fetch_v_tail(buf, k0, slot);
  };

  // Prologue: block ids of tiles 0..2, K and V of tile 0, K of tile 1, and
  // the scores of tile 0.
  uint32_t id_next = 0;
  if (threadIdx.x < kTk) {
    put_addrs(0, k_begin, table_entry(k_begin));
    put_addrs(1, k_begin + kTk, ntiles > 1 ? table_entry(k_begin + kTk) : 0u);
  }
  __syncthreads();
  if constexpr (Q8 == 0) {
    dma_rows(sk0, 0, false);
    if (ntiles > 1) dma_rows(sk1, 1, false);
    fetch_v(sv0, k_begin, 0);
  } else {
    dma_codes(sk0, 0, false);
    if (ntiles > 1) dma_codes(sk1, 1, false);
    dma_codes(sv0, 0, true);
    expand_codes(sk0, k_begin, false);
    if (ntiles > 1) expand_codes(sk1, k_begin + kTk, false);
    expand_codes(sv0, k_begin, true);
  }
  if (threadIdx.x < kTk)
    put_addrs(2, k_begin + 2 * kTk, ntiles > 2 ? table_entry(k_begin + 2 * kTk) : 0u);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's direct loads are in LDS
  __syncthreads();
  if (threadIdx.x < kTk && ntiles > 3) id_next = table_entry(k_begin + 3 * kTk);
  f32x4 sc[RS][4];
  scores(sc, sk0);
  __syncthreads();  // every wave is done with K(0) before K(2) replaces it

  // Iteration it (of parity P, a compile-time constant in each half of the
  // unrolled loop): reads K(it + 1) from sk[1 - P] and V(it) from sv[P].
  int slot = 0;  // it % 3
  auto iteration = [&](auto parity, int it) {
    constexpr int P = decltype(parity)::value;
    uint16_t *const sk_this = P ? sk1 : sk0;  // K(it), then K(it + 2)
    uint16_t *const sk_next = P ? sk0 : sk1;  // K(it + 1)
    uint16_t *const sv_this = P ? sv1 : sv0;  // V(it)
    uint16_t *const sv_next = P ? sv0 : sv1;  // V(it - 1), then V(it + 1)
    const int k0 = k_begin + it * kTk;
    const int slot1 = slot == 2 ? 0 : slot + 1;
    const int slot2 = slot1 == 2 ? 0 : slot1 + 1;
    // K(it + 2) into the buffer K(it) left (last read in iteration it - 1),
    // V(it + 1) into the one V(it - 1) left: they land during this
    // iteration (8-bit codes are widened at its end).
    if constexpr (Q8 == 0) {
      if (it + 2 < ntiles) dma_rows(sk_this, slot2, false);
      if (it + 1 < ntiles) fetch_v(sv_next, k0 + kTk, slot1);
    } else {
      if (it + 2 < ntiles) dma_codes(sk_this, slot2, false);
      if (it + 1 < ntiles) dma_codes(sv_next, slot1, true);
    }

    // Online softmax of tile it.  The running maximum m is kept on the raw
    // scores (sl2 > 0: q carries a negative scale's sign, and a zero scale
    // is raised to the least normal float, which gives every unmasked p = 1
    // as zero does).  The tile's scores arrive as x - m (x while m is -inf,
    // from the seed they were issued with), and p = 2^((x - m) sl2).  When
    // the tile's maximum passes m + slack, m moves to it and the scores shift
    // by the same amount, so p is exactly 1 at the new maximum.  Masked
    // positions (only in tiles that reach past the workgroup's first row)
    // become -inf, so p = 0.
    const bool masked = k0 + kTk - 1 > pos_first;
#pragma unroll
    for (int r = 0; r < RS; ++r) {
      if (masked) {
        // token k0 + 16 tb + 4 g4 + i lies past the row's position
        const int lim = pos[r] - k0 - 4 * g4;
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (16 * tb + i > lim) sc[r][tb][i] = neg_inf();
      }
      float cm = neg_inf();
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) cm = fmaxf(cm, sc[r][tb][i]);
      cm = group_max4(cm);  // relative to m (raw while m is -inf)
      const bool first = m[r] == neg_inf();
      // the tile's maximum passes m + slack (any finite score while m is
      // -inf); wave-uniform branch (lanes that need no rescale scale by
      // exactly 1 and shift by 0), so the accumulators are updated in place
      const bool up = first ? cm > neg_inf() : cm > slack;
      if (__builtin_amdgcn_ballot_w64(up)) {
        // 0 when m was -inf (nothing accumulated yet)
        const float alpha = up ? (first ? 0.f : __builtin_amdgcn_exp2f(-cm * sl2)) : 1.f;
        const float shift = up ? cm : 0.f;
        lsum[r] *= alpha;
#pragma unroll
        for (int b = 0; b < kDb; ++b) acc[r][b] *= alpha;
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) sc[r][tb] -= shift;
        m[r] = up ? (first ? cm : m[r] + cm) : m[r];
        seed[r] = up ? f32x4{-m[r], -m[r], -m[r], -m[r]} : seed[r];
      }
    }

    // The scores of tile it + 1 on the matrix cores while the vector unit
    // turns tile it's scores into the hi/lo probability operands (on the
    // last tile the products read a stale buffer and are discarded).
    __builtin_amdgcn_s_setprio(1);
    f32x4 sn[RS][4];
    scores(sn, sk_next);
    bf16x8 phi[RS][2], plo[RS][2];
#pragma unroll
    for (int r = 0; r < RS; ++r) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          float pr[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int jj = j + u;
            const int tb = 2 * kk + (jj >> 2);
            pr[u] = __builtin_amdgcn_exp2f(sc[r][tb][jj & 3] * sl2);
          }
          lsum[r] += pr[0] + pr[1];
          const uint32_t h = bf16x2_bits(pr[0], pr[1]);
          hw[j >> 1] = h;
          lw[j >> 1] = bf16x2_bits(pr[0] - __uint_as_float(h << 16),
                                   pr[1] - __uint_as_float(h & 0xFFFF0000u));
        }
        phi[r][kk] = __builtin_bit_cast(bf16x8, u32x4{hw[0], hw[1], hw[2], hw[3]});
        plo[r][kk] = __builtin_bit_cast(bf16x8, u32x4{lw[0], lw[1], lw[2], lw[3]});
      }
    }

    // O^T += V^T P^T.  gfx950's transposing LDS read: within each 16-lane
    // group, lane c points at 4 elements of row (base + c / 4) and receives,
    // from the rows base .. base + 3, the element in its own column -- here
    // element 16 b + c16 of tokens 32 kk + 4 g4 + 0..3 (and + 16).
    const uint16_t *sv = sv_this + sv_lane;
#pragma unroll
    for (int b = 0; b < kDb; ++b) {
      const uint16_t *vb = sv + 8 * ((2 * b + ((c16 & 3) >> 1)) ^ swv);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const u32x2 lo = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(vb + 32 * kk * D)));
        const u32x2 hi = __builtin_bit_cast(
            u32x2,
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(vb + (32 * kk + 16) * D)));
        const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
        for (int r = 0; r < RS; ++r) {
          acc[r][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, phi[r][kk], acc[r][b], 0, 0, 0);
          acc[r][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, plo[r][kk], acc[r][b], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int r = 0; r < RS; ++r)
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) sc[r][tb] = sn[r][tb];

    if constexpr (Q8 != 0) {
      if (it + 2 < ntiles) expand_codes(sk_this, k0 + 2 * kTk, false);
      if (it + 1 < ntiles) expand_codes(sv_next, k0 + kTk, true);
    }
    // the ids of tile it + 3 into the slot of tile it (last read when V(it)
    // was fetched)
    if (threadIdx.x < kTk && it + 3 < ntiles) put_addrs(slot, k0 + 3 * kTk, id_next);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's direct loads are in LDS
    __syncthreads();
    if (threadIdx.x < kTk && it + 4 < ntiles) id_next = table_entry(k0 + 4 * kTk);
    slot = slot1;
  };
  for (int it = 0; it < ntiles; it += 2) {
    iteration(std::integral_constant<int, 0>{}, it);
    if (it + 1 < ntiles) iteration(std::integral_constant<int, 1>{}, it + 1);
  }
  // normalise and write: lane (g4, c16) holds row c16 of each row set,
  // elements 16 b + 4 g4 .. +3.  A sequence whose context fits in one
  // partition goes straight to out (the merge skips it); the others leave
  // (max, sum, output) partials for the merge.
  const bool split = min((L + ps - 1) / ps, P) > 1;
#pragma unroll
  for (int r = 0; r < RS; ++r) {
    float l = lsum[r];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const int R = row0 + (wave * RS + r) * 16 + c16;
    if (R < row_end) {
      // (8-bit pools: the V scale multiplies the normalised output)
      const float inv = l > 0.f ? v_scale / l : 0.f;
      const int64_t orow = (int64_t)(qs + R / G) * hq + kvh * G + R % G;
      float *o = split ? ws_o + (orow * P + part) * D : out + orow * D;
#pragma unroll
      for (int b = 0; b < kDb; ++b)
        *reinterpret_cast<f32x4 *>(o + 16 * b + 4 * g4) = acc[r][b] * inv;
      if (split && g4 == 0) {
        ws_ml[(orow * P + part) * 2 + 0] = m[r] * sl2;  // log2 units
        ws_ml[(orow * P + part) * 2 + 1] = l;
      }
    }
  }
}

// Merge of the partition partials of the (query token, head) rows, one wave
// per row, kMqMergeRows rows per workgroup: row (s, i, h) is head h of token
// i of sequence s's chunk, and, when the sequence was split or has a shared
// prefix, combines its prefix partial (the row's last slot) and the
// partitions with private positions that the token's position reaches
// (log-sum-exp weights, prefix first, then ascending partition order).  Rows
// of sequences that fit in one partition and share no prefix were written
// to out directly.
constexpr int kMqMergeRows = 4;
// partials of a row loaded in one batch (as in the decode merge)
constexpr int kMqMergeAhead = 3;
template <int D>
__global__ __launch_bounds__(64 * kMqMergeRows) void paged_multi_query_merge_kernel(
    const int32_t *__restrict__ context_lens, const int32_t *__restrict__ query_start,
    const float *__restrict__ ws_o, const float *__restrict__ ws_ml, float *__restrict__ out,
    int num_tokens, int hq, int cap, int max_q, int ps, int P, int64_t rows,
    const int32_t *__restrict__ shared_lens, int slots) {
  constexpr int EPL = D / 64;  // elements per lane
  const int64_t rr =
      (int64_t)blockIdx.x * kMqMergeRows + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (rr >= rows) return;
  const int h = (int)(rr % hq);
  const int i = (int)((rr / hq) % max_q);
  const int s = (int)(rr / ((int64_t)hq * max_q));
  int L = context_lens[s];
  L = max(0, min(L, cap));
  const int sh = shared_lens ? min(max(shared_lens[s], 0), L) & ~15 : 0;
  if (min((L + ps - 1) / ps, P) <= 1 && sh == 0) return;  // written to out directly
  const int first = sh / ps;  // the first partition with private positions
  const int qs = max(0, min(query_start[s], num_tokens));
  int n = query_start[s + 1] - qs;
  n = max(0, min(min(n, L), min(max_q, num_tokens - qs)));
  if (i >= n) return;  // no such token in the chunk
  const int pos = L - n + i;
  const int np = min(pos / ps + 1, P);
  const int64_t row = (int64_t)(qs + i) * hq + h;
  const float *ml = ws_ml + row * slots * 2;
  const float *o = ws_o + row * slots * D + (threadIdx.x & 63) * EPL;
  const int pre = slots - 1;  // the prefix slot (used when sh > 0)
  // the partials in merge order (the prefix's, then the private partitions
  // ascending); the first kMqMergeAhead are loaded (max, sum and rows) in
  // one batch, so their rows do not wait on the maximum
  const int cnt = (sh > 0 ? 1 : 0) + max(np - first, 0);
  auto slot_at = [&](int k) { return sh > 0 ? (k == 0 ? pre : first + k - 1) : first + k; };
  float am[kMqMergeAhead], al[kMqMergeAhead], ao[kMqMergeAhead][EPL];
#pragma unroll
  for (int k = 0; k < kMqMergeAhead; ++k) {
    am[k] = neg_inf();
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
  float M = neg_inf();
#pragma unroll
  for (int k = 0; k < kMqMergeAhead; ++k) M = fmaxf(M, am[k]);
  for (int k = kMqMergeAhead; k < cnt; ++k) M = fmaxf(M, ml[2 * slot_at(k)]);
  float num[EPL], den = 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) num[e] = 0.f;
  auto add = [&](float mj, float lj, const float *oj) {
    const float w = mj == neg_inf() ? 0.f : lj * __builtin_amdgcn_exp2f(mj - M);
#pragma unroll
    for (int e = 0; e < EPL; ++e) num[e] = fmaf(w, oj[e], num[e]);
    den += w;
  };
#pragma unroll
  for (int k = 0; k < kMqMergeAhead; ++k)
    if (k < cnt) add(am[k], al[k], ao[k]);
  for (int k = kMqMergeAhead; k < cnt; ++k) {
    const int j = slot_at(k);
    float oj[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) oj[e] = o[(int64_t)j * D + e];
    add(ml[2 * j], ml[2 * j + 1], oj);
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e)
    out[row * D + (threadIdx.x & 63) * EPL + e] = den > 0.f ? num[e] / den : 0.f;
}

hipError_t launch_merge(const MultiQueryArgs &a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.num_seqs * a.max_query_len * a.num_q_heads;
  if (rows <= 0) return hipSuccess;
  const bool pfx = a.num_groups > 0;
  const int slots = a.num_partitions + (pfx ? 1 : 0);
  const int cap = (int)std::min<int64_t>((int64_t)a.max_blocks_per_seq << a.log2_block_size,
                                         INT32_MAX);
  const uint32_t grid = (uint32_t)((rows + kMqMergeRows - 1) / kMqMergeRows);
  if (a.head_dim == 64)
    hipLaunchKernelGGL((paged_multi_query_merge_kernel<64>), dim3(grid), dim3(64 * kMqMergeRows),
                       0, stream, a.context_lens, a.query_start, a.ws_o, a.ws_ml, a.out,
                       a.num_tokens, a.num_q_heads, cap, a.max_query_len, a.partition_size,
                       a.num_partitions, rows, pfx ? a.shared_lens : nullptr, slots);
  else
    hipLaunchKernelGGL((paged_multi_query_merge_kernel<128>), dim3(grid), dim3(64 * kMqMergeRows),
                       0, stream, a.context_lens, a.query_start, a.ws_o, a.ws_ml, a.out,
                       a.num_tokens, a.num_q_heads, cap, a.max_query_len, a.partition_size,
                       a.num_partitions, rows, pfx ? a.shared_lens : nullptr, slots);
  return hipGetLastError();
}

template <int D, int RS, int Q8>
hipError_t launch_typed(const MultiQueryArgs &a, hipStream_t stream) {
  const int G = a.num_q_heads / a.num_kv_heads;
  const int64_t rows = (int64_t)a.max_query_len * G;
  const int row_tiles = (int)((rows + 64 * RS - 1) / (64 * RS));
  const int64_t units = (int64_t)a.num_seqs * a.num_kv_heads * a.num_partitions;
  if (units <= 0 || row_tiles <= 0) return hipSuccess;
  const int64_t grid = (units + kXcds - 1) / kXcds * kXcds * row_tiles;
  // 8-bit pools: the K scale multiplies every score, so it joins the softmax
  // scale; the V scale multiplies the output
  const float sl2 = a.scale * (Q8 ? a.k_scale : 1.f) * kLog2e;
  hipLaunchKernelGGL((paged_multi_query_kernel<D, RS, Q8>), dim3((uint32_t)grid), dim3(kThreads),
                     0, stream, static_cast<const uint16_t *>(a.q), a.k_cache, a.v_cache,
                     a.block_tables, a.context_lens, a.query_start, a.out, a.ws_o, a.ws_ml, sl2,
                     Q8 ? a.v_scale : 1.f, a.num_tokens, a.num_kv_heads, G, a.log2_block_size,
                     a.num_blocks, a.max_blocks_per_seq, a.max_query_len, row_tiles, (int)units,
                     a.partition_size, a.num_partitions, a.order);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.num_partitions <= 1) return e;
  return launch_merge(a, stream);
}

template <int D, int Q8>
hipError_t launch_d(const MultiQueryArgs &a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.max_query_len * (a.num_q_heads / a.num_kv_heads);
  if (rows > 64) return launch_typed<D, 2, Q8>(a, stream);
  return launch_typed<D, 1, Q8>(a, stream);
}

template <int D>
hipError_t launch_kind(const MultiQueryArgs &a, hipStream_t stream) {
  switch (a.kv_dtype) {
    case 2: return launch_d<D, 1>(a, stream);  // FP8 E4M3
    case 3: return launch_d<D, 2>(a, stream);  // INT8
    default: return launch_d<D, 0>(a, stream);
  }
}

}  // namespace

bool multi_query_supported(int32_t dtype, int32_t head_dim) {
  return dtype == 1 && (head_dim == 64 || head_dim == 128);
}

int64_t multi_query_workgroups(int64_t num_seqs, int64_t num_q_heads, int64_t num_kv_heads,
                               int64_t head_dim, int64_t max_query_len, int64_t P) {
  const int64_t rows = max_query_len * (num_q_heads / num_kv_heads);
  const int64_t units = num_seqs * num_kv_heads * P;
  if (head_dim == 128 && rows <= kMqFewRows)  // the decode walk: 16-row column sets
    return (units + kXcds - 1) / kXcds * kXcds * multi_query_few_rows_groups((rows + 15) / 16);
  const int64_t rs = rows > 64 ? 2 : 1;
  return (units + kXcds - 1) / kXcds * kXcds * ((rows + 64 * rs - 1) / (64 * rs));
}

hipError_t launch_multi_query(const MultiQueryArgs &a, hipStream_t stream) {
  if (a.order && !a.order_ready) {
    const int cap = (int)std::min<int64_t>((int64_t)a.max_blocks_per_seq << a.log2_block_size,
                                           INT32_MAX);
    const bool pfx = a.num_groups > 0;
    const hipError_t e = launch_schedule(
        a.context_lens, a.order, a.num_seqs, a.num_partitions, a.partition_size, cap, stream,
        pfx ? a.groups : nullptr, pfx ? a.shared_lens : nullptr, pfx ? a.num_groups : 0, 0,
        false,
        pfx ? (int)mq_prefix_items_per_group(a.max_query_len, a.num_q_heads / a.num_kv_heads)
            : 4);
    if (e != hipSuccess) return e;
  }
  if (multi_query_few_rows_supported(a)) {
    // a few rows per KV head: the decode walk, one wave per 16-token tile
    hipError_t e = launch_multi_query_few_rows(a, stream);
    if (e != hipSuccess || (a.num_partitions <= 1 && a.num_groups == 0)) return e;
    return launch_merge(a, stream);
  }
  switch (a.head_dim) {
    case 64: return launch_kind<64>(a, stream);
    case 128: return launch_kind<128>(a, stream);
    default: return hipErrorNotSupported;
  }
}

}  // namespace pa
