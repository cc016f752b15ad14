// Mixed W4/W8 x A8 GEMM of the W4.4A8 layer for gfx950 (MI355X), with scatter epilogue.
//
// Method (MixLLM talk notes, 二段階逆量子化 "two-step dequantization"): per group of 128
// inputs, (1) partially dequantize the 4-bit weights to (W_q - z), which fits int8,
// (2) multiply with the int8 activations on the int8 matrix cores into an exact int32
// group partial, (3) scale the partial by s_w * s_a and add it to an fp32 accumulator
// (the per-group / global double accumulator of the summary page, 核心方法).  The 4-bit
// and 8-bit output channels form two disjoint sub-GEMMs (talk notes, 並列実行 "parallel
// execution"); here both run in one grid, each wave handling one 32-channel block of one
// subset, and the epilogue writes every channel's fp16 result to its original index.
//
// Differences from the pages' A100 design, for CDNA4:
//  * (W_q - z) is formed with byte-wise SWAR arithmetic on packed nibbles:
//    ((q | 0x80) - z) ^ 0x80 per byte, four codes per 32-bit op (the role of the pages'
//    vsub4; CDNA has no byte-vector subtract).
//  * int32 -> fp32 uses v_cvt_f32_i32, a full-rate VALU op on CDNA; the pages' 0x4b400000
//    bias trick replaces a slow conversion on their GPU and buys nothing here.
//  * The tile kernel stages the activation tile through LDS (shared by the four waves of
//    a workgroup) and streams each wave's own weights straight from HBM into registers,
//    one group ahead; the skinny kernel (small M) streams both from L2/HBM and splits the
//    groups over the waves of a workgroup, reducing through LDS.
//
// MFMA layouts used (gfx950):
//  * v_mfma_i32_32x32x32_i8: lane l supplies row/column (l % 32) and 16 bytes of k; the
//    two half-waves h = l / 32 cover the two 16-wide k halves.  Output register r of lane
//    l is row 8 (r / 4) + 4 h + (r % 4), column l % 32.
//  * v_mfma_i32_16x16x64_i8: lane l supplies row/column (l % 16), quarter q = l / 16 covers
//    16 of the 64 k.  Output register r of lane l is row 4 q + r, column l % 16.
//  The contraction is order-free, so any assignment of k to (lane group, byte) works as
//  long as both operands use the same one; the packer lays the weights out for the
//  assignment below and the activation reads follow it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mixllm.h"
#include "mixllm_layout.h"

namespace mixllm {
bool is_aligned16(const void *p);
}

namespace {

using namespace mixllm;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

struct GemmArgs {
  const int8_t *aq;
  const float *sa;
  const int32_t *asum;
  int M, N, K, G;
  const uint8_t *w4;
  const uint16_t *s4;
  const uint8_t *z4;
  const uint8_t *w8;
  const uint16_t *s8;
  const int32_t *idx;
  int n4, nb, nb4;
  uint16_t *y;
  int64_t ldy;
  int32_t *part;  // partials mode output [M][n_count][G]
  int n_begin, n_count;
  int tiles_m, tiles_n;
  int ks;       // split-K factor of the tile kernel
  float *ws;    // split-K partial tiles [tiles][ks][64 * 128]
  int *cnt;     // split-K arrival counters [tiles], zero between launches
};

__device__ __forceinline__ float h2f(uint16_t bits) { return (float)__builtin_bit_cast(_Float16, bits); }
__device__ __forceinline__ uint16_t f2h(float v) { return __builtin_bit_cast(uint16_t, (_Float16)v); }

// Four 4-bit codes (one per byte, 0..15) minus the zero point z (zz = z * 0x01010101),
// as four signed bytes in [-15, 15].  Biasing each byte by 0x80 keeps the subtraction
// from borrowing across bytes; the xor removes the bias.
__device__ __forceinline__ int w4_sub(uint32_t nib, uint32_t zz) {
  return (int)(((nib | 0x80808080u) - zz) ^ 0x80808080u);
}

// 16 int8 weight operands from 8 bytes of packed nibbles (words x0, x1).
__device__ __forceinline__ v4i w4_operand(uint32_t x0, uint32_t x1, uint32_t zz) {
  v4i r;
  r[0] = w4_sub(x0 & 0x0F0F0F0Fu, zz);
  r[1] = w4_sub((x0 >> 4) & 0x0F0F0F0Fu, zz);
  r[2] = w4_sub(x1 & 0x0F0F0F0Fu, zz);
  r[3] = w4_sub((x1 >> 4) & 0x0F0F0F0Fu, zz);
  return r;
}

__device__ __forceinline__ v4i ldg16(const void *p) { return *reinterpret_cast<const v4i *>(p); }

// The zero point held in the low (odd = 0) or high (odd = 1) nibble of byte zb, copied
// into all four bytes of a word (v_perm_b32 broadcast, then shift and mask).
__device__ __forceinline__ uint32_t zero_point_x4(uint32_t zb, int odd) {
  const uint32_t b4 = __builtin_amdgcn_perm(0u, zb, 0x00000000u);
  return (b4 >> (odd * 4)) & 0x0F0F0F0Fu;
}

// k-chunk (16 inputs) read by half-wave h at 32-wide step s of a group, 32x32x32 kernels.
// Steps 2p and 2p+1 of half h use chunks 2p+h and 2p+h+4: the two halves of one packed
// 4-bit unit.
__device__ __forceinline__ int chunk32(int s, int h) { return 4 * (s & 1) + 2 * (s >> 1) + h; }

template <int V>
struct IntC {
  static constexpr int value = V;
};

// Calls f(IntC<B>{}), ..., f(IntC<E-1>{}): compile-time indices for register rings.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (B < E) {
    f(IntC<B>{});
    static_for<B + 1, E>(f);
  }
}

// ------------------------------------------------------------------------------------
// Tile kernel: a workgroup of 4 waves owns 64 rows x 128 channels (4 blocks of 32); wave w
// computes block 4 tn + w for all 64 rows, one wave per SIMD.
//
// Per group and 32x32 output block a wave issues
//   * 4 x v_mfma_i32_32x32x32_i8: the group partial.  4-bit blocks feed the raw codes q;
//     the zero point is removed in the float domain (below), so decoding costs 3 VALU
//     ops per 8 codes;
//   * 1 x v_mfma_f32_32x32x16_bf16: the scale products s_a[m] s_w[n] of the whole block
//     as an outer product of exact bf16 splits (s_a = a0 + a1 + a2, s_w = b0 + b1);
//   * 4-bit blocks only: 1 x v_mfma_f32_32x32x16_bf16 that subtracts
//     (S_A[m] s_a[m]) (z[n] s_w[n]) from the accumulator, S_A being the group's code sum:
//     sum_k (q - z) a_k s_a s_w = s_a s_w sum_k q a_k - (S_A s_a) (z s_w);
//   * the fold acc += float(P) * scale: 2 VALU ops per output element.
// The integer partial is exact; only the fp32 fold differs from the fp64 definition.
//
// Two workgroups per CU: each CU runs two independent workgroups (two waves per SIMD)
// with their own barriers, so one wave's matrix-core phase overlaps the other's VALU
// phase.  When the grid has too few tiles for that, the groups of a tile are split over
// KS workgroups (contiguous ranges); each writes its fp32 partial tile to the workspace
// and the last one to arrive sums the KS partials in split order (deterministic) and
// writes the output.
//
// Latency hiding: every thread keeps a ring of S groups of its loads in registers (its
// share of the activation tile and of the scale/code-sum rows, its wave's weights and
// scales), requesting group g + S - 1 while group g is computed.  The compiler's
// per-register wait counters order each use after its load; the ring is refilled
// unconditionally and whole ring turns carry no guards, so those waits stay exact.
// ------------------------------------------------------------------------------------
constexpr int kTileBM = 64;
constexpr int kTileThreads = 256;

// LDS bank swizzles.  A ds_read_b128 wave is served in groups of 16 lanes over 64 banks;
// the rows one group reads must hit distinct banks.  Activation tile: 16-byte chunk c of
// row r sits at chunk position c ^ swz_a(r) of the row's 128 bytes.  Piece rows (32
// bytes): the two 16-byte halves are swapped when swz_p(r) is 1.
__device__ __forceinline__ int swz_a(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int swz_p(int r) { return (r >> 3) & 1; }

// The activation tile of group g lives in buffer g % 2 and is read only in step g.  The
// scale pieces of group g live in buffer g % 3: they are read in step g + 1 too (the
// delayed fold), and a wave may write step g + 2's pieces before a slower wave has left
// step g + 1, so two buffers would race.
struct TileSmem {
  uint8_t a[2][kTileBM * 128];   // [buffer] activation tile, swizzled 16 B chunks
  uint32_t pa[3][kTileBM][8];    // [buffer][row] bf16 pieces of s_a (one 16 B half) + zeros
  uint32_t pu[3][kTileBM][8];    // same for S_A * s_a
  int last;                      // split-K: this workgroup arrived last at its tile
};

__device__ __forceinline__ uint32_t pack_bf16(uint32_t lo, uint32_t hi) { return lo | (hi << 16); }

// x = p0 + p1 + p2 exactly, each a bf16 (returned as 16-bit patterns): truncate to
// bf16, the remainder keeps at most 16 significant bits, truncate again, the second
// remainder has at most 8 and is itself a bf16.
__device__ __forceinline__ void split3_bf16(float x, uint32_t &p0, uint32_t &p1, uint32_t &p2) {
  const uint32_t b0 = __float_as_uint(x) & 0xFFFF0000u;
  const float r1 = x - __uint_as_float(b0);
  const uint32_t b1 = __float_as_uint(r1) & 0xFFFF0000u;
  const float r2 = r1 - __uint_as_float(b1);
  p0 = b0 >> 16;
  p1 = b1 >> 16;
  p2 = __float_as_uint(r2) >> 16;
}

// x = p0 + p1 exactly for x with at most 16 significant bits (fp16 scales, z * s_w).
__device__ __forceinline__ void split2_bf16(float x, uint32_t &p0, uint32_t &p1) {
  const uint32_t b0 = __float_as_uint(x) & 0xFFFF0000u;
  p0 = b0 >> 16;
  p1 = __float_as_uint(x - __uint_as_float(b0)) >> 16;
}

__device__ __forceinline__ v16f mfma_bf16(v4i a, v4i b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0,
                                                 0, 0);
}

// Column operand of the piece products: lanes of the first half-wave carry
// [b0, b1, b0, b1, b0, b1, 0, 0], the second half-wave zeros (its k slots are unused).
__device__ __forceinline__ v4i col_pieces(float x, int h, bool negate) {
  uint32_t b0, b1;
  split2_bf16(x, b0, b1);
  uint32_t w = pack_bf16(b0, b1) ^ (negate ? 0x80008000u : 0u);
  w = h ? 0u : w;
  return v4i{(int)w, (int)w, (int)w, 0};
}

enum BlockKind { kNone = 0, kW4 = 1, kW8 = 2 };

template <int S, int KIND, bool PARTIALS>
__device__ __forceinline__ void tile_body(const GemmArgs &p, TileSmem &sm, int t, int ksplit, int m0, int blk,
                                          int wave, int lane) {
  constexpr int RB = kTileBM / 32;
  constexpr bool H4 = KIND == kW4;
  constexpr bool H8 = KIND == kW8;
  const int tid = wave * 64 + lane;
  const int ch32 = lane & 31, h = lane >> 5, half = ch32 >> 4, ch = ch32 & 15;
  const int G = p.G;
  const int gb = (int)((int64_t)G * ksplit / p.ks), ge = (int)((int64_t)G * (ksplit + 1) / p.ks);

  // Ring slots hold raw loaded bits only: converting a value right after its load would
  // make the wait for it a wait for every load issued before it.
  v4i aR[S][RB];
  float saR[S];
  int32_t asR[S];
  v4i b4R[S][2];
  uint32_t z8R[S];
  uint32_t s4R[S];
  v4i b8R[S][4];
  uint32_t s8R[S];

  const int prow = min(m0 + lane, p.M - 1);  // row whose scales this lane loads
  auto issue = [&](auto slot_c, int g) {
    constexpr int j = decltype(slot_c)::value;
#pragma unroll
    for (int q = 0; q < RB; ++q) {
      const int u = tid + 256 * q, r = u >> 3, c = u & 7;
      const int row = min(m0 + r, p.M - 1);  // rows past M load a valid row; never stored
      aR[j][q] = ldg16(p.aq + (int64_t)row * p.K + g * 128 + c * 16);
    }
    saR[j] = p.sa[(int64_t)g * p.M + prow];
    asR[j] = p.asum[(int64_t)g * p.M + prow];
    if (H4) {
      const size_t cidx = (size_t)blk * G + g;
      const uint8_t *chunk = p.w4 + cidx * kW4Chunk + half * 1024;
#pragma unroll
      for (int q = 0; q < 2; ++q) b4R[j][q] = ldg16(chunk + ((2 * q + h) * 16 + ch) * 16);
      // whole words only: the word holding this channel's scale, the one holding its zero
      s4R[j] = reinterpret_cast<const uint32_t *>(p.s4)[cidx * 16 + (ch32 >> 1)];
      z8R[j] = reinterpret_cast<const uint32_t *>(p.z4)[cidx * 4 + (ch32 >> 3)];
    }
    if (H8) {
      const size_t cidx = (size_t)(blk - p.nb4) * G + g;
      const uint8_t *chunk = p.w8 + cidx * kW8Chunk + half * 2048;
#pragma unroll
      for (int s = 0; s < 4; ++s) b8R[j][s] = ldg16(chunk + (chunk32(s, h) * 16 + ch) * 16);
      s8R[j] = reinterpret_cast<const uint32_t *>(p.s8)[cidx * 16 + (ch32 >> 1)];
    }
  };

  // The activation tile and the row pieces of group slot j into LDS buffer `buf`.  The
  // pieces of all 64 rows (lane = row) are computed by wave g % 4, so the work rotates.
  auto store_a = [&](auto slot_c, int buf, int pbuf, int g) {
    constexpr int j = decltype(slot_c)::value;
#pragma unroll
    for (int q = 0; q < RB; ++q) {
      const int u = tid + 256 * q, r = u >> 3, c = u & 7;
      *reinterpret_cast<v4i *>(&sm.a[buf][r * 128 + ((c ^ swz_a(r)) << 4)]) = aR[j][q];
    }
    if (wave == (g & 3)) {
      uint32_t a0, a1, a2, u0, u1, u2;
      split3_bf16(saR[j], a0, a1, a2);
      split3_bf16((float)asR[j] * saR[j], u0, u1, u2);
      const int sw = swz_p(lane) * 4;
      *reinterpret_cast<v4i *>(&sm.pa[pbuf][lane][sw]) =
          v4i{(int)pack_bf16(a0, a0), (int)pack_bf16(a1, a1), (int)pack_bf16(a2, a2), 0};
      *reinterpret_cast<v4i *>(&sm.pu[pbuf][lane][sw]) =
          v4i{(int)pack_bf16(u0, u0), (int)pack_bf16(u1, u1), (int)pack_bf16(u2, u2), 0};
    }
  };

  const int jp = blk * 32 + ch32;
  auto a_operand = [&](int buf, int rb, int chunk) {
    const int r = rb * 32 + ch32;
    return *reinterpret_cast<const v4i *>(&sm.a[buf][r * 128 + ((chunk ^ swz_a(r)) << 4)]);
  };
  auto row_pieces = [&](uint32_t (*arr)[kTileBM][8], int buf, int rb) {
    const int r = rb * 32 + ch32;
    return *reinterpret_cast<const v4i *>(&arr[buf][r][(h * 4) ^ (swz_p(r) * 4)]);
  };

  v16f acc[RB];
  v16i Pprev[RB];  // int32 partials of the previous group, folded during this step
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    acc[rb] = v16f{0};
    Pprev[rb] = v16i{0};
  }
  uint32_t swprev = 0, zprev = 0;  // that group's scale word and zero-point word
  int pbufprev = 0;                // and the LDS buffer of its scale pieces

  // Fold the previous group: its scale products come from the bf16 MFMA on the pieces
  // still held in its LDS buffer (written two steps apart) and its scale/zero words.
  auto fold_prev = [&]() {
    const float sw = h2f((uint16_t)(swprev >> ((ch32 & 1) * 16)));
    const uint32_t z = H4 ? ((zprev >> ((ch32 & 7) * 4)) & 15u) : 0u;
    const v4i bp = col_pieces(sw, h, false);
    const v4i bu = col_pieces((float)z * sw, h, true);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const v16f sc = mfma_bf16(row_pieces(sm.pa, pbufprev, rb), bp, v16f{0});
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[rb][r] = fmaf((float)Pprev[rb][r], sc[r], acc[rb][r]);
      if (H4) acc[rb] = mfma_bf16(row_pieces(sm.pu, pbufprev, rb), bu, acc[rb]);
    }
  };

  // Group g on the matrix core; returns its partials.  In the partials mode the
  // partials are written out instead.
  auto mma = [&](auto slot_c, int buf, int g, v16i (&Pi)[RB]) {
    constexpr int j = decltype(slot_c)::value;
    v4i bq[4];
    if (H4) {
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const uint32_t x0 = (uint32_t)b4R[j][q][2 * e], x1 = (uint32_t)b4R[j][q][2 * e + 1];
          bq[2 * q + e] = v4i{(int)(x0 & 0x0F0F0F0Fu), (int)((x0 >> 4) & 0x0F0F0F0Fu), (int)(x1 & 0x0F0F0F0Fu),
                              (int)((x1 >> 4) & 0x0F0F0F0Fu)};
        }
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) bq[s] = b8R[j][s];
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) Pi[rb] = v16i{0};
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        Pi[rb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a_operand(buf, rb, chunk32(s, h)), bq[s], Pi[rb], 0, 0, 0);
    if (PARTIALS) {
      const uint32_t z = H4 ? ((z8R[j] >> ((ch32 & 7) * 4)) & 15u) : 0u;
      const int orig = p.idx[jp];
      if (orig >= p.n_begin && orig < p.n_begin + p.n_count) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = m0 + rb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            if (row < p.M) {
              const int corr = H4 ? (int)z * p.asum[(int64_t)g * p.M + row] : 0;
              p.part[((int64_t)row * p.n_count + (orig - p.n_begin)) * G + g] = Pi[rb][r] - corr;
            }
          }
      }
    }
  };

  // One step: group g's activation tile into LDS, barrier, refill the ring, then the
  // matrix-core work of group g interleaved with the VALU fold of group g - 1.
  auto step = [&](auto jc, int g) {
    constexpr int j = decltype(jc)::value;
    const int buf = g & 1;
    const int pbuf = g % 3;
    store_a(jc, buf, pbuf, g);
    __syncthreads();
    // the words of group g leave the ring slot that the refill below reuses later
    const uint32_t swcur = H4 ? s4R[j] : s8R[j];
    const uint32_t zcur = H4 ? z8R[j] : 0u;
    // Always refill the ring (past the range end, reload the last group): a branch here
    // would merge two load histories and make the compiler's waits conservative.
    issue(IntC<(j + S - 1) % S>{}, min(g + S - 1, ge - 1));
    if (KIND != kNone) {
      v16i Pi[RB];
      mma(jc, buf, g, Pi);
      if (!PARTIALS) fold_prev();
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) Pprev[rb] = Pi[rb];
    }
    swprev = swcur;
    zprev = zcur;
    pbufprev = pbuf;
  };

  static_for<0, S - 1>([&](auto jc) { issue(jc, min(gb + (int)decltype(jc)::value, ge - 1)); });
  int g0 = gb;
  for (; g0 + S <= ge; g0 += S) static_for<0, S>([&](auto jc) { step(jc, g0 + decltype(jc)::value); });
  static_for<0, S>([&](auto jc) {
    if (g0 + (int)decltype(jc)::value < ge) step(jc, g0 + decltype(jc)::value);
  });
  if (!PARTIALS && KIND != kNone) fold_prev();  // the last group's fold
  if (PARTIALS) return;

  if (p.ks > 1) {
    // Split-K: publish this split's partial tile; the last workgroup of the tile to
    // arrive sums all splits in split order and writes the output.
    float *slots = p.ws + (size_t)t * p.ks * (kTileBM * 128);
    float *mine = slots + (size_t)ksplit * (kTileBM * 128);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mine[((wave * RB + rb) * 16 + r) * 64 + lane] = acc[rb][r];
    __threadfence();
    __syncthreads();
    if (tid == 0) sm.last = atomicAdd(&p.cnt[t], 1) == p.ks - 1;
    __syncthreads();
    if (!sm.last) return;
    __threadfence();
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = 0.0f;
        for (int k = 0; k < p.ks; ++k) {
          const float o = __builtin_nontemporal_load(&slots[(size_t)k * (kTileBM * 128) +
                                                            ((wave * RB + rb) * 16 + r) * 64 + lane]);
          v += k == ksplit ? acc[rb][r] : o;
        }
        acc[rb][r] = v;
      }
    if (tid == 0) p.cnt[t] = 0;  // leave the counter zero for the next launch
  }
  if (KIND == kNone) return;
  const int orig = p.idx[jp];
  if (orig < 0) return;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = m0 + rb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
      if (row < p.M) p.y[(int64_t)row * p.ldy + orig] = f2h(acc[rb][r]);
    }
}

// Register-ring depth (groups of loads in flight) per block kind.
#ifndef MIXLLM_RING_W4
#define MIXLLM_RING_W4 3
#endif
#ifndef MIXLLM_RING_W8
#define MIXLLM_RING_W8 2
#endif
constexpr int kRingW4 = MIXLLM_RING_W4;
constexpr int kRingW8 = MIXLLM_RING_W8;

template <bool PARTIALS>
__global__ __launch_bounds__(kTileThreads, 2) void gemm_tile_kernel(const GemmArgs p) {
  __shared__ __attribute__((aligned(16))) TileSmem sm;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;

  // Zero the piece arrays once: only one 16-byte half of each row is rewritten per group.
  for (int e = tid; e < (int)(sizeof(sm.pa) / 16); e += kTileThreads) {
    reinterpret_cast<v4i *>(&sm.pa[0][0][0])[e] = v4i{0, 0, 0, 0};
    reinterpret_cast<v4i *>(&sm.pu[0][0][0])[e] = v4i{0, 0, 0, 0};
  }
  __syncthreads();  // before any wave writes its first pieces

  // Workgroup w runs on XCD w % 8.  Give each XCD a contiguous range of tasks (tile,
  // split) with the split fastest and then the M tile, so the splits of a tile share an
  // XCD's L2 and its workgroups share weight blocks and activation tiles there.
  const int T = p.tiles_m * p.tiles_n * p.ks;
  const int xcd = blockIdx.x & 7, i = blockIdx.x >> 3;
  const int per = T >> 3, rem = T & 7;
  const int task = xcd * per + (xcd < rem ? xcd : rem) + i;
  const int ksplit = task % p.ks, t = task / p.ks;
  const int tm = t % p.tiles_m, tn = t / p.tiles_m;
  const int m0 = tm * kTileBM;
  const int blk = tn * 4 + wave;
  const int kind = blk >= p.nb ? kNone : (blk < p.nb4 ? kW4 : kW8);
  switch (kind) {
    case kW4: tile_body<kRingW4, kW4, PARTIALS>(p, sm, t, ksplit, m0, blk, wave, lane); break;
    case kW8: tile_body<kRingW8, kW8, PARTIALS>(p, sm, t, ksplit, m0, blk, wave, lane); break;
    default: tile_body<kRingW4, kNone, PARTIALS>(p, sm, t, ksplit, m0, blk, wave, lane); break;
  }
}

// ------------------------------------------------------------------------------------
// Skinny kernel (small M): one workgroup per 16-channel half block; its KS waves split
// the groups, each wave computes all M <= 16 RB rows for its groups with
// v_mfma_i32_16x16x64_i8, and the partial sums are reduced through LDS.
// ------------------------------------------------------------------------------------
template <int RB, bool PARTIALS>
__global__ __launch_bounds__(1024) void gemm_skinny_kernel(const GemmArgs p, int ks) {
  __shared__ float red[16][RB * 4][64];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int sub = blockIdx.x;
  const int blk = sub >> 1, half = sub & 1;
  const int ch = lane & 15, qd = lane >> 4, ch32 = half * 16 + ch;
  const int G = p.G;
  const int g0 = (int)((int64_t)G * wave / ks), g1 = (int)((int64_t)G * (wave + 1) / ks);
  const bool has4 = blk < p.nb4;
  const bool has8 = !has4;
  const int jp = blk * 32 + ch32;

  float acc[RB][4];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[rb][r] = 0.0f;

  auto a_load = [&](int rb, int g, int chunk) {
    const int row = rb * 16 + ch;
    return row < p.M ? ldg16(p.aq + (int64_t)row * p.K + g * 128 + chunk * 16) : v4i{0, 0, 0, 0};
  };
  auto fold_or_emit = [&](const v4i (&P)[RB], int g, float sw) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = rb * 16 + 4 * qd + r;
        if (PARTIALS) {
          const int orig = p.idx[jp];
          if (row < p.M && orig >= p.n_begin && orig < p.n_begin + p.n_count)
            p.part[((int64_t)row * p.n_count + (orig - p.n_begin)) * G + g] = P[rb][r];
        } else {
          const float s_a = row < p.M ? p.sa[(int64_t)g * p.M + row] : 0.0f;
          acc[rb][r] = fmaf((float)P[rb][r], sw * s_a, acc[rb][r]);
        }
      }
  };

  for (int g = g0; g < g1; ++g) {
    if (has4) {
      const size_t cidx = (size_t)blk * G + g;
      const v4i x = ldg16(p.w4 + cidx * kW4Chunk + half * 1024 + lane * 16);
      const uint32_t zz = zero_point_x4(p.z4[cidx * 16 + (ch32 >> 1)], ch32 & 1);
      const float sw = h2f(p.s4[cidx * 32 + ch32]);
      const v4i b0 = w4_operand((uint32_t)x[0], (uint32_t)x[1], zz);
      const v4i b1 = w4_operand((uint32_t)x[2], (uint32_t)x[3], zz);
      v4i P[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        P[rb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a_load(rb, g, qd), b0, v4i{0, 0, 0, 0}, 0, 0, 0);
        P[rb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a_load(rb, g, qd + 4), b1, P[rb], 0, 0, 0);
      }
      fold_or_emit(P, g, sw);
    }
    if (has8) {
      const size_t cidx = (size_t)(blk - p.nb4) * G + g;
      const uint8_t *chunk = p.w8 + cidx * kW8Chunk + half * 2048;
      const v4i b0 = ldg16(chunk + lane * 16);
      const v4i b1 = ldg16(chunk + 1024 + lane * 16);
      const float sw = h2f(p.s8[cidx * 32 + ch32]);
      v4i P[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        P[rb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a_load(rb, g, qd), b0, v4i{0, 0, 0, 0}, 0, 0, 0);
        P[rb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a_load(rb, g, qd + 4), b1, P[rb], 0, 0, 0);
      }
      fold_or_emit(P, g, sw);
    }
  }
  if (PARTIALS) return;

#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][rb * 4 + r][lane] = acc[rb][r];
  __syncthreads();
  for (int e = tid; e < RB * 4 * 64; e += ks * 64) {
    const int ri = e >> 6, ln = e & 63;
    float v = 0.0f;
    for (int w = 0; w < ks; ++w) v += red[w][ri][ln];
    const int rb = ri >> 2, r = ri & 3;
    const int row = rb * 16 + 4 * (ln >> 4) + r;
    const int orig = p.idx[blk * 32 + half * 16 + (ln & 15)];
    if (row < p.M && orig >= 0) p.y[(int64_t)row * p.ldy + orig] = f2h(v);
  }
}

// ------------------------------------------------------------------------------------
// Host side
// ------------------------------------------------------------------------------------

int check_common(const int8_t *aq, const float *sa, const int32_t *asum, int32_t M, int32_t N, int32_t K,
                 int32_t n8, const void *blob, size_t blob_bytes, mixllm_blob_info *L) {
  if (M < 0 || N <= 0 || K <= 0 || K % kGroup != 0) return MIXLLM_E_SHAPE;
  if (n8 < 0 || n8 > N) return MIXLLM_E_INDEX;
  if (!compute_layout(N, K, n8, L)) return MIXLLM_E_SHAPE;
  if (M == 0) return MIXLLM_OK;
  if (!aq || !sa || !asum || !blob) return MIXLLM_E_NULL;
  if (!is_aligned16(aq) || !is_aligned16(sa) || !is_aligned16(asum) || !is_aligned16(blob)) return MIXLLM_E_SHAPE;
  if (blob_bytes < L->total_bytes) return MIXLLM_E_SPACE;
  return MIXLLM_OK;
}

void fill_args(GemmArgs &a, const int8_t *aq, const float *sa, const int32_t *asum, int32_t M,
               const void *blob, const mixllm_blob_info &L) {
  const uint8_t *base = (const uint8_t *)blob;
  a.aq = aq;
  a.sa = sa;
  a.asum = asum;
  a.M = M;
  a.N = L.N;
  a.K = L.K;
  a.G = L.G;
  a.w4 = base + L.off_w4;
  a.s4 = (const uint16_t *)(base + L.off_s4);
  a.z4 = base + L.off_z4;
  a.w8 = base + L.off_w8;
  a.s8 = (const uint16_t *)(base + L.off_s8);
  a.idx = (const int32_t *)(base + L.off_idx);
  a.n4 = L.n4;
  a.nb = L.nb;
  a.nb4 = L.nb4;
  a.y = nullptr;
  a.ldy = 0;
  a.part = nullptr;
  a.n_begin = 0;
  a.n_count = 0;
  a.tiles_m = a.tiles_n = 0;
  a.ks = 1;
  a.ws = nullptr;
  a.cnt = nullptr;
}

// Launch plan of one GEMM call, a pure function of the shape (also sizes the workspace).
struct Plan {
  bool skinny;
  int rb;                      // skinny: 16-row blocks
  int ks;                      // skinny: waves per workgroup; tile: split-K factor
  int tiles_m, tiles_n;
  size_t ws_slots, ws_bytes;   // tile split-K: partial-tile bytes, total workspace bytes
};

constexpr int kCUs = 256;      // compute units of the MI355X
// Splitting the groups of a tile over workgroups needs an agent-scope release per
// workgroup, which costs a full L2 write-back here; measured slower than no split at
// every shape tried, so it is off.
constexpr bool kSplitK = false;

Plan make_plan(int M, const mixllm_blob_info &L, bool partials) {
  Plan pl{};
  if (M <= 64) {
    pl.skinny = true;
    pl.rb = (M + 15) / 16;
    const int subs = 2 * L.nb;
    int ks = (4096 + subs - 1) / subs;
    ks = ks < 1 ? 1 : (ks > 16 ? 16 : ks);
    pl.ks = ks > L.G ? L.G : ks;
    return pl;
  }
  pl.tiles_m = (M + kTileBM - 1) / kTileBM;
  pl.tiles_n = (L.nb + 3) / 4;
  const int64_t T = (int64_t)pl.tiles_m * pl.tiles_n;
  // Two workgroups per CU: split the groups of each tile when there are too few tiles.
  int ks = 1;
  if (kSplitK && !partials && T < 2 * kCUs) {
    ks = (int)((2 * kCUs + T - 1) / T);
    ks = ks > 8 ? 8 : ks;
    ks = ks > L.G ? L.G : ks;
  }
  pl.ks = ks;
  if (ks > 1) {
    pl.ws_slots = align256((size_t)T * ks * kTileBM * 128 * sizeof(float));
    pl.ws_bytes = pl.ws_slots + align256((size_t)T * sizeof(int));
  }
  return pl;
}

template <bool PARTIALS>
int launch(GemmArgs &a, const Plan &pl, void *workspace, hipStream_t stream) {
  (void)hipGetLastError();
  if (pl.skinny) {
    const int ks = pl.ks;
    const dim3 grid((unsigned)(2 * a.nb)), block((unsigned)(64 * ks));
    switch (pl.rb) {
      case 1: hipLaunchKernelGGL((gemm_skinny_kernel<1, PARTIALS>), grid, block, 0, stream, a, ks); break;
      case 2: hipLaunchKernelGGL((gemm_skinny_kernel<2, PARTIALS>), grid, block, 0, stream, a, ks); break;
      case 3: hipLaunchKernelGGL((gemm_skinny_kernel<3, PARTIALS>), grid, block, 0, stream, a, ks); break;
      default: hipLaunchKernelGGL((gemm_skinny_kernel<4, PARTIALS>), grid, block, 0, stream, a, ks); break;
    }
  } else {
    a.tiles_m = pl.tiles_m;
    a.tiles_n = pl.tiles_n;
    a.ks = pl.ks;
    a.ws = pl.ks > 1 ? (float *)workspace : nullptr;
    a.cnt = pl.ks > 1 ? (int *)((uint8_t *)workspace + pl.ws_slots) : nullptr;
    const int64_t T = (int64_t)a.tiles_m * a.tiles_n * a.ks;
    if (T > 0x7FFFFFFF) return MIXLLM_E_SHAPE;
    hipLaunchKernelGGL((gemm_tile_kernel<PARTIALS>), dim3((unsigned)T), dim3(kTileThreads), 0, stream, a);
  }
  return hipGetLastError() == hipSuccess ? MIXLLM_OK : MIXLLM_E_HIP;
}

}  // namespace

extern "C" size_t mixllm_gemm_workspace_bytes(int32_t M, int32_t N, int32_t K, int32_t n8) {
  mixllm_blob_info L;
  if (M <= 0 || !compute_layout(N, K, n8, &L)) return 0;
  return make_plan(M, L, false).ws_bytes;
}

extern "C" int mixllm_gemm_w4w8a8(const int8_t *aq, const float *sa, const int32_t *asum, int32_t M, int32_t N,
                                  int32_t K, int32_t n8, const void *blob, size_t blob_bytes, uint16_t *y,
                                  int64_t ldy, void *workspace, size_t workspace_bytes, void *stream) {
  mixllm_blob_info L;
  int st = check_common(aq, sa, asum, M, N, K, n8, blob, blob_bytes, &L);
  if (st != MIXLLM_OK || M == 0) return st;
  if (!y) return MIXLLM_E_NULL;
  if (ldy < N) return MIXLLM_E_SHAPE;
  const Plan pl = make_plan(M, L, false);
  if (pl.ws_bytes) {
    if (!workspace) return MIXLLM_E_NULL;
    if (workspace_bytes < pl.ws_bytes) return MIXLLM_E_SPACE;
    if (!is_aligned16(workspace)) return MIXLLM_E_SHAPE;
  }
  GemmArgs a;
  fill_args(a, aq, sa, asum, M, blob, L);
  a.y = y;
  a.ldy = ldy;
  return launch<false>(a, pl, workspace, (hipStream_t)stream);
}

extern "C" int mixllm_gemm_w4w8a8_partials(const int8_t *aq, const float *sa, const int32_t *asum, int32_t M,
                                           int32_t N, int32_t K, int32_t n8, const void *blob, size_t blob_bytes,
                                           int32_t n_begin, int32_t n_count, int32_t *part, void *stream) {
  mixllm_blob_info L;
  int st = check_common(aq, sa, asum, M, N, K, n8, blob, blob_bytes, &L);
  if (st != MIXLLM_OK) return st;
  if (n_begin < 0 || n_count < 0 || (int64_t)n_begin + n_count > N) return MIXLLM_E_SHAPE;
  if (M == 0 || n_count == 0) return MIXLLM_OK;
  if (!part) return MIXLLM_E_NULL;
  GemmArgs a;
  fill_args(a, aq, sa, asum, M, blob, L);
  a.part = part;
  a.n_begin = n_begin;
  a.n_count = n_count;
  return launch<true>(a, make_plan(M, L, true), nullptr, (hipStream_t)stream);
}
