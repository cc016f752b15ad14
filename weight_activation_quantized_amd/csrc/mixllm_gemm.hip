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

struct GemmArgs {
  const int8_t *aq;
  const float *sa;
  int M, N, K, G;
  const uint8_t *w4;
  const uint16_t *s4;
  const uint8_t *z4;
  const uint8_t *w8;
  const uint16_t *s8;
  const int32_t *idx;
  int n4, nb, nb4, b8s;
  uint16_t *y;
  int64_t ldy;
  int32_t *part;  // partials mode output [M][n_count][G]
  int n_begin, n_count;
  int tiles_m, tiles_n;
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
// Tile kernel: BM = 32 RB rows x 128 channels (4 blocks) per workgroup of 4 waves; wave w
// owns block 4 tn + w for all BM rows.
//
// Latency hiding: one workgroup per CU and one wave per SIMD is the natural fill at the
// large shapes, so the loads must run far ahead.  Every thread keeps a ring of S groups
// of its loads in registers (its share of the activation tile, its wave's weights and
// scales); group g + S - 1 is requested while group g is computed, and the compiler's
// per-register wait counters order each use after its load.  The activation tile goes
// through a double-buffered, XOR-swizzled LDS tile (one barrier per group); weights stay
// in the registers of the wave that owns them.  The loop body is instantiated per block
// kind (4-bit only, 8-bit only, the one block holding both, none), so a wave only holds
// the rings it uses.
// ------------------------------------------------------------------------------------
enum BlockKind { kNone = 0, kW4 = 1, kW8 = 2, kBoth = 3 };

template <int RB, int S, int KIND, bool PARTIALS>
__device__ __forceinline__ void tile_body(const GemmArgs &p, uint8_t (*a_lds)[32 * RB * 128],
                                          float (*sa_lds)[32 * RB], int m0, int blk, int tid, int lane) {
  constexpr int BM = 32 * RB;
  constexpr bool H4 = (KIND & kW4) != 0;
  constexpr bool H8 = (KIND & kW8) != 0;
  const int ch32 = lane & 31, h = lane >> 5, half = ch32 >> 4, ch = ch32 & 15;
  const int G = p.G;

  // Ring slots hold raw loaded bits only: converting a value right after its load would
  // make the wait for it a wait for every load issued before it.
  v4i aR[S][RB];
  float saR[S];
  v4i b4R[S][2];
  uint32_t z8R[S];   // byte holding this lane's zero point
  uint32_t s4R[S];   // fp16 bits of the 4-bit scale
  v4i b8R[S][4];
  uint32_t s8R[S];   // fp16 bits of the 8-bit scale

  auto issue = [&](auto slot_c, int g) {
    constexpr int j = decltype(slot_c)::value;
#pragma unroll
    for (int q = 0; q < RB; ++q) {
      const int u = tid + 256 * q, r = u >> 3, c = u & 7;
      const int row = min(m0 + r, p.M - 1);  // rows past M load a valid row; never stored
      aR[j][q] = ldg16(p.aq + (int64_t)row * p.K + g * 128 + c * 16);
    }
    saR[j] = p.sa[(int64_t)g * p.M + min(m0 + (tid & (BM - 1)), p.M - 1)];  // unconditional: no branch
    if (H4) {
      const size_t cidx = (size_t)blk * G + g;
      const uint8_t *chunk = p.w4 + cidx * kW4Chunk + half * 1024;
#pragma unroll
      for (int q = 0; q < 2; ++q) b4R[j][q] = ldg16(chunk + ((2 * q + h) * 16 + ch) * 16);
      s4R[j] = p.s4[cidx * 32 + ch32];
      z8R[j] = p.z4[cidx * 16 + (ch32 >> 1)];
    }
    if (H8) {
      const size_t cidx = (size_t)(blk - p.b8s) * G + g;
      const uint8_t *chunk = p.w8 + cidx * kW8Chunk + half * 2048;
#pragma unroll
      for (int s = 0; s < 4; ++s) b8R[j][s] = ldg16(chunk + (chunk32(s, h) * 16 + ch) * 16);
      s8R[j] = p.s8[cidx * 32 + ch32];
    }
  };

  float acc[RB][16];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[rb][r] = 0.0f;

  const int jp = blk * 32 + ch32;
  auto emit_partials = [&](const v16i(&P)[RB], int g, bool mine) {
    const int orig = mine ? p.idx[jp] : -1;
    if (orig < p.n_begin || orig >= p.n_begin + p.n_count) return;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + rb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (row < p.M) p.part[((int64_t)row * p.n_count + (orig - p.n_begin)) * G + g] = P[rb][r];
      }
  };
  auto fold = [&](const v16i(&P)[RB], int st, float sw) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 s4v = *reinterpret_cast<const float4 *>(&sa_lds[st][rb * 32 + 8 * j + 4 * h]);
        const float sv[4] = {s4v.x, s4v.y, s4v.z, s4v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q)
          acc[rb][4 * j + q] = fmaf((float)P[rb][4 * j + q], sw * sv[q], acc[rb][4 * j + q]);
      }
  };
  auto a_operand = [&](int st, int rb, int chunk) {
    const int r = rb * 32 + ch32;
    return *reinterpret_cast<const v4i *>(&a_lds[st][r * 128 + ((chunk ^ (r & 7)) << 4)]);
  };
  auto compute = [&](auto slot_c, int st, int g) {
    constexpr int j = decltype(slot_c)::value;
    if (H4) {
      const uint32_t zz = zero_point_x4(z8R[j], ch32 & 1);
      v16i P[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) P[rb] = v16i{0};
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const v4i bA = w4_operand((uint32_t)b4R[j][q][0], (uint32_t)b4R[j][q][1], zz);
        const v4i bB = w4_operand((uint32_t)b4R[j][q][2], (uint32_t)b4R[j][q][3], zz);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          P[rb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a_operand(st, rb, 2 * q + h), bA, P[rb], 0, 0, 0);
          P[rb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a_operand(st, rb, 2 * q + h + 4), bB, P[rb], 0, 0, 0);
        }
      }
      if (PARTIALS)
        emit_partials(P, g, jp < p.n4);
      else
        fold(P, st, h2f((uint16_t)s4R[j]));
    }
    if (H8) {
      v16i P[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) P[rb] = v16i{0};
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          P[rb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a_operand(st, rb, chunk32(s, h)), b8R[j][s], P[rb], 0, 0, 0);
      if (PARTIALS)
        emit_partials(P, g, jp >= p.n4 && jp < p.N);
      else
        fold(P, st, h2f((uint16_t)s8R[j]));
    }
  };
  auto store_a = [&](auto slot_c, int st) {
    constexpr int j = decltype(slot_c)::value;
#pragma unroll
    for (int q = 0; q < RB; ++q) {
      const int u = tid + 256 * q, r = u >> 3, c = u & 7;
      *reinterpret_cast<v4i *>(&a_lds[st][r * 128 + ((c ^ (r & 7)) << 4)]) = aR[j][q];
    }
    sa_lds[st][tid & (BM - 1)] = saR[j];  // all threads (duplicates agree): no branch
  };

  // prologue: groups 0 .. S-2 in flight
  static_for<0, S - 1>([&](auto jc) { issue(jc, min((int)decltype(jc)::value, G - 1)); });
  auto step = [&](auto jc, int g) {
    constexpr int j = decltype(jc)::value;
    const int st = g & 1;
    store_a(jc, st);
    __syncthreads();
    // Always refill the ring (past the last group, reload the last group): a branch here
    // would merge two load histories and make the compiler's waits conservative.
    issue(IntC<(j + S - 1) % S>{}, min(g + S - 1, G - 1));
    compute(jc, st, g);
  };
  // Whole turns of the ring carry no guards, so every wait the compiler derives is exact;
  // the last partial turn is guarded.
  int g0 = 0;
  for (; g0 + S <= G; g0 += S) static_for<0, S>([&](auto jc) { step(jc, g0 + decltype(jc)::value); });
  static_for<0, S>([&](auto jc) {
    if (g0 + (int)decltype(jc)::value < G) step(jc, g0 + decltype(jc)::value);
  });

  if (PARTIALS || KIND == kNone) return;
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

// Register-ring depth (groups of loads in flight) per block kind.  The block holding both
// subsets exists at most once per layer, so it gets the shallow ring.
#ifndef MIXLLM_RING_W4
#define MIXLLM_RING_W4 5
#endif
#ifndef MIXLLM_RING_W8
#define MIXLLM_RING_W8 4
#endif
constexpr int kRingW4 = MIXLLM_RING_W4;
constexpr int kRingW8 = MIXLLM_RING_W8;
constexpr int kRingBoth = 2;

template <int RB, bool PARTIALS>
__global__ __launch_bounds__(256) void gemm_tile_kernel(const GemmArgs p) {
  constexpr int BM = 32 * RB;
  __shared__ __attribute__((aligned(16))) uint8_t a_lds[2][BM * 128];
  __shared__ __attribute__((aligned(16))) float sa_lds[2][BM];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;

  // Workgroup w runs on XCD w % 8.  Give each XCD a contiguous range of tiles, ordered
  // with the M tile fastest, so the workgroups of one XCD share weight blocks and the
  // activation tiles in that XCD's L2.
  const int T = p.tiles_m * p.tiles_n;
  const int xcd = blockIdx.x & 7, i = blockIdx.x >> 3;
  const int per = T >> 3, rem = T & 7;
  const int t = xcd * per + (xcd < rem ? xcd : rem) + i;
  const int tm = t % p.tiles_m, tn = t / p.tiles_m;
  const int m0 = tm * BM;
  const int blk = tn * 4 + wave;
  const bool has4 = blk < p.nb4;
  const bool has8 = blk >= p.b8s && blk < p.nb;
  const int kind = (has4 ? kW4 : 0) | (has8 ? kW8 : 0);
  switch (kind) {
    case kW4: tile_body<RB, kRingW4, kW4, PARTIALS>(p, a_lds, sa_lds, m0, blk, tid, lane); break;
    case kW8: tile_body<RB, kRingW8, kW8, PARTIALS>(p, a_lds, sa_lds, m0, blk, tid, lane); break;
    case kBoth: tile_body<RB, kRingBoth, kBoth, PARTIALS>(p, a_lds, sa_lds, m0, blk, tid, lane); break;
    default: tile_body<RB, kRingW4, kNone, PARTIALS>(p, a_lds, sa_lds, m0, blk, tid, lane); break;
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
  const bool has8 = blk >= p.b8s;
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
  auto fold_or_emit = [&](const v4i (&P)[RB], int g, float sw, bool mine) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = rb * 16 + 4 * qd + r;
        if (PARTIALS) {
          const int orig = mine ? p.idx[jp] : -1;
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
      fold_or_emit(P, g, sw, jp < p.n4);
    }
    if (has8) {
      const size_t cidx = (size_t)(blk - p.b8s) * G + g;
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
      fold_or_emit(P, g, sw, jp >= p.n4 && jp < p.N);
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

int check_common(const int8_t *aq, const float *sa, int32_t M, int32_t N, int32_t K, int32_t n8,
                 const void *blob, size_t blob_bytes, mixllm_blob_info *L) {
  if (M < 0 || N <= 0 || K <= 0 || K % kGroup != 0) return MIXLLM_E_SHAPE;
  if (n8 < 0 || n8 > N) return MIXLLM_E_INDEX;
  if (!compute_layout(N, K, n8, L)) return MIXLLM_E_SHAPE;
  if (M == 0) return MIXLLM_OK;
  if (!aq || !sa || !blob) return MIXLLM_E_NULL;
  if (!is_aligned16(aq) || !is_aligned16(sa) || !is_aligned16(blob)) return MIXLLM_E_SHAPE;
  if (blob_bytes < L->total_bytes) return MIXLLM_E_SPACE;
  return MIXLLM_OK;
}

void fill_args(GemmArgs &a, const int8_t *aq, const float *sa, int32_t M, const void *blob,
               const mixllm_blob_info &L) {
  const uint8_t *base = (const uint8_t *)blob;
  a.aq = aq;
  a.sa = sa;
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
  a.b8s = L.b8s;
  a.y = nullptr;
  a.ldy = 0;
  a.part = nullptr;
  a.n_begin = 0;
  a.n_count = 0;
}

template <bool PARTIALS>
int launch(GemmArgs &a, hipStream_t stream) {
  (void)hipGetLastError();
  if (a.M <= 64) {
    const int rb = (a.M + 15) / 16;
    const int subs = 2 * a.nb;
    int ks = (4096 + subs - 1) / subs;
    ks = ks < 1 ? 1 : (ks > 16 ? 16 : ks);
    if (ks > a.G) ks = a.G;
    const dim3 grid((unsigned)subs), block((unsigned)(64 * ks));
    switch (rb) {
      case 1: hipLaunchKernelGGL((gemm_skinny_kernel<1, PARTIALS>), grid, block, 0, stream, a, ks); break;
      case 2: hipLaunchKernelGGL((gemm_skinny_kernel<2, PARTIALS>), grid, block, 0, stream, a, ks); break;
      case 3: hipLaunchKernelGGL((gemm_skinny_kernel<3, PARTIALS>), grid, block, 0, stream, a, ks); break;
      default: hipLaunchKernelGGL((gemm_skinny_kernel<4, PARTIALS>), grid, block, 0, stream, a, ks); break;
    }
  } else {
    constexpr int RB = 2;
    a.tiles_m = (a.M + 32 * RB - 1) / (32 * RB);
    a.tiles_n = (a.nb + 3) / 4;
    const int64_t T = (int64_t)a.tiles_m * a.tiles_n;
    if (T > 0x7FFFFFFF) return MIXLLM_E_SHAPE;
    hipLaunchKernelGGL((gemm_tile_kernel<RB, PARTIALS>), dim3((unsigned)T), dim3(256), 0, stream, a);
  }
  return hipGetLastError() == hipSuccess ? MIXLLM_OK : MIXLLM_E_HIP;
}

}  // namespace

extern "C" size_t mixllm_gemm_workspace_bytes(int32_t M, int32_t N, int32_t K, int32_t n8) {
  (void)M;
  (void)N;
  (void)K;
  (void)n8;
  return 0;
}

extern "C" int mixllm_gemm_w4w8a8(const int8_t *aq, const float *sa, int32_t M, int32_t N, int32_t K,
                                  int32_t n8, const void *blob, size_t blob_bytes, uint16_t *y, int64_t ldy,
                                  void *workspace, size_t workspace_bytes, void *stream) {
  (void)workspace;
  mixllm_blob_info L;
  int st = check_common(aq, sa, M, N, K, n8, blob, blob_bytes, &L);
  if (st != MIXLLM_OK || M == 0) return st;
  if (!y) return MIXLLM_E_NULL;
  if (ldy < N) return MIXLLM_E_SHAPE;
  if (workspace_bytes < mixllm_gemm_workspace_bytes(M, N, K, n8)) return MIXLLM_E_SPACE;
  GemmArgs a;
  fill_args(a, aq, sa, M, blob, L);
  a.y = y;
  a.ldy = ldy;
  return launch<false>(a, (hipStream_t)stream);
}

extern "C" int mixllm_gemm_w4w8a8_partials(const int8_t *aq, const float *sa, int32_t M, int32_t N, int32_t K,
                                           int32_t n8, const void *blob, size_t blob_bytes, int32_t n_begin,
                                           int32_t n_count, int32_t *part, void *stream) {
  mixllm_blob_info L;
  int st = check_common(aq, sa, M, N, K, n8, blob, blob_bytes, &L);
  if (st != MIXLLM_OK) return st;
  if (n_begin < 0 || n_count < 0 || (int64_t)n_begin + n_count > N) return MIXLLM_E_SHAPE;
  if (M == 0 || n_count == 0) return MIXLLM_OK;
  if (!part) return MIXLLM_E_NULL;
  GemmArgs a;
  fill_args(a, aq, sa, M, blob, L);
  a.part = part;
  a.n_begin = n_begin;
  a.n_count = n_count;
  return launch<true>(a, (hipStream_t)stream);
}
