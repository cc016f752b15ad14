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
//  * The tile kernel feeds raw 4-bit codes to the matrix cores and removes the zero point
//    in the float domain with one more matrix-core op per block (-(S_A s_a)(z s_w));
//    the scale products s_a s_w are matrix-core outer products of exact bf16 splits.
//    The skinny kernel (small M, bandwidth-bound) forms (W_q - z) with byte-wise SWAR
//    arithmetic: ((q | 0x80) - z) ^ 0x80 per byte, four codes per 32-bit op (the role of
//    the pages' vsub4; CDNA has no byte-vector subtract).
//  * int32 -> fp32: the tile kernel either converts with v_cvt_f32_i32 (exact fold) or
//    uses the pages' float-bits bias with the bias seeded into the MFMA accumulator and
//    its subtraction moved onto the matrix cores (bias fold, one VALU op per element).
//  * The tile kernel stages the activation tile and the row operands through LDS
//    (shared by the eight waves of a workgroup) with direct-to-LDS loads and streams
//    each wave's own weights into registers; the skinny kernel streams both from L2/HBM
//    and splits the groups over the waves of a workgroup, reducing through LDS.
//  * Small M has two more bandwidth-bound kernels: the gemv kernel (M <= 3; one lane per
//    channel, v_dot4_i32_i8 against activation codes held in SGPRs) and the strip kernel
//    (4 <= M <= 32; 16x16x64 integer MFMA tiles fed from a per-wave LDS ring).  They keep
//    one group of loads ahead (the strip kernel two, with two row blocks): with more, the
//    older waves of a CU fill its memory queue and the younger ones lag, leaving a long
//    tail.  make_plan picks the kernel for each call.
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
#include <stddef.h>
#include <stdint.h>
#include <string.h>

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
  const uint32_t *rowop;  // [G][M][8] row operand records of the scale products and corrections
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
  int spread;  // tile kernel: the grid fits the device at once (one workgroup per CU)
  int ident;   // tile kernel: packed channel j is original channel j, and y takes 16-byte stores
  int ileave;  // tile kernel: block bi of N tile tn is block bi * tiles_n + tn (else tn * NB + bi)
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
// Tile kernel.  A workgroup of 8 waves (4 with NB = 2) owns 64 rows x NB blocks of 32
// channels.  Wave (b, q) computes block NB tn + b for all 64 rows (two 32-row blocks)
// over the groups g = q, q + 2, q + 4, ... (two interleaved group slices; the two waves
// of a block share a SIMD); the slices' accumulators are summed through LDS at the end.
//
// Per group and wave:
//   * 2 x 4 v_mfma_i32_32x32x32_i8: the exact group partials of the two row blocks, from
//     the raw 4-bit codes q (3 VALU ops per 8 codes) or the 8-bit codes;
//   * per row block, 1 v_mfma_f32_32x32x16_bf16: the scale products s_a[m] s_w[n] as an
//     outer product of exact bf16 splits (s_a = a0 + a1 + a2 from the activation
//     quantizer, s_w = b0 + b1 from the packed blob);
//   * the fold acc += float(P) * scale: 2 VALU ops per output element;
//   * the zero point: sum_k (q - z) a_k = sum_k q a_k - z S_A (S_A the group's code sum),
//     so 4-bit channels need -sum_g (S_A s_a)[m, g] (z s_w)[n, g] added: a sum of rank-one
//     terms, put on the matrix cores two groups at a time (one per half-wave of a bf16
//     MFMA).  Wave (b, q) adds the terms of row block q for both slices' groups of each
//     step, so every output gets each group's term exactly once.
// Two conversions of the int32 partial to fp32 are built: v_cvt_f32_i32 (default), and
// the float-bits conversion of the talk notes (高速 I2F 変換), exact here: the partial's
// MFMA chain starts from the integer 0x4B400000, so its bits read as a float are exactly
// B + P (B = 1.5 * 2^23, |P| < 2^22), and one subtraction of B recovers P.
//
// Schedule.  A step (one group per wave) is two half-steps, one per row block.  In the
// half-step of row block r the matrix cores run r's scale product and partial chain while
// the vector ALUs fold the other row block's previous partials (and, in the first half,
// decode the step's 4-bit codes); the LDS reads for the next half-step are issued in the
// same window.  Every operand an MFMA reads was loaded one half-step earlier.
//
// Streams.  The activation tile of a group (64 rows x 128 B) and the rows' operand
// records (64 rows x 32 B) go from memory straight into LDS (buffer_load ... lds) in a
// ring of kSA stages shared by the workgroup; each wave's weights and column words go
// into a ring of kSA register slots.  Step s (between its two half-steps) publishes stage
// s + 1 with a workgroup barrier and refills the ring: stage s + kSA and the weights of
// step s + kSA - 1.  The loop is unrolled by kSA so every stage and slot index is a
// compile-time constant.  Every wave issues a fixed set of loads per step, so a wait for
// "at most 2 steps' loads outstanding" proves the next stage has landed; the wait is
// explicit because the compiler does not track LDS written by these loads.  Groups past
// the slice's last one clamp their loads to a valid group and read zero column words, so
// they add nothing.
// ------------------------------------------------------------------------------------
constexpr int kTileBM = 64;
constexpr int kTileNB = 4;                          // channel blocks per workgroup (at most; NB)
constexpr int kKS = 2;                              // interleaved group slices
constexpr int tile_threads(int nb) { return 64 * nb * kKS; }
constexpr int kSA = 4;                              // LDS stages = weight ring slots
#ifndef MIXLLM_ZERO_PRE
#define MIXLLM_ZERO_PRE 0
#endif
// Variant: subtract 4-bit zero points from the codes (byte-wise) before the matrix cores
// instead of the matrix-core correction (a measured ablation).
constexpr bool kZeroPre = MIXLLM_ZERO_PRE != 0;
#ifndef MIXLLM_FOLD_BIAS
#define MIXLLM_FOLD_BIAS 0
#endif
// Variant: the float-bits int32 -> fp32 conversion instead of v_cvt_f32_i32.
constexpr bool kFoldBias = MIXLLM_FOLD_BIAS != 0;
constexpr int kBiasBits = 0x4B400000;               // float bits of B = 1.5 * 2^23

// LDS bank swizzle of the activation tile: a ds_read_b128 wave is served in groups of
// 16 lanes over 64 banks, and the rows one group reads must hit distinct banks; the
// 16-byte chunk c of row r sits at position c ^ swz_a(r) of the row's 128 bytes.
__device__ __forceinline__ int swz_a(int r) { return (r >> 1) & 7; }

// CW: the column scales and zero points of the step's two groups go through LDS too
// (4-block tiles; a 2-block tile stays within 80 KB so that two fit a CU, and its waves
// load their own).
template <bool CW>
struct TileSmemT {
  uint8_t a[kSA][kKS][kTileBM * 128];           // [stage][slice] activation tiles
  uint8_t r[kSA][kKS][kTileBM * 32];            // [stage][slice] row operand records
};
template <>
struct TileSmemT<true> {
  uint8_t a[kSA][kKS][kTileBM * 128];
  uint8_t r[kSA][kKS][kTileBM * 32];
  uint8_t c[kSA][2048];  // [stage]: fp16 scales [block][group of the pair][32], zero points at 1024
};
template <int NB>
using TileSmem = TileSmemT<NB == kTileNB>;
constexpr int kAStage = kKS * kTileBM * 128;        // bytes per activation stage
constexpr int kRBase = kSA * kAStage;               // offset of the row operand stages
constexpr int kRStage = kKS * kTileBM * 32;
constexpr int kCBase = kRBase + kSA * kRStage;      // offset of the column stages
constexpr int kCStage = 2048;
constexpr int kCZero = 1024;                        // zero points within a column stage
static_assert(kTileNB * 2 * 64 <= kCZero && kCZero + 64 * 16 <= kCStage, "column stage");
static_assert(offsetof(TileSmemT<false>, r) == kRBase && offsetof(TileSmemT<true>, r) == kRBase &&
                  offsetof(TileSmemT<true>, c) == kCBase && sizeof(TileSmemT<false>) <= 80 * 1024,
              "LDS layout");
static_assert(kKS * kTileNB * 16 * 64 * 4 + kKS * kTileNB * 32 * 32 * 2 <= (int)sizeof(TileSmemT<false>::a),
              "reduction and output staging space");

__device__ __forceinline__ v16f mfma_bf16(v4i a, v4i b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0,
                                                 0, 0);
}

enum BlockKind { kNone = 0, kW4 = 1, kW8 = 2 };

// Buffer resources: the 128-bit descriptor of a byte range [base, base + bytes).  Loads
// through it take a per-lane 32-bit offset (computed once) plus a wave-uniform offset
// (per group, scalar arithmetic), so the inner loop spends no vector ops on addresses.
// Lanes whose per-lane offset is past `bytes` read zeros; the scalar offsets used here
// always stay inside the range.
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kRsrcFlags = 0x00020000;  // gfx9 raw buffer, 32-bit data format

__device__ __forceinline__ Rsrc make_rsrc(const void *base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0xFFFFFFFFll ? 0xFFFFFFFFll : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)(uint32_t)n, kRsrcFlags);
}
__device__ __forceinline__ v4i bload16(Rsrc r, int voff, int soff) {
  return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
// With the cache-policy bit nt (non-temporal), for weights that a kernel reads once.
constexpr int kNonTemporal = 2;
__device__ __forceinline__ v4i bload16_nt(Rsrc r, int voff, int soff) {
  return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kNonTemporal));
}
__device__ __forceinline__ uint32_t bload4(Rsrc r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
__device__ __forceinline__ uint32_t bload2(Rsrc r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}
__device__ __forceinline__ uint32_t bload1(Rsrc r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, voff, soff, 0);
}
// A per-lane offset past every descriptor's range: the load returns zeros, moves nothing.
constexpr int kOob = 0x7FFFFF00;

// x (at most 16 significant bits) as an exact sum of two bf16 values, packed as a word
// for a bf16 matrix-core operand: the leading 8 significant bits in the low half, the
// remainder (exact: at most 8 bits) in the high half.
__device__ __forceinline__ uint32_t bf16_pair(float x) {
  const uint32_t b0 = __float_as_uint(x) & 0xFFFF0000u;
  const uint32_t b1 = __float_as_uint(x - __uint_as_float(b0));
  // bytes 2, 3 of b0 into bytes 0, 1 and bytes 2, 3 of b1 into bytes 2, 3 (one v_perm_b32)
  return __builtin_amdgcn_perm(b1, b0, 0x07060302u);
}
typedef __attribute__((address_space(3))) void *LdsPtr;
// 16 bytes per lane from the buffer into LDS at dst + 16 * lane (dst wave-uniform).
__device__ __forceinline__ void bload16_lds(Rsrc r, void *dst, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LdsPtr)dst, 16, voff, soff, 0, 0);
}

// s_waitcnt with only the vector-memory count: wait until at most N vector-memory
// operations of this wave are outstanding (gfx9 encoding: vmcnt low bits [3:0], high
// bits [15:14]; expcnt 7 and lgkmcnt 15 mean "no wait").
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for LDS data: this wave's LDS reads and writes complete, then the
// barrier.  The scheduler barriers keep the compiler from moving memory operations
// across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// RDMA: this wave also loads 32 rows of the row operand records per step; CDMA: it also
// loads the column scales (wave 2) or zero points (wave 3) of the tile's four blocks.
template <int NB, int KIND, bool PARTIALS, bool RDMA, bool CDMA, int Q, bool WNT>
__device__ __forceinline__ void tile_body(const GemmArgs &p, TileSmem<NB> &sm, int m0, int blk, int bi, int lane) {
  constexpr int q = Q;  // group slice
  constexpr bool HASW = KIND != kNone;
  constexpr int NW = KIND == kW8 ? 4 : (KIND == kW4 ? 2 : 0);     // 16-byte weight loads per step
  // Zero-point word: partials mode, and the variant that subtracts the zero point from
  // the codes before the matrix cores.
  constexpr bool ZPRE = kZeroPre && !PARTIALS && KIND == kW4;
  constexpr int NZ = ((PARTIALS && KIND == kW4) || ZPRE) ? 1 : 0;
  constexpr bool CORR = KIND == kW4 && !ZPRE && !PARTIALS;
  constexpr bool BIAS = kFoldBias && !PARTIALS;
  constexpr int kDmaRows = 64 / NB;                               // activation rows this wave loads
  constexpr bool CLDS = NB == kTileNB;                            // column values from LDS
  constexpr bool CWORDS = CLDS && CDMA && !PARTIALS;               // (the partials need no column values)
  constexpr int NPW = (!CLDS && !PARTIALS) ? (CORR ? 2 : 1) : 0;  // column-value loads into registers
  constexpr int LD = kDmaRows / 8 + (RDMA ? 1 : 0) + (CWORDS ? 1 : 0);  // direct-to-LDS loads per step
  constexpr int LW = HASW ? NW + NPW + NZ : 0;                    // register-ring loads per step
  // Issue order.  A wave that folds (HASW, not partials) loads the weights of step
  // t + kSA - 1 in the first half of step t (their ring slot is free once step t - 1 has
  // decoded it) and stage t + kSA in the second half, after the barrier that frees it;
  // the prologue keeps the same order (weights t before stage t + 1).  Before the barrier
  // of step s, stage s + 1 must have landed; after it came the weights of steps s + 1 ..
  // s + kSA - 1 and the stages s + 2 .. s + kSA - 1.  Other waves issue both parts of
  // their batch after the barrier of step s (stage, then the weights of step s + kSA - 1):
  // after stage s + 1 came its batch's weights, already waited for by the decode of this
  // step, and the batches of the kSA - 2 steps since.
  constexpr bool WEARLY = HASW && !PARTIALS;
  constexpr int WAIT = WEARLY ? (kSA - 2) * LD + (kSA - 1) * LW : (kSA - 2) * (LD + LW);
  static_assert(WAIT < 64, "vmcnt range");
  const int ch32 = lane & 31, h = lane >> 5;
  const int G = p.G;
  const int nsteps = (G + kKS - 1) / kKS;                          // same for every wave
  const int niter = (nsteps + kSA - 1) / kSA;

  // Descriptors.  Activation rows past M load zeros; operand rows past M repeat row M - 1.
  const Rsrc ra = make_rsrc(p.aq + (int64_t)m0 * p.K, (int64_t)(p.M - m0) * p.K);
  const Rsrc rro = make_rsrc(p.rowop, (int64_t)G * p.M * 32);
  const int bq = KIND == kW8 ? blk - p.nb4 : blk;
  constexpr int kWChunk = KIND == kW8 ? (int)kW8Chunk : (int)kW4Chunk;
  const Rsrc rw = make_rsrc((KIND == kW8 ? p.w8 : p.w4) + (size_t)bq * G * kWChunk, (int64_t)G * kWChunk);
  // Column values of step s (groups 2s and 2s + 1): the fp16 scales s_w and, for the
  // corrections of 4-bit blocks, the zero points z.  Through LDS (4-block tiles) wave 2 of
  // slice 1 loads the scales of the tile's blocks (lane l < 32: block l / 8, group
  // l / 4 % 2, channels 8 (l % 4) .. + 8, from s4 or s8 through one descriptor over both
  // sections) and wave 3 their zero points (lane l < 8: block l / 2, group l % 2, 32
  // nibbles); other lanes, groups past the layer and blocks past it (or not 4-bit, for
  // the zero points) read zeros.  Else each wave loads its own channel's values.
  const uint8_t *s4b = reinterpret_cast<const uint8_t *>(p.s4);
  const int64_t s8off = reinterpret_cast<const uint8_t *>(p.s8) - s4b;
  const bool zrole = bi == 3;
  const Rsrc rcol = !CWORDS ? make_rsrc(s4b, 0)
                    : zrole ? make_rsrc(p.z4, (int64_t)p.nb4 * G * (int)kZ4Chunk)
                            : make_rsrc(s4b, s8off + (int64_t)(p.nb - p.nb4) * G * 64);
  int vcol = kOob, cgp = 0;  // DMA lane: offset of its chunk in group cgp (step 0), its group parity
  if constexpr (CWORDS) {
    const int j = zrole ? (lane >> 1) : (lane >> 3);                 // the lane's block in the tile
    const int tb = p.ileave ? blk + (j - bi) * p.tiles_n : blk - bi + j;
    cgp = zrole ? (lane & 1) : ((lane >> 2) & 1);
    if (zrole ? (lane < 8 && tb < p.nb4) : (lane < 32 && tb < p.nb))
      vcol = zrole ? (tb * G + cgp) * (int)kZ4Chunk
                   : (int)((tb < p.nb4 ? (int64_t)tb * G * 64 : s8off + (int64_t)(tb - p.nb4) * G * 64) + cgp * 64 +
                           (lane & 3) * 16);
  }
  const Rsrc rsw = make_rsrc((KIND == kW8 ? s4b + s8off + (size_t)bq * G * 64 : s4b + (size_t)blk * G * 64),
                             NPW ? (int64_t)G * 64 : 0);
  const Rsrc rzw = make_rsrc(p.z4 + (size_t)blk * G * kZ4Chunk, NPW == 2 ? (int64_t)G * kZ4Chunk : 0);
  const Rsrc rz = make_rsrc(p.z4 + (size_t)blk * G * kZ4Chunk, NZ ? (int64_t)G * kZ4Chunk : 0);

  // Per-lane offsets.
  int vdma[kDmaRows / 8];  // this wave loads rows [kDmaRows bi, + kDmaRows) of the slice's tile, 8 per load
#pragma unroll
  for (int i = 0; i < kDmaRows / 8; ++i) {
    const int r = kDmaRows * bi + 8 * i + (lane >> 3), pos = lane & 7;
    vdma[i] = r * p.K + ((pos ^ swz_a(r)) << 4);
  }
  // ... and (waves 0 and 1 of a slice) the 32-byte operand records of rows [32 bi, 32 bi + 32)
  const int vro = min(m0 + 32 * bi + (lane >> 1), p.M - 1) * 32 + (lane & 1) * 16;
  int vw[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
    vw[s] = KIND == kW8 ? ((ch32 >> 4) * 8 + chunk32(s, h)) * 256 + (ch32 & 15) * 16
                        : (((ch32 >> 4) * 4 + 2 * (s & 1) + h) * 16 + (ch32 & 15)) * 16;
  // LDS byte offsets of this lane's operands in stage 0, row block 0 (row block 1: + 32 rows)
  int va[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) va[s] = q * kTileBM * 128 + ch32 * 128 + ((chunk32(s, h) ^ swz_a(ch32)) << 4);
  const int vrs = kRBase + q * kTileBM * 32 + ch32 * 32;       // s-part of this slice's record
  const int vru = kRBase + h * kTileBM * 32 + ch32 * 32 + 16;  // u-part, slice h (corrections)
  uint8_t *const smb = reinterpret_cast<uint8_t *>(&sm);

  // Register ring (raw loaded bits): slot s % kSA holds step s.
  v4i bR[kSA][NW > 0 ? NW : 1];
  uint32_t cR[kSA][2];  // column values (2-block tiles): s_w and z of group 2s + h (s_w of 2s + q without z)
  uint32_t zR[kSA];

  // Stage s % kSA: the activation tile and the row operands of step s, in two pieces (the
  // first half of this wave's activation rows; the rest with the records and column values).
  constexpr int NA = kDmaRows / 8;
  auto issue_stage = [&](auto j_c, int s, int piece) {
    constexpr int J = decltype(j_c)::value;
    const int gl = min(kKS * s + q, G - 1);
#pragma unroll
    for (int i = piece ? (NA + 1) / 2 : 0; i < (piece ? NA : (NA + 1) / 2); ++i)
      bload16_lds(ra, smb + J * kAStage + q * kTileBM * 128 + (kDmaRows * bi + 8 * i) * 128, vdma[i], gl * 128);
    if (piece) {
      if constexpr (RDMA) bload16_lds(rro, smb + kRBase + J * kRStage + q * kTileBM * 32 + bi * 1024, vro, gl * p.M * 32);
      if constexpr (CWORDS)
        bload16_lds(rcol, smb + kCBase + J * kCStage + (zrole ? kCZero : 0),
                    vcol != kOob && 2 * s + cgp < G ? vcol + 2 * s * (zrole ? (int)kZ4Chunk : 64) : kOob, 0);
    }
  };
  auto issue_a = [&](auto j_c, int s) {
    issue_stage(j_c, s, 0);
    issue_stage(j_c, s, 1);
  };
  // Ring slot s % kSA: this wave's weights of step s (and in 2-block tiles its column
  // values; groups past the layer read zeros), in two pieces (the first half of the
  // weights; the rest with the column values and zero-point word).
  auto issue_weights = [&](auto j_c, int s, int piece) {
    constexpr int J = decltype(j_c)::value;
    if constexpr (HASW) {
      const int gl = min(kKS * s + q, G - 1);
#pragma unroll
      for (int t = piece ? (NW + 1) / 2 : 0; t < (piece ? NW : (NW + 1) / 2); ++t)
        bR[J][t] = WNT ? bload16_nt(rw, vw[t], gl * kWChunk) : bload16(rw, vw[t], gl * kWChunk);
      if (!piece) return;
      // (whole words: the lane's fp16 scale and zero-point byte are extracted when used;
      // 2-byte and 1-byte loads measured slower)
      if constexpr (NPW == 1) {
        cR[J][0] = bload4(rsw, (ch32 >> 1) * 4, (2 * s + q) * 64);
      } else if constexpr (NPW == 2) {
        cR[J][0] = bload4(rsw, h * 64 + (ch32 >> 1) * 4, 2 * s * 64);
        cR[J][1] = bload4(rzw, h * (int)kZ4Chunk + (ch32 >> 3) * 4, 2 * s * (int)kZ4Chunk);
      }
      if constexpr (NZ) zR[J] = bload4(rz, (ch32 >> 3) * 4, gl * (int)kZ4Chunk);
    }
  };
  auto issue_w = [&](auto j_c, int s) {
    issue_weights(j_c, s, 0);
    issue_weights(j_c, s, 1);
  };

  v16f acc0 = v16f{0}, acc1 = v16f{0};  // folded products of row blocks 0 and 1
  v16i P0, P1 = v16i{0};                // group partials (P1: block 1 of the previous step)
  v16f sc0, sc1 = v16f{0};              // and their scale products
  if constexpr (BIAS) {
#pragma unroll
    for (int r = 0; r < 16; ++r) P1[r] = kBiasBits;
  }
  v16i pinit;
#pragma unroll
  for (int r = 0; r < 16; ++r) pinit[r] = BIAS ? kBiasBits : 0;
  v4i a0[4], a1[4];                     // activation operands of row blocks 0 and 1
  v4i rs0, rs1;                         // s-parts of the row records
  const int jp = blk * 32 + ch32;
  // The channel's original index for the scatter epilogue, loaded now so its latency
  // overlaps the main loop instead of delaying the final stores.
  const int orig_out = (!PARTIALS && HASW) ? p.idx[jp] : -1;

  auto lds16 = [&](int off) { return *reinterpret_cast<const v4i *>(smb + off); };
  auto load_a = [&](auto j_c, int rb, v4i (&av)[4]) {
    constexpr int J = decltype(j_c)::value;
#pragma unroll
    for (int k = 0; k < 4; ++k) av[k] = lds16(va[k] + J * kAStage + rb * 32 * 128);
  };
  auto chain = [&](const v4i (&av)[4], const v4i (&bw)[4]) {
    v16i P = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[0], bw[0], pinit, 0, 0, 0);
#pragma unroll
    for (int k = 1; k < 4; ++k) P = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[k], bw[k], P, 0, 0, 0);
    return P;
  };
  // acc += float(P) * sc for the four output registers [4c, 4c + 4).
  auto fold4 = [&](v16f &acc, const v16i &P, const v16f &sc, int c) {
#pragma unroll
    for (int r = 4 * c; r < 4 * c + 4; ++r) {
      const float x = BIAS ? __int_as_float(P[r]) - 12582912.0f : (float)P[r];
      acc[r] = fmaf(x, sc[r], acc[r]);
    }
  };
  auto fold = [&](v16f &acc, const v16i &P, const v16f &sc) {
#pragma unroll
    for (int c = 0; c < 4; ++c) fold4(acc, P, sc, c);
  };
  auto fence = [] { __builtin_amdgcn_sched_barrier(0); };

  // Partials mode: the exact group partials of an active step, zero point removed.
  auto emit = [&](int rb, const v16i &Pc, int g, uint32_t zword) {
    const int orig = p.idx[jp];
    const uint32_t z = KIND == kW4 ? ((zword >> ((ch32 & 7) * 4)) & 15u) : 0u;
    if (orig >= p.n_begin && orig < p.n_begin + p.n_count) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + rb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (row < p.M) {
          const int corr = KIND == kW4 ? (int)z * p.asum[(int64_t)g * p.M + row] : 0;
          p.part[((int64_t)row * p.n_count + (orig - p.n_begin)) * G + g] = Pc[r] - corr;
        }
      }
    }
  };

  // Weight operand k (k-chunks of one 32-wide step) of ring slot W: 4-bit codes as bytes
  // (3 VALU ops per 8 codes; with the zero_pre variant, (q - z) per byte), or the 8-bit
  // codes as loaded.
  auto decode = [&](auto w_c, int k) -> v4i {
    constexpr int W = decltype(w_c)::value;
    if constexpr (KIND == kW4) {
      const int e = k >> 1, u = k & 1;
      const uint32_t x0 = (uint32_t)bR[W][e][2 * u], x1 = (uint32_t)bR[W][e][2 * u + 1];
      if constexpr (ZPRE) {
        const uint32_t zz = ((zR[W] >> ((ch32 & 7) * 4)) & 15u) * 0x01010101u;
        return w4_operand(x0, x1, zz);
      } else {
        return v4i{(int)(x0 & 0x0F0F0F0Fu), (int)((x0 >> 4) & 0x0F0F0F0Fu), (int)(x1 & 0x0F0F0F0Fu),
                   (int)((x1 >> 4) & 0x0F0F0F0Fu)};
      }
    } else {
      return bR[W][k];
    }
  };

  // Column operands of step s (stage / ring slot J), as exact bf16 pairs: s_w of this
  // wave's group (2s + q) for the scale products (zero in the upper half-wave, whose row
  // operand slots are unused), and for the corrections -z s_w of group 2s + h, the group
  // whose row operands half-wave h reads (z s_w has at most 15 significant bits, so it is
  // exact in fp32 too).  Each step forms the next step's, off its own critical path.
  struct ColOps {
    int sw, zw;
  };
  auto col_ops = [&](auto j_c) -> ColOps {
    constexpr int J = decltype(j_c)::value;
    uint32_t sq16, sh16 = 0, zh = 0;
    if constexpr (CLDS) {
      // (whole words, as for the loads below: the lane's half or byte is extracted)
      const uint8_t *cst = smb + kCBase + J * kCStage;
      auto word = [&](int off) { return *reinterpret_cast<const uint32_t *>(cst + off); };
      sq16 = word(bi * 128 + q * 64 + (ch32 >> 1) * 4) >> ((ch32 & 1) * 16);
      if constexpr (CORR) {
        sh16 = word(bi * 128 + h * 64 + (ch32 >> 1) * 4) >> ((ch32 & 1) * 16);
        zh = word(kCZero + (bi * 2 + h) * 16 + (ch32 >> 3) * 4) >> ((ch32 & 6) * 4);
      }
    } else if constexpr (CORR) {
      // s_w of group 2s + q is what half-wave q loaded: swapping the halves of two copies
      // leaves the lower half-wave's values in every lane of the first result and the
      // upper half-wave's in the second.
      sh16 = cR[J][0] >> ((ch32 & 1) * 16);
      zh = cR[J][1] >> ((ch32 & 6) * 4);  // the byte of channels ch32 & ~1, ch32 | 1
      const auto halves = __builtin_amdgcn_permlane32_swap(sh16, sh16, false, false);
      sq16 = halves[q];
    } else {
      sq16 = cR[J][0] >> ((ch32 & 1) * 16);
    }
    // (computed in every lane and pinned there: a conditional computation would become a
    // branch, which splits the step's schedule)
    uint32_t swl = bf16_pair(h2f((uint16_t)sq16));
    asm volatile("" : "+v"(swl));
    ColOps c{h ? 0 : (int)swl, 0};
    if constexpr (CORR) {
      const float zf = (float)((zh >> ((ch32 & 1) * 4)) & 15u);
      c.zw = (int)(bf16_pair(zf * h2f((uint16_t)sh16)) ^ 0x80008000u);
    }
    return c;
  };
  ColOps co{0, 0};  // this step's

  // One step s: stage J = s % kSA.  Entry: a0 and rs0 hold row block 0's operands of step
  // s (read during the previous step), P1 / sc1 the previous step's block 1.  The code is
  // written in issue order; the scheduler barriers between its pieces keep each MFMA
  // next to the vector work that overlaps it.
  auto step = [&](auto j_c, int s) {
    constexpr int J = decltype(j_c)::value;
    constexpr int JN = (J + 1) % kSA;
    if constexpr (!HASW) {
      wait_vm<WAIT>();
      lds_barrier();
      issue_a(IntC<J>{}, s + kSA);
      issue_w(IntC<(J + kSA - 1) % kSA>{}, s + kSA - 1);
      return;
    }
    v4i bw[4];
    if constexpr (PARTIALS) {
#pragma unroll
      for (int k = 0; k < 4; ++k) bw[k] = decode(j_c, k);
      const int g = kKS * s + q;
      const v16i Pa = chain(a0, bw);
      load_a(j_c, 1, a1);
      if (g < G) emit(0, Pa, g, zR[J]);
      wait_vm<0>();  // the partials' stores count too: wait for everything
      lds_barrier();
      issue_a(IntC<J>{}, s + kSA);
      issue_w(IntC<(J + kSA - 1) % kSA>{}, s + kSA - 1);
      const v16i Pb = chain(a1, bw);
      load_a(IntC<JN>{}, 0, a0);
      if (g < G) emit(1, Pb, g, zR[J]);
      return;
    }
    const v4i bs = v4i{co.sw, co.sw, co.sw, co.sw};
    v4i bz;
    if constexpr (CORR) bz = v4i{co.zw, co.zw, co.zw, co.zw};
    // First half: row block 0 on the matrix cores, row block 1 of the previous step folds
    // and this step's codes are decoded.
    sc0 = mfma_bf16(rs0, bs, v16f{0});
    bw[0] = decode(j_c, 0);
    fence();
    P0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0[0], bw[0], pinit, 0, 0, 0);
    bw[1] = decode(j_c, 1);
    fold4(acc1, P1, sc1, 0);
    a1[0] = lds16(va[0] + J * kAStage + 32 * 128);
    fence();
    P0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0[1], bw[1], P0, 0, 0, 0);
    issue_weights(IntC<(J + kSA - 1) % kSA>{}, s + kSA - 1, 0);  // slot of step s - 1, decoded
    bw[2] = decode(j_c, 2);
    fold4(acc1, P1, sc1, 1);
    a1[1] = lds16(va[1] + J * kAStage + 32 * 128);
    fence();
    P0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0[2], bw[2], P0, 0, 0, 0);
    issue_weights(IntC<(J + kSA - 1) % kSA>{}, s + kSA - 1, 1);
    bw[3] = decode(j_c, 3);
    fold4(acc1, P1, sc1, 2);
    a1[2] = lds16(va[2] + J * kAStage + 32 * 128);
    fence();
    P0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0[3], bw[3], P0, 0, 0, 0);
    fold4(acc1, P1, sc1, 3);
    a1[3] = lds16(va[3] + J * kAStage + 32 * 128);
    rs1 = lds16(vrs + J * kRStage + 32 * 32);
    // The correction's row operands come from stage s too, so they are read before the
    // barrier that frees it.
    v4i ru;
    if constexpr (CORR) ru = lds16(vru + J * kRStage + q * 32 * 32);
    fence();
    if constexpr (CORR && q == 0) acc0 = mfma_bf16(ru, bz, acc0);
    fence();
    wait_vm<WAIT>();
    lds_barrier();  // stage s + 1 is published; stage s is free
    fence();
    // Second half: row block 1 on the matrix cores, row block 0 folds, and stage s + kSA
    // goes out in two pieces between the matrix-core operations.  (Spreading the batch over
    // the step rather than issuing it at once after the barrier measured 3-7% faster: the
    // workgroup's loads reach the memory path spread out.)
    sc1 = mfma_bf16(rs1, bs, v16f{0});
    fence();
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      P1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1[k], bw[k], k ? P1 : pinit, 0, 0, 0);
      if (k == 0 || k == 2) issue_stage(j_c, s + kSA, k >> 1);
      fold4(acc0, P0, sc0, k);
      a0[k] = lds16(va[k] + JN * kAStage);
      if (k == 3) rs0 = lds16(vrs + JN * kRStage);
      fence();
    }
    const ColOps nxt = col_ops(IntC<JN>{});  // stage s + 1 was published at this step's barrier
    if constexpr (CORR && q == 1) acc1 = mfma_bf16(ru, bz, acc1);
    fence();
    co = nxt;
  };

  // Prologue: stages 0 .. kSA - 1 and the weights of steps 0 .. kSA - 2 in the loop's
  // order (see WAIT), then stage 0 is published and row block 0's operands of step 0 are
  // read.  Every load counted by the waits is one the code uses:
  // a load whose result is never read would be deleted by the compiler and break the count.
  static_for<0, kSA>([&](auto t_c) {
    constexpr int T = decltype(t_c)::value;  // virtual step T - kSA
    if constexpr (WEARLY) {
      issue_a(IntC<T>{}, T);
      if constexpr (T < kSA - 1) issue_w(IntC<T>{}, T);
    } else {
      issue_a(IntC<T>{}, T);
      if constexpr (T > 0) issue_w(IntC<T - 1>{}, T - 1);
    }
  });
  wait_vm<(kSA - 1) * (LD + LW)>();
  lds_barrier();
  if constexpr (HASW) {
    load_a(IntC<0>{}, 0, a0);
    rs0 = lds16(vrs);
    if constexpr (!PARTIALS) co = col_ops(IntC<0>{});
  }
  for (int it = 0; it < niter; ++it) {
    const int s = it * kSA;
    static_for<0, kSA>([&](auto j_c) { step(j_c, s + decltype(j_c)::value); });
  }
  if constexpr (!PARTIALS && HASW) fold(acc1, P1, sc1);
  // All direct-to-LDS loads (including those past the last step) have landed before the
  // stages' space is reused.
  wait_vm<0>();
  lds_barrier();
  if constexpr (PARTIALS) return;

  // Sum the two slices' accumulators and write the output: slice 0 finishes rows 0-31
  // (block 0) and slice 1 rows 32-63 (block 1), each adding the other slice's partial
  // sums taken from LDS; both compute slice 0's value + slice 1's value.
  static_assert(kKS == 2, "the epilogue pairs two slices");
  float *red = reinterpret_cast<float *>(&sm.a[0][0][0]);  // [block kept by the reader][wave][r][lane]
  const int give = 1 - q;                                   // the block this wave hands over
#pragma unroll
  for (int r = 0; r < 16; ++r) red[((give * NB + bi) * 16 + r) * 64 + lane] = q == 0 ? acc1[r] : acc0[r];
  lds_barrier();
  if (KIND == kNone) return;
  v16f mine = q == 0 ? acc0 : acc1;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float other = red[((q * NB + bi) * 16 + r) * 64 + lane];
    mine[r] = q == 0 ? mine[r] + other : other + mine[r];
  }
  if (p.ident) {
    // Channels in original order (all 4-bit or all 8-bit): no scatter.  The wave's
    // 32 x 32 block goes through LDS row-major, then out as 16-byte runs of 8 channels.
    uint16_t *st = reinterpret_cast<uint16_t *>(&sm.a[0][0][0] + kKS * kTileNB * 16 * 64 * 4) +
                   (q * NB + bi) * 32 * 32;
#pragma unroll
    for (int r = 0; r < 16; ++r) st[(8 * (r >> 2) + 4 * h + (r & 3)) * 32 + ch32] = f2h(mine[r]);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = i * 16 + (lane >> 2), c8 = (lane & 3) * 8;
      const uint4 v = *reinterpret_cast<const uint4 *>(st + row * 32 + c8);
      const int grow = m0 + q * 32 + row, col = blk * 32 + c8;
      if (grow >= p.M) continue;
      uint16_t *dst = p.y + (int64_t)grow * p.ldy + col;
      if (col + 8 <= p.N) {
        *reinterpret_cast<uint4 *>(dst) = v;
      } else {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (col + e < p.N) dst[e] = (uint16_t)(w[e >> 1] >> ((e & 1) * 16));
      }
    }
    return;
  }
  if (orig_out < 0) return;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = m0 + q * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
    if (row < p.M) p.y[(int64_t)row * p.ldy + orig_out] = f2h(mine[r]);
  }
}

// The body for one wave: its block kind, which shared loads it issues, its slice.  Waves
// 0 and 1 of each slice load the row operand records (32 rows each); in 4-block tiles the
// column words go to waves 2 and 3 of slice 1.
template <int NB, bool PARTIALS, int Q, bool RDMA, bool CDMA, bool WNT>
__device__ __forceinline__ void tile_kind(const GemmArgs &p, TileSmem<NB> &sm, int m0, int blk, int bi, int lane,
                                          int kind) {
  switch (kind) {
    case kW4: tile_body<NB, kW4, PARTIALS, RDMA, CDMA, Q, WNT>(p, sm, m0, blk, bi, lane); break;
    case kW8: tile_body<NB, kW8, PARTIALS, RDMA, CDMA, Q, WNT>(p, sm, m0, blk, bi, lane); break;
    default: tile_body<NB, kNone, PARTIALS, RDMA, CDMA, Q, WNT>(p, sm, m0, blk, bi, lane); break;
  }
}

template <int NB, bool PARTIALS, int Q, bool WNT>
__device__ __forceinline__ void tile_dispatch(const GemmArgs &p, TileSmem<NB> &sm, int m0, int blk, int bi,
                                              int lane, int kind) {
  if constexpr (NB != kTileNB) {
    tile_kind<NB, PARTIALS, Q, true, false, WNT>(p, sm, m0, blk, bi, lane, kind);
  } else {
    if (bi < 2)
      tile_kind<NB, PARTIALS, Q, true, false, WNT>(p, sm, m0, blk, bi, lane, kind);
    else if (Q == 1)
      tile_kind<NB, PARTIALS, Q, false, true, WNT>(p, sm, m0, blk, bi, lane, kind);
    else
      tile_kind<NB, PARTIALS, Q, false, false, WNT>(p, sm, m0, blk, bi, lane, kind);
  }
}

// Workgroup w runs on XCD w % 8.  The tiles go to the XCDs in contiguous ranges, ordered
// in bands of kTileBand M tiles (M tile fastest within a band), so the workgroups an XCD
// runs at once share both activation rows and weight blocks in its L2.
constexpr int kTileBand = 4;

// NB: channel blocks per workgroup (4; 2 on layers too narrow to fill the CUs with 4).
// WNT: the weights load with the non-temporal policy, for grids of one band, whose
// workgroups reading a weight block all run at once (with more bands a later band reads
// it again from L2: measured 7% slower with the policy at M = 512 and 2048, and 2-5% faster
// at M = 64-256).
template <int NB, bool PARTIALS, bool WNT>
__global__ __launch_bounds__(tile_threads(NB)) __attribute__((amdgpu_waves_per_eu(2))) void gemm_tile_kernel(
    const GemmArgs p) {
  __shared__ __attribute__((aligned(16))) TileSmem<NB> sm;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;  // wave: uniform
  const int bi = wave % NB, q = wave / NB;

  const int T = p.tiles_m * p.tiles_n;
  const int xcd = blockIdx.x & 7, i = blockIdx.x >> 3;
  const int per = T >> 3, rem = T & 7;
  const int t = xcd * per + (xcd < rem ? xcd : rem) + i;
  const int band = t / (kTileBand * p.tiles_n), in_band = t - band * (kTileBand * p.tiles_n);
  const int bm = min(kTileBand, p.tiles_m - band * kTileBand);  // M tiles in this band
  const int tm = band * kTileBand + in_band % bm, tr = in_band / bm;
  // When the whole grid runs at once, N tiles go in a stride-8 order so that the XCDs
  // sharing a band each get some of the 8-bit blocks (one in each of the last N tiles)
  // instead of one XCD getting all of them; in longer grids the contiguous order streams
  // the weights better.
  const int tn = (!p.spread || (p.tiles_n & 7)) ? tr : (tr & 7) * (p.tiles_n >> 3) + (tr >> 3);
  const int m0 = tm * kTileBM;
  // With ileave, block bi of N tile tn is block bi * tiles_n + tn: a tile's blocks are
  // tiles_n apart, so the 8-bit blocks (the last ones) go one to a tile instead of filling
  // the last tiles.
  const int blk = p.ileave ? bi * p.tiles_n + tn : tn * NB + bi;
  const int kind = blk >= p.nb ? kNone : (blk < p.nb4 ? kW4 : kW8);
  // Waves 0 and 1 of each slice also load the row operand records (32 rows each).
  if (q == 0)
    tile_dispatch<NB, PARTIALS, 0, WNT>(p, sm, m0, blk, bi, lane, kind);
  else
    tile_dispatch<NB, PARTIALS, 1, WNT>(p, sm, m0, blk, bi, lane, kind);
}
// ------------------------------------------------------------------------------------
// Skinny kernel (small M): one workgroup per 16-channel half block; its KS waves share
// the groups (wave w takes groups w, w + KS, w + 2 KS, ...), each wave computes all
// M <= 16 RB rows for its groups with v_mfma_i32_16x16x64_i8, and the partial sums are
// reduced through LDS.
// The kernel is bound by the weight stream from HBM: every wave keeps the loads of the
// next D - 1 groups in flight (a register ring, unrolled so the slot indices are
// constants; the compiler places the waits), then finishes the last cnt % D groups in an
// unrolled tail.  Loads issued ahead past a wave's last group re-read that group (the
// group index is clamped) and are never consumed.
// ------------------------------------------------------------------------------------
// A per-lane buffer offset beyond any skinny-kernel descriptor, even with the largest
// scalar offset added (the host checks M * K and G * M * 4 stay below it).
constexpr int kSkinnyOob = 0x7FFFFF00;

// The groups of wave `wave` among `ks` sharing G: wave, wave + ks, ... (interleaved, so
// the workgroup reads a block's group chunks in address order, ks chunks at a time:
// measured 2-14% faster on the Llama-3.1 8B and 70B layers at one to 32 tokens than
// contiguous ranges per wave, whose concurrent streams sit G / ks chunks apart).
__device__ __forceinline__ int wave_groups(int G, int wave, int ks) { return (G - wave + ks - 1) / ks; }

// Ring depths (measured on the Llama-3.1 8B and 70B layers): weights 8 groups for one
// 16-row block of 4-bit codes, else 4; activations 8 for one block, 4 for two, 2 for three
// or four (deeper rings spill there).
constexpr int skinny_wring(int rb, int kind) { return rb == 1 && kind == kW4 ? 8 : 4; }
constexpr int skinny_aring(int rb) { return rb == 1 ? 8 : (rb == 2 ? 4 : 2); }

template <int RB, int KIND, bool PARTIALS>
__device__ __forceinline__ void skinny_body(const GemmArgs &p, int blk, int half, int lane, int g0, int gstep,
                                            int cnt, float (&acc)[RB][4]) {
  constexpr int DW = skinny_wring(RB, KIND);         // weight ring: loads DW - 1 groups ahead
  constexpr int DA = skinny_aring(RB) < DW ? skinny_aring(RB) : DW;  // activation ring: DA - 1 ahead
  constexpr int NWL = KIND == kW8 ? 2 : 1;           // 16-byte weight loads per group
  const int ch = lane & 15, qd = lane >> 4, ch32 = half * 16 + ch;
  const int G = p.G;
  const int jp = blk * 32 + ch32;
  const int bq = KIND == kW8 ? blk - p.nb4 : blk;
  constexpr int kWChunk = KIND == kW8 ? (int)kW8Chunk : (int)kW4Chunk;
  const Rsrc rw = make_rsrc((KIND == kW8 ? p.w8 : p.w4) + (size_t)bq * G * kWChunk, (int64_t)G * kWChunk);
  const Rsrc rs = make_rsrc((KIND == kW8 ? p.s8 : p.s4) + (size_t)bq * G * 32, (int64_t)G * 64);
  const Rsrc rz = make_rsrc(p.z4 + (size_t)bq * G * kZ4Chunk, KIND == kW4 ? (int64_t)G * kZ4Chunk : 0);
  const Rsrc ra = make_rsrc(p.aq, (int64_t)p.M * p.K);
  const Rsrc rsa = make_rsrc(p.sa, (int64_t)G * p.M * 4);
  // Per-lane offsets.  Lanes of rows past M take an offset past the end of every
  // descriptor (kSkinnyOob), so their loads return zeros without touching memory.
  const int vw = KIND == kW8 ? half * 2048 + lane * 16 : half * 1024 + lane * 16;
  int va[RB][2], vsa[RB][4];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = rb * 16 + ch;
#pragma unroll
    for (int c = 0; c < 2; ++c) va[rb][c] = row < p.M ? row * p.K + (qd + 4 * c) * 16 : kSkinnyOob;
#pragma unroll
    for (int r = 0; r < 4; ++r) vsa[rb][r] = rb * 16 + 4 * qd + r < p.M ? (rb * 16 + 4 * qd + r) * 4 : kSkinnyOob;
  }

  v4i wR[DW][NWL];
  uint32_t zR[DW], sR[DW];
  v4i aR[DA][RB][2], saR[DA][RB];
  auto grp = [&](int s) { return g0 + min(s, cnt - 1) * gstep; };
  // The activation loads of step s go first in a step's batch: waiting for them then
  // leaves the deeper weight loads issued after them in flight.
  auto issue_a = [&](auto j_c, int s) {
    constexpr int J = decltype(j_c)::value;
    const int g = grp(s);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int c = 0; c < 2; ++c) aR[J][rb][c] = bload16(ra, va[rb][c], g * 128);
#pragma unroll
      for (int r = 0; r < 4; ++r) saR[J][rb][r] = (int)bload4(rsa, vsa[rb][r], g * p.M * 4);
    }
  };
  auto issue_w = [&](auto j_c, int s) {
    constexpr int J = decltype(j_c)::value;
    const int g = grp(s);
#pragma unroll
    for (int t = 0; t < NWL; ++t) wR[J][t] = bload16_nt(rw, vw + t * 1024, g * kWChunk);
    sR[J] = bload4(rs, (ch32 >> 1) * 4, g * 64);
    if constexpr (KIND == kW4) zR[J] = bload4(rz, (ch32 >> 3) * 4, g * (int)kZ4Chunk);
  };
  auto compute = [&](auto jw_c, auto ja_c, int s) {
    constexpr int JW = decltype(jw_c)::value, JA = decltype(ja_c)::value;
    const int g = grp(s);
    const float sw = h2f((uint16_t)(sR[JW] >> ((ch32 & 1) * 16)));
    v4i b0, b1;
    if constexpr (KIND == kW4) {
      const uint32_t zz = ((zR[JW] >> ((ch32 & 7) * 4)) & 15u) * 0x01010101u;
      const v4i x = wR[JW][0];
      b0 = w4_operand((uint32_t)x[0], (uint32_t)x[1], zz);
      b1 = w4_operand((uint32_t)x[2], (uint32_t)x[3], zz);
    } else {
      b0 = wR[JW][0];
      b1 = wR[JW][1];
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      v4i P = __builtin_amdgcn_mfma_i32_16x16x64_i8(aR[JA][rb][0], b0, v4i{0, 0, 0, 0}, 0, 0, 0);
      P = __builtin_amdgcn_mfma_i32_16x16x64_i8(aR[JA][rb][1], b1, P, 0, 0, 0);
      if constexpr (PARTIALS) {
        const int orig = p.idx[jp];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = rb * 16 + 4 * qd + r;
          if (row < p.M && orig >= p.n_begin && orig < p.n_begin + p.n_count)
            p.part[((int64_t)row * p.n_count + (orig - p.n_begin)) * G + g] = P[r];
        }
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[rb][r] = fmaf((float)P[r], sw * __int_as_float(saR[JA][rb][r]), acc[rb][r]);
      }
    }
  };

  // Prologue in the order the steps issue: step t issues activations for t + DA - 1, then
  // weights for t + DW - 1 (DA <= DW).
  static_assert(DW % DA == 0, "ring depths");
  static_for<0, DW - 1>([&](auto t_c) {
    constexpr int T = decltype(t_c)::value;  // "step" T - (DW - 1) of the prologue
    constexpr int SA = T - (DW - 1) + (DA - 1);
    if constexpr (SA >= 0) issue_a(IntC<SA % DA>{}, SA);
    issue_w(t_c, T);
  });
  const int nfull = cnt / DW * DW;
  for (int s = 0; s < nfull; s += DW) {
    static_for<0, DW>([&](auto j_c) {
      constexpr int J = decltype(j_c)::value;
      issue_a(IntC<(J + DA - 1) % DA>{}, s + J + DA - 1);
      issue_w(IntC<(J + DW - 1) % DW>{}, s + J + DW - 1);
      compute(j_c, IntC<J % DA>{}, s + J);
    });
  }
  // The last cnt % DW steps: their weights are already in flight; the activations of the
  // later ones still have to be issued.  (Wave-uniform branches.)
  const int rem = cnt - nfull;
  static_for<0, DW - 1>([&](auto j_c) {
    constexpr int J = decltype(j_c)::value;
    if (J < rem) {
      issue_a(IntC<(J + DA - 1) % DA>{}, nfull + J + DA - 1);
      compute(j_c, IntC<J % DA>{}, nfull + J);
    }
  });
}

constexpr int skinny_max_waves(int) { return 8; }  // waves per workgroup (up to 256 VGPRs each)

template <int RB, bool PARTIALS>
__global__ __launch_bounds__(64 * skinny_max_waves(RB)) void gemm_skinny_kernel(const GemmArgs p, int ks) {
  extern __shared__ float red_dyn[];  // [ks][RB * 4][64]
  float(*red)[RB * 4][64] = reinterpret_cast<float(*)[RB * 4][64]>(red_dyn);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int sub = blockIdx.x;
  const int blk = sub >> 1, half = sub & 1;
  const int G = p.G;
  const int cnt = wave_groups(G, wave, ks);

  float acc[RB][4];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[rb][r] = 0.0f;
  if (cnt > 0) {
    if (blk < p.nb4)
      skinny_body<RB, kW4, PARTIALS>(p, blk, half, lane, wave, ks, cnt, acc);
    else
      skinny_body<RB, kW8, PARTIALS>(p, blk, half, lane, wave, ks, cnt, acc);
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
// GEMV kernel (M = 1, one token: the decode case).  Every lane streams 64 bytes of one
// channel's codes per group and forms its part of the group partial with v_dot4_i32_i8
// against the token's activation codes, which all lanes share and which therefore come
// through scalar loads into SGPRs.  A 4-bit wave owns two blocks (64 channels, one per
// lane; the 64 bytes are the channel's 128 codes); an 8-bit wave owns one block, lanes c
// and c + 32 holding the first and second 64 inputs of channel c.  The zero point enters
// as - z * S_A.  A workgroup's waves share the groups (wave w takes every ks-th, from w)
// and reduce through LDS in a fixed order.  The vector memory path carries only weights and their
// scale and zero-point words, so the kernel is bound by the weight stream.
// ------------------------------------------------------------------------------------
constexpr int kGvWaves = 16;  // waves per workgroup at most
constexpr int kGvRing = 2;    // weight ring: loads one group ahead (deeper rings measured slower)
constexpr int kGvMaxRows = 3;  // tokens the gemv kernel takes
#ifndef MIXLLM_GV_WAVES_PER_SIMD
#define MIXLLM_GV_WAVES_PER_SIMD 7
#endif
// Waves per SIMD at most, whatever the registers allow: with all 8 the 70B gate at M = 1
// ran 30 µs instead of 24 (more waves per CU, more requests queued ahead of the youngest).
constexpr int kGvWavesPerSimd = MIXLLM_GV_WAVES_PER_SIMD;

typedef const __attribute__((address_space(4))) v16i *ConstV16;
typedef const __attribute__((address_space(4))) float *ConstF;
typedef const __attribute__((address_space(4))) int32_t *ConstI;

// 4-bit: lane c (c = lane & 31) computes packed channel 32 blk + c, blk being the strip's
// first block for lanes 0-31 and its second for lanes 32-63 (`second`; with `dup` the
// first block again, results unused).  8-bit, and 4-bit with SPLIT (one block per strip,
// for layers whose block pairs would leave CUs idle): blk0 is the block and kh = lane >> 5
// the half of the group's inputs.  MT tokens (rows): a lane decodes its codes of a group once
// and runs them against each row's activation codes; the rows' operands pass through a
// two-slot SGPR ring in (group, row) order, one item ahead.
template <int KIND, int MT, bool PARTIALS, bool SPLIT>
__device__ __forceinline__ void gemv_body(const GemmArgs &p, int blk0, int second, bool dup, int lane, int g0,
                                          int gstep, int cnt, float (&acc)[MT]) {
  constexpr int D = kGvRing;
  constexpr int kWChunk = KIND == kW8 ? (int)kW8Chunk : (int)kW4Chunk;
  const int c = lane & 31, half = c >> 4, ch = c & 15, kh = lane >> 5;
  const int G = p.G;
  const int bq = KIND == kW8 ? blk0 - p.nb4 : blk0;
  const Rsrc rw = make_rsrc((KIND == kW8 ? p.w8 : p.w4) + (size_t)bq * G * kWChunk, (int64_t)2 * G * kWChunk);
  const Rsrc rs = make_rsrc((KIND == kW8 ? p.s8 : p.s4) + (size_t)bq * G * 32, (int64_t)2 * G * 64);
  const Rsrc rz = make_rsrc(p.z4 + (size_t)bq * G * kZ4Chunk, KIND == kW4 ? (int64_t)2 * G * kZ4Chunk : 0);
  // 4-bit: unit (half * 4 + a) * 16 + ch holds k-chunks a and a + 4 of the channel (with
  // SPLIT this lane loads a = 2 kh, 2 kh + 1); 8-bit: unit (half * 8 + t) * 16 + ch holds
  // k-chunk t (this lane: t = 4 kh + a).
  constexpr int NWL = KIND == kW4 && SPLIT ? 2 : 4;  // 16-byte weight loads per group
  const int vw = KIND == kW8 ? ((half * 8 + 4 * kh) * 16 + ch) * 16
                 : SPLIT     ? ((half * 4 + 2 * kh) * 16 + ch) * 16
                             : second * G * kWChunk + ((half * 4) * 16 + ch) * 16;
  const int vs = (KIND == kW8 ? 0 : second * G * 64) + (c >> 1) * 4;
  const int vz = second * G * (int)kZ4Chunk + (c >> 3) * 4;
  const int jp = (blk0 + second) * 32 + c;
  const int64_t K = p.K;

  v4i wR[D][4];
  uint32_t sR[D], zR[D];
  v16i aR[2][2];
  float saR[2];
  int asR[2];
  auto grp = [&](int s) { return g0 + min(s, cnt - 1) * gstep; };
  // Item (s, m): row m's operands of step s's group into slot Q.
  auto issue_a = [&](auto q_c, int s, int m) {
    constexpr int Q = decltype(q_c)::value;
    const int g = grp(s);
    const int8_t *ap = p.aq + (int64_t)m * K + (int64_t)g * 128;
    aR[Q][0] = *(ConstV16)ap;
    aR[Q][1] = *(ConstV16)(ap + 64);
    saR[Q] = *(ConstF)(p.sa + (int64_t)g * MT + m);
    if constexpr (KIND == kW4) asR[Q] = *(ConstI)(p.asum + (int64_t)g * MT + m);
  };
  auto issue_w = [&](auto j_c, int s) {
    constexpr int J = decltype(j_c)::value;
    const int g = grp(s);
#pragma unroll
    for (int t = 0; t < NWL; ++t)
      wR[J][t] = bload16_nt(rw, vw + t * 256, g * kWChunk);
    sR[J] = bload4(rs, vs, g * 64);
    if constexpr (KIND == kW4) zR[J] = bload4(rz, vz, g * (int)kZ4Chunk);
  };
  // Step s (ring slot J of the weights; U = its position in the unrolled loop, which
  // fixes the activation slots): decode once, then every row, prefetching the next item.
  auto compute = [&](auto jw_c, auto u_c, int s, bool last) {
    constexpr int JW = decltype(jw_c)::value, U = decltype(u_c)::value;
    int wd[32];  // the lane's codes as 32 words of 4 consecutive inputs
    if constexpr (KIND == kW4 && SPLIT) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const v4i x = wR[JW][t];
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          // words 8w + 4t + [0, 4): the codes of inputs 64 w + 16 (2 kh + t) + [0, 16)
          const uint32_t x0 = (uint32_t)x[2 * w], x1 = (uint32_t)x[2 * w + 1];
          wd[8 * w + 4 * t + 0] = (int)(x0 & 0x0F0F0F0Fu);
          wd[8 * w + 4 * t + 1] = (int)((x0 >> 4) & 0x0F0F0F0Fu);
          wd[8 * w + 4 * t + 2] = (int)(x1 & 0x0F0F0F0Fu);
          wd[8 * w + 4 * t + 3] = (int)((x1 >> 4) & 0x0F0F0F0Fu);
        }
      }
    } else if constexpr (KIND == kW4) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const v4i x = wR[JW][a];
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          // words 2w, 2w + 1: the codes of inputs 64 w + 16 a + [0, 16)
          const uint32_t x0 = (uint32_t)x[2 * w], x1 = (uint32_t)x[2 * w + 1];
          wd[16 * w + 4 * a + 0] = (int)(x0 & 0x0F0F0F0Fu);
          wd[16 * w + 4 * a + 1] = (int)((x0 >> 4) & 0x0F0F0F0Fu);
          wd[16 * w + 4 * a + 2] = (int)(x1 & 0x0F0F0F0Fu);
          wd[16 * w + 4 * a + 3] = (int)((x1 >> 4) & 0x0F0F0F0Fu);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) wd[i] = wR[JW][i >> 2][i & 3];
    }
    const int z = KIND == kW4 ? (int)((zR[JW] >> ((c & 7) * 4)) & 15u) : 0;
    const float sw = h2f((uint16_t)(sR[JW] >> ((c & 1) * 16)));
    static_for<0, MT>([&](auto m_c) {
      constexpr int m = decltype(m_c)::value;
      constexpr int Q = (U * MT + m) % 2;
      // the next item: row m + 1 of this step, or row 0 of the next step
      if constexpr (m + 1 < MT)
        issue_a(IntC<(Q + 1) % 2>{}, s, m + 1);
      else if (!last)
        issue_a(IntC<(Q + 1) % 2>{}, s + 1, 0);
      int P = 0;
      if constexpr (KIND == kW4 && SPLIT) {
        // both halves' activation words against this lane's codes, then the lane's half;
        // the zero point's - z S_A (over the whole group) enters once, in half 0
        int P0 = 0, P1 = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int w = i >> 3, t = (i >> 2) & 1, j = i & 3;
          P0 = __builtin_amdgcn_sdot4(aR[Q][w][4 * t + j], wd[i], P0, false);
          P1 = __builtin_amdgcn_sdot4(aR[Q][w][8 + 4 * t + j], wd[i], P1, false);
        }
        P = kh ? P1 : P0 - z * asR[Q];
      } else if constexpr (KIND == kW4) {
#pragma unroll
        for (int i = 0; i < 32; ++i) P = __builtin_amdgcn_sdot4(aR[Q][i >> 4][i & 15], wd[i], P, false);
        P -= z * asR[Q];
      } else {
        // Both halves of the activation codes against this lane's codes (scalar operands
        // cannot differ between lanes), then keep the half this lane's inputs belong to.
        int P0 = 0, P1 = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          P0 = __builtin_amdgcn_sdot4(aR[Q][0][i], wd[i], P0, false);
          P1 = __builtin_amdgcn_sdot4(aR[Q][1][i], wd[i], P1, false);
        }
        P = kh ? P1 : P0;
      }
      if constexpr (PARTIALS) {
        if constexpr (KIND == kW8 || SPLIT) P += __shfl_xor(P, 32);  // both halves of the inputs
        const int orig = p.idx[jp];
        if (!dup && ((KIND == kW4 && !SPLIT) || kh == 0) && orig >= p.n_begin && orig < p.n_begin + p.n_count)
          p.part[((int64_t)m * p.n_count + (orig - p.n_begin)) * G + grp(s)] = P;
      } else {
        acc[m] = fmaf((float)P, sw * saR[Q], acc[m]);
      }
    });
  };

  // Prologue: weights of steps 0 .. D - 2, the first item.  The loop is unrolled by D (even)
  // so every slot index is a constant; the last cnt % D steps run in an unrolled tail
  // (wave-uniform branches).
  static_assert(D % 2 == 0, "ring sizes");
  issue_a(IntC<0>{}, 0, 0);
  static_for<0, D - 1>([&](auto t_c) { issue_w(t_c, decltype(t_c)::value); });
  const int nfull = cnt / D * D;
  for (int s = 0; s < nfull; s += D) {
    static_for<0, D>([&](auto j_c) {
      constexpr int J = decltype(j_c)::value;
      issue_w(IntC<(J + D - 1) % D>{}, s + J + D - 1);
      compute(j_c, j_c, s + J, false);
    });
  }
  const int rem = cnt - nfull;
  static_for<0, D - 1>([&](auto j_c) {
    constexpr int J = decltype(j_c)::value;
    if (J < rem) compute(j_c, j_c, nfull + J, J + 1 == rem);
  });
}

// Waves per workgroup at most: 16 for one row, 8 (more registers per wave) for more.
constexpr int gv_max_waves(int mt) { return mt == 1 ? kGvWaves : kGvWaves / 2; }

template <int MT, bool PARTIALS>
__global__ __launch_bounds__(64 * gv_max_waves(MT)) void gemm_gemv_kernel(const GemmArgs p, int ks, int nstrip4,
                                                                          int split) {
  __shared__ float red[gv_max_waves(MT)][MT][64];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int strip = blockIdx.x;
  // Strips [0, nstrip4) pair the 4-bit blocks (with an odd count the last strip has one
  // block, and its lanes 32-63 repeat lanes 0-31), or with `split` hold one 4-bit block
  // each, split over the two half-waves like the 8-bit blocks; the others hold one 8-bit
  // block each.
  const bool w4 = strip < nstrip4;
  const bool halves = !w4 || split;  // lanes c and c + 32 share channel c
  const int blk0 = w4 ? (split ? strip : 2 * strip) : p.nb4 + (strip - nstrip4);
  const bool dup = w4 && !split && (lane >> 5) >= min(2, p.nb4 - blk0);
  const int second = w4 && !split && !dup ? (lane >> 5) : 0;
  const int G = p.G;
  // (wave-uniform; read back into scalar registers for the loads' scalar offsets)
  const int cnt = wave_groups(G, wave, ks);
  float acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = 0.0f;
  if (cnt > 0) {
    if (w4 && split)
      gemv_body<kW4, MT, PARTIALS, true>(p, blk0, 0, false, lane, wave, ks, cnt, acc);
    else if (w4)
      gemv_body<kW4, MT, PARTIALS, false>(p, blk0, second, dup, lane, wave, ks, cnt, acc);
    else
      gemv_body<kW8, MT, PARTIALS, false>(p, blk0, 0, false, lane, wave, ks, cnt, acc);
  }
  if (PARTIALS) return;
#pragma unroll
  for (int m = 0; m < MT; ++m) red[wave][m][lane] = acc[m];
  __syncthreads();
  if (wave != 0 || dup || (halves && lane >= 32)) return;
  const int orig = p.idx[(blk0 + second) * 32 + (lane & 31)];
  if (orig < 0) return;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    float v = 0.0f;
    if (!halves) {
      for (int w = 0; w < ks; ++w) v += red[w][m][lane];
    } else {
      for (int w = 0; w < ks; ++w) v += red[w][m][lane] + red[w][m][lane + 32];
    }
    p.y[(int64_t)m * p.ldy + orig] = f2h(v);
  }
}

// ------------------------------------------------------------------------------------
// Strip kernel (4 <= M <= 32 on wide layers).  A wave owns a strip of channels (two
// 4-bit blocks, or one block) and all M rows (one or two 16-row blocks), as 16 x 16 tiles
// of v_mfma_i32_16x16x64_i8: it loads a group's activation operands once and reuses them
// for its four (or two) 16-channel column tiles, so the activation reads per channel are
// a quarter (a half) of the skinny kernel's.  The 4-bit codes go to the matrix cores raw
// and the zero point enters as - z * S_A on the exact integer partial.  Weights pass
// through a register ring and the activation codes, s_a and S_A through an LDS ring (its
// own stages per wave, filled by direct-to-LDS loads), 3 (two row blocks: 2) groups
// ahead; the workgroup's waves share the groups (wave w takes every ks-th, from w) and
// reduce through LDS in a fixed order.
// ------------------------------------------------------------------------------------
constexpr int kLdsPerCu = 160 * 1024;
constexpr int kStWaves = 8;  // waves per workgroup at most
#ifndef MIXLLM_ST_MIX
#define MIXLLM_ST_MIX 1  // mixed strips (see halves8_fit); 0 keeps whole 8-bit strips, to compare
#endif
constexpr int kStMaxRows = 32;  // tokens the strip kernel takes
// RB 16-row blocks (M <= 16 RB).  Weight ring (registers) and activation ring (LDS) of
// st_ring(RB) stages: one group ahead for one row block, 2 for two (measured: deeper rings
// let the older waves of a CU hog its memory queue; the explicit wait count below must
// also stay under the 6-bit vmcnt).
constexpr int st_ring(int rb) { return rb == 1 ? 2 : 3; }
// LDS stage of a wave: the group's activation codes [16 RB rows][128 B] (chunk c of row r
// at position c ^ (r & 7)), then s_a and S_A of up to 64 rows (4 B each, 256 B areas).
constexpr int st_stage(int rb) { return rb * 2048 + 256 + 256; }
constexpr int st_lds(int rb) { return kStWaves * st_ring(rb) * st_stage(rb); }
static_assert(st_lds(1) >= kStWaves * 16 * 64 * 4 && st_lds(2) >= kStWaves * 32 * 64 * 4,
              "the reduction reuses the stage space");

__device__ __forceinline__ void bload4_lds(Rsrc r, void *dst, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LdsPtr)dst, 4, voff, soff, 0, 0);
}

// NT column tiles: with SB = 2, 4-bit strips hold blocks blk0 and blk0 + second (tiles 2
// and 3 repeat tiles 0 and 1 when the strip has one block: dup); otherwise a strip is
// block blk0, or for 8-bit strips with SB = 1 (MODE 1) its 16-channel half `half`, or
// (MODE 2, a mixed strip) the half `half` of 8-bit block blk0 as tile 0 and the half
// `half` of 4-bit block `second` as tile 1.  `lds` is this wave's ring of st_ring(RB)
// stages.
template <int KIND, int SB, int RB, bool PARTIALS, int MODE = 0>
__device__ __forceinline__ void strip_body(const GemmArgs &p, int blk0, int second, bool dup, int half, int lane,
                                           int g0, int gstep, int cnt, uint8_t *lds, float (&acc)[4][RB][4]) {
  constexpr bool H8 = MODE == 1, MIX = MODE == 2;
  static_assert(!MIX || (KIND == kW8 && SB == 1), "mixed strips");
  // Column tiles: 4 (two 4-bit blocks), 2 (one 4-bit block, one 8-bit block, or a mixed
  // strip), or 1 (H8: the 16-channel half `half` of an 8-bit block).
  constexpr int NT = MIX ? 2 : (KIND == kW8 ? (H8 ? 1 : 2) : (SB == 1 ? 2 : 4));
  constexpr bool ANY4 = MIX || KIND == kW4;  // a 4-bit tile: the group's code sums are loaded
  constexpr bool ANY8 = MIX || KIND == kW8;
  constexpr int D = st_ring(RB);
  constexpr int kStage = st_stage(RB);
  // Vector-memory operations per step: the stage's direct-to-LDS loads, then the weight
  // ring's loads.  When step s computes, the loads issued after step s's stage are the
  // weight batch of the step that issued it and D - 1 full batches; a wait for at most
  // that many outstanding proves the stage has landed (the compiler does not track LDS
  // written by these loads).
  constexpr int LA = 2 * RB + (ANY4 ? 2 : 1);
  constexpr int LW = 3 * NT;  // per column tile: codes (or two loads of 8-bit codes) and scale
                              // word, plus the zero-point word for 4-bit
  constexpr int WAIT = LW + (D - 1) * (LA + LW);
  static_assert(WAIT < 64, "vmcnt range");
  const int ch = lane & 15, qd = lane >> 4;
  const int G = p.G, M = p.M;
  // The strip's 8-bit block (index among the 8-bit blocks) and 4-bit block.
  const int b8 = ANY8 ? blk0 - p.nb4 : 0, b4 = MIX ? second : (KIND == kW4 ? blk0 : 0);
  const Rsrc rw8 = make_rsrc(p.w8 + (size_t)b8 * G * kW8Chunk, ANY8 ? (int64_t)2 * G * kW8Chunk : 0);
  const Rsrc rs8 = make_rsrc(p.s8 + (size_t)b8 * G * 32, ANY8 ? (int64_t)2 * G * 64 : 0);
  const Rsrc rw4 = make_rsrc(p.w4 + (size_t)b4 * G * kW4Chunk, ANY4 ? (int64_t)2 * G * kW4Chunk : 0);
  const Rsrc rs4 = make_rsrc(p.s4 + (size_t)b4 * G * 32, ANY4 ? (int64_t)2 * G * 64 : 0);
  const Rsrc rz = make_rsrc(p.z4 + (size_t)b4 * G * kZ4Chunk, ANY4 ? (int64_t)2 * G * kZ4Chunk : 0);
  const Rsrc ra = make_rsrc(p.aq, (int64_t)M * p.K);
  const Rsrc rsa = make_rsrc(p.sa, (int64_t)G * M * 4);
  const Rsrc ras = make_rsrc(p.asum, ANY4 ? (int64_t)G * M * 4 : 0);
  // Column tile t: its kind, block offset bo(t) (in blocks from the strip's 4-bit block)
  // and half ht(t) of it; blkt(t) is its block.  (t is a constant in every unrolled loop,
  // so these fold.)
  auto is8 = [&](int t) { return MIX ? t == 0 : KIND == kW8; };
  auto bo = [&](int t) { return NT == 4 ? (t >> 1) * second : 0; };
  auto ht = [&](int t) { return (NT == 1 || MIX) ? half : (t & 1); };
  auto blkt = [&](int t) { return MIX ? (t == 0 ? blk0 : second) : blk0 + bo(t); };
  // Direct-to-LDS offsets: load i of a stage fills rows 8i .. 8i + 7 (lane l: row
  // 8i + l / 8, position l % 8, which holds chunk (l % 8) ^ (row & 7)); the scale loads
  // fill row l's word.  Rows past M load from past every descriptor (zeros, no traffic).
  int vdma[2 * RB];
#pragma unroll
  for (int i = 0; i < 2 * RB; ++i) {
    const int r = 8 * i + (lane >> 3);
    vdma[i] = r < M ? r * p.K + (((lane & 7) ^ (r & 7)) << 4) : kSkinnyOob;
  }
  const int vrow = lane < M ? lane * 4 : kSkinnyOob;
  // LDS offsets of this lane's MFMA operands: row 16 rb + ch, chunks qd and qd + 4.
  int va[RB][2];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int c = 0; c < 2; ++c) va[rb][c] = (16 * rb + ch) * 128 + (((qd + 4 * c) ^ (ch & 7)) << 4);

  v4i wR[D][NT][ANY8 ? 2 : 1];
  uint32_t sR[D][NT], zR[D][NT];
  auto grp = [&](int s) { return g0 + min(s, cnt - 1) * gstep; };
  auto issue_a = [&](auto j_c, int s) {
    constexpr int J = decltype(j_c)::value;
    const int g = grp(s);
    uint8_t *st = lds + J * kStage;
#pragma unroll
    for (int i = 0; i < 2 * RB; ++i) bload16_lds(ra, st + i * 1024, vdma[i], g * 128);
    bload4_lds(rsa, st + RB * 2048, vrow, g * M * 4);
    if constexpr (ANY4) bload4_lds(ras, st + RB * 2048 + 256, vrow, g * M * 4);
  };
  auto issue_w = [&](auto j_c, int s) {
    constexpr int J = decltype(j_c)::value;
    const int g = grp(s);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int cw = ht(t) * 16 + ch;  // the lane's channel within its block
      if (is8(t)) {
        if constexpr (ANY8) {
#pragma unroll
          for (int mf = 0; mf < 2; ++mf)
            wR[J][t][mf] = bload16_nt(rw8, ht(t) * 2048 + mf * 1024 + lane * 16, g * (int)kW8Chunk);
          sR[J][t] = bload4(rs8, (cw >> 1) * 4, g * 64);
        }
      } else {
        wR[J][t][0] = bload16_nt(rw4, bo(t) * G * (int)kW4Chunk + ht(t) * 1024 + lane * 16, g * (int)kW4Chunk);
        zR[J][t] = bload4(rz, bo(t) * G * (int)kZ4Chunk + (cw >> 3) * 4, g * (int)kZ4Chunk);
        sR[J][t] = bload4(rs4, bo(t) * G * 64 + (cw >> 1) * 4, g * 64);
      }
    }
  };
  auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
  auto compute = [&](auto j_c, int s, bool tail) {
    constexpr int J = decltype(j_c)::value;
    // This step's stage has landed.  In the tail, where no later loads follow, and in the
    // partials mode, whose stores count too and which drops the unused scale loads, wait
    // for everything.
    if (tail || PARTIALS)
      wait_vm<0>();
    else
      wait_vm<WAIT>();
    fence();
    const uint8_t *st = lds + J * kStage;
    v4i a0[RB], a1[RB], sa4[RB], as4[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      a0[rb] = *reinterpret_cast<const v4i *>(st + va[rb][0]);
      a1[rb] = *reinterpret_cast<const v4i *>(st + va[rb][1]);
      sa4[rb] = *reinterpret_cast<const v4i *>(st + RB * 2048 + (16 * rb + 4 * qd) * 4);
      as4[rb] = ANY4 ? *reinterpret_cast<const v4i *>(st + RB * 2048 + 256 + (16 * rb + 4 * qd) * 4)
                     : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int cw = ht(t) * 16 + ch;
      v4i b0, b1;
      if (!is8(t)) {
        const v4i x = wR[J][t][0];
        const uint32_t x0 = (uint32_t)x[0], x1 = (uint32_t)x[1], x2 = (uint32_t)x[2], x3 = (uint32_t)x[3];
        b0 = v4i{(int)(x0 & 0x0F0F0F0Fu), (int)((x0 >> 4) & 0x0F0F0F0Fu), (int)(x1 & 0x0F0F0F0Fu),
                 (int)((x1 >> 4) & 0x0F0F0F0Fu)};
        b1 = v4i{(int)(x2 & 0x0F0F0F0Fu), (int)((x2 >> 4) & 0x0F0F0F0Fu), (int)(x3 & 0x0F0F0F0Fu),
                 (int)((x3 >> 4) & 0x0F0F0F0Fu)};
      } else {
        b0 = wR[J][t][0];
        if constexpr (ANY8) b1 = wR[J][t][1];
      }
      const int z = !is8(t) ? (int)((zR[J][t] >> ((cw & 7) * 4)) & 15u) : 0;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        v4i P = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0[rb], b0, v4i{0, 0, 0, 0}, 0, 0, 0);
        P = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1[rb], b1, P, 0, 0, 0);
        if (!is8(t)) {
#pragma unroll
          for (int r = 0; r < 4; ++r) P[r] -= z * as4[rb][r];
        }
        if constexpr (PARTIALS) {
          const int orig = p.idx[blkt(t) * 32 + cw];
          if (!(dup && t >= 2) && orig >= p.n_begin && orig < p.n_begin + p.n_count) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int row = 16 * rb + 4 * qd + r;
              if (row < M) p.part[((int64_t)row * p.n_count + (orig - p.n_begin)) * G + grp(s)] = P[r];
            }
          }
        } else {
          const float sw = h2f((uint16_t)(sR[J][t] >> ((cw & 1) * 16)));
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[t][rb][r] = fmaf((float)P[r], sw * __int_as_float(sa4[rb][r]), acc[t][rb][r]);
        }
      }
    }
    fence();
  };

  // Prologue: the loads of steps 0 .. D - 2, stage then weights per step, the order the
  // loop issues them in.  The loop is unrolled by D so every slot index is a constant; the
  // last cnt % D steps run in an unrolled tail (wave-uniform branches).  A step's loads
  // refill the slots of the previous step, whose LDS reads completed before its matrix
  // operations were issued.
  static_for<0, D - 1>([&](auto t_c) {
    issue_a(t_c, decltype(t_c)::value);
    issue_w(t_c, decltype(t_c)::value);
  });
  const int nfull = cnt / D * D;
  for (int s = 0; s < nfull; s += D) {
    static_for<0, D>([&](auto j_c) {
      constexpr int J = decltype(j_c)::value;
      fence();
      issue_a(IntC<(J + D - 1) % D>{}, s + J + D - 1);
      issue_w(IntC<(J + D - 1) % D>{}, s + J + D - 1);
      compute(j_c, s + J, false);
    });
  }
  const int rem = cnt - nfull;
  static_for<0, D - 1>([&](auto j_c) {
    constexpr int J = decltype(j_c)::value;
    if (J < rem) compute(j_c, nfull + J, true);
  });
  wait_vm<0>();  // no load into this wave's stages is in flight past here
}

// SB: 4-bit blocks per strip (2 on wide layers; 1 doubles the strips of narrower ones).
// RB: 16-row blocks.
template <int SB, int RB, bool PARTIALS>
__global__ __launch_bounds__(64 * kStWaves) void gemm_strip_kernel(const GemmArgs p, int ks, int nstrip4,
                                                                   int mode8) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[st_lds(RB)];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int strip = blockIdx.x;
  // Strips [0, nstrip4) hold SB 4-bit blocks each (with SB = 2 an odd count leaves the
  // last strip one block, repeated in tiles 2 and 3); the others one 8-bit block each, or
  // with SB = 1 and mode8 = 1 one 16-channel half of an 8-bit block (every strip then
  // streams 16 bytes of weights per input, as a one-block 4-bit strip does), or with
  // mode8 = 2 a mixed strip: half j of 8-bit block i and half j of 4-bit block nstrip4 + i
  // (the last nb8 4-bit blocks go in halves beside the 8-bit ones: 24 bytes per input).
  const bool w4 = strip < nstrip4;
  const bool h8 = SB == 1 && mode8 == 1 && !w4;
  const bool mix = SB == 1 && mode8 == 2 && !w4;
  const int s8 = strip - nstrip4;
  const int half = h8 || mix ? (s8 & 1) : 0;
  const int blk0 = w4 ? SB * strip : p.nb4 + (h8 || mix ? (s8 >> 1) : s8);
  const int blk4 = mix ? nstrip4 + (s8 >> 1) : 0;  // a mixed strip's 4-bit block
  const bool dup = SB == 2 && w4 && p.nb4 - blk0 < 2;
  const int second = SB == 2 && w4 && !dup ? 1 : 0;
  const int G = p.G;
  // (wave-uniform; read back into scalar registers for the loads' scalar offsets)
  const int cnt = wave_groups(G, wave, ks);
  uint8_t *lds = smem + wave * st_ring(RB) * st_stage(RB);
  float acc[4][RB][4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[t][rb][r] = 0.0f;
  if (cnt > 0) {
    if (w4)
      strip_body<kW4, SB, RB, PARTIALS>(p, blk0, second, dup, 0, lane, wave, ks, cnt, lds, acc);
    else if (SB == 1 && h8)
      strip_body<kW8, 1, RB, PARTIALS, 1>(p, blk0, 0, false, half, lane, wave, ks, cnt, lds, acc);
    else if (SB == 1 && mix)
      strip_body<kW8, 1, RB, PARTIALS, 2>(p, blk0, blk4, false, half, lane, wave, ks, cnt, lds, acc);
    else
      strip_body<kW8, SB, RB, PARTIALS>(p, blk0, 0, false, 0, lane, wave, ks, cnt, lds, acc);
  }
  if (PARTIALS) return;
  __syncthreads();  // every wave's stages are done; the space becomes the reduction area
  float(*red)[16 * RB][64] = reinterpret_cast<float(*)[16 * RB][64]>(smem);
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave][(t * RB + rb) * 4 + r][lane] = acc[t][rb][r];
  __syncthreads();
  // Output: the workgroup's waves share the 16 RB (tile, row block, row) slots; each sums
  // its slot over the waves in order and writes the row's channel.
  const bool four = SB == 2 && w4;  // four column tiles (two blocks)
  const bool one = h8;              // one column tile (half an 8-bit block)
  const int nt = four && !dup ? 4 : (one ? 1 : 2);
  const int ch = lane & 15, qd = lane >> 4;
  for (int e = wave; e < 16 * RB; e += ks) {
    const int t = e / (4 * RB), rb = (e >> 2) % RB, r = e & 3;
    const int rowo = 16 * rb + 4 * qd + r;
    if (t >= nt || rowo >= p.M) continue;
    float v = 0.0f;
    for (int w = 0; w < ks; ++w) v += red[w][e][lane];
    const int cw = (four ? (t & 1) : (one || mix ? half : t)) * 16 + ch;
    const int orig = p.idx[(mix ? (t == 0 ? blk0 : blk4) : blk0 + (four ? (t >> 1) : 0)) * 32 + cw];
    if (orig >= 0) p.y[(int64_t)rowo * p.ldy + orig] = f2h(v);
  }
}

// ------------------------------------------------------------------------------------
// Host side
// ------------------------------------------------------------------------------------

int check_common(const int8_t *aq, const float *sa, const int32_t *asum, const uint32_t *rowop, int32_t M,
                 int32_t N, int32_t K, int32_t n8, const mixllm_blob_info *info, const void *blob, size_t blob_bytes,
                 mixllm_blob_info *L) {
  if (M < 0 || N <= 0 || K <= 0 || K % kGroup != 0) return MIXLLM_E_SHAPE;
  if (n8 < 0 || n8 > N) return MIXLLM_E_INDEX;
  if (!compute_layout(N, K, n8, L)) return MIXLLM_E_SHAPE;
  // The blob's host header must describe exactly this layer in this format: the device
  // copy cannot be read back without synchronizing, so the header copy the caller took
  // with mixllm_blob_get_info is what stands for it.
  if (!info) return MIXLLM_E_NULL;
  if (memcmp(info, L, sizeof(*L)) != 0) return MIXLLM_E_FORMAT;
  if (M == 0) return MIXLLM_OK;
  if (!aq || !sa || !rowop || !blob) return MIXLLM_E_NULL;
  if (!asum && L->nb4 > 0) return MIXLLM_E_NULL;  // read only by the 4-bit blocks' zero points
  if (!is_aligned16(aq) || !is_aligned16(sa) || (asum && !is_aligned16(asum)) || !is_aligned16(rowop) ||
      !is_aligned16(blob))
    return MIXLLM_E_SHAPE;
  if (blob_bytes < L->total_bytes) return MIXLLM_E_SPACE;
  return MIXLLM_OK;
}

void fill_args(GemmArgs &a, const int8_t *aq, const float *sa, const int32_t *asum, const uint32_t *rowop,
               int32_t M, const void *blob, const mixllm_blob_info &L) {
  const uint8_t *base = (const uint8_t *)blob;
  a.aq = aq;
  a.sa = sa;
  a.asum = asum;
  a.rowop = rowop;
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
  a.spread = 0;
  a.ident = 0;
  a.ileave = 0;
}

// Compute units of the current device (cached per device).
int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cus[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cus[dev] = v;
  }
  return cus[dev];
}

// Launch plan of one GEMM call, a pure function of the shape.
struct Plan {
  bool gemv;                   // M <= 3: the one-lane-per-channel kernel
  bool strip;                  // 4 <= M <= 16 on wide layers: the strip kernel
  int sb;                      // strip, gemv: 4-bit blocks per strip
  bool h8;                     // strip with sb = 1: 8-bit blocks in 16-channel halves
  bool mix;                    // strip with sb = 1: 8-bit halves paired with 4-bit halves
  int nstrip4, nstrip;         // gemv: strips of 4-bit blocks, all strips
  bool skinny;
  int rb;                      // skinny: 16-row blocks
  int ks;                      // skinny: waves per workgroup
  int tiles_m, tiles_n;        // tile kernel grid
  int nbt;                     // tile kernel: channel blocks per workgroup
};

// Waves of the skinny kernel that fit a SIMD at once (its register count, read once).
template <int RB>
int skinny_waves_per_simd() {
  static int cached = 0;
  if (cached == 0) {
    hipFuncAttributes at;
    int regs = 128;
    if (hipFuncGetAttributes(&at, reinterpret_cast<const void *>(gemm_skinny_kernel<RB, false>)) == hipSuccess &&
        at.numRegs > 0)
      regs = at.numRegs;
    regs = (regs + 7) / 8 * 8;
    const int w = 512 / regs;
    cached = w < 1 ? 1 : (w > 8 ? 8 : w);
  }
  return cached;
}

int skinny_waves_per_simd_rb(int rb) {
  switch (rb) {
    case 1: return skinny_waves_per_simd<1>();
    case 2: return skinny_waves_per_simd<2>();
    case 3: return skinny_waves_per_simd<3>();
    default: return skinny_waves_per_simd<4>();
  }
}

// Waves of the strip kernel that fit a SIMD at once (its register count, read once).
template <int SB, int RB>
int strip_waves_per_simd_sb() {
  static int cached = 0;
  if (cached == 0) {
    hipFuncAttributes at;
    int regs = 128;
    if (hipFuncGetAttributes(&at, reinterpret_cast<const void *>(gemm_strip_kernel<SB, RB, false>)) == hipSuccess &&
        at.numRegs > 0)
      regs = at.numRegs;
    regs = (regs + 7) / 8 * 8;
    const int w = 512 / regs;
    cached = w < 1 ? 1 : (w > 8 ? 8 : w);
  }
  return cached;
}
int strip_waves_per_simd(int sb, int rb) {
  if (rb == 1) return sb == 2 ? strip_waves_per_simd_sb<2, 1>() : strip_waves_per_simd_sb<1, 1>();
  return sb == 2 ? strip_waves_per_simd_sb<2, 2>() : strip_waves_per_simd_sb<1, 2>();
}

// Waves of the gemv kernel for MT rows that fit a SIMD at once (its register count, read once).
template <int MT>
int gemv_waves_per_simd() {
  static int cached = 0;
  if (cached == 0) {
    hipFuncAttributes at;
    int regs = 128;
    if (hipFuncGetAttributes(&at, reinterpret_cast<const void *>(gemm_gemv_kernel<MT, false>)) == hipSuccess &&
        at.numRegs > 0)
      regs = at.numRegs;
    regs = (regs + 7) / 8 * 8;
    const int w = 512 / regs;
    cached = w < 1 ? 1 : (w > kGvWavesPerSimd ? kGvWavesPerSimd : w);
  }
  return cached;
}

// Waves per workgroup at most for one token: 6 with one-block strips, 8 with block pairs.
// A single row gives a wave little arithmetic per weight byte, so few waves keep the
// weight stream going, and more of them only queue more requests: measured on the
// Llama-3.1 70B layers at M = 1, the o, down and q/k/v projections took 10.6, 28.1 and
// 13.7 us with the counts the cost alone picks (16, 16, 13) against 9.1, 24.6 and 12.5
// with 6; the gate (block pairs) 23.5 with 13 against 22.7 with 8.
int gv_one_row_waves(int sb) { return sb == 1 ? 6 : 8; }

int gemv_waves_per_simd_m(int m) {
  static_assert(kGvMaxRows == 3, "one case per row count");
  switch (m) {
    case 1: return gemv_waves_per_simd<1>();
    case 2: return gemv_waves_per_simd<2>();
    default: return gemv_waves_per_simd<3>();
  }
}

// Waves per workgroup for a grid of nwg workgroups whose waves share G groups: the
// count that minimizes (rounds of workgroups) x (groups per wave),
// a CU holding floor(wpc / k) workgroups of k waves (wpc: waves per CU the kernel's
// registers allow), and at most wg_cap (its LDS).  Ties keep the smaller count (fewer
// rounds, longer loops).
int pick_waves(int64_t nwg, int G, int wpc, int kmax, int cus, int wg_cap = 64) {
  int best = 1;
  int64_t best_cost = INT64_MAX;
  for (int k = 1; k <= kmax && k <= G; ++k) {
    const int per_cu = min(wpc / k, wg_cap);
    if (per_cu < 1) break;
    const int64_t fit = (int64_t)cus * per_cu;
    const int64_t cost = (nwg + fit - 1) / fit * ((G + k - 1) / k);
    if (cost < best_cost) {
      best_cost = cost;
      best = k;
    }
  }
  return best;
}

// Relative cost per weight byte of the skinny kernel against a full round of the tile
// kernel, in thousandths, for M rows (measured on the Llama-3.1 8B and 70B layers: it grows
// with the 16-row blocks the skinny kernel computes).
int skinny_cost_pm(int M) {
  const int rb = (M + 15) / 16;
  return rb == 1 ? 1000 + 1000 * M / 48 : (rb == 2 ? 2100 : (rb == 3 ? 3900 : 4400));
}

// M <= 64 rows: the tile kernel runs one 64-row tile per 128 channels, so a layer with
// fewer tiles than CUs leaves CUs idle (a round of tiles takes about as long as the skinny
// kernel takes to stream the same weights at M = 1); the skinny kernel keeps every CU busy
// but costs more per weight byte as M grows.  The tile kernel is taken when
// tiles * cost > 0.9 * CUs (0.45 * CUs where the layer runs 2-block tiles).
// One-block strips of the strip kernel: an 8-bit block streams twice the bytes of a
// 4-bit one, so it goes in two 16-channel halves, each as heavy as a 4-bit strip, when
// all the strips still fit the CUs at one each (measured: 6144 x 8192 at M = 8 10.2 ->
// 8.4 us, 6144 x 4096 at M = 16 7.4 -> 6.5 us).  With more strips than CUs some CUs would
// run two, which measured slower than the 2:1 imbalance it removes (Llama-3.1-70B down
// projection at M = 4 / 8: 28.3 / 29.6 us against 33.7 / 35.6).  (The same split of the
// one-lane-per-channel kernel's 8-bit strips, inputs in quarters, measured 2-6% slower at
// M = 1..3 on 4096 x 4096 and 6144 x 4096, and is not used.)  Where the halves do not fit,
// mixed strips pair each half of an 8-bit block with the same half of one of the last nb8
// 4-bit blocks: as many strips as blocks, the heaviest streaming 24 bytes per input instead
// of 32 (70B down projection at M = 4 / 8 / 16: 28.4 / 29.8 / 32.7 -> 26.3 / 27.7 / 30.3 us).
bool halves8_fit(const mixllm_blob_info &L, int cus) { return L.nb4 + 2 * (int64_t)L.nb8 <= cus; }

Plan make_plan(int M, const mixllm_blob_info &L) {
  Plan pl{};
  const int cus = device_cus() > 0 ? device_cus() : 256;
  // One to three tokens: the gemv kernel, when the layer has enough one-block strips (one
  // workgroup each) to occupy at least half the CUs; narrower layers run the skinny
  // kernel, whose grid is twice as fine.  (At four tokens the gemv kernel lost to the tile
  // kernel on the 70B layers.)
  const int nstrip4 = (L.nb4 + 1) / 2, nstrip = nstrip4 + L.nb8;
  if (M <= kGvMaxRows && 2 * (L.nb4 + L.nb8) >= cus) {
    pl.gemv = true;
    // Fewer block pairs than CUs: one 4-bit block per strip, its inputs split over the
    // half-waves, so the strips cover the CUs.
    pl.sb = nstrip < cus ? 1 : 2;
    pl.nstrip4 = pl.sb == 2 ? nstrip4 : L.nb4;
    pl.nstrip = pl.nstrip4 + L.nb8;
    pl.ks = pick_waves(pl.nstrip, L.G, 4 * gemv_waves_per_simd_m(M), M == 1 ? gv_one_row_waves(pl.sb) : gv_max_waves(M),
                       cus);
    return pl;
  }
  // Up to 32 tokens on layers with a strip (one workgroup) for at least 3/4 of the CUs:
  // the strip kernel, with two 4-bit blocks per strip, or one if that gives the strips
  // (its workgroups are large, so a narrower layer would leave CUs idle; the skinny
  // kernel's grid is finer).
  if (M <= kStMaxRows && (4 * (int64_t)nstrip >= 3 * (int64_t)cus || 4 * (int64_t)L.nb >= 3 * (int64_t)cus)) {
    pl.strip = true;
    pl.rb = (M + 15) / 16;
    pl.sb = 4 * (int64_t)nstrip >= 3 * (int64_t)cus ? 2 : 1;
    pl.nstrip4 = pl.sb == 2 ? nstrip4 : L.nb4;
    pl.h8 = pl.sb == 1 && halves8_fit(L, cus);
    pl.mix = MIXLLM_ST_MIX && pl.sb == 1 && !pl.h8 && L.nb8 > 0 && L.nb4 >= L.nb8;
    if (pl.mix) pl.nstrip4 = L.nb4 - L.nb8;
    pl.nstrip = pl.sb == 2 ? nstrip : L.nb4 + (pl.h8 ? 2 : 1) * L.nb8;
    pl.ks = pick_waves(pl.nstrip, L.G, 4 * strip_waves_per_simd(pl.sb, pl.rb), kStWaves, cus,
                       kLdsPerCu / st_lds(pl.rb));
    return pl;
  }
  // (A layer with fewer 4-block tiles than CUs runs 2-block tiles, each half the work: the
  // tile kernel's side of the comparison halves.)
  const int64_t tiles_n = (L.nb + kTileNB - 1) / kTileNB;
  const int64_t thr_pm = tiles_n < cus ? 450 : 900;
  if (M <= 64 && tiles_n * skinny_cost_pm(M) <= thr_pm * cus) {
    pl.skinny = true;
    pl.rb = (M + 15) / 16;
    pl.ks = pick_waves(2 * (int64_t)L.nb, L.G, 4 * skinny_waves_per_simd_rb(pl.rb), skinny_max_waves(pl.rb), cus);
    return pl;
  }
  // Tile width: 4 blocks, or 2 when 4-block tiles would leave CUs without a tile (twice
  // the workgroups, up to two per CU; where 4-block tiles fill the device their shared
  // activation reads win).
  pl.tiles_m = (M + kTileBM - 1) / kTileBM;
  pl.nbt = (int64_t)pl.tiles_m * ((L.nb + 3) / 4) < cus ? 2 : 4;
  pl.tiles_n = (L.nb + pl.nbt - 1) / pl.nbt;
  return pl;
}

// The tile kernel addresses the row operands with 32-bit offsets (G * M * 32 bytes), a
// block's weights likewise, an activation tile as 64 rows of K, and the column scales of
// every block from the start of s4 to the end of s8 (and the zero points) below kOob.
bool tile_offsets_fit(int M, const mixllm_blob_info &L) {
  const int64_t scales = (int64_t)(L.off_s8 - L.off_s4) + (int64_t)L.nb8 * L.G * 64;
  return (int64_t)L.G * M * 32 <= 0x7FFFFFFF && (int64_t)L.G * (int64_t)kW8Chunk <= 0x7FFFFFFF &&
         scales + 2 * (int64_t)L.G * 64 <= kOob && (int64_t)L.nb4 * L.G * (int64_t)kZ4Chunk + 256 <= kOob &&
         (int64_t)kTileBM * L.K + (int64_t)L.G * 128 <= 0x7FFFFFFF;
}

// The skinny kernel addresses an activation row set (M * K bytes), a group's scales
// (G * M * 4) and a block's weights (G * 4096) with 32-bit offsets.
bool skinny_offsets_fit(int M, const mixllm_blob_info &L) {
  return (int64_t)M * L.K + 256 <= kSkinnyOob && (int64_t)L.G * M * 4 + 256 <= kSkinnyOob &&
         (int64_t)L.G * (int64_t)kW8Chunk <= 0x7FFFFFFF &&
         (int64_t)kSkinnyOob + (int64_t)L.G * 128 + (int64_t)L.G * M * 4 < ((int64_t)1 << 32);
}

// The gemv kernel addresses two blocks' weights of all groups with 32-bit offsets.
bool gemv_offsets_fit(const mixllm_blob_info &L) { return (int64_t)(2 * L.G + 1) * (int64_t)kW8Chunk <= 0x7FFFFFFF; }

bool offsets_fit(const Plan &pl, int M, const mixllm_blob_info &L) {
  if (pl.gemv) return gemv_offsets_fit(L);
  if (pl.strip) return gemv_offsets_fit(L) && skinny_offsets_fit(M, L);
  return pl.skinny ? skinny_offsets_fit(M, L) : tile_offsets_fit(M, L);
}

template <bool PARTIALS>
int launch(GemmArgs &a, const Plan &pl, hipStream_t stream) {
  (void)hipGetLastError();
  if (pl.gemv) {
    const dim3 grid((unsigned)pl.nstrip), block((unsigned)(64 * pl.ks));
    switch (a.M) {
      case 1: hipLaunchKernelGGL((gemm_gemv_kernel<1, PARTIALS>), grid, block, 0, stream, a, pl.ks, pl.nstrip4, pl.sb == 1); break;
      case 2: hipLaunchKernelGGL((gemm_gemv_kernel<2, PARTIALS>), grid, block, 0, stream, a, pl.ks, pl.nstrip4, pl.sb == 1); break;
      default: hipLaunchKernelGGL((gemm_gemv_kernel<3, PARTIALS>), grid, block, 0, stream, a, pl.ks, pl.nstrip4, pl.sb == 1); break;
    }
  } else if (pl.strip) {
    const dim3 grid((unsigned)pl.nstrip), block((unsigned)(64 * pl.ks));
    if (pl.rb == 1) {
      if (pl.sb == 2)
        hipLaunchKernelGGL((gemm_strip_kernel<2, 1, PARTIALS>), grid, block, 0, stream, a, pl.ks, pl.nstrip4, pl.h8 ? 1 : (pl.mix ? 2 : 0));
      else
        hipLaunchKernelGGL((gemm_strip_kernel<1, 1, PARTIALS>), grid, block, 0, stream, a, pl.ks, pl.nstrip4, pl.h8 ? 1 : (pl.mix ? 2 : 0));
    } else {
      if (pl.sb == 2)
        hipLaunchKernelGGL((gemm_strip_kernel<2, 2, PARTIALS>), grid, block, 0, stream, a, pl.ks, pl.nstrip4, pl.h8 ? 1 : (pl.mix ? 2 : 0));
      else
        hipLaunchKernelGGL((gemm_strip_kernel<1, 2, PARTIALS>), grid, block, 0, stream, a, pl.ks, pl.nstrip4, pl.h8 ? 1 : (pl.mix ? 2 : 0));
    }
  } else if (pl.skinny) {
    const int ks = pl.ks;
    const dim3 grid((unsigned)(2 * a.nb)), block((unsigned)(64 * ks));
    const size_t lds = (size_t)ks * pl.rb * 4 * 64 * sizeof(float);
    switch (pl.rb) {
      case 1: hipLaunchKernelGGL((gemm_skinny_kernel<1, PARTIALS>), grid, block, lds, stream, a, ks); break;
      case 2: hipLaunchKernelGGL((gemm_skinny_kernel<2, PARTIALS>), grid, block, lds, stream, a, ks); break;
      case 3: hipLaunchKernelGGL((gemm_skinny_kernel<3, PARTIALS>), grid, block, lds, stream, a, ks); break;
      default: hipLaunchKernelGGL((gemm_skinny_kernel<4, PARTIALS>), grid, block, lds, stream, a, ks); break;
    }
  } else {
    a.tiles_m = pl.tiles_m;
    a.tiles_n = pl.tiles_n;
    const int64_t T = (int64_t)a.tiles_m * a.tiles_n;
    if (T > 0x7FFFFFFF) return MIXLLM_E_SHAPE;
    a.spread = T <= device_cus() ? 1 : 0;
    // Interleaved blocks when each tile gets at most one 8-bit block and the grid runs in
    // several rounds or has 2-block tiles.  Same box, against consecutive blocks:
    // Llama-3.1-70B q/o at M = 512 66.2 -> 62.8 us, gate 216.9 -> 210.5, 4096 x 4096 at
    // M = 128 13.9 -> 13.4; with half the channels 8-bit (two per tile) 19.9 -> 21.0.  A
    // single round of 4-block tiles (4096 x 4096 at M = 512) ran within 1% either way but
    // wrote 8.2 MB instead of 7.0 (more workgroups writing partial output lines), so it
    // keeps consecutive blocks.
    a.ileave = a.nb - a.nb4 <= a.tiles_n && !(a.spread && pl.nbt == 4) ? 1 : 0;
    const dim3 grid((unsigned)T);
    if (!PARTIALS && a.tiles_m <= kTileBand) {
      if (pl.nbt == 2)
        hipLaunchKernelGGL((gemm_tile_kernel<2, PARTIALS, !PARTIALS>), grid, dim3(tile_threads(2)), 0, stream, a);
      else
        hipLaunchKernelGGL((gemm_tile_kernel<4, PARTIALS, !PARTIALS>), grid, dim3(tile_threads(4)), 0, stream, a);
    } else if (pl.nbt == 2) {
      hipLaunchKernelGGL((gemm_tile_kernel<2, PARTIALS, false>), grid, dim3(tile_threads(2)), 0, stream, a);
    } else {
      hipLaunchKernelGGL((gemm_tile_kernel<4, PARTIALS, false>), grid, dim3(tile_threads(4)), 0, stream, a);
    }
  }
  return hipGetLastError() == hipSuccess ? MIXLLM_OK : MIXLLM_E_HIP;
}

}  // namespace

extern "C" size_t mixllm_gemm_workspace_bytes(int32_t M, int32_t N, int32_t K, int32_t n8) {
  // No kernel needs scratch memory: the slices of a tile are reduced inside its workgroup.
  (void)M;
  (void)N;
  (void)K;
  (void)n8;
  return 0;
}

extern "C" int mixllm_gemm_w4w8a8(const int8_t *aq, const float *sa, const int32_t *asum, const uint32_t *rowop,
                                  int32_t M, int32_t N, int32_t K, int32_t n8, const mixllm_blob_info *blob_info,
                                  const void *blob, size_t blob_bytes, uint16_t *y, int64_t ldy, void *workspace,
                                  size_t workspace_bytes, void *stream) {
  mixllm_blob_info L;
  int st = check_common(aq, sa, asum, rowop, M, N, K, n8, blob_info, blob, blob_bytes, &L);
  if (st != MIXLLM_OK || M == 0) return st;
  if (!y) return MIXLLM_E_NULL;
  if (ldy < N) return MIXLLM_E_SHAPE;
  (void)workspace;
  (void)workspace_bytes;
  const Plan pl = make_plan(M, L);
  if (!offsets_fit(pl, M, L)) return MIXLLM_E_SHAPE;
  GemmArgs a;
  fill_args(a, aq, sa, asum, rowop, M, blob, L);
  a.y = y;
  a.ldy = ldy;
  // All channels of one kind: the packed order is the original order.
  a.ident = (L.n8 == 0 || L.n8 == L.N) && ldy % 8 == 0 && is_aligned16(y) ? 1 : 0;
  return launch<false>(a, pl, (hipStream_t)stream);
}

extern "C" int mixllm_gemm_w4w8a8_partials(const int8_t *aq, const float *sa, const int32_t *asum,
                                           const uint32_t *rowop, int32_t M, int32_t N, int32_t K, int32_t n8,
                                           const mixllm_blob_info *blob_info, const void *blob, size_t blob_bytes,
                                           int32_t n_begin, int32_t n_count, int32_t *part, void *stream) {
  mixllm_blob_info L;
  int st = check_common(aq, sa, asum, rowop, M, N, K, n8, blob_info, blob, blob_bytes, &L);
  if (st != MIXLLM_OK) return st;
  if (n_begin < 0 || n_count < 0 || (int64_t)n_begin + n_count > N) return MIXLLM_E_SHAPE;
  if (M == 0 || n_count == 0) return MIXLLM_OK;
  if (!part) return MIXLLM_E_NULL;
  const Plan pl = make_plan(M, L);
  if (!offsets_fit(pl, M, L)) return MIXLLM_E_SHAPE;
  GemmArgs a;
  fill_args(a, aq, sa, asum, rowop, M, blob, L);
  a.part = part;
  a.n_begin = n_begin;
  a.n_count = n_count;
  return launch<true>(a, pl, (hipStream_t)stream);
}
