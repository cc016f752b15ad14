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
  const uint32_t *rowop;  // [G][2][M][4] row operands of the scale products
  int M, N, K, G;
  const uint8_t *w4;
  const uint16_t *s4;
  const uint8_t *z4;
  const uint8_t *w8;
  const uint16_t *s8;
  const int32_t *idx;
  const uint32_t *pw;
  int n4, nb, nb4;
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
// Tile kernel (M > 64).  A workgroup of 4 x KS waves owns 64 rows x 128 channels (4
// blocks of 32 channels).  Wave (b, q) computes block 4 tn + b for all 64 rows over the
// q-th of KS contiguous slices of the groups; the KS partial accumulators are summed
// through LDS at the end in slice order.  Several waves per SIMD let one wave's
// matrix-core work cover another's VALU work and memory waits.
//
// Per group and wave (two 32-row blocks):
//   * 4 x 2 v_mfma_i32_32x32x32_i8: the exact group partials.  4-bit blocks feed the raw
//     codes q (3 VALU ops per 8 codes); the zero point is removed in the float domain;
//   * per block, 1 v_mfma_f32_32x32x16_bf16 for the scale products s_a[m] s_w[n] as an
//     outer product of exact bf16 splits: the row operand [a0 a0 a1 a1 a2 a2 0 0]
//     (s_a = a0 + a1 + a2, written by the activation quantizer) against the column
//     operand [b0 b1] x 4 (s_w = b0 + b1, from the packed weights);
//   * 4-bit blocks: 1 more that adds -(S_A[m] s_a[m]) (z[n] s_w[n]) to the accumulator,
//     S_A being the group's activation code sum: sum_k (q - z) a_k s_a s_w =
//     s_a s_w sum_k q a_k - (S_A s_a) (z s_w);
//   * the fold acc += float(P) * scale: 2 VALU ops per output element.
// The integer partial is exact; only the fp32 fold differs from the fp64 definition.
// Software pipeline: block 0 of a group runs on the matrix cores while block 1 of the
// previous group folds, then block 1 while block 0 folds.
//
// Streams.  The activation tile of a group (64 rows x 128 B) and the rows' scale
// operands (2 x 64 x 16 B) go from memory straight into LDS (buffer_load ... lds)
// kD = kSA - 2 groups ahead of their use, in a ring of kSA stages (a stage is read during
// its step and the next); a wave's weights and scale words stream into a register ring
// SW groups deep.  Every wave issues the same fixed set of loads per step, so a wait for
// "at most N loads outstanding" (N counting the later steps' loads) proves that the
// current step's stage has landed; a workgroup barrier after that wait publishes it.  The
// wait is explicit because the compiler does not track LDS written by these loads.
// ------------------------------------------------------------------------------------
constexpr int kTileBM = 64;
constexpr int kTileNB = 4;                          // channel blocks per workgroup
#ifndef MIXLLM_TILE_KS
#define MIXLLM_TILE_KS 2
#endif
constexpr int kKS = MIXLLM_TILE_KS;                 // group slices per workgroup
constexpr int kTileWaves = kTileNB * kKS;
constexpr int kTileThreads = 64 * kTileWaves;
#ifndef MIXLLM_TILE_SA
#define MIXLLM_TILE_SA 6
#endif
constexpr int kSA = MIXLLM_TILE_SA;                 // LDS stages
constexpr int kD = kSA - 2;                         // prefetch distance (groups)
#ifndef MIXLLM_SW4
#define MIXLLM_SW4 2
#endif
constexpr int kSW4 = MIXLLM_SW4, kSW8 = 2;          // weight ring depth, 4-bit / 8-bit blocks

// LDS bank swizzle of the activation tile: a ds_read_b128 wave is served in groups of
// 16 lanes over 64 banks, and the rows one group reads must hit distinct banks; the
// 16-byte chunk c of row r sits at position c ^ swz_a(r) of the row's 128 bytes.
__device__ __forceinline__ int swz_a(int r) { return (r >> 1) & 7; }

struct TileSmem {
  uint8_t a[kSA][kKS][kTileBM * 128];           // [stage][slice] activation tiles
  uint32_t rp[kSA][kKS][4][64][4];              // [stage][slice][row / 16][lane] row operands:
                                                // lane < 16: s_a of row 16 b + lane; 16..31: S_A s_a; rest unused
};
static_assert((kKS - 1) * kTileNB * kTileBM * 32 * 4 <= (int)sizeof(TileSmem::a), "reduction space");

__device__ __forceinline__ v16f mfma_bf16(v4i a, v4i b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0,
                                                 0, 0);
}

enum BlockKind { kNone = 0, kW4 = 1, kW8 = 2 };

// Buffer resources: the 128-bit descriptor of a byte range [base, base + bytes).  Loads
// through it take a per-lane 32-bit offset (computed once) plus a wave-uniform offset
// (per group, scalar arithmetic), so the inner loop spends no vector ops on addresses,
// and loads past `bytes` return zeros instead of touching memory.
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kRsrcFlags = 0x00020000;  // gfx9 raw buffer, 32-bit data format

__device__ __forceinline__ Rsrc make_rsrc(const void *base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0xFFFFFFFFll ? 0xFFFFFFFFll : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)(uint32_t)n, kRsrcFlags);
}
__device__ __forceinline__ v4i bload16(Rsrc r, int voff, int soff) {
  return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ uint32_t bload4(Rsrc r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
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
// Wait until at most N vector-memory operations are outstanding, N = min(s, CAP) * L.
template <int L, int CAP>
__device__ __forceinline__ void wait_vm_steps(int s) {
  static_assert(CAP <= 3, "extend the cases below");
  if (CAP >= 3 && s >= 3) {
    wait_vm<(CAP >= 3 ? 3 : 0) * L>();
  } else if (CAP >= 2 && s >= 2) {
    wait_vm<(CAP >= 2 ? 2 : 0) * L>();
  } else if (CAP >= 1 && s >= 1) {
    wait_vm<L>();
  } else {
    wait_vm<0>();
  }
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

template <int KIND, bool PARTIALS>
__device__ __forceinline__ void tile_body(const GemmArgs &p, TileSmem &sm, int m0, int blk, int bi, int q,
                                          int lane) {
  constexpr int SW = KIND == kW8 ? kSW8 : kSW4;
  constexpr int NW = KIND == kW8 ? 4 : (KIND == kW4 ? 2 : 0);     // 16-byte weight loads per step
  constexpr int NPW = KIND == kW4 ? 2 : (KIND == kW8 ? 1 : 0);    // scale words per step
  constexpr int NZ = (PARTIALS && KIND == kW4) ? 1 : 0;           // zero-point word (partials)
  constexpr int L = 3 + NW + NPW + NZ;                            // loads per step
  static_assert(kD >= 2 && (kD - 1) * L < 64, "prefetch distance");
  const int ch32 = lane & 31, h = lane >> 5, half = ch32 >> 4, ch = ch32 & 15;
  const int G = p.G;
  const int gb = G * q / kKS, ge = G * (q + 1) / kKS;             // this slice's groups
  const int nsteps = (G + kKS - 1) / kKS;                          // same for every wave
  const int glast = max(ge - 1, gb);
  auto grp = [&](int s) { return min(gb + s, glast); };            // clamped: always a valid group

  // Descriptors.  Activation rows past M load zeros; operand rows past M read other
  // rows (finite, never stored) or zeros past the end.
  const Rsrc ra = make_rsrc(p.aq + (int64_t)m0 * p.K, (int64_t)(p.M - m0) * p.K);
  const Rsrc rro = make_rsrc(p.rowop, (int64_t)G * 2 * p.M * 16);
  const int bq = KIND == kW8 ? blk - p.nb4 : blk;
  const Rsrc rw = KIND == kW8 ? make_rsrc(p.w8 + (size_t)bq * G * kW8Chunk, (int64_t)G * kW8Chunk)
                              : make_rsrc(p.w4 + (size_t)bq * G * kW4Chunk, (int64_t)G * kW4Chunk);
  const Rsrc rpw = make_rsrc((const uint8_t *)p.pw + (size_t)blk * G * kPwChunk, (int64_t)G * kPwChunk);

  // Per-lane offsets.
  int vdma[2];  // this wave loads rows [16 bi, 16 bi + 16) of the slice's tile, 8 rows per load
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 16 * bi + 8 * i + (lane >> 3), pos = lane & 7;
    vdma[i] = r * p.K + ((pos ^ swz_a(r)) << 4);
  }
  // ... and the operands of the same 16 rows: lanes 0-15 s_a, lanes 16-31 S_A s_a (lanes
  // 32-63 repeat them into the unused half of the wave's operand area)
  const int vro = (((lane >> 4) & 1) * p.M + m0 + 16 * bi + (lane & 15)) * 16;
  const int vpw = ch32 * 8;
  int vw[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
    vw[s] = KIND == kW8 ? ((half * 8 + chunk32(s, h)) * 16 + ch) * 16 : ((half * 4 + 2 * (s & 1) + h) * 16 + ch) * 16;
  int va[4];  // LDS byte offset of this lane's A operand for k-step s, 32-row block 0
#pragma unroll
  for (int s = 0; s < 4; ++s) va[s] = ch32 * 128 + ((chunk32(s, h) ^ swz_a(ch32)) << 4);
  // (row + 32 has the same swizzle as row, so block 1 is block 0 + 32 * 128.)
  // byte offset of row ch32's s_a operand within a [stage][slice] operand area (S_A s_a at
  // + 256 bytes, block 1 at + 2 * 1024 bytes)
  const int vrp = ((ch32 >> 4) * 64 + (ch32 & 15)) * 16;
  constexpr int kAStage = kKS * kTileBM * 128, kRStage = kKS * 4 * 64 * 16;  // bytes per stage
  uint8_t *const abase = &sm.a[0][q][0];
  uint8_t *const rbase = reinterpret_cast<uint8_t *>(&sm.rp[0][q][0][0][0]);

  // Register ring (raw loaded bits only), two steps deep: slot = step parity.
  static_assert(SW == 2, "the step loop is unrolled by two");
  v4i bR[2][NW > 0 ? NW : 1];
  uint32_t swR[2], zwR[2];
  uint32_t zpR[2];

  // Stage st: the activation tile and the row operands of group g, straight into LDS.
  auto issue_a = [&](int st, int g) {
#pragma unroll
    for (int i = 0; i < 2; ++i) bload16_lds(ra, abase + st * kAStage + (16 * bi + 8 * i) * 128, vdma[i], g * 128);
    bload16_lds(rro, rbase + st * kRStage + bi * 1024, vro, g * 2 * p.M * 16);
  };
  // Ring slot j: this wave's weights and scale words of group g.
  auto issue_w = [&](auto j_c, int g) {
    constexpr int j = decltype(j_c)::value;
    if constexpr (KIND != kNone) {
#pragma unroll
      for (int s = 0; s < NW; ++s) bR[j][s] = bload16(rw, vw[s], g * (KIND == kW8 ? (int)kW8Chunk : (int)kW4Chunk));
      swR[j] = bload4(rpw, vpw, g * (int)kPwChunk);
      if constexpr (KIND == kW4) zwR[j] = bload4(rpw, vpw + 4, g * (int)kPwChunk);
      if constexpr (NZ) zpR[j] = bload4(make_rsrc(p.z4, (int64_t)p.nb4 * G * kZ4Chunk), (ch32 >> 3) * 4,
                                        (int)(((size_t)blk * G + g) * kZ4Chunk));
    }
  };

  v16f acc[2] = {v16f{0}, v16f{0}};
  v16i P1[2] = {v16i{0}, v16i{0}};  // block-1 partials of the even / odd steps
  uint32_t swprev = 0, zwprev = 0;  // column words of the previous step (0: nothing to fold)
  const int jp = blk * 32 + ch32;

  // The row operands (s_a and S_A s_a pieces) of one 32-row block of stage st.
  auto load_rows = [&](int rb, int st, v4i &rs, v4i &ru) {
    const uint8_t *o = rbase + st * kRStage + vrp + rb * 2048;
    rs = *reinterpret_cast<const v4i *>(o);
    if constexpr (KIND == kW4) ru = *reinterpret_cast<const v4i *>(o + 256);
  };
  // Scale products of one 32-row block on the matrix cores (row operand rs, column word
  // sw).  The column words are zero in the second half-wave (its k slots must add
  // nothing) and for a step that folds nothing.
  auto scales = [&](const v4i &rs, uint32_t sw) {
    return mfma_bf16(rs, v4i{(int)sw, (int)sw, (int)sw, (int)sw}, v16f{0});
  };
  // acc[rb] += float(P) * scale, then (4-bit blocks) the zero-point term.
  auto fold = [&](int rb, const v16i &Pp, const v16f &sc, const v4i &ru, uint32_t zw) {
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[rb][r] = fmaf((float)Pp[r], sc[r], acc[rb][r]);
    if constexpr (KIND == kW4) acc[rb] = mfma_bf16(ru, v4i{(int)zw, (int)zw, (int)zw, (int)zw}, acc[rb]);
  };

  // The A operands of one 32-row block of stage st (4 LDS reads, issued together).
  auto load_a = [&](int st, int rb, v4i (&av)[4]) {
    const uint8_t *at = abase + st * kAStage + rb * 32 * 128;
#pragma unroll
    for (int k = 0; k < 4; ++k) av[k] = *reinterpret_cast<const v4i *>(at + va[k]);
  };
  // The group partial of one 32-row block on the matrix cores.
  auto block_mma = [&](const v4i (&av)[4], const v4i (&bq)[4]) {
    v16i P = v16i{0};
#pragma unroll
    for (int k = 0; k < 4; ++k) P = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[k], bq[k], P, 0, 0, 0);
    return P;
  };

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

  // One step s (parity j = s % 2 known at compile time; stage st = s mod kSA).  The
  // prologue waited for stages 0 .. kD - 1; stage s >= kD was issued at step s - kD, and
  // the kD - 1 later steps issued L loads each, so "at most (kD - 1) L outstanding" means
  // stage s has landed.
  auto step = [&](auto j_c, int s, int st) {
    constexpr int j = decltype(j_c)::value;
    wait_vm<(kD - 1) * L>();
    lds_barrier();
    // the column words of step s leave the ring slot that the refill below reuses
    const uint32_t swcur = KIND != kNone ? swR[j] : 0u;
    const uint32_t zwcur = KIND == kW4 ? zwR[j] : 0u;
    // Refill (unconditionally, clamped, so every step issues the same loads): stage
    // s + kD (the slot of step s - 2, read for the last time during step s - 1), and the
    // weights of step s + 1 (the slot of step s - 1).
    const int st_next = st + kD >= kSA ? st + kD - kSA : st + kD;
    issue_a(st_next, grp(s + kD));
    issue_w(IntC<1 - j>{}, grp(s + 1));
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (KIND != kNone) {
      // Branch-free: an inactive step (past this slice's range, on clamped data) computes
      // partials that are never folded (its column words are replaced by zeros).
      const bool act = gb + s < ge;
      const uint32_t sw = (act && h == 0) ? swcur : 0u, zw = (act && h == 0) ? zwcur : 0u;
      v4i bq[4];
      if constexpr (KIND == kW4) {
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const uint32_t x0 = (uint32_t)bR[j][e][2 * u], x1 = (uint32_t)bR[j][e][2 * u + 1];
            bq[2 * e + u] = v4i{(int)(x0 & 0x0F0F0F0Fu), (int)((x0 >> 4) & 0x0F0F0F0Fu), (int)(x1 & 0x0F0F0F0Fu),
                                (int)((x1 >> 4) & 0x0F0F0F0Fu)};
          }
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) bq[k] = bR[j][k];
      }
      const int st_prev = st == 0 ? kSA - 1 : st - 1;
      if constexpr (PARTIALS) {
        v4i av[4];
        load_a(st, 0, av);
        const v16i P0 = block_mma(av, bq);
        if (act) emit(0, P0, gb + s, zpR[j]);
        load_a(st, 1, av);
        const v16i Pb = block_mma(av, bq);
        if (act) emit(1, Pb, gb + s, zpR[j]);
      } else {
        // Block 0 of this step on the matrix cores while block 1 of the previous step
        // folds, then block 1 of this step while block 0 of this step folds.  Each block's
        // LDS operand reads are issued together ahead of its matrix-core ops.
        v4i av[4], rs, ru;
        load_a(st, 0, av);
        load_rows(1, st_prev, rs, ru);
        __builtin_amdgcn_sched_barrier(0);
        const v16f sc1 = scales(rs, swprev);
        const v16i P0 = block_mma(av, bq);
        fold(1, P1[1 - j], sc1, ru, zwprev);
        load_a(st, 1, av);
        load_rows(0, st, rs, ru);
        __builtin_amdgcn_sched_barrier(0);
        const v16f sc0 = scales(rs, sw);
        P1[j] = block_mma(av, bq);
        fold(0, P0, sc0, ru, zw);
      }
      swprev = sw;
      zwprev = zw;
    }
  };

  // Prologue: stages 0 .. kD - 1 and the weights of step 0, all landed before step 0.
  for (int st = 0; st < kD; ++st) issue_a(st, grp(st));
  issue_w(IntC<0>{}, grp(0));
  wait_vm<0>();

  int s = 0, st = 0;
  for (; s + 2 <= nsteps; s += 2) {
    step(IntC<0>{}, s, st);
    st = st + 1 == kSA ? 0 : st + 1;
    step(IntC<1>{}, s + 1, st);
    st = st + 1 == kSA ? 0 : st + 1;
  }
  if (s < nsteps) {
    step(IntC<0>{}, s, st);
    ++s;
  }
  // Block 1 of the last step still has to fold; its stage is intact (the last refill went
  // to the slot of step nsteps - 2).
  if constexpr (!PARTIALS && KIND != kNone) {
    v4i rs, ru;
    load_rows(1, (nsteps - 1) % kSA, rs, ru);
    const v16f sc = scales(rs, swprev);
    if ((nsteps - 1) & 1)
      fold(1, P1[1], sc, ru, zwprev);
    else
      fold(1, P1[0], sc, ru, zwprev);
  }
  // All direct-to-LDS loads (including the clamped refills) have landed before the
  // stages' space is reused.
  wait_vm<0>();
  lds_barrier();
  if constexpr (PARTIALS) return;

  // Sum the slices' accumulators in slice order and write the output.
  float *red = reinterpret_cast<float *>(&sm.a[0][0][0]);
  if (q > 0) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int r = 0; r < 16; ++r) red[((((q - 1) * kTileNB + bi) * 2 + rb) * 16 + r) * 64 + lane] = acc[rb][r];
  }
  lds_barrier();
  if (q > 0 || KIND == kNone) return;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int qq = 1; qq < kKS; ++qq) acc[rb][r] += red[((((qq - 1) * kTileNB + bi) * 2 + rb) * 16 + r) * 64 + lane];
  const int orig = p.idx[jp];
  if (orig < 0) return;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = m0 + rb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
      if (row < p.M) p.y[(int64_t)row * p.ldy + orig] = f2h(acc[rb][r]);
    }
}

template <bool PARTIALS>
__global__ __launch_bounds__(kTileThreads) void gemm_tile_kernel(const GemmArgs p) {
  __shared__ __attribute__((aligned(16))) TileSmem sm;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;  // wave: uniform
  const int bi = wave & 3, q = wave >> 2;

  // Zero the operand stages: a fold before the first group reads a stage not loaded yet
  // (with zero column words, which must meet finite values).
  for (int e = tid; e < (int)(sizeof(sm.rp) / 16); e += kTileThreads)
    reinterpret_cast<v4i *>(&sm.rp[0][0][0][0][0])[e] = v4i{0, 0, 0, 0};
  __syncthreads();

  // Workgroup w runs on XCD w % 8.  Give each XCD a contiguous range of tiles, ordered in
  // bands of kBandM M tiles (M tile fastest within a band), so the workgroups an XCD runs
  // at once share both activation rows and weight blocks in its L2.
  constexpr int kBandM = 4;
  const int T = p.tiles_m * p.tiles_n;
  const int xcd = blockIdx.x & 7, i = blockIdx.x >> 3;
  const int per = T >> 3, rem = T & 7;
  const int t = xcd * per + (xcd < rem ? xcd : rem) + i;
  const int band = t / (kBandM * p.tiles_n), in_band = t - band * (kBandM * p.tiles_n);
  const int bm = min(kBandM, p.tiles_m - band * kBandM);  // M tiles in this band
  const int tm = band * kBandM + in_band % bm, tn = in_band / bm;
  const int m0 = tm * kTileBM;
  const int blk = tn * kTileNB + bi;
  const int kind = blk >= p.nb ? kNone : (blk < p.nb4 ? kW4 : kW8);
  switch (kind) {
    case kW4: tile_body<kW4, PARTIALS>(p, sm, m0, blk, bi, q, lane); break;
    case kW8: tile_body<kW8, PARTIALS>(p, sm, m0, blk, bi, q, lane); break;
    default: tile_body<kNone, PARTIALS>(p, sm, m0, blk, bi, q, lane); break;
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

int check_common(const int8_t *aq, const float *sa, const int32_t *asum, const uint32_t *rowop, int32_t M,
                 int32_t N, int32_t K, int32_t n8, const void *blob, size_t blob_bytes, mixllm_blob_info *L) {
  if (M < 0 || N <= 0 || K <= 0 || K % kGroup != 0) return MIXLLM_E_SHAPE;
  if (n8 < 0 || n8 > N) return MIXLLM_E_INDEX;
  if (!compute_layout(N, K, n8, L)) return MIXLLM_E_SHAPE;
  if (M == 0) return MIXLLM_OK;
  if (!aq || !sa || !asum || !rowop || !blob) return MIXLLM_E_NULL;
  if (!is_aligned16(aq) || !is_aligned16(sa) || !is_aligned16(asum) || !is_aligned16(rowop) || !is_aligned16(blob))
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
  a.pw = (const uint32_t *)(base + L.off_pw);
  a.n4 = L.n4;
  a.nb = L.nb;
  a.nb4 = L.nb4;
  a.y = nullptr;
  a.ldy = 0;
  a.part = nullptr;
  a.n_begin = 0;
  a.n_count = 0;
  a.tiles_m = a.tiles_n = 0;
}

// Launch plan of one GEMM call, a pure function of the shape.
struct Plan {
  bool skinny;
  int rb;                      // skinny: 16-row blocks
  int ks;                      // skinny: waves per workgroup
  int tiles_m, tiles_n;        // tile kernel grid
};

Plan make_plan(int M, const mixllm_blob_info &L) {
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
  pl.tiles_n = (L.nb + kTileNB - 1) / kTileNB;
  return pl;
}

// The tile kernel addresses the row operands with 32-bit offsets (G * M * 32 bytes) and a
// block's weights likewise (G * 4096).
bool tile_offsets_fit(int M, const mixllm_blob_info &L) {
  return (int64_t)L.G * M * 32 <= 0x7FFFFFFF && (int64_t)L.G * (int64_t)kW8Chunk <= 0x7FFFFFFF &&
         (int64_t)kTileBM * L.K + (int64_t)L.G * 128 <= 0x7FFFFFFF;
}

template <bool PARTIALS>
int launch(GemmArgs &a, const Plan &pl, hipStream_t stream) {
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
    const int64_t T = (int64_t)a.tiles_m * a.tiles_n;
    if (T > 0x7FFFFFFF) return MIXLLM_E_SHAPE;
    hipLaunchKernelGGL((gemm_tile_kernel<PARTIALS>), dim3((unsigned)T), dim3(kTileThreads), 0, stream, a);
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
                                  int32_t M, int32_t N, int32_t K, int32_t n8, const void *blob, size_t blob_bytes,
                                  uint16_t *y, int64_t ldy, void *workspace, size_t workspace_bytes, void *stream) {
  mixllm_blob_info L;
  int st = check_common(aq, sa, asum, rowop, M, N, K, n8, blob, blob_bytes, &L);
  if (st != MIXLLM_OK || M == 0) return st;
  if (!y) return MIXLLM_E_NULL;
  if (ldy < N) return MIXLLM_E_SHAPE;
  (void)workspace;
  (void)workspace_bytes;
  const Plan pl = make_plan(M, L);
  if (!pl.skinny && !tile_offsets_fit(M, L)) return MIXLLM_E_SHAPE;
  GemmArgs a;
  fill_args(a, aq, sa, asum, rowop, M, blob, L);
  a.y = y;
  a.ldy = ldy;
  return launch<false>(a, pl, (hipStream_t)stream);
}

extern "C" int mixllm_gemm_w4w8a8_partials(const int8_t *aq, const float *sa, const int32_t *asum,
                                           const uint32_t *rowop, int32_t M, int32_t N, int32_t K, int32_t n8,
                                           const void *blob, size_t blob_bytes, int32_t n_begin, int32_t n_count,
                                           int32_t *part, void *stream) {
  mixllm_blob_info L;
  int st = check_common(aq, sa, asum, rowop, M, N, K, n8, blob, blob_bytes, &L);
  if (st != MIXLLM_OK) return st;
  if (n_begin < 0 || n_count < 0 || (int64_t)n_begin + n_count > N) return MIXLLM_E_SHAPE;
  if (M == 0 || n_count == 0) return MIXLLM_OK;
  if (!part) return MIXLLM_E_NULL;
  const Plan pl = make_plan(M, L);
  if (!pl.skinny && !tile_offsets_fit(M, L)) return MIXLLM_E_SHAPE;
  GemmArgs a;
  fill_args(a, aq, sa, asum, rowop, M, blob, L);
  a.part = part;
  a.n_begin = n_begin;
  a.n_count = n_count;
  return launch<true>(a, pl, (hipStream_t)stream);
}
