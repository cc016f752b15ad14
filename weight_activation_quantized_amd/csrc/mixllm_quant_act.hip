// Activation quantization of the W4.4A8 layer: fp16 -> int8, one symmetric
// round-to-nearest scale per token and per group of 128 inputs (MixLLM talk notes,
// 設計判断の概要 "design decisions": 8-bit symmetric group-wise RTN activations;
// アブレーション研究 "ablation": activation groups of 128).
//
// The pages do not describe this kernel.  It is a streaming pass (2 bytes in, 1 + 4/128
// (+ 4/128) bytes out per element), so its roofline is HBM bandwidth.  Layout: one
// 16-lane quarter of a wave owns one (token, group) pair; each lane loads 8 fp16 values
// (16 bytes), the quarter reduces the group maximum and the code sum with DPP lane moves,
// and each lane stores its 8 codes (8 bytes).  Consecutive quarters own consecutive
// groups of the same token, so a wave reads 1 KB of contiguous fp16 input.
//
// Arithmetic matches the definition bit for bit: the maximum of |x| is exact, the scale
// is an IEEE fp32 division amax / 127, each code is rne(x / s) of the correctly rounded
// quotient (a reciprocal product where that provably rounds the same way, else hipcc's
// default correctly rounded division; no fast-math), clamped to [-127, 127].
//
// Optionally the kernel also writes the row operands of the GEMM's matrix-core scale
// products and zero-point corrections: s and u = fp32(S_A * s) each as an exact sum of
// three bf16 values (truncate to bf16, the remainder has at most 16 significant bits,
// truncate again, the second remainder has at most 8), as two 16-byte bf16 MFMA row
// operands: [s0 s0 s1 s1 s2 s2 0 0] and [u0 u0 u1 u1 u2 u2 0 0].
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mixllm.h"

namespace mixllm {
bool is_aligned16(const void *p);
}

namespace {

#ifndef MIXLLM_QA_DIV
#define MIXLLM_QA_DIV 0
#endif
#ifndef MIXLLM_QA_PPL
#define MIXLLM_QA_PPL 1
#endif
#ifndef MIXLLM_QA_MAXBLOCKS
#define MIXLLM_QA_MAXBLOCKS 0x7FFFFFFF
#endif
constexpr int kThreads = 256;
constexpr int kPairsPerBlock = kThreads / 16;
// Up to this many tokens the pairs go in group-major order (see quant_act_kernel):
// 512 x 4096 4.69 -> 4.18 us, 1024 x 28672 25.8 -> 24.8 us; 2048 x 8192 17.0 -> 17.7 us.
constexpr int32_t kGroupMajorMaxM = 1024;

__device__ __forceinline__ float h2f(uint32_t bits16) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)));
}

// Reductions over the 16 lanes of a quarter (a DPP row) with DPP lane moves, no LDS: swap
// neighbours, swap pairs (quad permutes), then mirror each 8-lane half and the row; after
// the four steps every lane holds the combination of all 16 lanes.
constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}

__device__ __forceinline__ float quarter_max(float v) {
  v = fmaxf(v, __int_as_float(dpp<kDppXor1>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp<kDppXor2>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp<kDppHalfMirror>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp<kDppMirror>(__float_as_int(v))));
  return v;
}

__device__ __forceinline__ int quarter_sum(int v) {
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  v += dpp<kDppMirror>(v);
  return v;
}

// x = p0 + p1 + p2 exactly, each a bf16 (returned as p | p << 16 words).
__device__ __forceinline__ void split3(float x, uint32_t w[3]) {
  const uint32_t b0 = __float_as_uint(x) & 0xFFFF0000u;
  const float r1 = x - __uint_as_float(b0);
  const uint32_t b1 = __float_as_uint(r1) & 0xFFFF0000u;
  const uint32_t b2 = __float_as_uint(r1 - __uint_as_float(b1)) & 0xFFFF0000u;
  w[0] = b0 | (b0 >> 16);
  w[1] = b1 | (b1 >> 16);
  w[2] = b2 | (b2 >> 16);
}

// One (token, group) pair per 16-lane quarter: load, reduce, quantize, store.
__device__ __forceinline__ void quant_pair(uint4 raw, bool live, int64_t m, int g, int sub, int32_t M, int32_t K,
                                           int8_t *__restrict__ aq, float *__restrict__ sa,
                                           int32_t *__restrict__ asum, uint4 *__restrict__ rowop) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = h2f(w[i] & 0xFFFFu);
    x[2 * i + 1] = h2f(w[i] >> 16);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
  amax = quarter_max(amax);
  const float s = amax / 127.0f;

  int q[8];
  int qsum = 0;
#if MIXLLM_QA_DIV
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float v = amax > 0.0f ? __builtin_rintf(x[i] / s) : 0.0f;
    v = fminf(fmaxf(v, -127.0f), 127.0f);
    q[i] = (int)v;
    qsum += q[i];
  }
#else
  // rne(x / s) without a division per code: t = x * rcp(s) differs from the correctly
  // rounded quotient by less than 6e-5 (|x / s| <= 127, v_rcp_f32 within 1 ulp, one more
  // rounding in the product), so rne(t) is rne(x / s) unless t lies within 2^-12 of a
  // half-integer; those codes take the IEEE division.
  const float r = __builtin_amdgcn_rcpf(s);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float t = x[i] * r;
    float v = __builtin_rintf(t);
    if (fabsf(t - v) > 0.5f - 0x1p-12f) v = __builtin_rintf(x[i] / s);
    v = amax > 0.0f ? fminf(fmaxf(v, -127.0f), 127.0f) : 0.0f;
    q[i] = (int)v;
    qsum += q[i];
  }
#endif
  qsum = quarter_sum(qsum);
  if (!live) return;

  uint2 packed;
  packed.x = (uint32_t)(q[0] & 0xFF) | ((uint32_t)(q[1] & 0xFF) << 8) | ((uint32_t)(q[2] & 0xFF) << 16) |
             ((uint32_t)(q[3] & 0xFF) << 24);
  packed.y = (uint32_t)(q[4] & 0xFF) | ((uint32_t)(q[5] & 0xFF) << 8) | ((uint32_t)(q[6] & 0xFF) << 16) |
             ((uint32_t)(q[7] & 0xFF) << 24);
  *reinterpret_cast<uint2 *>(aq + m * K + (int64_t)g * MIXLLM_GROUP + sub * 8) = packed;
  if (sub == 0) {
    sa[(int64_t)g * M + m] = s;
    if (asum) asum[(int64_t)g * M + m] = qsum;
  }
  if (rowop && sub < 2) {
    uint32_t ws[3], wu[3];
    split3(s, ws);
    split3((float)qsum * s, wu);
    rowop[((int64_t)g * M + m) * 2 + sub] =
        sub == 0 ? make_uint4(ws[0], ws[1], ws[2], 0u) : make_uint4(wu[0], wu[1], wu[2], 0u);
  }
}

// Each quarter handles pairs pair0, pair0 + stride, ... with PPL of them in flight.  Pair
// order: token-major (consecutive quarters take consecutive groups of one token: a wave
// reads 1 KB of one row) or, with GMAJOR, group-major (consecutive quarters take one group
// of consecutive tokens: a wave's scales, code sums and row records are contiguous, which
// is faster while the outputs are small; measured on the Llama shapes).
template <int PPL, bool GMAJOR>
__global__ __launch_bounds__(kThreads) void quant_act_kernel(const uint16_t *__restrict__ a, int64_t lda,
                                                             int32_t M, int32_t K, int8_t *__restrict__ aq,
                                                             float *__restrict__ sa, int32_t *__restrict__ asum,
                                                             uint4 *__restrict__ rowop) {
  const int G = K / MIXLLM_GROUP;
  const int sub = threadIdx.x & 15;
  const int64_t npairs = (int64_t)M * G;
  const int64_t stride = (int64_t)gridDim.x * kPairsPerBlock;
  for (int64_t base = (int64_t)blockIdx.x * kPairsPerBlock + (threadIdx.x >> 4); base < npairs;
       base += stride * PPL) {
    uint4 raw[PPL];
    int64_t m[PPL];
    int g[PPL];
    bool live[PPL];
#pragma unroll
    for (int i = 0; i < PPL; ++i) {
      const int64_t pair = base + i * stride;
      live[i] = pair < npairs;
      if (GMAJOR) {
        g[i] = live[i] ? (int)(pair / M) : 0;
        m[i] = live[i] ? pair - (int64_t)g[i] * M : 0;
      } else {
        m[i] = live[i] ? pair / G : 0;
        g[i] = live[i] ? (int)(pair - m[i] * G) : 0;
      }
      raw[i] = make_uint4(0, 0, 0, 0);
      if (live[i]) raw[i] = *reinterpret_cast<const uint4 *>(a + m[i] * lda + (int64_t)g[i] * MIXLLM_GROUP + sub * 8);
    }
#pragma unroll
    for (int i = 0; i < PPL; ++i) quant_pair(raw[i], live[i], m[i], g[i], sub, M, K, aq, sa, asum, rowop);
  }
}

// The Llama MLP activation between the gate/up and down projections, fused with the
// down projection's activation quantization: h = SiLU(gate) * up, computed in fp32
// (SiLU(x) = x / (1 + e^-x), IEEE division, the library exp) and rounded once to fp16,
// then quantized exactly as quant_act quantizes an fp16 input (same code path), so the
// outputs equal quant_act applied to h.  Optionally writes h.
__global__ __launch_bounds__(kThreads) void silu_mul_quant_kernel(const uint16_t *__restrict__ gate,
                                                                  const uint16_t *__restrict__ up, int64_t ld,
                                                                  int32_t M, int32_t I, int8_t *__restrict__ aq,
                                                                  float *__restrict__ sa, int32_t *__restrict__ asum,
                                                                  uint4 *__restrict__ rowop, uint16_t *__restrict__ h) {
  const int G = I / MIXLLM_GROUP;
  const int sub = threadIdx.x & 15;
  const int64_t npairs = (int64_t)M * G;
  const int64_t pair = (int64_t)blockIdx.x * kPairsPerBlock + (threadIdx.x >> 4);
  const bool live = pair < npairs;
  const int64_t m = live ? pair / G : 0;
  const int g = live ? (int)(pair - m * G) : 0;
  uint4 gr = make_uint4(0, 0, 0, 0), ur = make_uint4(0, 0, 0, 0);
  if (live) {
    const int64_t off = m * ld + (int64_t)g * MIXLLM_GROUP + sub * 8;
    gr = *reinterpret_cast<const uint4 *>(gate + off);
    ur = *reinterpret_cast<const uint4 *>(up + off);
  }
  const uint32_t gw[4] = {gr.x, gr.y, gr.z, gr.w}, uw[4] = {ur.x, ur.y, ur.z, ur.w};
  uint32_t hw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t out = 0;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const float gv = h2f((gw[i] >> (16 * half)) & 0xFFFFu), uv = h2f((uw[i] >> (16 * half)) & 0xFFFFu);
      const float silu = gv / (1.0f + expf(-gv));
      const float hv = silu * uv;
      out |= (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hv) << (16 * half);
    }
    hw[i] = out;
  }
  const uint4 raw = make_uint4(hw[0], hw[1], hw[2], hw[3]);
  if (live && h) *reinterpret_cast<uint4 *>(h + m * I + (int64_t)g * MIXLLM_GROUP + sub * 8) = raw;
  quant_pair(raw, live, m, g, sub, M, I, aq, sa, asum, rowop);
}

}  // namespace

extern "C" int mixllm_quant_act(const uint16_t *a, int64_t lda, int32_t M, int32_t K, int32_t group,
                                int8_t *aq, float *sa, int32_t *asum, uint32_t *rowop, void *stream) {
  if (group != MIXLLM_GROUP) return MIXLLM_E_GROUP;
  if (M < 0 || K <= 0 || K % MIXLLM_GROUP != 0 || lda < K || lda % 8 != 0) return MIXLLM_E_SHAPE;
  if (M == 0) return MIXLLM_OK;
  if (!a || !aq || !sa) return MIXLLM_E_NULL;
  if (!mixllm::is_aligned16(a) || !mixllm::is_aligned16(aq) || !mixllm::is_aligned16(sa) ||
      (asum && !mixllm::is_aligned16(asum)) || (rowop && !mixllm::is_aligned16(rowop)))
    return MIXLLM_E_SHAPE;
  const int64_t npairs = (int64_t)M * (K / MIXLLM_GROUP);
  constexpr int kPPL = MIXLLM_QA_PPL;
  int64_t blocks = (npairs + kPairsPerBlock * kPPL - 1) / (kPairsPerBlock * kPPL);
  if (blocks > MIXLLM_QA_MAXBLOCKS) blocks = MIXLLM_QA_MAXBLOCKS;
  if (M <= kGroupMajorMaxM)
    hipLaunchKernelGGL((quant_act_kernel<kPPL, true>), dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)stream,
                       a, lda, M, K, aq, sa, asum, reinterpret_cast<uint4 *>(rowop));
  else
    hipLaunchKernelGGL((quant_act_kernel<kPPL, false>), dim3((unsigned)blocks), dim3(kThreads), 0,
                       (hipStream_t)stream, a, lda, M, K, aq, sa, asum, reinterpret_cast<uint4 *>(rowop));
  return hipGetLastError() == hipSuccess ? MIXLLM_OK : MIXLLM_E_HIP;
}

extern "C" int mixllm_silu_mul_quant(const uint16_t *gate, const uint16_t *up, int64_t ld, int32_t M, int32_t I,
                                     int32_t group, int8_t *aq, float *sa, int32_t *asum, uint32_t *rowop, uint16_t *h,
                                     void *stream) {
  if (group != MIXLLM_GROUP) return MIXLLM_E_GROUP;
  if (M < 0 || I <= 0 || I % MIXLLM_GROUP != 0 || ld < I || ld % 8 != 0) return MIXLLM_E_SHAPE;
  if (M == 0) return MIXLLM_OK;
  if (!gate || !up || !aq || !sa) return MIXLLM_E_NULL;
  if (!mixllm::is_aligned16(gate) || !mixllm::is_aligned16(up) || !mixllm::is_aligned16(aq) ||
      !mixllm::is_aligned16(sa) || (asum && !mixllm::is_aligned16(asum)) ||
      (rowop && !mixllm::is_aligned16(rowop)) || (h && !mixllm::is_aligned16(h)))
    return MIXLLM_E_SHAPE;
  const int64_t npairs = (int64_t)M * (I / MIXLLM_GROUP);
  const int64_t blocks = (npairs + kPairsPerBlock - 1) / kPairsPerBlock;
  if (blocks > 0x7FFFFFFF) return MIXLLM_E_SHAPE;
  hipLaunchKernelGGL(silu_mul_quant_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)stream, gate,
                     up, ld, M, I, aq, sa, asum, reinterpret_cast<uint4 *>(rowop), h);
  return hipGetLastError() == hipSuccess ? MIXLLM_OK : MIXLLM_E_HIP;
}
