// Host-side weight packer of the W4.4A8 mixed-precision linear layer.
//
// Quantizes an fp16 weight matrix per output channel and group of 128 inputs -- 8-bit
// symmetric for the salient channel set, 4-bit asymmetric for the rest (MixLLM talk
// notes, 設計判断の概要 "design decisions"; 二段階逆量子化 "two-step dequantization") --
// and writes the codes in the order the GEMM kernels read them (ソフトウェアパイプライン:
// weights are packed and interleaved ahead of time so no permutation runs in the kernel).
//
// Float semantics: every step is a single IEEE binary32 operation (this file is built
// with -ffp-contract=off and without fast-math), ties of the round-to-nearest steps go
// to even, and fp16 conversions round to nearest even.  These are the readings of
// "RTN" and of the scale dtype stated in the header mixllm.h.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "mixllm.h"
#include "mixllm_hostquant.h"
#include "mixllm_layout.h"

namespace mixllm {

float f16_to_f32(uint16_t h) {
  const uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  const uint32_t e = (h >> 10) & 0x1Fu;
  const uint32_t m = h & 0x3FFu;
  float out;
  if (e == 0) {
    out = (float)m * 5.9604644775390625e-08f;  // m * 2^-24, exact
    return sign ? -out : out;
  }
  uint32_t bits;
  if (e == 31) {
    bits = sign | 0x7F800000u | (m << 13);
  } else {
    bits = sign | ((e + 112u) << 23) | (m << 13);
  }
  memcpy(&out, &bits, 4);
  return out;
}

// binary32 -> binary16, round to nearest, ties to even.
uint16_t f32_to_f16_rne(float f) {
  uint32_t x;
  memcpy(&x, &f, 4);
  const uint16_t sign = (uint16_t)((x >> 16) & 0x8000u);
  const uint32_t ax = x & 0x7FFFFFFFu;
  if (ax >= 0x7F800000u) return sign | (ax > 0x7F800000u ? 0x7E00u : 0x7C00u);
  if (ax >= 0x477FF000u) return sign | 0x7C00u;  // >= 65520 rounds to infinity
  if (ax >= 0x38800000u) {                       // normal binary16 range
    const uint32_t r = ax - 0x38000000u;         // rebias exponent 127 -> 15
    return sign | (uint16_t)((r + 0x0FFFu + ((r >> 13) & 1u)) >> 13);
  }
  // Below 2^-14: the result is round(|f| / 2^-24) subnormal units (1024 is 2^-14).
  const uint32_t e = ax >> 23;
  const uint32_t m = e ? ((ax & 0x7FFFFFu) | 0x800000u) : ax;
  const int shift = 126 - (int)(e ? e : 1);  // |f| = m * 2^(e-150) = (m >> shift) units
  if (shift >= 25) return sign;              // below half a unit
  uint32_t q = m >> shift;
  const uint32_t rem = m & ((1u << shift) - 1u);
  const uint32_t half = 1u << (shift - 1);
  if (rem > half || (rem == half && (q & 1u))) ++q;
  return sign | (uint16_t)q;
}

static inline float clampf(float v, float lo, float hi) { return v < lo ? lo : (v > hi ? hi : v); }

// One group of an 8-bit symmetric channel.
void quant_group_w8(const uint16_t *w, int8_t *q, uint16_t *s16_out) {
  float x[kGroup];
  float amax = 0.0f;
  for (int i = 0; i < kGroup; ++i) {
    x[i] = f16_to_f32(w[i]);
    amax = std::max(amax, fabsf(x[i]));
  }
  if (!(amax > 0.0f)) {
    memset(q, 0, kGroup);
    *s16_out = 0;
    return;
  }
  const float s32 = amax / 127.0f;
  uint16_t s16 = f32_to_f16_rne(s32);
  if (s16 == 0) s16 = 1;  // underflow: smallest subnormal, 2^-24
  const float s = f16_to_f32(s16);
  for (int i = 0; i < kGroup; ++i) q[i] = (int8_t)clampf(rintf(x[i] / s), -127.0f, 127.0f);
  *s16_out = s16;
}

// One group of a 4-bit asymmetric channel.
void quant_group_w4(const uint16_t *w, uint8_t *q, uint8_t *z_out, uint16_t *s16_out) {
  float x[kGroup];
  float lo = 0.0f, hi = 0.0f;
  for (int i = 0; i < kGroup; ++i) {
    x[i] = f16_to_f32(w[i]);
    lo = std::min(lo, x[i]);
    hi = std::max(hi, x[i]);
  }
  const float range = hi - lo;
  if (!(range > 0.0f)) {
    memset(q, 0, kGroup);
    *z_out = 0;
    *s16_out = 0;
    return;
  }
  const float s32 = range / 15.0f;
  uint16_t s16 = f32_to_f16_rne(s32);
  if (s16 == 0) s16 = 1;
  const float s = f16_to_f32(s16);
  const float z = clampf(rintf(-lo / s), 0.0f, 15.0f);
  for (int i = 0; i < kGroup; ++i) q[i] = (uint8_t)clampf(rintf(x[i] / s) + z, 0.0f, 15.0f);
  *z_out = (uint8_t)z;
  *s16_out = s16;
}

}  // namespace mixllm

namespace {

using mixllm::f16_to_f32;
using mixllm::f32_to_f16_rne;
using mixllm::kBlock;
using mixllm::kGroup;
using mixllm::quant_group_w4;
using mixllm::quant_group_w8;

// Position of the byte holding the code of group input k inside a 4-bit unit:
// returns byte offset within the (block, group) chunk and whether it is the high nibble.
inline void w4_code_pos(int ch32, int k, size_t *byte_off, int *hi) {
  const int c = k >> 4;            // k-chunk 0..7
  const int a = c & 3;             // unit index within the half
  const int part = c >> 2;         // 0: bytes 0..7, 1: bytes 8..15
  const int r = k & 15;            // position inside the k-chunk
  const int w = r >> 3;            // word 0 or 1
  const int i = r & 3;             // byte inside the word
  *hi = (r >> 2) & 1;              // inputs k0+8w+4..7 live in the high nibble
  const int half = ch32 >> 4, ch = ch32 & 15;
  const size_t unit = (size_t)((half * 4 + a) * 16 + ch);
  *byte_off = unit * 16 + (size_t)part * 8 + (size_t)w * 4 + (size_t)i;
}

inline size_t w8_code_pos(int ch32, int k) {
  const int c = k >> 4;
  const int half = ch32 >> 4, ch = ch32 & 15;
  const size_t unit = (size_t)((half * 8 + c) * 16 + ch);
  return unit * 16 + (size_t)(k & 15);
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" {

const char *mixllm_status_str(int status) {
  switch (status) {
    case MIXLLM_OK: return "MIXLLM_OK";
    case MIXLLM_E_NULL: return "MIXLLM_E_NULL: a required pointer is NULL";
    case MIXLLM_E_SHAPE: return "MIXLLM_E_SHAPE: invalid shape, stride, alignment or size";
    case MIXLLM_E_GROUP: return "MIXLLM_E_GROUP: group size must be 128";
    case MIXLLM_E_INDEX: return "MIXLLM_E_INDEX: invalid 8-bit channel index or count";
    case MIXLLM_E_SPACE: return "MIXLLM_E_SPACE: caller buffer too small";
    case MIXLLM_E_FORMAT: return "MIXLLM_E_FORMAT: bad packed-weight blob";
    case MIXLLM_E_HIP: return "MIXLLM_E_HIP: HIP runtime error";
    default: return "MIXLLM: unknown status";
  }
}

size_t mixllm_packed_bytes(int32_t N, int32_t K, int32_t group, int32_t n8) {
  mixllm_blob_info L;
  if (group != kGroup || !mixllm::compute_layout(N, K, n8, &L)) return 0;
  return (size_t)L.total_bytes;
}

int mixllm_pack_weights(const uint16_t *w, int32_t N, int32_t K, int32_t group, const int32_t *idx8,
                        int32_t n8, void *blob, size_t blob_bytes) {
  if (!w || !blob || (n8 > 0 && !idx8)) return MIXLLM_E_NULL;
  if (group != kGroup) return MIXLLM_E_GROUP;
  if (N <= 0 || K <= 0 || K % kGroup != 0) return MIXLLM_E_SHAPE;
  if (n8 < 0 || n8 > N) return MIXLLM_E_INDEX;
  mixllm_blob_info L;
  if (!mixllm::compute_layout(N, K, n8, &L)) return MIXLLM_E_SHAPE;
  if (blob_bytes < L.total_bytes) return MIXLLM_E_SPACE;

  std::vector<uint8_t> is8((size_t)N, 0);
  for (int32_t i = 0; i < n8; ++i) {
    const int32_t c = idx8[i];
    if (c < 0 || c >= N || is8[(size_t)c]) return MIXLLM_E_INDEX;
    is8[(size_t)c] = 1;
  }
  // Packed order: 4-bit channels ascending, then 8-bit channels ascending.
  std::vector<int32_t> perm;
  perm.reserve((size_t)N);
  for (int32_t c = 0; c < N; ++c)
    if (!is8[(size_t)c]) perm.push_back(c);
  for (int32_t c = 0; c < N; ++c)
    if (is8[(size_t)c]) perm.push_back(c);

  uint8_t *base = (uint8_t *)blob;
  memset(base, 0, (size_t)L.total_bytes);
  memcpy(base, &L, sizeof(L));
  const int G = L.G;
  uint8_t *w4 = base + L.off_w4;
  uint16_t *s4 = (uint16_t *)(base + L.off_s4);
  uint8_t *z4 = base + L.off_z4;
  int8_t *w8 = (int8_t *)(base + L.off_w8);
  uint16_t *s8 = (uint16_t *)(base + L.off_s8);
  uint8_t *zp = base + L.off_zp;
  int32_t *idx = (int32_t *)(base + L.off_idx);

  for (int64_t j = 0; j < (int64_t)L.nb * kBlock; ++j) idx[j] = j < N ? perm[(size_t)j] : -1;

  const int64_t j8 = (int64_t)L.nb4 * kBlock;  // first packed channel of the 8-bit blocks
  uint8_t q4[kGroup];
  int8_t q8[kGroup];
  for (int64_t j = 0; j < N; ++j) {
    const int32_t n = perm[(size_t)j];
    const uint16_t *row = w + (size_t)n * (size_t)K;
    const int64_t b = j / kBlock;
    const int ch32 = (int)(j % kBlock);
    for (int g = 0; g < G; ++g) {
      if (j < j8) {  // a whole 4-bit block: packed nibbles
        uint8_t z;
        uint16_t s16;
        quant_group_w4(row + (size_t)g * kGroup, q4, &z, &s16);
        const size_t cidx = (size_t)b * G + g;
        uint8_t *chunk = w4 + cidx * mixllm::kW4Chunk;
        for (int k = 0; k < kGroup; ++k) {
          size_t off;
          int hi;
          w4_code_pos(ch32, k, &off, &hi);
          chunk[off] |= (uint8_t)(q4[k] << (hi ? 4 : 0));
        }
        s4[cidx * 32 + ch32] = s16;
        z4[cidx * 16 + ch32 / 2] |= (uint8_t)(z << ((ch32 & 1) ? 4 : 0));
        continue;
      }
      const size_t cidx = (size_t)(b - L.nb4) * G + g;
      int8_t *chunk = w8 + cidx * mixllm::kW8Chunk;
      uint16_t s16;
      if (j < L.n4) {  // leftover 4-bit channel: int8 partial dequantization q - z
        uint8_t z;
        quant_group_w4(row + (size_t)g * kGroup, q4, &z, &s16);
        for (int k = 0; k < kGroup; ++k) chunk[w8_code_pos(ch32, k)] = (int8_t)((int)q4[k] - (int)z);
        zp[(size_t)(j - j8) * G + g] = z;
      } else {
        quant_group_w8(row + (size_t)g * kGroup, q8, &s16);
        for (int k = 0; k < kGroup; ++k) chunk[w8_code_pos(ch32, k)] = q8[k];
      }
      s8[cidx * 32 + ch32] = s16;
    }
  }
  return MIXLLM_OK;
}

int mixllm_blob_get_info(const void *blob, size_t blob_bytes, mixllm_blob_info *info) {
  if (!blob || !info) return MIXLLM_E_NULL;
  if (blob_bytes < mixllm::kHeaderBytes) return MIXLLM_E_SPACE;
  mixllm_blob_info H, L;
  memcpy(&H, blob, sizeof(H));
  if (H.magic != MIXLLM_BLOB_MAGIC || H.version != MIXLLM_BLOB_VERSION || H.group != kGroup)
    return MIXLLM_E_FORMAT;
  if (!mixllm::compute_layout(H.N, H.K, H.n8, &L) || memcmp(&H, &L, sizeof(H)) != 0)
    return MIXLLM_E_FORMAT;
  if (blob_bytes < L.total_bytes) return MIXLLM_E_SPACE;
  *info = L;
  return MIXLLM_OK;
}

int mixllm_unpack_weights(const void *blob, size_t blob_bytes, uint8_t *q, uint8_t *z, uint16_t *s,
                          uint8_t *is8) {
  if (!q || !z || !s || !is8) return MIXLLM_E_NULL;
  mixllm_blob_info L;
  const int st = mixllm_blob_get_info(blob, blob_bytes, &L);
  if (st != MIXLLM_OK) return st;
  const uint8_t *base = (const uint8_t *)blob;
  const uint8_t *w4 = base + L.off_w4;
  const uint16_t *s4 = (const uint16_t *)(base + L.off_s4);
  const uint8_t *z4 = base + L.off_z4;
  const int8_t *w8 = (const int8_t *)(base + L.off_w8);
  const uint16_t *s8 = (const uint16_t *)(base + L.off_s8);
  const uint8_t *zp = base + L.off_zp;
  const int32_t *idx = (const int32_t *)(base + L.off_idx);
  const int G = L.G, K = L.K;
  const int64_t j8 = (int64_t)L.nb4 * kBlock;
  for (int64_t j = 0; j < L.N; ++j) {
    const int32_t n = idx[j];
    if (n < 0 || n >= L.N) return MIXLLM_E_FORMAT;
    const int64_t b = j / kBlock;
    const int ch32 = (int)(j % kBlock);
    is8[n] = j >= L.n4;
    for (int g = 0; g < G; ++g) {
      uint8_t *qrow = q + (size_t)n * K + (size_t)g * kGroup;
      if (j < j8) {
        const size_t cidx = (size_t)b * G + g;
        const uint8_t *chunk = w4 + cidx * mixllm::kW4Chunk;
        for (int k = 0; k < kGroup; ++k) {
          size_t off;
          int hi;
          w4_code_pos(ch32, k, &off, &hi);
          qrow[k] = hi ? (chunk[off] >> 4) : (chunk[off] & 15);
        }
        s[(size_t)n * G + g] = s4[cidx * 32 + ch32];
        z[(size_t)n * G + g] = (z4[cidx * 16 + ch32 / 2] >> ((ch32 & 1) ? 4 : 0)) & 15;
        continue;
      }
      const size_t cidx = (size_t)(b - L.nb4) * G + g;
      const int8_t *chunk = w8 + cidx * mixllm::kW8Chunk;
      const int zz = j < L.n4 ? zp[(size_t)(j - j8) * G + g] : 0;
      for (int k = 0; k < kGroup; ++k) qrow[k] = (uint8_t)(chunk[w8_code_pos(ch32, k)] + zz);
      s[(size_t)n * G + g] = s8[cidx * 32 + ch32];
      z[(size_t)n * G + g] = (uint8_t)zz;
    }
  }
  return MIXLLM_OK;
}

}  // extern "C"

// Used by the device entry points for pointer checks.
namespace mixllm {
bool is_aligned16(const void *p) { return aligned16(p); }
}  // namespace mixllm
