// Packed-blob layout shared by the host packer and the GEMM launchers.
//
// The blob is a 256-byte header followed by sections, each 256-byte aligned:
//
//   w4   [nb4 blocks][G groups] 2048 B: 32 channels x 128 4-bit codes
//   s4   [nb4][G][32]  fp16 scales of the 4-bit blocks
//   z4   [nb4][G][16]  4-bit zero points, channel c in byte c/2 (low nibble for even c)
//   w8   [nb8 blocks][G] 4096 B: 32 channels x 128 int8 codes
//   s8   [nb8][G][32]  fp16 scales of the 8-bit blocks
//   zp   [32][G]       zero points of the promoted 4-bit channels (unpacking only)
//   idx  [nb * 32]     int32 original channel index of every packed channel (-1: empty)
//
// Packed channel order: the n4 4-bit channels (ascending original index), then the n8
// 8-bit channels (ascending), then empty channels up to nb * 32 = 32 ceil(N / 32).
// Block b holds packed channels [32b, 32b + 32).  The first nb4 = floor(n4 / 32) blocks
// are 4-bit blocks.  The remaining nb8 = nb - nb4 blocks are 8-bit blocks; the first of
// them starts with the r = n4 - 32 nb4 leftover 4-bit channels, stored as their partially
// dequantized int8 codes (q - z) in [-15, 15] with their fp16 scale.  Two-step
// dequantization computes the same partial sum_k (q - z) a_k and the same scale
// product for them either way, so every block has one kind, and the block count is
// ceil(N / 32): no tile is spent on padding between the two subsets.
//
// The tile kernel's matrix-core scale products take s_w (an fp16, at most 11 significant
// bits) and z * s_w (at most 15) as exact sums of two bf16 values, which it forms from
// s4 / s8 and z4 as it reads them.
//
// Inside a 4-bit (block, group) chunk of 2048 B, 16-byte unit u = ((half * 4 + a) * 16 + ch)
// holds channel 16 * half + ch, k-chunks a (bytes 0..7) and a + 4 (bytes 8..15) of the
// group, where k-chunk c covers the group's inputs [16c, 16c + 16).  The 8 bytes of a
// k-chunk starting at input k0 are two little-endian words: byte i (i = 0..3) of word w
// (w = 0, 1) holds the code of input k0 + 8w + i in its low nibble and the code of
// input k0 + 8w + 4 + i in its high nibble.  Masking a word with 0x0F0F0F0F, or its copy
// shifted right by 4, therefore yields four consecutive input codes as bytes.
//
// Inside an 8-bit (block, group) chunk of 4096 B, unit u = ((half * 8 + c) * 16 + ch)
// holds the 16 codes of channel 16 * half + ch for inputs [16c, 16c + 16).
//
// A 64-lane wave reading units [64j, 64j + 64) of a chunk touches 1 KB of contiguous
// memory; the 16x16x64 kernels read exactly that, and the 32x32x32 kernels read
// contiguous 256-byte runs.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "mixllm.h"

namespace mixllm {

constexpr int kGroup = 128;
constexpr int kBlock = 32;          // channels per block
constexpr size_t kHeaderBytes = 256;
constexpr size_t kW4Chunk = 2048;   // bytes per (block, group), 4-bit part
constexpr size_t kW8Chunk = 4096;   // bytes per (block, group), 8-bit part
constexpr size_t kS4Chunk = 64;     // 32 fp16 scales
constexpr size_t kZ4Chunk = 16;     // 32 nibbles
constexpr size_t kS8Chunk = 64;

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Fills the layout for (N, K, n8).  Returns false when the parameters are invalid or
// the size overflows.
inline bool compute_layout(int32_t N, int32_t K, int32_t n8, mixllm_blob_info *L) {
  if (N <= 0 || K <= 0 || K % kGroup != 0 || n8 < 0 || n8 > N) return false;
  const int64_t G = K / kGroup;
  const int64_t n4 = (int64_t)N - n8;
  const int64_t nb = ((int64_t)N + kBlock - 1) / kBlock;
  const int64_t nb4 = n4 / kBlock;
  const int64_t nb8 = nb - nb4;
  // Keep every byte count well inside 2^62 so the sums below cannot overflow.
  if (nb > (int64_t(1) << 26) || G > (int64_t(1) << 26)) return false;
  L->magic = MIXLLM_BLOB_MAGIC;
  L->version = MIXLLM_BLOB_VERSION;
  L->N = N;
  L->K = K;
  L->group = kGroup;
  L->n8 = n8;
  L->n4 = (int32_t)n4;
  L->G = (int32_t)G;
  L->nb = (int32_t)nb;
  L->nb4 = (int32_t)nb4;
  L->nb8 = (int32_t)nb8;
  L->n4_promoted = (int32_t)(n4 - nb4 * kBlock);
  size_t off = kHeaderBytes;
  L->off_w4 = off;
  off = align256(off + (size_t)nb4 * G * kW4Chunk);
  L->off_s4 = off;
  off = align256(off + (size_t)nb4 * G * kS4Chunk);
  L->off_z4 = off;
  off = align256(off + (size_t)nb4 * G * kZ4Chunk);
  L->off_w8 = off;
  off = align256(off + (size_t)nb8 * G * kW8Chunk);
  L->off_s8 = off;
  off = align256(off + (size_t)nb8 * G * kS8Chunk);
  L->off_zp = off;
  off = align256(off + (size_t)kBlock * G);
  L->off_idx = off;
  off = align256(off + (size_t)nb * kBlock * 4);
  L->total_bytes = off;
  return true;
}

}  // namespace mixllm
