/*
 * mixllm.h -- C ABI of the MI355X (gfx950) W4.4A8 output-channel mixed-precision
 * linear layer (the MixLLM hot path).
 *
 * What the layer computes (sources: the MixLLM talk notes on notes.yuuk.io, MLSys 2026,
 * sections 設計判断の概要 "design decisions", 二段階逆量子化 "two-step dequantization",
 * 並列実行 "parallel execution"; and the awesome-system-papers summary page of the same
 * paper, section 核心方法 "core method"):
 *
 *   * activations A (fp16 [M][K]) are quantized per token and per 128-wide group of
 *     input features to int8 with a symmetric round-to-nearest scale;
 *   * a set S8 of output channels (~10%) holds 8-bit symmetric group-128 weights,
 *     the other channels hold 4-bit asymmetric group-128 weights (code, 4-bit zero
 *     point, fp16 scale);
 *   * Y[m][n] = sum_g s_w[n][g] * s_a[m][g] * sum_{k in g} (W_q[n][k] - z[n][g]) * A_q[m][k]
 *     -- an exact int32 dot product per group, then one fp32 scale-and-accumulate per
 *     group -- written as fp16 to the channel's original index n.
 *
 * Conventions shared by every entry point:
 *   * Every function returns a mixllm_status: 0 on success, a negative code on error.
 *     No function aborts, prints, or allocates device memory.
 *   * All argument checks run on the host before any HIP call; on error nothing is
 *     launched and no output is written.
 *   * Device entry points are asynchronous on the given stream (NULL = the default
 *     stream) and never synchronize.  A launch failure returns MIXLLM_E_HIP.
 *   * The caller owns every buffer.  Device pointers must be 16-byte aligned.
 *   * The quantization group size is fixed at 128 (MIXLLM_GROUP); K must be a
 *     multiple of it.  M = 0 is a valid no-op.
 *   * Inputs must be finite; non-finite activations or weights give unspecified codes.
 *
 * Calls that overlap on one device and share an output buffer race; calls on
 * different streams with distinct outputs are independent.
 */
#ifndef MIXLLM_H_
#define MIXLLM_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MIXLLM_GROUP 128
#define MIXLLM_BLOB_MAGIC 0x344C584Du /* "MXL4" little-endian */
#define MIXLLM_BLOB_VERSION 6u

typedef enum mixllm_status {
  MIXLLM_OK = 0,
  MIXLLM_E_NULL = -1,   /* a required pointer is NULL */
  MIXLLM_E_SHAPE = -2,  /* M < 0, N or K <= 0, K % 128 != 0, misaligned pointer, size overflow, bad stride */
  MIXLLM_E_GROUP = -3,  /* group != 128 */
  MIXLLM_E_INDEX = -4,  /* an 8-bit channel index is out of [0, N) or repeated, or n8 out of [0, N] */
  MIXLLM_E_SPACE = -5,  /* a caller buffer (blob, workspace, output window) is too small */
  MIXLLM_E_FORMAT = -6, /* a packed blob has a bad magic, version or shape */
  MIXLLM_E_HIP = -7     /* the HIP runtime reported an error at launch */
} mixllm_status;

/* Host-side copy of the packed-blob header (the first 256 bytes of every blob). */
typedef struct mixllm_blob_info {
  uint32_t magic, version;
  int32_t N, K, group, n8, n4;  /* n4 = N - n8 */
  int32_t G;                    /* K / 128 groups per channel */
  int32_t nb;                   /* 32-channel blocks: ceil(N / 32) */
  int32_t nb4;                  /* 4-bit blocks: floor(n4 / 32) */
  int32_t nb8;                  /* 8-bit blocks: nb - nb4 */
  int32_t n4_promoted;          /* n4 - 32 nb4 4-bit channels stored in the first 8-bit block */
  uint64_t off_w4, off_s4, off_z4, off_w8, off_s8, off_zp, off_idx, total_bytes;
} mixllm_blob_info;

/* Human-readable name of a status code (static string, never NULL). */
const char *mixllm_status_str(int status);

/* ------------------------------------------------------------------------------------
 * Weight packing (host, offline, once per layer).
 *
 * Quantizes an fp16 weight matrix per output channel and group of 128 input features
 * (talk notes, 二段階逆量子化 and ルーフラインモデル: 4-bit asymmetric channels store
 * 0.5 + 2.5/G bytes per element, 8-bit symmetric channels 1 + 2/G) and lays the codes
 * out in the order the GEMM kernels consume them, so no permutation happens at run
 * time (talk notes, ソフトウェアパイプライン: pre-packed, interleaved weight layout).
 *
 *   8-bit channel n, group g:  amax = max |W|;  s = fp16(amax / 127)  (fp32 division,
 *       round to nearest even; a non-zero group whose scale underflows gets 2^-24);
 *       q = clamp(rne(W / s), -127, 127);  s = 0 and q = 0 for an all-zero group.
 *   4-bit channel n, group g:  lo = min(min W, 0), hi = max(max W, 0);
 *       s = fp16((hi - lo) / 15);  z = clamp(rne(-lo / s), 0, 15);
 *       q = clamp(rne(W / s) + z, 0, 15);  dequantized value (q - z) * s.
 *
 * Channel order inside the blob: the 4-bit channels in ascending original index, then
 * the 8-bit channels in ascending original index, padded with empty channels (index -1)
 * to a multiple of 32, in blocks of 32 channels.  Whole blocks of 4-bit channels keep
 * packed nibbles; the n4 % 32 leftover 4-bit channels share the first 8-bit block,
 * stored as their int8 partial dequantization (q - z) (the same two-step arithmetic).
 * The blob is position independent: a byte copy of it to device memory is what the GEMM
 * reads.
 * ------------------------------------------------------------------------------------ */

/* Size in bytes of the blob for these parameters, or 0 if they are invalid. */
size_t mixllm_packed_bytes(int32_t N, int32_t K, int32_t group, int32_t n8);

/*
 * w_fp16_host: [N][K] row-major IEEE fp16 bit patterns (nn.Linear layout [out][in]).
 * idx8_host:   n8 distinct 8-bit channel indices in [0, N), any order (NULL if n8 == 0).
 * blob_host:   output, blob_bytes >= mixllm_packed_bytes(N, K, group, n8).
 * Host-only, synchronous, pure (no global state).  Errors: E_NULL, E_SHAPE, E_GROUP,
 * E_INDEX, E_SPACE.
 */
int mixllm_pack_weights(const uint16_t *w_fp16_host, int32_t N, int32_t K, int32_t group,
                        const int32_t *idx8_host, int32_t n8, void *blob_host, size_t blob_bytes);

/* Reads and checks the header of a host blob.  Errors: E_NULL, E_SPACE, E_FORMAT. */
int mixllm_blob_get_info(const void *blob_host, size_t blob_bytes, mixllm_blob_info *info);

/*
 * Inverse of the packing, for tests: codes in original channel order.
 * q: [N][K] bytes (uint4 code for 4-bit channels, int8 code bits for 8-bit channels);
 * z: [N][G] (zero point; 0 for 8-bit channels); s_fp16: [N][G] scale bits;
 * is8: [N] (1 for 8-bit channels).  Host-only.  Errors: E_NULL, E_SPACE, E_FORMAT.
 */
int mixllm_unpack_weights(const void *blob_host, size_t blob_bytes, uint8_t *q, uint8_t *z,
                          uint16_t *s_fp16, uint8_t *is8);

/* ------------------------------------------------------------------------------------
 * Global output-channel precision search (host): the step before packing that decides
 * which channels get 8 bits (talk notes, グローバル混合精度探索; summary page, 核心方法).
 *
 * mixllm_channel_salience: for every output channel n of one layer,
 *   S_n = (1/D) sum_d | t_dn + t_dn^2 / 2 |,  t_dn = sum_k grads[d][n][k] * delta_n[k],
 * the loss change of quantizing only channel n by a second-order Taylor expansion with the
 * Fisher approximation of the Hessian (first-order term kept), where delta_n = c_q - c_0
 * is the channel dequantized from this library's 4-bit asymmetric group-128 quantizer
 * minus its fp16 weights.  Computed in fp64.
 * w_fp16: [N][K] fp16 weights (host).  grads: [D][N][K] fp32 per-sample gradients of the
 * loss with respect to those weights (host; the caller computes them on a model and
 * calibration data).  s_out: [N] fp64.  Errors: E_NULL, E_SHAPE (N, K or D <= 0,
 * K % 128 != 0), E_GROUP.
 *
 * mixllm_assign_channels: the pages' Algorithm 1.  scores: the salience of every channel
 * of L layers, concatenated layer by layer (layer l has layer_n[l] channels).  The T
 * highest scores over all layers get 8 bits; equal scores go to the lower layer, then the
 * lower channel, first.  idx8_out: [T] the chosen channels, layer by layer, ascending
 * within a layer (each layer's run is the idx8 argument of mixllm_pack_weights);
 * layer_n8_out: [L] how many each layer got.  idx8_out may be NULL when T == 0.  Errors:
 * E_NULL, E_SHAPE (L <= 0, a layer_n <= 0, T < 0 or above the total, a non-finite score).
 * ------------------------------------------------------------------------------------ */
int mixllm_channel_salience(const uint16_t *w_fp16, const float *grads, int32_t N, int32_t K, int32_t group,
                            int32_t D, double *s_out);

int mixllm_assign_channels(const double *scores, const int32_t *layer_n, int32_t L, int64_t T, int32_t *idx8_out,
                           int32_t *layer_n8_out);

/* ------------------------------------------------------------------------------------
 * Activation quantization (device).
 *
 * Per token m and group g (talk notes, 設計判断の概要: 8-bit symmetric group-wise RTN
 * activations): amax = max |A[m][g*128 .. +128)| in fp32; s = amax / 127 (fp32 IEEE
 * division); A_q = clamp(rne(A / s), -127, 127) (IEEE division); s = 0, A_q = 0 for an
 * all-zero group; S_A = sum of the group's codes.
 *
 * a_fp16_dev: [M][lda] fp16, lda >= K, lda % 8 == 0.
 * aq_dev:     output int8 [M][K] row-major.
 * sa_dev:     output fp32 [G][M] (group-major: the scales of one group for consecutive
 *             tokens are contiguous).
 * asum_dev:   output int32 [G][M] code sums, or NULL to skip.
 * rowop_dev:  output uint32 [G][M][8], or NULL to skip: the row operands of the GEMM's
 *             scale products and zero-point corrections.  s and u = fp32(S_A * s) are
 *             each split into three bf16 values p0 + p1 + p2 that sum to them exactly
 *             (p0 = the value truncated to bf16, p1 = the remainder truncated, p2 = the
 *             rest); with the word w(p) = p | p << 16, record [g][m] is {w(s0), w(s1),
 *             w(s2), 0, w(u0), w(u1), w(u2), 0}.
 * Errors: E_NULL, E_SHAPE, E_GROUP, E_HIP.
 * ------------------------------------------------------------------------------------ */
int mixllm_quant_act(const uint16_t *a_fp16_dev, int64_t lda, int32_t M, int32_t K, int32_t group,
                     int8_t *aq_dev, float *sa_dev, int32_t *asum_dev, uint32_t *rowop_dev, void *stream);

/* ------------------------------------------------------------------------------------
 * Llama MLP activation fused with the down projection's activation quantization (device).
 *
 * The step between the gate/up and down projections of the Llama MLP blocks whose layer
 * shapes the pages time (talk notes, A100 GPU でのシステム性能; the activation itself is
 * the standard Llama one, not described on the pages): h = SiLU(gate) * up with
 * SiLU(x) = x / (1 + e^-x), computed in fp32 and rounded once to fp16 (nearest even), then
 * quantized for the down projection exactly as mixllm_quant_act quantizes an fp16 input
 * (the outputs equal mixllm_quant_act applied to h).
 *
 * gate_dev, up_dev: fp16 [M][ld] each (for one GEMM over the packed gate ∪ up channels,
 *                   up_dev = gate_dev + I and ld = 2 I); ld >= I, ld % 8 == 0.
 * aq_dev, sa_dev, asum_dev, rowop_dev: as mixllm_quant_act with K = I.
 * h_dev:            fp16 [M][I] copy of h, or NULL to skip.
 * Errors: E_NULL, E_SHAPE, E_GROUP, E_HIP.
 * ------------------------------------------------------------------------------------ */
int mixllm_silu_mul_quant(const uint16_t *gate_dev, const uint16_t *up_dev, int64_t ld, int32_t M, int32_t I,
                          int32_t group, int8_t *aq_dev, float *sa_dev, int32_t *asum_dev, uint32_t *rowop_dev,
                          uint16_t *h_dev, void *stream);

/* ------------------------------------------------------------------------------------
 * Mixed W4/W8 x A8 GEMM with scatter epilogue (device).
 *
 * Two-step dequantization (talk notes, 二段階逆量子化): for each group, the exact
 * int32 dot product of (W_q - z) with A_q on the int8 matrix cores, then one fp32
 * multiply-add by s_w * s_a into a per-element fp32 accumulator (double accumulator:
 * per group and global, summary page, 核心方法).  The 4-bit and 8-bit channel subsets
 * are disjoint sub-GEMMs run in one grid (talk notes, 並列実行); the epilogue writes each
 * channel's fp16 result (round to nearest even) to its original index.  The zero point
 * of a 4-bit channel enters as sum_k (q - z) a_k = sum_k q a_k - z S_A, with S_A the
 * group's activation code sum.
 *
 * aq_dev, sa_dev, asum_dev, rowop_dev: as produced by mixllm_quant_act for the same M and K.
 *                 asum_dev may be NULL when the blob has no whole 4-bit block (nb4 == 0: no
 *                 zero points to correct); the other three are always required.
 * N, K, n8:       the layer the caller expects (output channels, inputs, 8-bit channels).
 * blob_info:      host pointer to the header of the packed blob, as mixllm_blob_get_info
 *                 returned it for the host blob whose byte copy is blob_dev.  It must equal,
 *                 field by field, the header a blob packed now for (N, K, n8) would carry
 *                 (magic, format version, shape, section offsets, size); otherwise the call
 *                 returns MIXLLM_E_FORMAT and launches nothing.  This is how a blob packed for
 *                 another layer, another 8-bit count or an older format is rejected: the
 *                 library does not read device memory back to check it.
 * blob_dev:       device copy of that blob (blob_bytes long, at least blob_info->total_bytes).
 * y_fp16_dev:     output fp16 [M][ldy], ldy >= N; only columns 0..N-1 are written.
 * workspace_dev:  reserved; pass NULL and 0 (mixllm_gemm_workspace_bytes returns 0: no
 *                 kernel needs scratch memory).
 * Kernel choice: M > 64 runs the tile kernel; M <= 3 runs the one-lane-per-channel gemv
 * kernel on layers with at least (CUs / 2) 32-channel blocks, in 64-channel strips, or in
 * 32-channel strips with each channel's inputs split over two lanes when there are fewer
 * 64-channel strips than CUs; 4 <= M <= 32 runs the strip
 * kernel on layers with at least (3 CUs / 4) strips of one or two blocks; otherwise
 * M <= 64 runs the skinny kernel unless the layer has enough 128-channel tiles to keep
 * the device busy (a cost rule on M, N and the CU count).  All give results within the
 * same tolerance; the int32 partials are identical.
 * Errors: E_NULL, E_SHAPE (also when the tile kernel runs and G * M * 32 exceeds
 * 2^31 - 1), E_GROUP, E_INDEX, E_SPACE, E_FORMAT, E_HIP.
 * ------------------------------------------------------------------------------------ */
size_t mixllm_gemm_workspace_bytes(int32_t M, int32_t N, int32_t K, int32_t n8);

int mixllm_gemm_w4w8a8(const int8_t *aq_dev, const float *sa_dev, const int32_t *asum_dev, const uint32_t *rowop_dev,
                       int32_t M, int32_t N, int32_t K, int32_t n8, const mixllm_blob_info *blob_info,
                       const void *blob_dev, size_t blob_bytes, uint16_t *y_fp16_dev, int64_t ldy,
                       void *workspace_dev, size_t workspace_bytes, void *stream);

/*
 * Test entry point: the same integer inner loop as mixllm_gemm_w4w8a8, but instead of
 * folding, it writes the int32 group partials P[m][j][g] = sum_{k in g} (W_q - z) * A_q
 * for the original channels n_begin + j, 0 <= j < n_count.
 * p_dev: int32 [M][n_count][G].  Errors: as mixllm_gemm_w4w8a8, plus E_SHAPE when the
 * window is outside [0, N).
 */
int mixllm_gemm_w4w8a8_partials(const int8_t *aq_dev, const float *sa_dev, const int32_t *asum_dev,
                                const uint32_t *rowop_dev, int32_t M, int32_t N, int32_t K, int32_t n8,
                                const mixllm_blob_info *blob_info, const void *blob_dev, size_t blob_bytes,
                                int32_t n_begin, int32_t n_count, int32_t *p_dev, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MIXLLM_H_ */
