// Global output-channel precision search of the W4.4A8 layer, host side (MixLLM talk
// notes, グローバル混合精度探索 "global mixed-precision search"; summary page, 核心方法).
//
// Salience of output channel c: the change of the model loss when only c is quantized,
// expanded to second order with the Hessian replaced by the empirical Fisher matrix
// (1/|D|) sum_d g_d g_d^T.  That leaves one dot product per calibration sample d, and
// the first-order term is kept:
//
//   S_c = (1/|D|) sum_d | t_d + t_d^2 / 2 |,   t_d = g_d . (c_q - c_0)
//
// with g_d the per-sample gradient of the loss with respect to c's weights, c_0 the
// original weights and c_q the channel as the 4-bit asymmetric path stores it
// (dequantized; the library's own quantizer).  The assignment (the pages' Algorithm 1)
// puts every channel of every layer in one list, ranks it by S descending and gives the
// first T channels 8 bits.  The gradients themselves come from a model and calibration
// data, which are outside this library: the caller supplies them.
//
// Arithmetic: c_q - c_0 is exact in fp64 (a small integer times an fp16 scale minus an
// fp16 value); each t_d is an fp64 dot product in input order; S is accumulated in fp64.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "mixllm.h"
#include "mixllm_hostquant.h"
#include "mixllm_layout.h"

extern "C" int mixllm_channel_salience(const uint16_t *w, const float *grads, int32_t N, int32_t K, int32_t group,
                                       int32_t D, double *s_out) {
  if (group != mixllm::kGroup) return MIXLLM_E_GROUP;
  if (N <= 0 || K <= 0 || K % mixllm::kGroup != 0 || D <= 0) return MIXLLM_E_SHAPE;
  if (!w || !grads || !s_out) return MIXLLM_E_NULL;
  const int G = K / mixllm::kGroup;
  std::vector<double> delta((size_t)K);
  uint8_t q[mixllm::kGroup];
  for (int64_t n = 0; n < N; ++n) {
    const uint16_t *row = w + (size_t)n * (size_t)K;
    for (int g = 0; g < G; ++g) {
      uint8_t z;
      uint16_t s16;
      mixllm::quant_group_w4(row + (size_t)g * mixllm::kGroup, q, &z, &s16);
      const double s = (double)mixllm::f16_to_f32(s16);
      for (int i = 0; i < mixllm::kGroup; ++i) {
        const size_t k = (size_t)g * mixllm::kGroup + i;
        delta[k] = ((double)q[i] - (double)z) * s - (double)mixllm::f16_to_f32(row[k]);
      }
    }
    double acc = 0.0;
    for (int64_t d = 0; d < D; ++d) {
      const float *gr = grads + ((size_t)d * (size_t)N + (size_t)n) * (size_t)K;
      double t = 0.0;
      for (int k = 0; k < K; ++k) t += (double)gr[k] * delta[(size_t)k];
      acc += fabs(t + 0.5 * t * t);
    }
    s_out[n] = acc / (double)D;
  }
  return MIXLLM_OK;
}

extern "C" int mixllm_assign_channels(const double *scores, const int32_t *layer_n, int32_t L, int64_t T,
                                      int32_t *idx8_out, int32_t *layer_n8_out) {
  if (L <= 0) return MIXLLM_E_SHAPE;
  if (!scores || !layer_n || !layer_n8_out) return MIXLLM_E_NULL;
  int64_t total = 0;
  for (int32_t l = 0; l < L; ++l) {
    if (layer_n[l] <= 0) return MIXLLM_E_SHAPE;
    total += layer_n[l];
  }
  if (T < 0 || T > total) return MIXLLM_E_SHAPE;
  if (T > 0 && !idx8_out) return MIXLLM_E_NULL;
  for (int64_t i = 0; i < total; ++i)
    if (!std::isfinite(scores[i])) return MIXLLM_E_SHAPE;
  // One entry per channel: (layer, channel); the position in the concatenated score
  // array orders ties by layer, then channel.
  struct Entry {
    double s;
    int64_t pos;
    int32_t layer, chan;
  };
  std::vector<Entry> all((size_t)total);
  int64_t pos = 0;
  for (int32_t l = 0; l < L; ++l)
    for (int32_t c = 0; c < layer_n[l]; ++c, ++pos) all[(size_t)pos] = Entry{scores[pos], pos, l, c};
  std::sort(all.begin(), all.end(), [](const Entry &a, const Entry &b) {
    return a.s > b.s || (a.s == b.s && a.pos < b.pos);
  });
  // The first T, regrouped by layer in channel order.
  std::vector<std::vector<int32_t>> pick((size_t)L);
  for (int64_t i = 0; i < T; ++i) pick[(size_t)all[(size_t)i].layer].push_back(all[(size_t)i].chan);
  int64_t o = 0;
  for (int32_t l = 0; l < L; ++l) {
    std::vector<int32_t> &v = pick[(size_t)l];
    std::sort(v.begin(), v.end());
    layer_n8_out[l] = (int32_t)v.size();
    if (!v.empty()) memcpy(idx8_out + o, v.data(), v.size() * sizeof(int32_t));
    o += (int64_t)v.size();
  }
  return MIXLLM_OK;
}
