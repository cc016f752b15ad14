// Host-side quantizer helpers shared by the packer and the channel-salience search
// (library-internal; not part of the C ABI).
#pragma once

#include <stdint.h>

namespace mixllm {

// fp16 bits -> fp32 value, exactly.
float f16_to_f32(uint16_t h);
// fp32 -> fp16 bits, round to nearest even.
uint16_t f32_to_f16_rne(float f);
// One group of 128 weights of an 8-bit symmetric channel: codes and the fp16 scale.
void quant_group_w8(const uint16_t *w, int8_t *q, uint16_t *s16_out);
// One group of 128 weights of a 4-bit asymmetric channel: codes, zero point, fp16 scale.
void quant_group_w4(const uint16_t *w, uint8_t *q, uint8_t *z_out, uint16_t *s16_out);

}  // namespace mixllm
