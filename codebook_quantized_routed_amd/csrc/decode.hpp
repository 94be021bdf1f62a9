// Per-group decoding of the two codebook formats on the device.
//
// IQ2_XS-like group code (u16): bits 0-8 grid index, bits 9-15 signs of weights 0-6;
// weight 7 takes the parity of those seven bits, so a group always has an even number
// of negatives.  IQ1_M-like group code: 8 index bits from ql, a nibble from qh holding
// index bits 8-10 and the delta sign.  ("Red Lite dev10 — standalone native Metal
// path", section "Quant grids": IQ2_XS 512 x 8 over 0x08/0x19/0x2b, IQ1_M on the
// IQ1_S 2048 x 8 grid over -1/0/+1.)
#pragma once

#include "common.hpp"

namespace moe {

// Sign byte of an IQ2 group: bits 0-6 from the code, bit 7 their parity.
__device__ __forceinline__ uint32_t iq2_sign_byte(uint32_t code) {
  uint32_t s7 = (code >> 9) & 0x7Fu;
  return s7 | ((__builtin_popcount(s7) & 1u) << 7);
}

// IQ2 super-block factor d * (2s + 1) / 8 for sub-block `sub` (0..7): exact in fp32.
__device__ __forceinline__ float iq2_factor(uint32_t sc_word, uint32_t d_bits, int sub) {
  uint32_t s = (sc_word >> (4 * sub)) & 15u;
  return half_bits_to_float(d_bits) * (float)(2 * s + 1) * 0.125f;
}

// IQ1 factor d * (2s + 1) for sub-block `sub` (0..15): exact in fp32.
__device__ __forceinline__ float iq1_factor(uint64_t sd, int sub) {
  uint32_t s = (uint32_t)(sd >> (16 + 3 * sub)) & 7u;
  return half_bits_to_float((uint32_t)(sd & 0xFFFFu)) * (float)(2 * s + 1);
}

// Signed grid values of one IQ2 group (without the scale factor), from the u8 grid.
__device__ __forceinline__ void iq2_group_values(uint32_t code, const uint8_t *grid, float v[8]) {
  uint32_t idx = code & 0x1FFu, sg = iq2_sign_byte(code);
  uint2 row = *(const uint2 *)(grid + idx * 8);
#pragma unroll
  for (int j = 0; j < 8; j++) {
    uint32_t byte = ((j < 4 ? row.x : row.y) >> (8 * (j & 3))) & 0xFFu;
    float f = (float)byte;
    v[j] = ((sg >> j) & 1u) ? -f : f;
  }
}

// Grid values plus delta of one IQ1 group (without the scale factor), from the i8 grid.
// code12: bits 0-10 grid index, bit 11 delta sign.
__device__ __forceinline__ void iq1_group_values(uint32_t code12, const int8_t *grid, float v[8]) {
  uint32_t idx = code12 & 0x7FFu;
  float delta = (code12 & 0x800u) ? -0.125f : 0.125f;
  uint2 row = *(const uint2 *)(grid + idx * 8);
#pragma unroll
  for (int j = 0; j < 8; j++) {
    int b = (int)(int8_t)(((j < 4 ? row.x : row.y) >> (8 * (j & 3))) & 0xFFu);
    v[j] = (float)b + delta;
  }
}

// IQ1 12-bit code of group g of a row: ql byte and the qh nibble.
__device__ __forceinline__ uint32_t iq1_code(const uint8_t *ql_row, const uint8_t *qh_row, int g) {
  uint32_t nib = (qh_row[g >> 1] >> (4 * (g & 1))) & 15u;
  return (uint32_t)ql_row[g] | (nib << 8);
}

}  // namespace moe
