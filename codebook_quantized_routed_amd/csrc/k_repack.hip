// Load-time repacking of IQ1_S-like matrices into the IQ1_M-like layout that every
// kernel of the path decodes ("Red Lite dev10 — standalone native Metal path", section
// "Quant grids": IQ1_M reuses the IQ1_S 2048 x 8 grid).  Both formats give a weight as
// d * (2s + 1) * (grid[idx][j] +/- 1/8); IQ1_S-like carries one scale and one delta sign
// per 32 weights where IQ1_M-like has them per 16 and per 8, so repeating them is exact:
// every repacked weight is the same bits.  The cost is 6 bytes per 256 weights more in
// HBM (56 instead of 50), which the latency-bound decode does not notice.
//
// One thread per (row, 256-weight super-block):
//   in : ql u8[32], qh u16[8] (bits 3i..3i+2: index bits 8-10 of group i of the 32-weight
//        sub-block, bits 12-14: 3-bit scale, bit 15: delta sign), d u16
//   out: ql u8[32] (copied), qh u8[16] (group g: nibble g & 1 of byte g / 2, bits 0-2 the
//        index high bits, bit 3 the delta sign), sd u64 (d in bits 0-15, the 3-bit scale of
//        16-weight sub-block i in bits 16 + 3i .. 18 + 3i)
#include "common.hpp"
#include "repack.hpp"

namespace moe {

__global__ void k_repack_iq1s(const uint8_t *__restrict__ ql, const uint16_t *__restrict__ qh,
                              const uint16_t *__restrict__ d, size_t n_blocks, uint8_t *__restrict__ ql_out,
                              uint8_t *__restrict__ qh_out, uint64_t *__restrict__ sd_out) {
  const size_t b = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= n_blocks) return;
  const uint4 *src = (const uint4 *)(ql + b * 32);
  uint4 *dst = (uint4 *)(ql_out + b * 32);
  const uint4 q0 = src[0], q1 = src[1];
  dst[0] = q0;
  dst[1] = q1;
  const uint4 hw = *(const uint4 *)(qh + b * 8);  // the eight sub-block words
  const uint32_t words[4] = {hw.x, hw.y, hw.z, hw.w};
  uint64_t sd = d[b];
  uint32_t out[4];
#pragma unroll
  for (int k = 0; k < 4; k++) {  // u32 k holds sub-blocks 2k (low half) and 2k + 1
    uint32_t o = 0;
#pragma unroll
    for (int h = 0; h < 2; h++) {
      const uint32_t w = (words[k] >> (16 * h)) & 0xFFFFu;
      const uint32_t sign = (w >> 15) & 1u, scale = (w >> 12) & 7u;
      const int sb = 2 * k + h;
      // groups 4 sb .. 4 sb + 3 -> bytes 2 sb, 2 sb + 1 of the output; 8 bits per 2 groups
#pragma unroll
      for (int i = 0; i < 4; i++) o |= (((w >> (3 * i)) & 7u) | (sign << 3)) << (16 * h + 4 * i);
      sd |= (uint64_t)scale << (16 + 3 * (2 * sb));
      sd |= (uint64_t)scale << (16 + 3 * (2 * sb + 1));
    }
    out[k] = o;
  }
  *(uint4 *)(qh_out + b * 16) = make_uint4(out[0], out[1], out[2], out[3]);
  sd_out[b] = sd;
}

hipError_t launch_repack_iq1s(const uint8_t *ql, const uint16_t *qh, const uint16_t *d, size_t n_blocks,
                              uint8_t *ql_out, uint8_t *qh_out, uint64_t *sd_out, hipStream_t s) {
  const unsigned grid = (unsigned)((n_blocks + 255) / 256);
  hipLaunchKernelGGL(k_repack_iq1s, dim3(grid), dim3(256), 0, s, ql, qh, d, n_blocks, ql_out, qh_out, sd_out);
  return hipGetLastError();
}

}  // namespace moe
