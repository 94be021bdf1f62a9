// Grid expansion and bit-exact dequantization to fp32.
#include "decode.hpp"
#include "mfma_dec.hpp"

namespace moe {

// Compact rows (symbol j in bits 2j..2j+1) to value rows, once per process.
__global__ void __launch_bounds__(256) k_grids_expand(const uint16_t *c2, const uint16_t *c1, uint8_t *grids) {
  for (int i = threadIdx.x; i < kIq2Rows * 8; i += blockDim.x) {
    uint32_t s = (c2[i >> 3] >> (2 * (i & 7))) & 3u;
    grids[kGridIq2Off + i] = s == 0 ? kIq2SymVal[0] : (s == 1 ? kIq2SymVal[1] : (s == 2 ? kIq2SymVal[2] : 0));
  }
  for (int i = threadIdx.x; i < kIq1Rows * 8; i += blockDim.x) {
    uint32_t s = (c1[i >> 3] >> (2 * (i & 7))) & 3u;
    grids[kGridIq1Off + i] =
        (uint8_t)(int8_t)(s == 0 ? kIq1SymVal[0] : (s == 1 ? kIq1SymVal[1] : (s == 2 ? kIq1SymVal[2] : 0)));
  }
  for (int i = threadIdx.x; i < kIq2Rows; i += blockDim.x) ((uint16_t *)(grids + kGridIq2CompactOff))[i] = c2[i];
  for (int i = threadIdx.x; i < kIq1Rows; i += blockDim.x) ((uint16_t *)(grids + kGridIq1CompactOff))[i] = c1[i];
  // the matrix-core decode tables, from the compact rows, in their LDS layout
  DecTableRegs r;
  const int t = threadIdx.x, n = blockDim.x;
#pragma unroll
  for (int i = 0; i < 2; i++) r.c2[i] = t + i * n < kIq2Rows ? c2[t + i * n] : 0u;
#pragma unroll
  for (int i = 0; i < 8; i++) r.c1[i] = t + i * n < kIq1Rows ? c1[t + i * n] : 0u;
  dec_tables_store(r, MOE_Q_IQ2XS_LIKE | MOE_Q_IQ1M_LIKE, dec_tables(MOE_Q_IQ2XS_LIKE | MOE_Q_IQ1M_LIKE),
                   grids + kGridDecOff, t, n);
}

hipError_t launch_grids_expand(const uint16_t *c2, const uint16_t *c1, uint8_t *grids, hipStream_t s) {
  hipLaunchKernelGGL(k_grids_expand, dim3(1), dim3(256), 0, s, c2, c1, grids);
  return hipGetLastError();
}

// One thread per 8-weight group; writes the group's 8 fp32 weights.
template <int QT>
__global__ void __launch_bounds__(256) k_dequant(int rows, int cols, QMat m, const uint8_t *grids, float *out) {
  const int ng = cols / 8, nb = cols / 256;
  size_t gid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (size_t)rows * ng) return;
  int r = (int)(gid / ng), g = (int)(gid % ng);
  int b = g / 32;
  float v[8], f;
  if (QT == MOE_Q_IQ2XS_LIKE) {
    uint32_t code = ((const uint16_t *)m.s0)[(size_t)r * ng + g];
    uint32_t sc = ((const uint32_t *)m.s1)[(size_t)r * nb + b];
    uint32_t d = ((const uint16_t *)m.s2)[(size_t)r * nb + b];
    iq2_group_values(code, grids + kGridIq2Off, v);
    f = iq2_factor(sc, d, (g % 32) / 4);
  } else {
    uint32_t code = iq1_code(m.s0 + (size_t)r * ng, m.s1 + (size_t)r * (ng / 2), g);
    uint64_t sd = ((const uint64_t *)m.s2)[(size_t)r * nb + b];
    iq1_group_values(code, (const int8_t *)(grids + kGridIq1Off), v);
    f = iq1_factor(sd, (g % 32) / 2);
  }
  float4 *o = (float4 *)(out + (size_t)r * cols + (size_t)g * 8);
  o[0] = make_float4(v[0] * f, v[1] * f, v[2] * f, v[3] * f);
  o[1] = make_float4(v[4] * f, v[5] * f, v[6] * f, v[7] * f);
}

hipError_t launch_dequant(int qt, int rows, int cols, QMat m, const uint8_t *grids, float *out, hipStream_t s) {
  size_t groups = (size_t)rows * (cols / 8);
  dim3 grid((unsigned)((groups + 255) / 256));
  if (qt == MOE_Q_IQ2XS_LIKE)
    hipLaunchKernelGGL(k_dequant<MOE_Q_IQ2XS_LIKE>, grid, dim3(256), 0, s, rows, cols, m, grids, out);
  else
    hipLaunchKernelGGL(k_dequant<MOE_Q_IQ1M_LIKE>, grid, dim3(256), 0, s, rows, cols, m, grids, out);
  return hipGetLastError();
}

}  // namespace moe
