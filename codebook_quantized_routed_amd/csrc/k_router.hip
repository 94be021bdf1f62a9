// Router projection: logits[t][e] = sum_c x[t][c] * wr[e][c], and optionally the gate of
// the shared expert, sw[t] = 1 / (1 + exp(-sum_c x[t][c] * wsg[c])) ("Red Lite dev9 —
// native runtime foundation", closing paragraph, and "Red Lite dev10 — standalone native
// Metal path", section "What dev10 does not yet claim": the router network that feeds
// the top-k path is the pages' next step; here it is one linear map, fp32 weights).
//
// A workgroup of kRouterWaves waves takes kRouterWaves consecutive rows (the gate vector
// is row E) and kRouterTok tokens; wave w owns row 8 b + w and keeps it in registers
// (lane l: columns 4 l + 256 m .. 4 l + 256 m + 3), the tokens are staged in LDS, and
// every (token, row) dot is: fmaf over the lane's columns in order, then the wave sum
// (DPP row shifts, then the four row sums by readlane).  The order depends on the width
// only, so a token's logits are the same bits whatever the batch.  HBM-bound at decode
// (E rows x H x 4 bytes per call, 4 MiB at the field shape).
#include "common.hpp"
#include "router.hpp"

namespace moe {

constexpr int kRouterWaves = 8, kRouterTok = 8;

template <int NB>  // NB = hidden / 256 float4 columns per lane
__global__ void __launch_bounds__(64 * kRouterWaves) k_router(const float *__restrict__ x,
                                                             const float *__restrict__ wr,
                                                             const float *__restrict__ wsg, int T, int E,
                                                             float *__restrict__ logits, float *__restrict__ sw) {
  constexpr int H = 256 * NB;
  __shared__ __align__(16) float xs[kRouterTok * H];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.y * kRouterTok, nt = min(kRouterTok, T - t0);
  const int r = blockIdx.x * kRouterWaves + wave;
  const bool is_gate = wsg != nullptr && r == E;
  // the row (clamped for waves past the last row: they load row E - 1 and store nothing)
  const float4 *wrow = (const float4 *)(is_gate ? wsg : wr + (size_t)min(r, E - 1) * H);
  float4 w[NB];
#pragma unroll
  for (int m = 0; m < NB; m++) w[m] = wrow[lane + 64 * m];
  const float4 *xg = (const float4 *)(x + (size_t)t0 * H);
  for (int i = threadIdx.x; i < nt * (H / 4); i += blockDim.x) ((float4 *)xs)[i] = xg[i];
  __syncthreads();
  if (r > E || (r == E && !is_gate)) return;
  for (int t = 0; t < nt; t++) {
    const float4 *xr = (const float4 *)(xs + t * H);
    float s = 0.0f;
#pragma unroll
    for (int m = 0; m < NB; m++) {
      const float4 f = xr[lane + 64 * m];
      s = fmaf(f.x, w[m].x, s);
      s = fmaf(f.y, w[m].y, s);
      s = fmaf(f.z, w[m].z, s);
      s = fmaf(f.w, w[m].w, s);
    }
    s = group_sum_first<64>(s);
    if (lane == 0) {
      if (is_gate)
        sw[t0 + t] = 1.0f / (1.0f + expf(-s));
      else
        logits[(size_t)(t0 + t) * E + r] = s;
    }
  }
}

// The shared expert's weight of each token (slot kprime - 1) from the gate values.
__global__ void k_shared_weight(const float *__restrict__ sw, int T, int kprime, float *__restrict__ w) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t < T) w[(size_t)t * kprime + kprime - 1] = sw[t];
}

hipError_t launch_router(const float *x, const float *wr, const float *wsg, int T, int H, int E, float *logits,
                         float *sw, hipStream_t s) {
  const int rows = E + (wsg ? 1 : 0);
  const dim3 grid((unsigned)((rows + kRouterWaves - 1) / kRouterWaves), (unsigned)((T + kRouterTok - 1) / kRouterTok));
  const dim3 block(64 * kRouterWaves);
  switch (H) {
    case 256: hipLaunchKernelGGL(k_router<1>, grid, block, 0, s, x, wr, wsg, T, E, logits, sw); break;
    case 512: hipLaunchKernelGGL(k_router<2>, grid, block, 0, s, x, wr, wsg, T, E, logits, sw); break;
    case 1024: hipLaunchKernelGGL(k_router<4>, grid, block, 0, s, x, wr, wsg, T, E, logits, sw); break;
    default: hipLaunchKernelGGL(k_router<8>, grid, block, 0, s, x, wr, wsg, T, E, logits, sw); break;
  }
  return hipGetLastError();
}

hipError_t launch_shared_weight(const float *sw, int T, int kprime, float *w, hipStream_t s) {
  hipLaunchKernelGGL(k_shared_weight, dim3((unsigned)((T + 255) / 256)), dim3(256), 0, s, sw, T, kprime, w);
  return hipGetLastError();
}

}  // namespace moe
