// Weighted accumulation of expert outputs and the unit-weight RMSNorm.
#include "common.hpp"

namespace moe {

// "Red Metal dev8 — resident routed top-k layer", step 5: accumulator +=
// router_weight * expert_output.  One thread per (token, column); the token's slots
// are taken in ascending expert id (ties, which a valid selection never has, by slot),
// each step one rounded multiply and one rounded add, so the result is a pure function
// of (acc, w, y) and does not depend on the order the router listed the experts in.
__global__ void __launch_bounds__(256) k_accumulate(const float *__restrict__ y, const float *__restrict__ w,
                                                    const int32_t *__restrict__ ids,
                                                    const int32_t *__restrict__ slot_pos, int kprime, int H,
                                                    float *__restrict__ acc) {
  __shared__ int order[MOE_MAX_K + 1];
  const int t = blockIdx.y;
  const int32_t *id = ids + (size_t)t * kprime;
  if (threadIdx.x < kprime) {
    int j = threadIdx.x, me = id[j], r = 0;
    for (int i = 0; i < kprime; i++) {
      int o = id[i];
      r += (o < me || (o == me && i < j)) ? 1 : 0;
    }
    order[r] = j;
  }
  __syncthreads();
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= H) return;
  float a = acc[(size_t)t * H + c];
  for (int q = 0; q < kprime; q++) {
    int s = t * kprime + order[q];
    float prod = __fmul_rn(w[s], y[(size_t)slot_pos[s] * H + c]);
    a = __fadd_rn(a, prod);
  }
  acc[(size_t)t * H + c] = a;
}

hipError_t launch_accumulate(const float *y, const float *w, const int32_t *ids, const int32_t *slot_pos, int T,
                             int kprime, int H, float *acc, hipStream_t s) {
  hipLaunchKernelGGL(k_accumulate, dim3((H + 255) / 256, T), dim3(256), 0, s, y, w, ids, slot_pos, kprime, H, acc);
  return hipGetLastError();
}

// "Red Lite dev16 — complete full-attention parity": the routed MoE reads the
// post-attention RMSNorm of the hidden state.  One workgroup per row.
// Thread t of 512 sums, with fmaf in column order, the squares of columns
// 4t .. 4t+3, 4t+2048 .. 4t+2051, ...; the waves' sums (first lane of a DPP/readlane
// tree) are combined as ((w0 + w1) + (w2 + w3)) + ((w4 + w5) + (w6 + w7)).  The decode
// of a stack of layers computes the same scale with the same operations.
__global__ void __launch_bounds__(512) k_rmsnorm(const float *h, int H, float eps,
                                                 float *x) {  // h and x may alias
  __shared__ float part[8];
  const float *hr = h + (size_t)blockIdx.x * H;
  float ss = 0.0f;
  for (int c = 4 * threadIdx.x; c < H; c += 2048)
    for (int j = 0; j < 4 && c + j < H; j++) ss = fmaf(hr[c + j], hr[c + j], ss);
  ss = group_sum_first<64>(ss);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = ((part[0] + part[1]) + (part[2] + part[3])) + ((part[4] + part[5]) + (part[6] + part[7]));
  const float r = 1.0f / sqrtf(tot / (float)H + eps);
  for (int c = threadIdx.x; c < H; c += blockDim.x) x[(size_t)blockIdx.x * H + c] = hr[c] * r;
}

hipError_t launch_rmsnorm(const float *h, int T, int H, float eps, float *x, hipStream_t s) {
  hipLaunchKernelGGL(k_rmsnorm, dim3(T), dim3(512), 0, s, h, H, eps, x);
  return hipGetLastError();
}

}  // namespace moe
