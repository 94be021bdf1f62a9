// Router top-k with renormalised softmax weights, and the token-to-expert grouping.
//
// "Red Metal dev8 — resident routed top-k layer": the layer pins every selected expert
// and runs each one; router weights are positive and sum to about one.  Selection is by
// (logit descending, expert id ascending) on the raw logits, so no rounding of exp can
// create or break a tie; the weights are exp(l_j - m) / sum_selected exp(l_i - m), the
// sum taken in selection order.
#include "route_dev.hpp"

namespace moe {

template <int VPL>
__global__ void __launch_bounds__(256) k_topk(const float *__restrict__ logits, int T, int E, int k, int kprime,
                                              int add_shared, int32_t *__restrict__ ids, float *__restrict__ w) {
  __shared__ TopkLds S[4];
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  topk_wave<VPL>(logits + (size_t)t * E, E, k, add_shared, ids + (size_t)t * kprime, w + (size_t)t * kprime,
                 nullptr, nullptr, S[threadIdx.x >> 6]);
}

// ----------------------------------------------------------------------------- grouping
// Stable counting sort of the n = T * kprime slots by expert id, in one workgroup of
// 16 waves.  Wave w owns a contiguous range of slots.  Pass 1 builds a histogram per
// wave in LDS; an exclusive scan over (expert, wave) in expert-major order gives every
// wave its starting cursor per expert; pass 2 walks the wave's slots 64 at a time and
// ranks each lane among the earlier lanes holding the same expert (found by ballots
// over the bits of the id).  Integer-only and
// order-defined, so the output is unique and identical run to run.

constexpr int kGroupWaves = 16;

struct GroupLds {
  int hist[kGroupWaves][MOE_MAX_IDS];
  int offs[MOE_MAX_IDS];
  int arank[MOE_MAX_IDS];
  int4 wave_tot[kGroupWaves];
  int4 total;
};

// Inclusive prefix sum over a wave: DPP row shifts inside the 16-lane rows, then the
// row totals carried by row broadcasts (lanes whose source falls outside take 0).
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// Exclusive prefix sums of four values over the workgroup in thread order, and their
// totals in S.total.  Integer sums: any order gives the same result.  S.wave_tot and
// S.total are read after the last barrier: a second call needs a barrier in between.
__device__ __forceinline__ int4 block_exclusive_scan4(int4 v, GroupLds &S) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int4 inc = make_int4(wave_inclusive_scan(v.x), wave_inclusive_scan(v.y), wave_inclusive_scan(v.z),
                             wave_inclusive_scan(v.w));
  if (lane == 63) S.wave_tot[wave] = inc;
  __syncthreads();
  if (threadIdx.x < 64) {  // the wave totals scanned by wave 0, lane i holding wave i's
    const int4 c = lane < kGroupWaves ? S.wave_tot[lane] : make_int4(0, 0, 0, 0);
    const int4 ic = make_int4(wave_inclusive_scan(c.x), wave_inclusive_scan(c.y), wave_inclusive_scan(c.z),
                              wave_inclusive_scan(c.w));
    if (lane < kGroupWaves) S.wave_tot[lane] = make_int4(ic.x - c.x, ic.y - c.y, ic.z - c.z, ic.w - c.w);
    if (lane == kGroupWaves - 1) S.total = ic;
  }
  __syncthreads();
  const int4 b = S.wave_tot[wave];
  return make_int4(b.x + inc.x - v.x, b.y + inc.y - v.y, b.z + inc.z - v.z, b.w + inc.w - v.w);
}


// ids: global or LDS.  Must be called by all 1024 threads.
__device__ void group_block(const int32_t *ids, int n, int n_ids, int max_narrow, int32_t *__restrict__ counts,
                            int32_t *__restrict__ offsets, int32_t *__restrict__ sorted_slot,
                            int32_t *__restrict__ slot_pos, WorkRec *__restrict__ work, GroupLds &S) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int id_bits = n_ids > 1 ? 32 - __builtin_clz((unsigned)(n_ids - 1)) : 0;
  const int per = (((n + kGroupWaves - 1) / kGroupWaves) + 63) / 64 * 64;
  const int lo = wave * per, hi = min(n, lo + per);
  const int nw = min(kGroupWaves, (n + per - 1) / per);  // the waves that hold slots

  for (int i = threadIdx.x; i < nw * MOE_MAX_IDS; i += blockDim.x) (&S.hist[0][0])[i] = 0;
  __syncthreads();
  for (int s = lo + lane; s < hi; s += 64) {
    int e = ids[s];
    if (e >= 0 && e < n_ids) atomicAdd(&S.hist[wave][e], 1);
  }
  __syncthreads();
  const int e = threadIdx.x;  // n_ids <= MOE_MAX_IDS == blockDim.x
  // the expert's count per wave (rows past nw were not cleared: not counted), all read
  // before any is used
  int hv[kGroupWaves], c = 0;
#pragma unroll
  for (int w = 0; w < kGroupWaves; w++) hv[w] = S.hist[w][e];
#pragma unroll
  for (int w = 0; w < kGroupWaves; w++) c += (w < nw && e < n_ids) ? hv[w] : 0;
  const bool wide = c > max_narrow;
  const int tiles = wide ? (c + MOE_MFMA_TILE_TOKENS - 1) / MOE_MFMA_TILE_TOKENS : 0;
  // slots, mat-vec experts, matrix-core experts, tiles
  const int4 ex = block_exclusive_scan4(make_int4(c, c > 0 && !wide ? 1 : 0, wide ? 1 : 0, tiles), S);
  const int4 tot = S.total;
  const int excl = ex.x, nex = ex.y, tex = ex.w;
  const int n_total = tot.x, n_narrow = tot.y, n_wide = tot.z, n_tiles = tot.w;
  if (e < n_ids) {
    counts[e] = c;
    offsets[e] = excl;
    S.offs[e] = excl;
    S.arank[e] = c > 0 && !wide ? 1 + nex : -1;  // the expert's record in the first set
    if (c > 0 && !wide) {
      WorkRec &r = work[1 + nex];
      r.e = e;
      r.p0 = excl;
      r.p1 = excl + c;
    }
    for (int i = 0; i < tiles; i++)
      work[n_ids + 1 + tex + i] =
          WorkRec{e, excl + i * MOE_MFMA_TILE_TOKENS, excl + min(c, (i + 1) * MOE_MFMA_TILE_TOKENS), 0};
  }
  if (e == 0) {
    offsets[n_ids] = n_total;
    work[0] = WorkRec{n_narrow, n_total, n_wide, n_tiles};
  }
  if (e < n_ids) {  // each wave's first position for the expert
    int run = excl;
#pragma unroll
    for (int w = 0; w < kGroupWaves; w++) {
      if (w < nw) {
        S.hist[w][e] = run;
        run += hv[w];
      }
    }
  }
  __syncthreads();

  for (int base = lo; base < hi; base += 64) {
    int s = base + lane;
    int my = -1;
    if (s < hi) {
      int v = ids[s];
      my = (v >= 0 && v < n_ids) ? v : -1;
    }
    // the lanes holding the same expert: one ballot per bit of the id (ids < 2^id_bits),
    // intersected, among the lanes that hold a slot; rank = those below this lane
    uint64_t peers = __ballot(my >= 0);
    for (int b = 0; b < id_bits; b++) {
      const bool bit = (my >> b) & 1;
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    const int rank = lanes_below(peers), tot = (int)__popcll(peers);
    if (my >= 0) {
      int pos = S.hist[wave][my] + rank;
      sorted_slot[pos] = s;
      slot_pos[s] = pos;
      if (pos == S.offs[my] && S.arank[my] > 0) work[S.arank[my]].slot0 = s;
    }
    __builtin_amdgcn_wave_barrier();
    if (my >= 0 && rank == 0) S.hist[wave][my] += tot;
    __builtin_amdgcn_wave_barrier();
  }
}

__global__ void __launch_bounds__(1024) k_group(const int32_t *__restrict__ ids, int T, int kprime, int n_ids,
                                                int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
                                                int32_t *__restrict__ sorted_slot, int32_t *__restrict__ slot_pos,
                                                WorkRec *__restrict__ work) {
  __shared__ GroupLds S;
  group_block(ids, T * kprime, n_ids, matvec_max_tokens(T), counts, offsets, sorted_slot, slot_pos, work, S);
}

// Small batches: top-k and grouping in one workgroup; the ids stay in LDS between them.
constexpr int kSmallMaxSlots = 1024;

template <int VPL>
__global__ void __launch_bounds__(1024) k_route_group_small(const float *__restrict__ logits, int T, int E, int k,
                                                            int add_shared, int32_t *__restrict__ ids,
                                                            float *__restrict__ w, int32_t *__restrict__ counts,
                                                            int32_t *__restrict__ offsets,
                                                            int32_t *__restrict__ sorted_slot,
                                                            int32_t *__restrict__ slot_pos,
                                                            WorkRec *__restrict__ work) {
  __shared__ GroupLds S;
  __shared__ TopkLds TS[kGroupWaves];
  __shared__ int32_t ids_l[kSmallMaxSlots];
  const int kprime = k + add_shared;
  const int wave = threadIdx.x >> 6;
  for (int t = wave; t < T; t += kGroupWaves)
    topk_wave<VPL>(logits + (size_t)t * E, E, k, add_shared, ids + (size_t)t * kprime, w + (size_t)t * kprime,
                   ids_l + t * kprime, nullptr, TS[wave]);
  __syncthreads();
  if (T * kprime <= kTinySlots)
    group_tiny(ids_l, T * kprime, E + add_shared, matvec_max_tokens(T), counts, offsets, sorted_slot, slot_pos, work);
  else
    group_block(ids_l, T * kprime, E + add_shared, matvec_max_tokens(T), counts, offsets, sorted_slot, slot_pos, work, S);
}

#define MOE_VPL_DISPATCH(E, KERNEL, ...)                      \
  do {                                                        \
    if ((E) <= 64) hipLaunchKernelGGL(KERNEL<1>, __VA_ARGS__); \
    else if ((E) <= 128) hipLaunchKernelGGL(KERNEL<2>, __VA_ARGS__); \
    else if ((E) <= 256) hipLaunchKernelGGL(KERNEL<4>, __VA_ARGS__); \
    else if ((E) <= 512) hipLaunchKernelGGL(KERNEL<8>, __VA_ARGS__); \
    else hipLaunchKernelGGL(KERNEL<16>, __VA_ARGS__);         \
  } while (0)

hipError_t launch_route_group(const float *logits, int T, int E, int k, int add_shared, int32_t *ids, float *w,
                              int32_t *counts, int32_t *offsets, int32_t *sorted_slot, int32_t *slot_pos,
                              WorkRec *work, hipStream_t s) {
  const int kprime = k + add_shared;
  // one launch for small batches; above 512 experts the 16 keys per lane do not fit
  // the register budget of a 1024-thread workgroup, so those go through two launches
  if (T * kprime <= kSmallMaxSlots && T <= 4 * kGroupWaves && E <= 512) {
    if (E <= 64)
      hipLaunchKernelGGL(k_route_group_small<1>, dim3(1), dim3(1024), 0, s, logits, T, E, k, add_shared, ids, w,
                         counts, offsets, sorted_slot, slot_pos, work);
    else if (E <= 128)
      hipLaunchKernelGGL(k_route_group_small<2>, dim3(1), dim3(1024), 0, s, logits, T, E, k, add_shared, ids, w,
                         counts, offsets, sorted_slot, slot_pos, work);
    else if (E <= 256)
      hipLaunchKernelGGL(k_route_group_small<4>, dim3(1), dim3(1024), 0, s, logits, T, E, k, add_shared, ids, w,
                         counts, offsets, sorted_slot, slot_pos, work);
    else
      hipLaunchKernelGGL(k_route_group_small<8>, dim3(1), dim3(1024), 0, s, logits, T, E, k, add_shared, ids, w,
                         counts, offsets, sorted_slot, slot_pos, work);
  } else {
    MOE_VPL_DISPATCH(E, k_topk, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, k, kprime, add_shared, ids, w);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(k_group, dim3(1), dim3(1024), 0, s, ids, T, kprime, E + add_shared, counts, offsets,
                       sorted_slot, slot_pos, work);
  }
  return hipGetLastError();
}

// Explicit selection: only the shared slot is written, then the grouping.
__global__ void k_fill_shared(int T, int E, int k, int kprime, int32_t *ids, float *w) {
  int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t < T) {
    ids[(size_t)t * kprime + k] = E;
    w[(size_t)t * kprime + k] = 1.0f;
  }
}

hipError_t launch_group_explicit(int T, int E, int k, int add_shared, int32_t *ids, float *w, int32_t *counts,
                                 int32_t *offsets, int32_t *sorted_slot, int32_t *slot_pos, WorkRec *work,
                                 hipStream_t s) {
  const int kprime = k + add_shared;
  if (add_shared) {
    hipLaunchKernelGGL(k_fill_shared, dim3((T + 255) / 256), dim3(256), 0, s, T, E, k, kprime, ids, w);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(k_group, dim3(1), dim3(1024), 0, s, ids, T, kprime, E + add_shared, counts, offsets,
                     sorted_slot, slot_pos, work);
  return hipGetLastError();
}

}  // namespace moe
