// Router top-k with renormalised softmax weights, and the token-to-expert grouping.
//
// "Red Metal dev8 — resident routed top-k layer": the layer pins every selected expert
// and runs each one; router weights are positive and sum to about one.  Selection is by
// (logit descending, expert id ascending) on the raw logits, so no rounding of exp can
// create or break a tie; the weights are exp(l_j - m) / sum_selected exp(l_i - m), the
// sum taken in selection order.
#include "common.hpp"

namespace moe {

// Float -> u32 with the same order; every finite value maps above 0x007FFFFF, so 0 can
// stand for "taken / no value".
__device__ __forceinline__ uint32_t orderable(float f) {
  uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float from_orderable(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Wave-wide max / min of a u32 through DPP row shifts and row broadcasts (lane 63 ends
// with the result), then read lane 63.  Lanes outside a shift's row take the identity.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false));  // row_shr:1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false));  // row_shr:2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false));  // row_shr:4
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false));  // row_shr:8
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false));  // row_bcast:15
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  const int I = -1;  // 0xFFFFFFFF, identity of min
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(I, (int)v, 0x111, 0xf, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(I, (int)v, 0x112, 0xf, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(I, (int)v, 0x114, 0xf, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(I, (int)v, 0x118, 0xf, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(I, (int)v, 0x142, 0xa, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(I, (int)v, 0x143, 0xc, 0xf, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Top-k of one token by one wave.  Lane l holds the logits of experts e = l + 64 i as
// orderable keys, sorted in the lane (descending key, ascending id on ties).
//
// Fast path: tau = the k-th largest of the 64 lane maxima is a lower bound on the k-th
// largest key (those k maxima are k keys >= tau), so every selected key is >= tau.
// tau comes from a bitwise search over ballots; the few keys >= tau (about k to 2k for
// N(0,1) logits) are packed into LDS, one per lane, and each is ranked against the
// others by (key descending, id ascending) through lane reads; rank < k is selected.
// If more than 64 keys reach tau (heavy ties), the selection falls back to k rounds of
// a wave-wide arg-max over the lanes' sorted lists.  Both give the same result.
constexpr int kCand = 64;

struct TopkLds {
  uint32_t cand_key[kCand];
  int cand_id[kCand];
  uint32_t sel_key[MOE_MAX_K];
  int sel_id[MOE_MAX_K];
};

template <int VPL>
__device__ __forceinline__ void topk_select_rounds(uint32_t (&key)[VPL], int (&eid)[VPL], int k, TopkLds &S) {
  const int lane = threadIdx.x & 63;
  for (int j = 0; j < k; j++) {
    const uint32_t m = wave_max_u32(key[0]);
    const uint64_t hit = __ballot(key[0] == m);
    int id;
    if (__popcll(hit) == 1)
      id = __builtin_amdgcn_readlane(eid[0], __ffsll((unsigned long long)hit) - 1);
    else
      id = (int)wave_min_u32(key[0] == m ? (uint32_t)eid[0] : 0xFFFFFFFFu);
    if (key[0] == m && eid[0] == id) {
#pragma unroll
      for (int i = 0; i + 1 < VPL; i++) {
        key[i] = key[i + 1];
        eid[i] = eid[i + 1];
      }
      key[VPL - 1] = 0u;
    }
    if (lane == 0) {
      S.sel_key[j] = m;
      S.sel_id[j] = id;
    }
  }
}

// Number of set bits of m in the lanes below this one.
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

template <int VPL>
__device__ __forceinline__ void topk_wave(const float *__restrict__ l, int E, int k, int add_shared,
                                          int32_t *__restrict__ ids, float *__restrict__ w, int32_t *ids_copy,
                                          TopkLds &S) {
  const int lane = threadIdx.x & 63;
  uint32_t key[VPL];
  int eid[VPL];
  float lv[VPL];
  // every lane loads (clamped index), so the loads are issued back to back
#pragma unroll
  for (int i = 0; i < VPL; i++) lv[i] = l[min(i * 64 + lane, E - 1)];
#pragma unroll
  for (int i = 0; i < VPL; i++) {
    const int e = i * 64 + lane;
    key[i] = e < E ? orderable(lv[i]) : 0u;
    eid[i] = e;
  }
#pragma unroll
  for (int i = 1; i < VPL; i++)
#pragma unroll
    for (int j = i; j > 0; j--) {
      const bool swap = key[j] > key[j - 1];  // equal keys keep the lower id first
      const uint32_t tk = swap ? key[j - 1] : key[j];
      const int te = swap ? eid[j - 1] : eid[j];
      key[j - 1] = swap ? key[j] : key[j - 1];
      eid[j - 1] = swap ? eid[j] : eid[j - 1];
      key[j] = tk;
      eid[j] = te;
    }
  // tau: the largest t with at least k lane maxima >= t (the set of such t is closed
  // downwards, so it is found bit by bit from the top).  At least k lanes hold a key.
  uint32_t tau = 0u;
  for (int b = 31; b >= 0; b--) {
    const uint32_t c = tau | (1u << b);
    if (__popcll(__ballot(key[0] >= c)) >= k) tau = c;
  }
  // candidates: keys >= tau (each lane's come first in its sorted list); invalid keys
  // are 0 < tau.  Position = candidates of lower lanes + index in the lane.
  int base = 0, total = 0;
#pragma unroll
  for (int i = 0; i < VPL; i++) {
    const uint64_t m = __ballot(key[i] >= tau);
    base += lanes_below(m);
    total += __popcll(m);
  }
  if (total <= kCand) {
#pragma unroll
    for (int i = 0; i < VPL; i++)
      if (key[i] >= tau) {
        S.cand_key[base + i] = key[i];
        S.cand_id[base + i] = eid[i];
      }
    __builtin_amdgcn_wave_barrier();
    const uint32_t ck = lane < total ? S.cand_key[lane] : 0u;
    const int cid = lane < total ? S.cand_id[lane] : 0x7FFFFFFF;
    int rank = 0;
    for (int j = 0; j < total; j++) {
      const uint32_t ok = (uint32_t)__builtin_amdgcn_readlane((int)ck, j);
      const int oid = __builtin_amdgcn_readlane(cid, j);
      rank += (ok > ck || (ok == ck && oid < cid)) ? 1 : 0;
    }
    if (lane < total && rank < k) {
      S.sel_key[rank] = ck;
      S.sel_id[rank] = cid;
    }
  } else {
    topk_select_rounds<VPL>(key, eid, k, S);
  }
  __builtin_amdgcn_wave_barrier();
  // weights: lane j exponentiates selection j; the sum runs over j in order
  float ex = 0.0f, top = 0.0f;
  int myid = 0;
  if (lane < k) {
    myid = S.sel_id[lane];
    top = from_orderable(S.sel_key[0]);
    ex = expf(__fsub_rn(from_orderable(S.sel_key[lane]), top));
  }
  float sum = 0.0f;
  for (int j = 0; j < k; j++) sum = __fadd_rn(sum, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), j)));
  if (lane < k) {
    ids[lane] = myid;
    w[lane] = __fdiv_rn(ex, sum);
    if (ids_copy) ids_copy[lane] = myid;
  }
  if (add_shared && lane == k) {
    ids[k] = E;
    w[k] = 1.0f;
    if (ids_copy) ids_copy[k] = E;
  }
}

template <int VPL>
__global__ void __launch_bounds__(256) k_topk(const float *__restrict__ logits, int T, int E, int k, int kprime,
                                              int add_shared, int32_t *__restrict__ ids, float *__restrict__ w) {
  __shared__ TopkLds S[4];
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  topk_wave<VPL>(logits + (size_t)t * E, E, k, add_shared, ids + (size_t)t * kprime, w + (size_t)t * kprime,
                 nullptr, S[threadIdx.x >> 6]);
}

// ----------------------------------------------------------------------------- grouping
// Stable counting sort of the n = T * kprime slots by expert id, in one workgroup of
// 16 waves.  Wave w owns a contiguous range of slots.  Pass 1 builds a histogram per
// wave in LDS; an exclusive scan over (expert, wave) in expert-major order gives every
// wave its starting cursor per expert; pass 2 walks the wave's slots 64 at a time and
// ranks each lane among the earlier lanes holding the same expert.  Integer-only and
// order-defined, so the output is unique and identical run to run.

constexpr int kGroupWaves = 16;

struct GroupLds {
  int hist[kGroupWaves][MOE_MAX_IDS];
  int offs[MOE_MAX_IDS];
  int arank[MOE_MAX_IDS];
  int wave_tot[kGroupWaves];
  int total;
};

__device__ __forceinline__ int block_exclusive_scan(int v, GroupLds &S) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int n = __shfl_up(inc, o, 64);
    if (lane >= o) inc += n;
  }
  if (lane == 63) S.wave_tot[wave] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int i = 0; i < kGroupWaves; i++) {
      int c = S.wave_tot[i];
      S.wave_tot[i] = run;
      run += c;
    }
    S.total = run;
  }
  __syncthreads();
  int r = S.wave_tot[wave] + inc - v;
  __syncthreads();
  return r;
}

// ids: global or LDS.  Must be called by all 1024 threads.
__device__ void group_block(const int32_t *ids, int n, int n_ids, int32_t *__restrict__ counts,
                            int32_t *__restrict__ offsets, int32_t *__restrict__ sorted_slot,
                            int32_t *__restrict__ slot_pos, WorkRec *__restrict__ work, GroupLds &S) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int per = (((n + kGroupWaves - 1) / kGroupWaves) + 63) / 64 * 64;
  const int lo = wave * per, hi = min(n, lo + per);

  for (int i = threadIdx.x; i < kGroupWaves * MOE_MAX_IDS; i += blockDim.x) (&S.hist[0][0])[i] = 0;
  __syncthreads();
  for (int s = lo + lane; s < hi; s += 64) {
    int e = ids[s];
    if (e >= 0 && e < n_ids) atomicAdd(&S.hist[wave][e], 1);
  }
  __syncthreads();
  const int e = threadIdx.x;  // n_ids <= MOE_MAX_IDS == blockDim.x
  int c = 0;
  if (e < n_ids) {
    for (int w = 0; w < kGroupWaves; w++) {
      int h = S.hist[w][e];
      S.hist[w][e] = c;
      c += h;
    }
  }
  const int excl = block_exclusive_scan(c, S);
  const int n_total = S.total;
  const bool wide = c > MOE_MATVEC_MAX_TOKENS;
  const int tiles = wide ? (c + MOE_MFMA_TILE_TOKENS - 1) / MOE_MFMA_TILE_TOKENS : 0;
  const int nex = block_exclusive_scan(c > 0 && !wide ? 1 : 0, S);
  const int n_narrow = S.total;
  block_exclusive_scan(wide ? 1 : 0, S);
  const int n_wide = S.total;
  const int tex = block_exclusive_scan(tiles, S);
  const int n_tiles = S.total;
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
  __syncthreads();
  if (e < n_ids)
    for (int w = 0; w < kGroupWaves; w++) S.hist[w][e] += S.offs[e];
  __syncthreads();

  for (int base = lo; base < hi; base += 64) {
    int s = base + lane;
    int my = -1;
    if (s < hi) {
      int v = ids[s];
      my = (v >= 0 && v < n_ids) ? v : -1;
    }
    int rank = 0, tot = 0;
    for (int j = 0; j < 64; j++) {
      int ej = __builtin_amdgcn_readlane(my, j);
      if (ej == my) {
        tot++;
        rank += j < lane ? 1 : 0;
      }
    }
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
  group_block(ids, T * kprime, n_ids, counts, offsets, sorted_slot, slot_pos, work, S);
}

// Grouping of at most 64 slots (decode): the same outputs as group_block, computed
// from lane reads of the slot ids, with no LDS traffic and no barrier.  Wave 0 ranks
// every slot among the others (stable: by id, then slot index) and writes the work
// records; every thread e counts the slots below and at its id.
constexpr int kTinySlots = 64;

__device__ void group_tiny(const int32_t *ids_l, int n, int n_ids, int32_t *__restrict__ counts,
                           int32_t *__restrict__ offsets, int32_t *__restrict__ sorted_slot,
                           int32_t *__restrict__ slot_pos, WorkRec *__restrict__ work) {
  const int lane = threadIdx.x & 63;
  const int my = lane < n ? ids_l[lane] : 0x7FFFFFFF;
  if (threadIdx.x < 64) {
    int rank = 0, same = 0, first = 1;
    for (int j = 0; j < n; j++) {
      const int o = __builtin_amdgcn_readlane(my, j);
      rank += (o < my || (o == my && j < lane)) ? 1 : 0;
      same += o == my ? 1 : 0;
      first &= (o == my && j < lane) ? 0 : 1;
    }
    const bool wide = same > MOE_MATVEC_MAX_TOKENS;
    const uint64_t firsts = __ballot(lane < n && first);
    const uint64_t wides = __ballot(lane < n && first && wide);
    // first set: distinct experts below mine; tiles: the tiles of wide experts below mine
    int below = 0, tiles_below = 0, n_tiles = 0;
    for (int j = 0; j < n; j++) {
      const int oj = __builtin_amdgcn_readlane(my, j), sj = __builtin_amdgcn_readlane(same, j);
      const bool fj = (firsts >> j) & 1u, wj = (wides >> j) & 1u;
      const int tj = (sj + MOE_MFMA_TILE_TOKENS - 1) / MOE_MFMA_TILE_TOKENS;
      if (fj && oj < my) {
        if (wj)
          tiles_below += tj;
        else
          below++;
      }
      n_tiles += wj ? tj : 0;
    }
    if (lane < n) {
      sorted_slot[rank] = lane;
      slot_pos[lane] = rank;
      if (first && !wide) work[1 + below] = WorkRec{my, rank, rank + same, lane};
      if (first && wide)
        for (int p = 0; p < same; p += MOE_MFMA_TILE_TOKENS)
          work[n_ids + 1 + tiles_below + p / MOE_MFMA_TILE_TOKENS] =
              WorkRec{my, rank + p, rank + min(same, p + MOE_MFMA_TILE_TOKENS), 0};
    }
    if (lane == 0) {
      offsets[n_ids] = n;
      const int n_wide = (int)__popcll(wides);
      work[0] = WorkRec{(int)__popcll(firsts) - n_wide, n, n_wide, n_tiles};
    }
  }
  for (int e = threadIdx.x; e < n_ids; e += blockDim.x) {
    int below = 0, at = 0;
    for (int j = 0; j < n; j++) {
      const int o = __builtin_amdgcn_readlane(my, j);
      below += o < e ? 1 : 0;
      at += o == e ? 1 : 0;
    }
    counts[e] = at;
    offsets[e] = below;
  }
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
                   ids_l + t * kprime, TS[wave]);
  __syncthreads();
  if (T * kprime <= kTinySlots)
    group_tiny(ids_l, T * kprime, E + add_shared, counts, offsets, sorted_slot, slot_pos, work);
  else
    group_block(ids_l, T * kprime, E + add_shared, counts, offsets, sorted_slot, slot_pos, work, S);
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
