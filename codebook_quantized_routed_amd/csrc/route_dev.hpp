// Device functions of the router top-k and of the grouping of a few slots, shared by
// the routing kernels and the fused decode-layer kernel.
#pragma once
#include "common.hpp"

namespace moe {

// Float -> u32 with the order of IEEE comparison: key = 2^31 + m for +m and 2^31 - m for
// -m (m = the magnitude bits), so -0.0 and +0.0 share the key 2^31 and tie, as they
// compare equal (the tie then goes to the lower id).  Every finite value maps above
// 0x007FFFFF, so 0 can stand for "taken / no value".
__device__ __forceinline__ uint32_t orderable(float f) {
  const uint32_t b = __float_as_uint(f), m = b & 0x7FFFFFFFu;
  return (b & 0x80000000u) ? 0x80000000u - m : 0x80000000u + m;
}
// The inverse (a zero key gives +0.0, which behaves as -0.0 in every use of it here).
__device__ __forceinline__ float from_orderable(uint32_t k) {
  return __uint_as_float(k >= 0x80000000u ? k - 0x80000000u : (0x80000000u - k) | 0x80000000u);
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
// orderable keys (no order within the lane).
//
// Fast path: tau = the k-th largest of the 64 lane maxima is a lower bound on the k-th
// largest key (those k maxima are k keys >= tau), so every selected key is >= tau.
// tau comes from a bitwise search over ballots; the few keys >= tau (about k to 2k for
// N(0,1) logits) are packed into LDS, one per lane, and each is ranked against the
// others by (key descending, id ascending) from broadcast LDS reads; rank < k is selected.
// If more than 64 keys reach tau (heavy ties), the selection falls back to k rounds of
// a wave-wide arg-max.  Both give the same result.
// Outputs: ids / w (global, skipped when ids is null) and the optional copies; returns
// the lane's slot (TopkSlot).
constexpr int kCand = 64;

struct TopkLds {
  // candidate j: (key << 32) | ~id, so one unsigned compare orders by (key descending,
  // id ascending)
  alignas(16) uint64_t cand[kCand];
  uint32_t sel_key[MOE_MAX_K];
  int sel_id[MOE_MAX_K];
  int sel_pos[MOE_MAX_K];
};

// A lane's slot after the top-k.  Lane j < k: selection j, with its expert id, its
// position among the token's slots in ascending expert id, and its router weight; lane k
// with a shared expert: id E, position k (E is above every routed id), weight 1; other
// lanes: id 0x7FFFFFFF, position -1.
struct TopkSlot {
  int id, pos;
  float w;
};

// k rounds of: the largest remaining key, ties to the lowest expert id; the winner is
// removed (key 0 = taken / no value).
template <int VPL>
__device__ __forceinline__ void topk_select_rounds(uint32_t (&key)[VPL], int k, TopkLds &S) {
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));
  for (int j = 0; j < k; j++) {
    uint32_t lmax = key[0];
#pragma unroll
    for (int i = 1; i < VPL; i++) lmax = max(lmax, key[i]);
    const uint32_t m = wave_max_u32(lmax);
    uint32_t lid = 0xFFFFFFFFu;  // the lane's lowest id holding m
#pragma unroll
    for (int i = VPL - 1; i >= 0; i--)
      if (key[i] == m) lid = (uint32_t)(i * 64 + lane);
    const int id = (int)wave_min_u32(lid);
#pragma unroll
    for (int i = 0; i < VPL; i++)
      if (i * 64 + lane == id) key[i] = 0u;
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

// The token's logits as lane l holds them (experts l + 64 i); every lane loads (clamped
// index), so the loads are issued back to back.
template <int VPL>
struct TopkVals {
  float v[VPL];
};

template <int VPL>
__device__ __forceinline__ TopkVals<VPL> topk_load(const float *__restrict__ l, int E) {
  // hidden from loop-invariant code motion (a kernel that routes in a loop would keep
  // every lane address and bound live across the loop)
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));
  TopkVals<VPL> t;
#pragma unroll
  for (int i = 0; i < VPL; i++) t.v[i] = l[min(i * 64 + lane, E - 1)];
  return t;
}

// TAU_BITS: bits of tau per search step (1, 2 or 4).  Fewer steps shorten the chain of
// ballot -> scalar count -> select, more ballots per step cost issue slots: one bit is
// the faster where the wave has its SIMD mostly to itself, two where it shares it with
// busy waves (the next layer's routing inside the stack kernel).  TAU_LOW: tau's bits
// below this one are not searched (stay zero); every caller takes 16, measured the
// faster (or as fast) in each kernel.  The selection is the same.
//
// topk_choose makes the selection and leaves it in S: sel_key / sel_id / sel_pos by rank
// (rank j = slot j; sel_pos = the position in ascending expert id); topk_weights then
// computes the router weights from it.
template <int VPL, int TAU_BITS = 1, int TAU_LOW = 0>
__device__ __forceinline__ void topk_choose(const TopkVals<VPL> &tv, int E, int k, TopkLds &S) {
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));
  uint32_t key[VPL], lmax = 0u;
#pragma unroll
  for (int i = 0; i < VPL; i++) {
    key[i] = i * 64 + lane < E ? orderable(tv.v[i]) : 0u;
    lmax = max(lmax, key[i]);
  }
  // tau: the largest t whose low TAU_LOW bits are zero with at least k lane maxima
  // >= t (the set of such t is closed downwards, so it is found from the top, TAU_BITS
  // bits per step: the count of the 2^TAU_BITS - 1 nonzero digits that keep at least k
  // maxima is the largest such digit, and their ballots are independent of each other).
  // It is at most the k-th largest lane maximum, so still a lower bound on the k-th
  // largest key; the low bits would only trim the candidates (stopping at bit 16, after
  // the sign, the exponent and 7 mantissa bits, leaves about one more for normal
  // logits).  At least k lanes hold a key.
  static_assert(TAU_BITS == 1 || TAU_BITS == 2 || TAU_BITS == 4, "tau digits must tile the searched bits");
  static_assert((32 - TAU_LOW) % TAU_BITS == 0, "tau digits must tile the searched bits");
  uint32_t tau = 0u;
#pragma unroll
  for (int sh = 32 - TAU_BITS; sh >= TAU_LOW; sh -= TAU_BITS) {
    uint32_t digit = 0u;
#pragma unroll
    for (uint32_t j = 1; j < (1u << TAU_BITS); j++) digit += __popcll(__ballot(lmax >= (tau | (j << sh)))) >= k ? 1u : 0u;
    tau |= digit << sh;
  }
  // candidates: keys >= tau (invalid keys are 0 < tau), packed in (i, lane) order
  int pos[VPL], total = 0;
#pragma unroll
  for (int i = 0; i < VPL; i++) {
    const uint64_t m = __ballot(key[i] >= tau);
    pos[i] = total + lanes_below(m);
    total += (int)__popcll(m);
  }
  if (total <= kCand) {
#pragma unroll
    for (int i = 0; i < VPL; i++)
      if (key[i] >= tau) S.cand[pos[i]] = ((uint64_t)key[i] << 32) | (uint32_t)~(uint32_t)(i * 64 + lane);
    __builtin_amdgcn_wave_barrier();
    // each lane ranks its candidate against all of them, two per 16-byte read (every
    // lane reads the same address: one broadcast read), four reads issued back to back
    // per trip (j0 <= 56, so j0 + 7 stays within the 64 entries; entries at or past
    // total are not counted)
    const uint64_t mine = lane < total ? S.cand[lane] : 0u;
    int rank = 0;
    for (int j0 = 0; j0 < total; j0 += 8) {
      uint4 pr[4];
#pragma unroll
      for (int u = 0; u < 4; u++) pr[u] = *(const uint4 *)&S.cand[j0 + 2 * u];
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const int j = j0 + 2 * u;
        rank += (j < total && (((uint64_t)pr[u].y << 32) | pr[u].x) > mine) ? 1 : 0;
        rank += (j + 1 < total && (((uint64_t)pr[u].w << 32) | pr[u].z) > mine) ? 1 : 0;
      }
    }
    // the candidates are packed in ascending expert id, so a selected candidate's
    // position among the selected ids is the count of selected candidates before it
    const bool chosen = lane < total && rank < k;
    const int pos = lanes_below(__ballot(chosen));
    if (chosen) {
      S.sel_key[rank] = (uint32_t)(mine >> 32);
      S.sel_id[rank] = (int)~(uint32_t)mine;
      S.sel_pos[rank] = pos;
    }
  } else {
    topk_select_rounds<VPL>(key, k, S);
    __builtin_amdgcn_wave_barrier();
    // positions in ascending expert id by counting (the ids are distinct)
    const int sid = lane < k ? S.sel_id[lane] : 0x7FFFFFFF;
    int pos = 0;
    for (int j = 0; j < k; j++) pos += __builtin_amdgcn_readlane(sid, j) < sid ? 1 : 0;
    if (lane < k) S.sel_pos[lane] = pos;
  }
}

__device__ __forceinline__ TopkSlot topk_weights(int E, int k, int add_shared, int32_t *__restrict__ ids,
                                                 float *__restrict__ w, int32_t *ids_copy, float *w_copy,
                                                 const TopkLds &S) {
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));
  // weights: lane j exponentiates selection j; the sum runs over j in order
  float ex = 0.0f, top = 0.0f;
  int myid = 0, mypos = -1;
  if (lane < k) {
    myid = S.sel_id[lane];
    mypos = S.sel_pos[lane];
    top = from_orderable(S.sel_key[0]);
    ex = expf(__fsub_rn(from_orderable(S.sel_key[lane]), top));
  }
  // the sum in selection order; lanes k.. hold +0, which leaves the (positive) sum as it
  // is, so the loop runs over the largest k, unrolled, with its lane reads back to back
  float sum = 0.0f;
#pragma unroll
  for (int j = 0; j < MOE_MAX_K; j++) sum = __fadd_rn(sum, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), j)));
  float wl = 0.0f;
  if (lane < k) {
    wl = __fdiv_rn(ex, sum);
    if (ids) {
      ids[lane] = myid;
      w[lane] = wl;
    }
    if (ids_copy) ids_copy[lane] = myid;
    if (w_copy) w_copy[lane] = wl;
  }
  if (add_shared && lane == k) {
    if (ids) {
      ids[k] = E;
      w[k] = 1.0f;
    }
    if (ids_copy) ids_copy[k] = E;
    if (w_copy) w_copy[k] = 1.0f;
  }
  if (lane < k) return TopkSlot{myid, mypos, wl};
  if (add_shared && lane == k) return TopkSlot{E, k, 1.0f};
  return TopkSlot{0x7FFFFFFF, -1, 0.0f};
}

template <int VPL, int TAU_BITS = 1, int TAU_LOW = 0>
__device__ __forceinline__ TopkSlot topk_select(const TopkVals<VPL> &tv, int E, int k, int add_shared,
                                            int32_t *__restrict__ ids, float *__restrict__ w, int32_t *ids_copy,
                                            float *w_copy, TopkLds &S) {
  topk_choose<VPL, TAU_BITS, TAU_LOW>(tv, E, k, S);
  __builtin_amdgcn_wave_barrier();
  return topk_weights(E, k, add_shared, ids, w, ids_copy, w_copy, S);
}

template <int VPL>
__device__ __forceinline__ void topk_wave(const float *__restrict__ l, int E, int k, int add_shared,
                                          int32_t *__restrict__ ids, float *__restrict__ w, int32_t *ids_copy,
                                          float *w_copy, TopkLds &S) {
  topk_select<VPL, 1, 16>(topk_load<VPL>(l, E), E, k, add_shared, ids, w, ids_copy, w_copy, S);
}

// Grouping of at most 64 slots (decode): the same outputs as group_block, computed
// from lane reads of the slot ids, with no LDS traffic and no barrier.  Wave 0 ranks
// every slot among the others (stable: by id, then slot index) and writes the work
// records; every thread e counts the slots below and at its id.
constexpr int kTinySlots = 64;

__device__ inline void group_tiny(const int32_t *ids_l, int n, int n_ids, int max_narrow, int32_t *__restrict__ counts,
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
    const bool wide = same > max_narrow;
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

}  // namespace moe
