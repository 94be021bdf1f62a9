// The whole decode step of one layer for one token in a single launch.
//
// "Red Metal dev8 — resident routed top-k layer", steps 3-6: the router selects the
// experts, each selected expert runs gate, up, SiLU(gate) * up and down, and the
// outputs are accumulated as acc += router_weight * expert_output in one command, with
// only the final output leaving the layer.  Here that command is one kernel:
//
//  1. every workgroup selects the same experts (top-k of the token's logits, or the
//     caller's explicit list) -- no exchange is needed for routing; the routing
//     outputs of moe_route_group are written by a wave with no down work meanwhile;
//  2. gate / up items (2 rows of one expert) are dealt to the waves of the whole grid,
//     the items of the first sorted positions to the waves of the highest issue
//     priority; each h value goes to global memory in sorted order, paired with the
//     call's tag in one 64-bit agent-scope atomic store;
//  3. down + the weighted accumulation in ascending expert id for the workgroup's
//     block of output rows: a wave reads the h row of its sorted position as soon as
//     its own gate / up work is done, and reads again the values whose tag is not yet
//     the call's (their writers have not finished), so no grid-wide barrier is needed.
// The call's tag comes from a per-call count: each workgroup adds one to its group's
// counter at the start, and every launch on a device has the same number of
// workgroups, so each call moves every counter by exactly one round.
// The arithmetic of every step is the one of moe_route_group, moe_expert_gateup_q and
// moe_expert_down_accumulate_q, so the results are the same bits.
//
// The wait for h is bounded: if an h value never gets the call's tag (which needs a
// workgroup that never runs, i.e. another kernel holding compute units meanwhile), the
// waiting wave gives up after about a second, sets the error word and finishes; the
// results of that call are then undefined.
//
// The second kernel of this file, k_stack_decode, runs the decode step of a whole chain
// of layers (RMSNorm, this layer, residual) in one launch with the same machinery.
#include "gemv_dev.hpp"
#include "route_dev.hpp"

namespace moe {

constexpr int kFusedWaves = 12;
// waves that take a slot each in the down phase (in the stack kernel the last wave
// routes the next layer meanwhile)
constexpr int kDownWaves = kFusedWaves - 1;
constexpr int kFusedMaxSlots = MOE_MAX_K + 1;

// Position of the lane's slot among the token's slots in (expert id, slot) order, from
// the expert ids held one per lane (lanes past the last slot hold 0x7FFFFFFF, which no
// slot counts).  Unrolled over the largest slot count, so the lane reads issue back to
// back instead of one per loop trip.
__device__ __forceinline__ int slot_rank(int my, int lane) {
  int rank = 0;
#pragma unroll
  for (int j = 0; j < kFusedMaxSlots; j++) {
    const int o = __builtin_amdgcn_readlane(my, j);
    rank += (o < my || (o == my && j < lane)) ? 1 : 0;
  }
  return rank;
}
constexpr int kFusedSlotsPerWave = (kFusedMaxSlots + kDownWaves - 1) / kDownWaves;
constexpr int kSpinLimit = 1 << 20;  // polls of a few hundred ns: a fraction of a second

// Workspace of the fused call: the synchronisation words, then h [kprime][inter] as
// 64-bit (value bits, tag) pairs.  Workgroup g counts calls on the counter of its group
// g / kBarGroup (counters in separate 128-byte lines, so few workgroups share one);
// error is set if a wait timed out.
constexpr int kBarGroup = 16;
constexpr int kBarGroups = 32;  // up to 512 workgroups
struct FusedSync {
  uint64_t reserved[16];
  uint32_t error, pad1[31];
  struct Line {
    uint64_t count, pad[15];
  } group[kBarGroups];
};
static_assert(sizeof(FusedSync) == 4352, "h follows the synchronisation words");
static_assert(offsetof(FusedSync, error) == 128 && offsetof(FusedSync, group) == 256, "documented offsets");

// Activations staged in LDS: lane l of a wave takes columns 32 l .. 32 l + 31 (hidden
// 2048), stored at l * kXsRow floats (the padding spreads the lanes over the banks).
constexpr int kXsRow = 36;

// The expert at one sorted position: its id, slot and bank.
struct PosRec {
  int32_t e, slot, bank, pad;
};

struct FusedLds {
  BankLds banks[MOE_MAX_BANKS];
  PosRec pos[kFusedMaxSlots];          // sorted position p -> its expert
  TopkLds topk;
  int32_t ids[kFusedMaxSlots];         // slot j -> expert
  float w[kFusedMaxSlots];             // slot j -> router weight
  int32_t slot_at[kFusedMaxSlots];     // sorted position p -> slot
  float wpos[kFusedMaxSlots];          // sorted position p -> router weight
  float ydot[kFusedMaxSlots][16];      // down outputs of the block's rows, per sorted position
  float xs[64 * kXsRow];               // the token's activations, lane l's 32 at l * kXsRow
  uint32_t tag;                        // the call's tag
};

__host__ __device__ inline size_t fused_stage_floats(int lpr) {
  return (size_t)kFusedWaves * lpr * kChunkPad;
}

// The call's tag (nonzero): one more than the number of earlier calls, from this
// workgroup's count on its group's counter.
__device__ inline uint32_t call_tag(FusedSync *s) {
  const uint32_t g = blockIdx.x / kBarGroup, n = gridDim.x;
  const uint32_t size = min((uint32_t)kBarGroup, n - g * kBarGroup);
  const uint64_t prev =
      __hip_atomic_fetch_add(&s->group[g].count, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return (uint32_t)(prev / size) + 1u;
}

// The h row of one slot (I pairs) into a wave's LDS area as floats (64-value chunks
// padded to kChunkPad floats): lane l takes pairs l, l + 64, ...; pairs whose tag is
// not yet the call's are read again after a pause, a bounded number of times.
template <int LPR>
__device__ inline void stage_h_row(const uint64_t *src, uint32_t tag, float *hs, FusedSync *s) {
  const int lane = threadIdx.x & 63;
  uint64_t v[LPR];
#pragma unroll
  for (int i = 0; i < LPR; i++) v[i] = __hip_atomic_load(src + lane + 64 * i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int spin = 0;; spin++) {
    bool ok = true;
#pragma unroll
    for (int i = 0; i < LPR; i++) ok = ok && (uint32_t)(v[i] >> 32) == tag;
    if (__ballot(!ok) == 0ull) break;
    if (spin == kSpinLimit) {
      if (lane == 0) __hip_atomic_store(&s->error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
#pragma unroll
    for (int i = 0; i < LPR; i++)
      if ((uint32_t)(v[i] >> 32) != tag)
        v[i] = __hip_atomic_load(src + lane + 64 * i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
#pragma unroll
  for (int i = 0; i < LPR; i++) hs[i * kChunkPad + lane] = __uint_as_float((uint32_t)v[i]);
}

// True when a matrix of format qt is IQ2_XS-like, decided at compile time when the
// kernel instance serves one format only.
template <int FMT>
__device__ __forceinline__ bool fmt_iq2(int qt) {
  return FMT == MOE_Q_IQ2XS_LIKE || (FMT != MOE_Q_IQ1M_LIKE && qt == MOE_Q_IQ2XS_LIKE);
}

// FMT: the layer's formats (MOE_Q_* bits), a template parameter so that a layer of one
// format runs an instance without the other format's code.
template <int LPR, int FMT>
__global__ void __launch_bounds__(64 * kFusedWaves) k_layer_decode(LayerArgs L, const float *__restrict__ logits,
                                                                    const float *__restrict__ x, int E, int k,
                                                                    int add_shared, int32_t *__restrict__ ids,
                                                                    float *__restrict__ w, int32_t *__restrict__ counts,
                                                                    int32_t *__restrict__ offsets,
                                                                    int32_t *__restrict__ sorted_slot,
                                                                    int32_t *__restrict__ slot_pos,
                                                                    WorkRec *__restrict__ work, float *__restrict__ acc,
                                                                    FusedSync *__restrict__ sync) {
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ FusedLds S;
  constexpr int RPP = 64 / LPR, HS = LPR * kChunkPad;
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
  const int kprime = k + add_shared, n_ids = E + add_shared;
  const int H = L.hidden, I = L.inter;
  uint64_t *h = (uint64_t *)(sync + 1);
  constexpr int formats = FMT;
  const TableLayout TL = table_layout(formats, kTabIq1 | kTabIq1Delta);
  float *hs = (float *)(lds + TL.bytes) + wave * HS;
  // wave 0's logits are the first loads of the kernel; the table rows are loaded by
  // waves 1.. while wave 0 routes (vector loads complete in order)
  TopkVals<8> tv;
  if (wave == 0 && logits) tv = topk_load<8>(logits, E);
  const TableRegs tr = tables_load(L.grids, formats, threadIdx.x - 64, blockDim.x - 64);
  uint32_t tag = 0;
  if (threadIdx.x == 64) tag = call_tag(sync);
  // waves 1..: the activations, one float4 per thread (hidden 2048), staged in LDS with
  // the tables (loading each wave's slice from global memory instead was measured 0.6 us
  // slower)
  const int xt = threadIdx.x - 64;
  float4 xv;
  if (xt >= 0 && xt < 512) xv = ((const float4 *)x)[xt];

  // ---- 1. routing, in every workgroup, by wave 0; the other waves expand the grid
  // tables into LDS meanwhile
  if (wave == 0) {
    if (logits) {
      // the selection only: the router weights are needed by the accumulation alone,
      // so they are computed later, while the wave waits for h
      topk_choose<8, 1, 16>(tv, E, k, S.topk);
    } else {
      if (lane < k) {
        S.ids[lane] = ids[lane];
        S.w[lane] = w[lane];
      }
      if (add_shared && lane == k) {
        S.ids[k] = E;
        S.w[k] = 1.0f;
        if (blockIdx.x == 0) {
          ids[k] = E;
          w[k] = 1.0f;
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
    // routed: slot j's expert and position as the selection left them (the shared
    // expert last); explicit: as copied to LDS above, positions by counting
    const bool shared_lane = add_shared && lane == k;
    const int my = logits ? (lane < k ? S.topk.sel_id[lane] : (shared_lane ? E : 0x7FFFFFFF))
                          : (lane < kprime ? S.ids[lane] : 0x7FFFFFFF);
    const int rank = logits ? (lane < k ? S.topk.sel_pos[lane] : (shared_lane ? k : -1)) : slot_rank(my, lane);
    if (lane < kprime) {
      if (logits) S.ids[lane] = my;
      S.slot_at[rank] = lane;
      S.pos[rank] = PosRec{my, lane, bank_index(L, my), 0};
      if (!logits) S.wpos[rank] = S.w[lane];
    }
  } else {
    tables_store(tr, formats, TL, lds, threadIdx.x - 64, blockDim.x - 64, false);
    if (xt >= 0 && xt < 512) *(float4 *)&S.xs[(xt >> 3) * kXsRow + (xt & 7) * 4] = xv;
    if (threadIdx.x == 64) {
      S.tag = tag;
      fill_banks(L, S.banks);
    }
  }
  __syncthreads();
  tag = S.tag;

  // ---- 2. gate / up items dealt over the grid's waves (at most one per wave when the
  // grid has as many waves as items): the wave's first item is issued before anything
  // waits, its activations come from LDS; later items are issued one at a time
  const int q = lane, lq = lane % LPR, sub = lane / LPR;
  constexpr int ipe = 64 * LPR / kWideRows;  // items per expert (inter = 64 LPR rows)
  const int n_items = kprime * ipe, nw = gridDim.x * kFusedWaves;
  // wave w of workgroup b takes item (w / 4) G + 4 b + w % 4 (G = 4 x grid): the waves
  // w / 4 = g of the grid (one per SIMD) hold the items of positions 4g .. 4g + 3
  const int item0 = (wave >> 2) * (4 * (int)gridDim.x) + blockIdx.x * 4 + (wave & 3);
  WideItem It;
  int cur_tok = 0;
  // the bank's bases and sizes come from the kernel arguments (scalar loads), so the
  // only LDS read before the loads leave is the position's record
  auto issue_bank = [&](const BankArgs &B, int e, int p, int slot, int item) {
    It.W = WorkRec{e, p, p + 1, slot};
    const QMat Wg = global_mat(expert_mat(B, e, kGate, I, H)), Wu = global_mat(expert_mat(B, e, kUp, I, H));
    if constexpr (FMT == MOE_Q_IQ2XS_LIKE || FMT == MOE_Q_IQ1M_LIKE)
      wide_issue_fmt<FMT>(It, Wg, Wu, H, item - p * ipe, q);
    else
      wide_issue_mats(It, Wg, Wu, uniform(B.qtype), H, item - p * ipe, q);
  };
  // a layer of one bank (the usual layout) addresses its experts from fixed argument
  // offsets, which the scalar loads can fetch before the expert is known
  auto issue = [&](int item) {
    const int p = item / ipe;
    const int e = uniform(S.pos[p].e), slot = uniform(S.pos[p].slot);
    if (L.n_banks == 1)
      issue_bank(L.banks[0], e, p, slot, item);
    else
      issue_bank(bank_of(L, e), e, p, slot, item);
  };
  // the first item's loads leave before the activations are read from LDS (its
  // addresses need only the routing records)
  if (item0 < n_items) issue(item0);
  // on each SIMD the wave of the lowest positions goes first, so those positions' h rows
  // are complete early and their down dots overlap the other waves' gate / up
  if (wave < 4)
    __builtin_amdgcn_s_setprio(3);
  else if (wave < 8)
    __builtin_amdgcn_s_setprio(2);
  else
    __builtin_amdgcn_s_setprio(1);
  X32 X;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const float4 f = *(const float4 *)&S.xs[lane * kXsRow + 4 * i];
    X.v[4 * i] = f.x, X.v[4 * i + 1] = f.y, X.v[4 * i + 2] = f.z, X.v[4 * i + 3] = f.w;
  }
  for (int item = item0; item < n_items; item += nw) {
    if (item != item0) issue(item);
    if (fmt_iq2<FMT>(It.qt))
      wide_run<MOE_Q_IQ2XS_LIKE, true>(L, It, X, cur_tok, q, kprime, XSource{x, H, 32}, sorted_slot, lds, TL, h, tag);
    else
      wide_run<MOE_Q_IQ1M_LIKE, true>(L, It, X, cur_tok, q, kprime, XSource{x, H, 32}, sorted_slot, lds, TL, h, tag);
  }

  // ---- the grouping outputs of moe_route_group (one token: every count is 0 or 1),
  // from the last wave, which takes no down position, while the others run the down
  // phase: counts and offsets spread over the workgroups, the rest from workgroup 0
  if (wave == kFusedWaves - 1) {
    for (int e = blockIdx.x + gridDim.x * lane; e < n_ids; e += gridDim.x * 64) {
      int below = 0, at = 0;
      for (int j = 0; j < kprime; j++) {
        below += S.ids[j] < e ? 1 : 0;
        at += S.ids[j] == e ? 1 : 0;
      }
      counts[e] = at;
      offsets[e] = below;
    }
    if (blockIdx.x == 0 && lane < kprime) {
      const int p = lane, slot = S.slot_at[p];
      sorted_slot[p] = slot;
      slot_pos[slot] = p;
      work[1 + p] = WorkRec{S.ids[slot], p, p + 1, slot};
      if (p == 0) {
        offsets[n_ids] = kprime;
        work[0] = WorkRec{kprime, kprime, 0, 0};
      }
    }
  }

  // ---- 3. the down rows of the wave's first sorted position (position = wave) in the
  // workgroup's first block, and its acc values, are loaded as soon as the wave's
  // gate / up work is done
  const int tiles = H / RPP;
  int tile = blockIdx.x;
  const bool down_wave = wave < kDownWaves;
  RowRaw Rd0;
  int dqt0 = 0;
  if (down_wave && wave < kprime && tile < tiles) {
    const PosRec &P = S.pos[wave];
    const BankLds &B = S.banks[uniform(P.bank)];
    const QMat Wd = bank_mat(B, uniform(P.e), kDown);
    dqt0 = uniform(B.qt);
    Rd0 = fmt_iq2<FMT>(dqt0) ? load_row<MOE_Q_IQ2XS_LIKE>(Wd, I, tile * RPP + sub, lq)
                                   : load_row<MOE_Q_IQ1M_LIKE>(Wd, I, tile * RPP + sub, lq);
  }
  float acc_in = 0.0f;
  if (threadIdx.x < RPP && tile < tiles) acc_in = acc[tile * RPP + threadIdx.x];
  // wave 0: the router weights of the selection (the arithmetic of topk_select), read
  // by the accumulation after the down phase's barrier
  if (wave == 0 && logits) {
    const TopkSlot ts = topk_weights(E, k, add_shared, blockIdx.x == 0 ? ids : nullptr, w, nullptr, nullptr, S.topk);
    if (lane < kprime) S.wpos[ts.pos] = ts.w;
  }

  // ---- 4. down + accumulation, block by block of RPP output rows; a wave takes the
  // sorted positions wave, wave + kDownWaves, ... one after the other
  for (bool first = true; tile < tiles; tile += gridDim.x, first = false) {
#pragma unroll 1
    for (int i = 0; i < kFusedSlotsPerWave; i++) {
      const int pj = wave + kDownWaves * i;  // sorted position
      if (!down_wave || pj >= kprime) break;
      RowRaw R;
      int qt;
      if (first && i == 0) {
        R = Rd0;
        qt = dqt0;
      } else {
        const PosRec &P = S.pos[pj];
        const BankLds &B = S.banks[uniform(P.bank)];
        const QMat Wd = bank_mat(B, uniform(P.e), kDown);
        qt = uniform(B.qt);
        R = fmt_iq2<FMT>(qt) ? load_row<MOE_Q_IQ2XS_LIKE>(Wd, I, tile * RPP + sub, lq)
                                   : load_row<MOE_Q_IQ1M_LIKE>(Wd, I, tile * RPP + sub, lq);
      }
      // the slot's h row (written by other workgroups) into the wave's LDS area
      stage_h_row<LPR>(h + (size_t)pj * I, tag, hs, sync);
      __builtin_amdgcn_wave_barrier();
      const float *hrow = hs + lq * kChunkPad;
      const float v = fmt_iq2<FMT>(qt) ? down_slot_dot<MOE_Q_IQ2XS_LIKE, LPR>(R, hrow, lq, lds, TL)
                                             : down_slot_dot<MOE_Q_IQ1M_LIKE, LPR>(R, hrow, lq, lds, TL);
      if (lq == 0) S.ydot[pj][sub] = v;
      __builtin_amdgcn_wave_barrier();  // the staging area is reused by the next slot
    }
    __syncthreads();
    if (threadIdx.x < RPP) {
      // acc += w * y over the sorted positions, i.e. in ascending expert id; every
      // operand is read before the first add (positions past the last slot are read and
      // not used), so the reads overlap instead of forming a chain
      const int r = tile * RPP + threadIdx.x;
      float wv[kFusedMaxSlots], yv[kFusedMaxSlots];
#pragma unroll
      for (int p = 0; p < kFusedMaxSlots; p++) {
        wv[p] = S.wpos[p];
        yv[p] = S.ydot[p][threadIdx.x];
      }
      float a = first ? acc_in : acc[r];
#pragma unroll
      for (int p = 0; p < kFusedMaxSlots; p++)
        if (p < kprime) a = __fadd_rn(a, __fmul_rn(wv[p], yv[p]));
      acc[r] = a;
    }
    __syncthreads();
  }
}

// ============================================================================ stack
// The decode step of a stack of layers for one token in a single launch:
// h <- h + MoE_l(RMSNorm(h)) for l = 0 .. L-1 ("Red Lite dev16 — complete
// full-attention parity", section "Pinned full-attention graph": the routed MoE follows
// the post-attention RMSNorm and feeds the residual stream; section "Scope boundary":
// the 48-layer scheduler is the next gate).  Per layer, every workgroup:
//  1. stages the layer's input residual (layer 0: the caller's h; later layers: the
//     previous layer's output rows, tagged pairs written by every workgroup) and
//     computes RMSNorm with the arithmetic of k_rmsnorm;
//  2. runs its gate / up items (waves 0..kDownWaves-1, one item each at the field
//     shape; h as tagged pairs, as k_layer_decode) while wave kDownWaves routes the
//     next layer (its logits do not depend on h) and copies the next layer's bank table;
//  3. down + the weighted accumulation for its block of output rows, added to the
//     input residual and stored as tagged pairs for the next layer (the last layer:
//     plain floats to the caller's output);
//  4. issues the loads of its first gate / up item of the next layer, whose routing is
//     now known, so that they arrive during the hand-off of the residual (with fewer
//     workgroups than row blocks: at the start of the next layer instead).
// Each layer has its own h and residual regions in the workspace, so the call's tag
// alone tells a value of this call from an older one.  The arithmetic is that of
// k_rmsnorm followed by k_layer_decode, so the result is the same bits as that chain.

struct RouteLds {
  PosRec pos[kFusedMaxSlots];  // sorted position -> its expert
  float wpos[kFusedMaxSlots];  // sorted position -> router weight
};

struct StackLds {
  BankLds banks[2][MOE_MAX_BANKS];  // this layer's and the next layer's
  RouteLds route[2];
  TopkLds topk;
  float ydot[kFusedMaxSlots][16];   // down outputs of the block's rows, per sorted position
  float hres[2048];                 // the layer's input residual
  float xs[64 * kXsRow];            // the same values, lane l's 32 at l * kXsRow (no bank conflicts)
  float part[8];
  uint32_t tag;
};

// One wave: the token's routing of one layer into R (as k_layer_decode's wave 0), the
// selection also to ids_out / w_out when given.
__device__ inline void route_wave(const float *logits, const LayerArgs &L, int E, int k, int add_shared,
                                  int32_t *ids_out, float *w_out, RouteLds &R, TopkLds &T) {
  const int lane = threadIdx.x & 63, kprime = k + add_shared;
  const TopkVals<8> tv = topk_load<8>(logits, E);
  // positions by counting, not the ones the top-k returns: with those, this kernel (at
  // its register limit) was scheduled 8 % slower
  const TopkSlot ts = topk_select<8, 2, 16>(tv, E, k, add_shared, ids_out, w_out, nullptr, nullptr, T);
  const int my = ts.id;
  const int rank = slot_rank(my, lane);
  if (lane < kprime) {
    R.pos[rank] = PosRec{my, lane, bank_index(L, my), 0};
    R.wpos[rank] = ts.w;
  }
}

// Four residual values (tagged pairs written by other workgroups), read again until
// all carry the call's tag (bounded).
__device__ inline float4 load_pairs4(const uint64_t *src, uint32_t tag, FusedSync *s) {
  uint64_t v[4];
#pragma unroll
  for (int i = 0; i < 4; i++) v[i] = __hip_atomic_load(src + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int spin = 0;; spin++) {
    bool ok = true;
#pragma unroll
    for (int i = 0; i < 4; i++) ok = ok && (uint32_t)(v[i] >> 32) == tag;
    if (__ballot(!ok) == 0ull) break;
    if (spin == kSpinLimit) {
      if ((threadIdx.x & 63) == 0) __hip_atomic_store(&s->error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
#pragma unroll
    for (int i = 0; i < 4; i++)
      if ((uint32_t)(v[i] >> 32) != tag) v[i] = __hip_atomic_load(src + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return make_float4(__uint_as_float((uint32_t)v[0]), __uint_as_float((uint32_t)v[1]), __uint_as_float((uint32_t)v[2]),
                     __uint_as_float((uint32_t)v[3]));
}

template <int LPR, bool ONE_TILE>
__global__ void __launch_bounds__(64 * kFusedWaves) k_stack_decode(
    const LayerArgs *__restrict__ tab, int n_layers, int formats, const uint8_t *__restrict__ grids,
    const float *__restrict__ logits, const float *__restrict__ h_in, float *__restrict__ h_out, int E, int k,
    int add_shared, float eps, int32_t *__restrict__ ids_out, float *__restrict__ w_out, FusedSync *__restrict__ sync,
    uint64_t *__restrict__ hp, uint64_t *__restrict__ rp) {
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ StackLds S;
  constexpr int H = 2048, I = 64 * LPR, RPP = 64 / LPR, HS = LPR * kChunkPad;
  constexpr int ipe = I / kWideRows;
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
  const int kprime = k + add_shared;
  const TableLayout TL = table_layout(formats, kTabIq1 | kTabIq1Delta);
  float *hs = (float *)(lds + TL.bytes) + wave * HS;
  const TableRegs tr = tables_load(grids, formats, threadIdx.x - 64, blockDim.x - 64);
  uint32_t tag = 0;
  if (threadIdx.x == 64) tag = call_tag(sync);
  if (wave == 0) {
    route_wave(logits, tab[0], E, k, add_shared, blockIdx.x == 0 ? ids_out : nullptr, w_out, S.route[0], S.topk);
  } else {
    tables_store(tr, formats, TL, lds, threadIdx.x - 64, blockDim.x - 64, false);
    if (threadIdx.x == 64) {
      S.tag = tag;
      fill_banks(tab[0], S.banks[0]);
    }
  }
  __syncthreads();
  tag = S.tag;

  const bool item_wave = wave < kDownWaves;  // the last wave routes the next layer instead
  const int n_items = kprime * ipe, nw = gridDim.x * kDownWaves;
  const int tiles = H / RPP;
  // ONE_TILE: the launch has at least as many workgroups as tiles of output rows
  // The loads of gate / up item `item` of the layer routed in Rr / Bb.
  WideItem It = {};
  auto issue = [&](const RouteLds &Rr, const BankLds *Bb, int item, int q) {
    const int p = item / ipe;
    const int e = uniform(Rr.pos[p].e), slot = uniform(Rr.pos[p].slot);
    const BankLds &B = Bb[uniform(Rr.pos[p].bank)];
    It.W = WorkRec{e, p, p + 1, slot};
    wide_issue_mats(It, bank_mat(B, e, kGate), bank_mat(B, e, kUp), uniform(B.qt), H, item - p * ipe, q);
  };
  // ---- 1. the wave's first gate / up item of layer 0 (of later layers: issued during
  // the previous layer's accumulation, as soon as that layer's routing is visible)
  // item of wave w of workgroup b: waves 0-3, 4-7 and 8-10 (one per SIMD each) take the
  // items of positions 0-3, 4-7 and 8-10 in that order of priority, so those positions'
  // h rows are complete in turn and their down dots overlap the later items
  auto first_item = [&](int b, int wv) {
    return wv < 8 ? (wv >> 2) * (4 * (int)gridDim.x) + 4 * b + (wv & 3) : 8 * (int)gridDim.x + 3 * b + (wv - 8);
  };
  if (wave < 4)
    __builtin_amdgcn_s_setprio(3);
  else if (wave < 8)
    __builtin_amdgcn_s_setprio(2);
  else
    __builtin_amdgcn_s_setprio(1);
  if (item_wave && first_item(blockIdx.x, wave) < n_items) issue(S.route[0], S.banks[0], first_item(blockIdx.x, wave), lane);
  int cur = 0;
  for (int l = 0; l < n_layers; l++, cur ^= 1) {
    // the lane and item indices are hidden from loop-invariant code motion: hoisted out
    // of the layer loop, every address derived from them stayed live for all layers
    int q = lane, item0 = first_item(blockIdx.x, wave), tid = threadIdx.x;
    asm volatile("" : "+v"(q));
    asm volatile("" : "+s"(item0));
    asm volatile("" : "+v"(tid));
    const int lq = q % LPR, sub = q / LPR;
    const RouteLds &R = S.route[cur];
    const BankLds *Bk = S.banks[cur];
    uint64_t *hpl = hp + (size_t)l * kprime * I;
    if constexpr (!ONE_TILE) {
      if (l > 0) It = WideItem{};  // not carried around the loop
      if (l > 0 && item_wave && item0 < n_items) issue(R, Bk, item0, q);
    }
    // ---- 2. the input residual into LDS, and its RMSNorm scale
    if (tid < H / 4) {  // as k_rmsnorm: thread t squares columns 4t .. 4t+3
      const float4 v = l == 0 ? ((const float4 *)h_in)[tid]
                              : load_pairs4(rp + (size_t)(l - 1) * H + 4 * tid, tag, sync);
      *(float4 *)&S.hres[4 * tid] = v;
      *(float4 *)&S.xs[(tid >> 3) * kXsRow + (tid & 7) * 4] = v;
      float ss = fmaf(v.x, v.x, 0.0f);
      ss = fmaf(v.y, v.y, ss);
      ss = fmaf(v.z, v.z, ss);
      ss = fmaf(v.w, v.w, ss);
      ss = group_sum_first<64>(ss);
      if (lane == 0) S.part[wave] = ss;
    }
    __syncthreads();
    const float tot =
        ((S.part[0] + S.part[1]) + (S.part[2] + S.part[3])) + ((S.part[4] + S.part[5]) + (S.part[6] + S.part[7]));
    const float rs = 1.0f / sqrtf(tot / (float)H + eps);
    // ---- 3. gate / up (waves 0 .. kDownWaves-1); the last wave routes the next layer
    if (item_wave) {
      X32 X;
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const float4 f = *(const float4 *)&S.xs[lane * kXsRow + 4 * i];
        X.v[4 * i] = f.x * rs;
        X.v[4 * i + 1] = f.y * rs;
        X.v[4 * i + 2] = f.z * rs;
        X.v[4 * i + 3] = f.w * rs;
      }
      for (int item = item0; item < n_items; item += nw) {
        if (item != item0) issue(R, Bk, item, q);
        if (It.qt == MOE_Q_IQ2XS_LIKE)
          wide_run_one<MOE_Q_IQ2XS_LIKE>(It, X, q, I, lds, TL, hpl, tag);
        else
          wide_run_one<MOE_Q_IQ1M_LIKE>(It, X, q, I, lds, TL, hpl, tag);
      }
    } else if (l + 1 < n_layers) {
      route_wave(logits + (size_t)(l + 1) * E, tab[l + 1], E, k, add_shared,
                 blockIdx.x == 0 && ids_out ? ids_out + (size_t)(l + 1) * kprime : nullptr,
                 w_out ? w_out + (size_t)(l + 1) * kprime : nullptr, S.route[cur ^ 1], S.topk);
      if (lane == 0) fill_banks(tab[l + 1], S.banks[cur ^ 1]);
    }
    // ---- 4. down + accumulation for the workgroup's block(s) of output rows
    auto tile_down = [&](int tile) {
#pragma unroll 1
      for (int i = 0; i < kFusedSlotsPerWave; i++) {
        const int pj = wave + kDownWaves * i;  // sorted position
        if (!item_wave || pj >= kprime) break;
        const PosRec &P = R.pos[pj];
        const BankLds &B = Bk[uniform(P.bank)];
        const QMat Wd = bank_mat(B, uniform(P.e), kDown);
        const int qt = uniform(B.qt);
        const RowRaw Rw = qt == MOE_Q_IQ2XS_LIKE ? load_row<MOE_Q_IQ2XS_LIKE>(Wd, I, tile * RPP + sub, lq)
                                                 : load_row<MOE_Q_IQ1M_LIKE>(Wd, I, tile * RPP + sub, lq);
        stage_h_row<LPR>(hpl + (size_t)pj * I, tag, hs, sync);
        __builtin_amdgcn_wave_barrier();
        const float *hrow = hs + lq * kChunkPad;
        const float v = qt == MOE_Q_IQ2XS_LIKE ? down_slot_dot<MOE_Q_IQ2XS_LIKE, LPR>(Rw, hrow, lq, lds, TL)
                                               : down_slot_dot<MOE_Q_IQ1M_LIKE, LPR>(Rw, hrow, lq, lds, TL);
        if (lq == 0) S.ydot[pj][sub] = v;
        __builtin_amdgcn_wave_barrier();  // the staging area is reused by the next slot
      }
      __syncthreads();
    };
    auto tile_accumulate = [&](int tile, bool sync_after) {
      if (tid < RPP) {
        const int r = tile * RPP + tid;
        float a = S.hres[r];
        for (int p = 0; p < kprime; p++) a = __fadd_rn(a, __fmul_rn(R.wpos[p], S.ydot[p][tid]));
        if (l + 1 < n_layers)
          __hip_atomic_store(rp + (size_t)l * H + r, ((uint64_t)tag << 32) | __float_as_uint(a), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        else
          h_out[r] = a;
      }
      if (sync_after) __syncthreads();
    };
    const bool next_item = l + 1 < n_layers && item_wave && item0 < n_items;
    if constexpr (ONE_TILE) {
      // at most one tile per workgroup: the next layer's first gate / up loads go out as
      // soon as its routing is visible (after the down barrier), under the accumulation,
      // the residual hand-off and the RMSNorm
      if (blockIdx.x < tiles) {
        tile_down(blockIdx.x);
        tile_accumulate(blockIdx.x, false);
      }
      if (next_item) issue(S.route[cur ^ 1], S.banks[cur ^ 1], item0, q);
      __syncthreads();
    } else {
      for (int tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
        tile_down(tile);
        tile_accumulate(tile, true);
      }
    }
    __syncthreads();  // the next layer rewrites the residual staging and reads the other buffers
  }
}

hipError_t launch_stack_decode(const LayerArgs *d_tab, int n_layers, int formats, const uint8_t *grids, int inter,
                               const float *logits, const float *h_in, float *h_out, int E, int k, int add_shared,
                               float eps, int32_t *ids, float *w, void *ws, hipStream_t s) {
  int dev = 0, cus = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (err != hipSuccess) return err;
  const int kprime = k + add_shared, lpr = inter / 64;
  FusedSync *sync = (FusedSync *)ws;
  uint64_t *hp = (uint64_t *)((uint8_t *)ws + stack_pairs_offset(n_layers));
  uint64_t *rp = hp + (size_t)n_layers * kprime * inter;
  const dim3 grid((unsigned)(cus < kBarGroup * kBarGroups ? cus : kBarGroup * kBarGroups)), block(64 * kFusedWaves);
  const size_t lds_bytes = table_layout(formats, kTabIq1 | kTabIq1Delta).bytes + fused_stage_floats(lpr) * sizeof(float);
  const bool one_tile = grid.x >= (unsigned)(2048 / (64 / lpr));
  auto kern = lpr == 8 ? (one_tile ? k_stack_decode<8, true> : k_stack_decode<8, false>)
                       : (one_tile ? k_stack_decode<4, true> : k_stack_decode<4, false>);
  hipLaunchKernelGGL(kern, grid, block, lds_bytes, s, d_tab, n_layers, formats, grids, logits, h_in, h_out, E, k,
                     add_shared, eps, ids, w, sync, hp, rp);
  return hipGetLastError();
}

size_t fused_sync_bytes() { return sizeof(FusedSync); }

size_t fused_lds_bytes(const LayerArgs &L) {
  return table_layout(L.formats, kTabIq1 | kTabIq1Delta).bytes + fused_stage_floats(L.inter / 64) * sizeof(float);
}

hipError_t launch_layer_decode(const LayerArgs &L, const float *logits, const float *x, int E, int k, int add_shared,
                               int32_t *ids, float *w, int32_t *counts, int32_t *offsets, int32_t *sorted_slot,
                               int32_t *slot_pos, WorkRec *work, float *acc, void *ws, hipStream_t s) {
  int dev = 0, cus = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (err != hipSuccess) return err;
  // one workgroup per compute unit, whatever the layer's shape: the barrier counters of
  // a workspace advance by the same round on every call
  const int lpr = L.inter / 64;
  const dim3 grid((unsigned)(cus < kBarGroup * kBarGroups ? cus : kBarGroup * kBarGroups)), block(64 * kFusedWaves);
  FusedSync *sync = (FusedSync *)ws;
  const bool both = L.formats == (MOE_Q_IQ2XS_LIKE | MOE_Q_IQ1M_LIKE), iq2 = L.formats == MOE_Q_IQ2XS_LIKE;
  auto kern = lpr == 8 ? (both ? k_layer_decode<8, MOE_Q_IQ2XS_LIKE | MOE_Q_IQ1M_LIKE>
                              : iq2 ? k_layer_decode<8, MOE_Q_IQ2XS_LIKE> : k_layer_decode<8, MOE_Q_IQ1M_LIKE>)
                       : (both ? k_layer_decode<4, MOE_Q_IQ2XS_LIKE | MOE_Q_IQ1M_LIKE>
                              : iq2 ? k_layer_decode<4, MOE_Q_IQ2XS_LIKE> : k_layer_decode<4, MOE_Q_IQ1M_LIKE>);
  hipLaunchKernelGGL(kern, grid, block, fused_lds_bytes(L), s, L, logits, x, E, k, add_shared, ids, w, counts, offsets,
                     sorted_slot, slot_pos, work, acc, sync);
  return hipGetLastError();
}

}  // namespace moe
