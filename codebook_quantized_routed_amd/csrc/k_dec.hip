// Gate / up for calls of a few tokens, on the matrix cores (decode).
//
// "Red Metal dev8 — resident routed top-k layer", step 4: each selected expert runs
// gate, up and SiLU(gate) * up from its resident weights for the tokens routed to it.
//
// Every weight is decoded once per call (an expert's tokens share its fragments) and
// the multiply-adds run on v_mfma_f32_16x16x32_f16 (see mfma_dec.hpp for the operand
// layout and the exactness argument).  A unit is 8 rows of one expert, gate and up
// (16 B columns); the hidden dimension is split into parts of two super-blocks, one
// wave each; the parts' partials are added in part order, then scaled back by 2^-e of
// the token.  The down projection of these calls stays on the vector kernels
// (k_gemv.hip): with about one token per selected expert a 16-row A operand is
// mostly empty, and the decode through LDS tables measured slower there.
#include "mfma_dec.hpp"
#include "route_dev.hpp"

namespace moe {

constexpr int kDecWaves = 16;

// ----------------------------------------------------------------------------- gate + up
// Unit u of the call: record a = u / (inter / 8) of the work list's first set, rows
// 8 rb .. 8 rb + 7 (rb = u % (inter / 8)) of its gate and up.
template <int NSB>
struct GuUnit {
  SbCodes c[NSB];
  int active, p0, ntok, rb;
  int arow;  // the staged A row of the lane's fragment row m (token i = m / 2 of the unit), or -1
};

// The first expert of the layer's first bank of format QT: a valid source for the loads
// of an idle unit (every load is issued, so no load sits behind a branch and the waits
// can count exactly how many are still in flight).
template <int QT>
__device__ __forceinline__ int first_expert_of(const LayerArgs &L) {
  int e = 0;
#pragma unroll
  for (int b = MOE_MAX_BANKS - 1; b >= 0; b--)
    if (b < L.n_banks && L.banks[b].qtype == QT) e = L.banks[b].first;
  return e;
}

// The loads of unit u given its record W (wave-uniform) and the token of each of the
// expert's sorted positions (tok_of, LDS; read once the copy is visible).
template <int QT, int NSB>
__device__ __forceinline__ GuUnit<NSB> gu_issue(const LayerArgs &L, const WorkRec &W, int rb, bool active, int kp) {
  GuUnit<NSB> U;
  const int H = L.hidden, I = L.inter, lane = threadIdx.x & 63, q = lane >> 4, n = lane & 15;
  U.active = active && bank_of(L, W.e).qtype == QT;
  const int e = U.active ? W.e : first_expert_of<QT>(L);
  const BankArgs &B = bank_of(L, e);
  U.p0 = W.p0;
  U.ntok = W.p1 - W.p0;
  U.rb = rb;
  const QMat M = pick_mat(n < 8, expert_mat(B, e, kGate, I, H), expert_mat(B, e, kUp, I, H));
  // an idle unit past the last record can have rb >= inter / 8: its loads stay in row
  // block inter / 8 - 1 (rb >= 0 always)
  const int row = 8 * min(rb, I / 8 - 1) + (n & 7);
#pragma unroll
  for (int i = 0; i < NSB; i++) U.c[i] = load_sb<QT>(M, H, row, kp * NSB + i, q);
  U.arow = -1;
  return U;
}

// Records and sorted positions of a call of at most kDecMaxTokens tokens fit LDS.
constexpr int kDecMaxSlots = kDecMaxTokens * (MOE_MAX_K + 1);

template <int QT, int NSB>
__global__ void __launch_bounds__(64 * kDecWaves) __attribute__((amdgpu_waves_per_eu(4, 4)))
k_gateup_dec(LayerArgs L, const float *__restrict__ x, int T, int kprime, const int32_t *__restrict__ sorted_slot,
             const WorkRec *__restrict__ work, int n_ids, float *__restrict__ h) {
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ float xinv[8];
  __shared__ __align__(16) uint32_t wmax[8 * 16];
  __shared__ int4 uinfo[2][kDecWaves];     // per unit slot of a round: (active, p0, ntok, rb), by round parity
  __shared__ __align__(16) _Float16 zero8[8];  // the A fragment of a missing token
  __shared__ WorkRec recs[kDecMaxSlots + 1];  // the work list's record 0 and first set
  __shared__ int tok_of[kDecMaxSlots];     // sorted position -> token
  const int H = L.hidden, I = L.inter, tid = threadIdx.x;
  constexpr int SB = NSB;                  // super-blocks per wave
  const int KP = (H >> 8) / SB, UPR = kDecWaves / KP, rbs = I / 8;
  // wave-uniform in scalar registers: the first unit's record then comes through the
  // scalar cache and its bank through scalar loads of the kernel arguments
  const int wave = uniform(tid >> 6), lane = tid & 63, q = lane >> 4, n = lane & 15;
  const int us = wave / KP, kp = wave - us * KP, stride = gridDim.x * UPR;
  const int nslots = T * kprime, nrec = min(nslots, n_ids) + 1;
  // the small inputs first, one load per thread (clamped: no load behind a branch)
  const WorkRec rec = work[min(tid, nrec - 1)];
  const int slot = sorted_slot[min(tid, nslots - 1)];
  const int ic = min(tid, H / 4 - 1);
  float4 v[8];
#pragma unroll
  for (int t = 0; t < 8; t++) v[t] = ((const float4 *)(x + (size_t)min(t, T - 1) * H))[ic];
  // the decode tables next: issued before the first unit's weight loads, so waiting for
  // them (vector loads complete in order) does not also wait for the weights
  const DecTables D = dec_tables(QT);
  const DecTableCopy tc = dec_tables_copy_load<QT>(L.grids, tid, blockDim.x);
  // the first unit's record through the scalar cache (its index does not depend on the
  // record count), so its weight loads leave without waiting for the copy
  int u = blockIdx.x * UPR + us;
  const int total = sload(&work[0].e) * rbs;
  if ((int)blockIdx.x * UPR >= total) return;  // no unit for this workgroup (uniform)
  const int a0 = min(u / rbs, n_ids - 1);
  GuUnit<NSB> cur = gu_issue<QT, NSB>(L, load_work(work, 1 + a0), u - a0 * rbs, u < total, kp);
  const int XR = stage_row_halves(H);
  _Float16 *xs = (_Float16 *)(lds + D.bytes);
  // partials [2 (round parity)][UPR][KP][8 tokens][16 columns]: a round writes one half
  // while the previous round's epilogue may still read the other, so one barrier a round
  float *red = (float *)(xs + (size_t)2 * T * XR);
  if (tid < 8) zero8[tid] = (_Float16)0.0f;
  // unconditional stores (a conditional one lets the compiler move the load into the
  // branch, where it waits for every older load): threads past the counts write
  // entries never read, or at the clamped last index the value that entry holds
  // (their loads were clamped to the last record / slot)
  recs[min(tid, kDecMaxSlots)] = rec;
  tok_of[min(tid, kDecMaxSlots - 1)] = slot / kprime;
  dec_tables_copy_store<QT>(tc, lds, tid, blockDim.x);
  // activations: per token the largest magnitude (wave max, then the 16 wave maxima),
  // then the hi / lo rows
  const bool mine = 4 * tid < H;
#pragma unroll
  for (int t = 0; t < 8; t++) {
    if (t < T) {
      const float m = mine ? fmaxf(fmaxf(fabsf(v[t].x), fabsf(v[t].y)), fmaxf(fabsf(v[t].z), fabsf(v[t].w))) : 0.0f;
      const uint32_t wm = wave_max_u32(__float_as_uint(m));
      if (lane == 0) wmax[t * 16 + wave] = wm;
    }
  }
  lds_barrier();
#pragma unroll
  for (int t = 0; t < 8; t++) {
    if (t < T) {
      uint32_t m = 0;
      const uint4 *wm = (const uint4 *)(wmax + t * 16);
#pragma unroll
      for (int k = 0; k < 4; k++) {
        const uint4 v4 = wm[k];
        m = max(max(m, max(v4.x, v4.y)), max(v4.z, v4.w));
      }
      const int e = stage_exponent(__uint_as_float(m));
      if (tid == 0) xinv[t] = pow2f(-e);
      if (mine) stage4(xs + (size_t)(2 * t) * XR, xs + (size_t)(2 * t + 1) * XR, 4 * tid, v[t], pow2f(e));
    }
  }
  lds_barrier();
  const int rounds = (total - (int)blockIdx.x * UPR + stride - 1) / stride;
  // the loads of the unit `ahead` rounds after u (record from LDS)
  auto issue_ahead = [&](int uu) __attribute__((always_inline)) {
    const int an = min(uu / rbs, nrec - 2);  // within the copied records
    const WorkRec Wn{uniform(recs[1 + an].e), uniform(recs[1 + an].p0), uniform(recs[1 + an].p1), 0};
    return gu_issue<QT, NSB>(L, Wn, uu - an * rbs, uu < total, kp);
  };
  // one round: the unit's partials, then the parts added in order and h written; buf
  // (the round's parity) picks the half of the partials and unit information
  auto round = [&](const GuUnit<NSB> &U, int buf) __attribute__((always_inline)) {
    float *redb = red + (size_t)buf * UPR * KP * 8 * 16;
    if (U.active) {
      const int ti = n >> 1;
      const int arow = ti < U.ntok ? 2 * tok_of[U.p0 + ti] + (n & 1) : -1;
      float r0 = 0.0f, r1 = 0.0f;
      dot_sb<QT, SB>(U.c, kp * SB, xs, XR, arow, q, lds, D, zero8, r0, r1);
      float *rp = redb + (size_t)(us * KP + kp) * 8 * 16;
      if (2 * q < U.ntok) rp[(2 * q) * 16 + n] = r0;
      if (2 * q + 1 < U.ntok) rp[(2 * q + 1) * 16 + n] = r1;
    }
    if (kp == 0 && lane == 0) uinfo[buf][us] = make_int4(U.active, U.p0, U.ntok, U.rb);
    lds_barrier();
    // epilogue: thread (unit slot, token i, row r) adds the parts in order; the next
    // round writes the other half, so no barrier follows
    const int us2 = tid >> 6, i = (tid >> 3) & 7, r = tid & 7;
    if (us2 < UPR) {
      const int4 inf = uinfo[buf][us2];
      if (inf.x && i < inf.z) {
        const float *rp = redb + (size_t)us2 * KP * 8 * 16 + i * 16;
        float g = rp[r], vu = rp[8 + r];
        for (int p = 1; p < KP; p++) {
          g += rp[p * 8 * 16 + r];
          vu += rp[p * 8 * 16 + 8 + r];
        }
        const float inv = xinv[tok_of[inf.y + i]];
        h[(size_t)(inf.y + i) * I + 8 * inf.w + r] = silu(g * inv) * (vu * inv);
      }
    }
  };
  // unrolled by two: each unit keeps its own registers while the other's loads travel
  // (a copy of in-flight registers would wait for their loads)
  GuUnit<NSB> nxt;
  for (int rd = 0;;) {
    nxt = issue_ahead(u + stride);
    round(cur, 0);
    if (++rd >= rounds) break;
    u += stride;
    cur = issue_ahead(u + stride);
    round(nxt, 1);
    if (++rd >= rounds) break;
    u += stride;
  }
}

// ----------------------------------------------------------------------------- launch
static hipError_t device_cus(int *cus) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err == hipSuccess) err = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
  return err;
}

bool dec_path_ok(const LayerArgs &L, int T) { return T >= 2 && T <= kDecMaxTokens && L.inter <= 512; }

size_t gateup_dec_lds(const LayerArgs &L, int qt, int T) {
  const int H = L.hidden, KP = (H >> 8) >= 2 ? (H >> 8) / 2 : 1, UPR = kDecWaves / KP;
  return dec_tables(qt).bytes + (size_t)2 * T * stage_row_halves(H) * sizeof(_Float16) +
         (size_t)2 * UPR * KP * 8 * 16 * sizeof(float);
}

hipError_t launch_gateup_dec(const LayerArgs &L, const float *x, int T, int kprime, const int32_t *sorted_slot,
                             const WorkRec *work, int n_ids, float *h, hipStream_t s) {
  int cus = 0;
  hipError_t err = device_cus(&cus);
  if (err != hipSuccess) return err;
  const long active = n_ids < (long)T * kprime ? n_ids : (long)T * kprime;
  const int KP = (L.hidden >> 8) >= 2 ? (L.hidden >> 8) / 2 : 1, UPR = kDecWaves / KP;
  const long units = active * (L.inter / 8);
  const long need = (units + UPR - 1) / UPR;
  const dim3 grid((unsigned)(need < cus ? (need < 1 ? 1 : need) : cus)), block(64 * kDecWaves);
  for (int qt : {MOE_Q_IQ2XS_LIKE, MOE_Q_IQ1M_LIKE}) {
    if (!(L.formats & qt)) continue;
    const size_t bytes = gateup_dec_lds(L, qt, T);
    if (qt == MOE_Q_IQ2XS_LIKE) {
      if (L.hidden >= 512)
        hipLaunchKernelGGL((k_gateup_dec<MOE_Q_IQ2XS_LIKE, 2>), grid, block, bytes, s, L, x, T, kprime, sorted_slot, work, n_ids, h);
      else
        hipLaunchKernelGGL((k_gateup_dec<MOE_Q_IQ2XS_LIKE, 1>), grid, block, bytes, s, L, x, T, kprime, sorted_slot, work, n_ids, h);
    } else {
      if (L.hidden >= 512)
        hipLaunchKernelGGL((k_gateup_dec<MOE_Q_IQ1M_LIKE, 2>), grid, block, bytes, s, L, x, T, kprime, sorted_slot, work, n_ids, h);
      else
        hipLaunchKernelGGL((k_gateup_dec<MOE_Q_IQ1M_LIKE, 1>), grid, block, bytes, s, L, x, T, kprime, sorted_slot, work, n_ids, h);
    }
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace moe
