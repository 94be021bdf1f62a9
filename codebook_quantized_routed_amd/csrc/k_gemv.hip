// Fused dequantize + mat-vec kernels for experts with few tokens.
//
// "Red Metal dev8 — resident routed top-k layer", step 4: each selected expert runs
// gate, up, SiLU(gate) * up and down from its resident weights.  The weights stay
// quantized in HBM and are decoded in registers.
//
// Lane layout: a lane owns a 64-column chunk of a row (8 groups of 8 weights): one
// 16-byte load brings its IQ2 codes (8-byte + 4-byte loads its IQ1 index streams);
// cols/64 lanes share a row and reduce through DPP.  A wave handles one "pass" (64/LPR
// rows of one expert; gate and up together in the first kernel) at a time and loops
// over passes on its own; the only workgroup barrier follows the LDS table build.
//
// Decode arithmetic: the grid values are held in LDS as fp16 (8, 25, 43 and -1, 0, +1
// are exact) and each weight enters one mixed-precision multiply-add (fp16 value times
// fp32 activation plus fp32 accumulator, v_fma_mix_f32):
//  IQ2_XS-like: the 7 explicit sign bits of a group select a row of a 128-entry table
//    of fp16 sign masks (the 8th sign is their parity), applied with one XOR per pair
//    of weights; d * (2s+1) / 8 scales each 32-column sub-block sum.
//  IQ1_M-like: sum_j (G_j + delta) x_j = sum_j G_j x_j + delta * sum_j x_j, the group
//    sums of x formed once per activation row; d * (2s+1) scales each 16-column
//    sub-block sum.
// Every dequantized weight is exact; products and sums are rounded in fp32.
#include "gemv_dev.hpp"

namespace moe {

// ----------------------------------------------------------------------------- gate + up
// A pass = rows [rp*RPP, rp*RPP + RPP) of one active expert, gate and up together.  A
// wave issues the loads of its next pass (work record, then the two rows and the first
// token's activations) before it does anything else, so the first pass's loads are in
// flight while the workgroup builds its LDS tables.
struct GatePass {
  WorkRec W;
  RowRaw g, u;
  XChunk X;
  int r, qt;
};

template <int LPR>
__device__ __forceinline__ void gateup_issue(const LayerArgs &L, GatePass &P, int a, int rp, int q, int sub,
                                             int kprime, const float *x) {
  constexpr int RPP = 64 / LPR;
  const int H = L.hidden, I = L.inter;
  const BankArgs &B = bank_of(L, P.W.e);
  P.qt = B.qtype;
  P.r = rp * RPP + sub;
  const QMat Wg = expert_mat(B, P.W.e, kGate, I, H), Wu = expert_mat(B, P.W.e, kUp, I, H);
  if (P.qt == MOE_Q_IQ2XS_LIKE) {
    P.g = load_row<MOE_Q_IQ2XS_LIKE>(Wg, H, P.r, q);
    P.u = load_row<MOE_Q_IQ2XS_LIKE>(Wu, H, P.r, q);
  } else {
    P.g = load_row<MOE_Q_IQ1M_LIKE>(Wg, H, P.r, q);
    P.u = load_row<MOE_Q_IQ1M_LIKE>(Wu, H, P.r, q);
  }
  load_x<MOE_Q_IQ2XS_LIKE>(x + (size_t)(P.W.slot0 / kprime) * H + 64 * q, P.X);  // values only
  (void)a;
}

template <int QT, int LPR>
__device__ __forceinline__ void gateup_run(const LayerArgs &L, GatePass &P, int q, int kprime, const float *x,
                                           const int32_t *sorted_slot, const uint8_t *lds, const TableLayout &TL,
                                           float *h) {
  const int H = L.hidden, I = L.inter;
  for (int p = P.W.p0; p < P.W.p1; p++) {
    if (p > P.W.p0) load_x<QT>(x + (size_t)(sload(sorted_slot + p) / kprime) * H + 64 * q, P.X);
    else if constexpr (QT == MOE_Q_IQ1M_LIKE) {
#pragma unroll
      for (int g = 0; g < 8; g++) {
        float s = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; j++) s += P.X.v[8 * g + j];
        P.X.gs8[g] = s * 0.125f;
      }
    }
    RowRaw g = P.g, u = P.u;
    opaque(g);
    opaque(u);
    float vg = dot_chunk<QT>(g, q, lds, TL, P.X);
    float vu = dot_chunk<QT>(u, q, lds, TL, P.X);
    vg = group_sum_first<LPR>(vg);
    vu = group_sum_first<LPR>(vu);
    if (q == 0) h[(size_t)p * I + P.r] = silu(vg) * vu;
  }
}

template <int LPR>
__global__ void __launch_bounds__(256) k_gateup(LayerArgs L, const float *__restrict__ x, int kprime,
                                                const int32_t *__restrict__ sorted_slot,
                                                const WorkRec *__restrict__ work, int max_tokens, int n_ids,
                                                float *__restrict__ h) {
  extern __shared__ __align__(16) uint8_t lds[];
  constexpr int RPP = 64 / LPR;
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6), q = lane % LPR, sub = lane / LPR;
  const int formats = layer_formats(L);
  const TableLayout TL = table_layout(formats);
  const int ppe = L.inter / RPP, stride = gridDim.x * 4;
  int pass = blockIdx.x * 4 + wave;
  // the record index stays within the n_ids + 1 records even before the count is known
  const int a0 = min(pass / ppe, n_ids - 1);
  const WorkRec rec0 = load_work(work, 1 + a0);
  const int total = sload(&work[0].e) * ppe;
  if ((int)blockIdx.x * 4 >= total) return;  // no pass for this workgroup (uniform)
  GatePass P;
  bool have = pass < total;
  if (have) {
    P.W = rec0;
    gateup_issue<LPR>(L, P, a0, pass - a0 * ppe, q, sub, kprime, x);
  }
  build_tables(L.grids, formats, TL, lds);
  while (have) {
    if (P.W.p1 - P.W.p0 <= max_tokens) {
      if (P.qt == MOE_Q_IQ2XS_LIKE)
        gateup_run<MOE_Q_IQ2XS_LIKE, LPR>(L, P, q, kprime, x, sorted_slot, lds, TL, h);
      else
        gateup_run<MOE_Q_IQ1M_LIKE, LPR>(L, P, q, kprime, x, sorted_slot, lds, TL, h);
    }
    pass += stride;
    have = pass < total;
    if (have) {
      const int a = pass / ppe;
      P.W = load_work(work, 1 + a);
      gateup_issue<LPR>(L, P, a, pass - a * ppe, q, sub, kprime, x);
    }
  }
}

// gate + up for hidden 2048 (one row per wave, 32 columns per lane; see the item
// layout in gemv_dev.hpp), persistent: at most one workgroup of kWideWaves waves per
// compute unit, so the grid tables are built once per compute unit; wave w of
// workgroup b takes items kWideWaves b + w, then every stride-th, and keeps the loads
// of its next two items in flight while it computes one (a single item of lookahead
// left each item waiting out the memory latency).  With at most kXStageTokens tokens,
// the tokens' activations are staged in LDS.
constexpr int kWideWaves = 12;
static_assert(64 * kWideWaves >= 2048 / 4 && 2 * 64 * kWideWaves >= MOE_MAX_IDS,
              "staging: one float4 of each token per thread; two work records per thread");
constexpr int kXStageTokens = 8;
constexpr int kXLaneRow = 36;                 // floats per lane slice in the staging
constexpr int kXTokRow = 64 * kXLaneRow;      // floats per staged token

// LDS after the grid tables: the staged activations (room for kXStageTokens tokens,
// when staged), then the work records (room for MOE_MAX_IDS).  Fixed sizes let the
// copies be unconditional, so their loads issue back to back.
__host__ __device__ inline size_t wide_stage_bytes(int T) {
  return T <= kXStageTokens ? (size_t)kXStageTokens * kXTokRow * sizeof(float) : 0;
}
constexpr size_t kWideRecsBytes = (size_t)MOE_MAX_IDS * sizeof(WorkRec);

template <bool STAGED, int QT>
__global__ void __launch_bounds__(64 * kWideWaves) k_gateup_wide(LayerArgs L, const float *__restrict__ x, int T,
                                                                 int kprime, const int32_t *__restrict__ sorted_slot,
                                                                 const WorkRec *__restrict__ work, int max_tokens,
                                                                 int n_ids, float *__restrict__ h) {
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ BankLds banks[MOE_MAX_BANKS];
  const int q = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
  const TableLayout TL = table_layout(QT, kTabIq1Delta);
  const TableRegs tr = tables_load(L.grids, QT);
  const int ipe = L.inter / kWideRows, stride = gridDim.x * kWideWaves;
  const int n1 = sload(&work[0].e), total = n1 * ipe;
  if ((int)blockIdx.x * kWideWaves >= total) return;  // no item for this workgroup (uniform)
  // the work records and the bank table in LDS: items are issued from there (two LDS
  // reads) instead of a scalar load and kernel-argument loads each.  The records and
  // the staged activations go through registers into LDS before any item is issued.
  WorkRec *recs = (WorkRec *)(lds + TL.bytes + wide_stage_bytes(T));
  float *xs = (float *)(lds + TL.bytes);
  {
    // all copies unconditional (clamped sources), loads first: one wait covers them
    constexpr int kXf4 = 2048 / 4;  // float4 per token (hidden 2048)
    const WorkRec r0 = work[1 + min((int)threadIdx.x, n1 - 1)];  // n1 <= MOE_MAX_IDS <= 2 blockDim.x
    const WorkRec r1 = work[1 + min((int)(threadIdx.x + blockDim.x), n1 - 1)];
    if (STAGED && threadIdx.x < kXf4) {  // thread i < 512 takes float4 i of every token
      const float4 *xf = (const float4 *)x + threadIdx.x;
      const int tl = T - 1;
      const float4 x0 = xf[0], x1 = xf[min(1, tl) * kXf4], x2 = xf[min(2, tl) * kXf4], x3 = xf[min(3, tl) * kXf4],
                   x4 = xf[min(4, tl) * kXf4], x5 = xf[min(5, tl) * kXf4], x6 = xf[min(6, tl) * kXf4],
                   x7 = xf[min(7, tl) * kXf4];
      const int c = 4 * threadIdx.x;  // column c goes to lane c / 32's slice
      float4 *d = (float4 *)(xs + (c >> 5) * kXLaneRow + (c & 31));
      static_assert(kXStageTokens == 8, "eight staged tokens");
      d[0] = x0, d[kXTokRow / 4] = x1, d[2 * kXTokRow / 4] = x2, d[3 * kXTokRow / 4] = x3;
      d[4 * kXTokRow / 4] = x4, d[5 * kXTokRow / 4] = x5, d[6 * kXTokRow / 4] = x6, d[7 * kXTokRow / 4] = x7;
    }
    recs[threadIdx.x] = r0;
    if (threadIdx.x + blockDim.x < MOE_MAX_IDS) recs[threadIdx.x + blockDim.x] = r1;
  }
  if (threadIdx.x == 0) fill_banks(L, banks);
  tables_store(tr, QT, TL, lds);  // also publishes the records, the activations and the bank table
  // three items in flight per wave: A is computed while B and C load.  Items of the
  // other format are skipped (a layer with both formats runs this kernel once per format).
  // (items are passed by value: a by-reference hand-off put them in scratch memory, whose
  // loads share the vector-memory counter and made every item wait for all in flight)
  auto issue = [&](int it) {
    WideItem D;
    D.qt = 0;
    if (it < total) {
      const int a = it / ipe;
      D.W = WorkRec{uniform(recs[a].e), uniform(recs[a].p0), uniform(recs[a].p1), uniform(recs[a].slot0)};
      const BankLds &Bk = banks[bank_index(L, D.W.e)];
      if (uniform(Bk.qt) == QT)
        wide_issue_fmt<QT>(D, bank_mat(Bk, D.W.e, kGate), bank_mat(Bk, D.W.e, kUp), L.hidden, it - a * ipe, q);
    }
    return D;
  };
  const XSource xsrc = STAGED ? XSource{xs, kXTokRow, kXLaneRow} : XSource{x, L.hidden, 32};
  X32 X;
  int cur_tok = -1;
  auto run = [&](WideItem &D) {
    if (D.qt == QT && D.W.p1 - D.W.p0 <= max_tokens)
      wide_run<QT>(L, D, X, cur_tok, q, kprime, xsrc, sorted_slot, lds, TL, h);
  };
  // unrolled by three so that each buffer keeps its registers (no copies between them)
  int it = blockIdx.x * kWideWaves + wave;
  if (it >= total) return;
  WideItem A = issue(it), B = issue(it + stride), C;
  for (;;) {
    C = issue(it + 2 * stride);
    run(A);
    if ((it += stride) >= total) break;
    A = issue(it + 2 * stride);
    run(B);
    if ((it += stride) >= total) break;
    B = issue(it + 2 * stride);
    run(C);
    if ((it += stride) >= total) break;
  }
}

// ----------------------------------------------------------------------------- down
template <int QT, int LPR>
__device__ __forceinline__ void down_pass(const LayerArgs &L, const WorkRec &W, int r, int q, const float *h,
                                          const uint8_t *lds, const TableLayout &TL, float *y) {
  const int H = L.hidden, I = L.inter;
  const BankArgs &B = bank_of(L, W.e);
  const RowRaw rd = load_row<QT>(expert_mat(B, W.e, kDown, H, I), I, r, q);
  for (int p = W.p0; p < W.p1; p++) {
    RowRaw d = rd;
    opaque(d);
    XChunk X;
    load_x<QT>(h + (size_t)p * I + 64 * q, X);
    const float v = group_sum_first<LPR>(dot_chunk<QT>(d, q, lds, TL, X));
    if (q == 0) y[(size_t)p * H + r] = v;
  }
}

template <int LPR>
__global__ void __launch_bounds__(256) k_down(LayerArgs L, const float *__restrict__ h,
                                              const WorkRec *__restrict__ work, int max_tokens,
                                              float *__restrict__ y) {
  extern __shared__ __align__(16) uint8_t lds[];
  constexpr int RPP = 64 / LPR;
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6), q = lane % LPR, sub = lane / LPR;
  const int formats = layer_formats(L);
  const TableLayout TL = table_layout(formats);
  const int ppe = L.hidden / RPP;
  const int total = sload(&work[0].e) * ppe;
  if ((int)blockIdx.x * 4 >= total) return;  // no pass for this workgroup (uniform)
  build_tables(L.grids, formats, TL, lds);
  for (int pass = blockIdx.x * 4 + wave; pass < total; pass += gridDim.x * 4) {
    const int a = pass / ppe, rp = pass - a * ppe;
    const WorkRec W = load_work(work, 1 + a);
    if (W.p1 - W.p0 > max_tokens) continue;
    const int r = rp * RPP + sub;
    if (bank_of(L, W.e).qtype == MOE_Q_IQ2XS_LIKE)
      down_pass<MOE_Q_IQ2XS_LIKE, LPR>(L, W, r, q, h, lds, TL, y);
    else
      down_pass<MOE_Q_IQ1M_LIKE, LPR>(L, W, r, q, h, lds, TL, y);
  }
}

// ----------------------------------------------------------------------------- down + accumulate
// One workgroup of 4 waves per (token, block of NT x RPP output rows); wave w takes the
// token's slots w, w + 4, ...: the down rows of each slot's expert are dotted with its
// h, and the outputs are accumulated as acc += w * y in ascending expert id ("Red Metal
// dev8", step 5), one rounded multiply and one rounded add per slot, so the result
// equals the separate accumulation exactly.  A wave reads a slot's activation chunk (and
// its group sums) once and dots it with NT rows per lane, so the LDS tables, the h
// staging and the chunk are built once for NT row groups.
//
// Every global load is issued before the first wait: LDS tables, the slots' h rows
// (when STAGE, copied whole into the wave's LDS area in coalesced 16-byte pieces, each
// 64-float chunk padded to 68 floats so the lanes of different chunks hit different
// banks), the slots' weight rows, acc and w.  The slot scalars come through the scalar
// cache, so issuing the weight loads never waits on a vector load.
template <int NT>
struct SlotRows {  // one slot's weight rows of a lane, one per row group
  RowRaw r[NT];
};

template <int LPR, bool STAGE, int NT>
__global__ void __launch_bounds__(256) k_down_acc(LayerArgs L, const float *__restrict__ h, int kprime,
                                                  const int32_t *__restrict__ ids, const float *__restrict__ w,
                                                  const int32_t *__restrict__ slot_pos, float *__restrict__ acc) {
  extern __shared__ __align__(16) uint8_t lds[];
  constexpr int RPP = 64 / LPR, HS = LPR * kChunkPad, F4 = LPR * 16;  // F4: float4 pieces of one h row
  constexpr int ROWS = NT * RPP;
  __shared__ float ydot[MOE_MAX_K + 1][ROWS];
  __shared__ float wsorted[MOE_MAX_K + 1];
  __shared__ int order[MOE_MAX_K + 1];
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6), q = lane % LPR, sub = lane / LPR;
  const int H = L.hidden, I = L.inter, tiles = H / ROWS;
  const int t = blockIdx.x / tiles, tile = blockIdx.x - t * tiles;
  const int r0 = tile * ROWS + sub;
  const int formats = layer_formats(L);
  const TableLayout TL = table_layout(formats);
  const int ns = (kprime + kDaWaves - 1) / kDaWaves;  // staged slots per wave
  float *hs = (float *)(lds + TL.bytes) + wave * ns * HS;
  const TableRegs tr = tables_load(L.grids, formats);
  const int32_t *tok_ids = ids + (size_t)t * kprime;
  const int32_t *tok_pos = slot_pos + (size_t)t * kprime;

  // h rows first (L2 / MALL resident), then the weight rows (HBM)
  u32x4 hv[STAGE ? kDaSlots : 1][STAGE ? (F4 + 63) / 64 : 1];
  int p[kDaSlots];
#pragma unroll
  for (int i = 0; i < kDaSlots; i++) {
    const int j = wave + kDaWaves * i;
    p[i] = j < kprime ? sload(tok_pos + j) : 0;
    if constexpr (STAGE) {
      if (j < kprime) {
        const u32x4 *src = (const u32x4 *)(h + (size_t)p[i] * I);
#pragma unroll
        for (int v = 0; v < (F4 + 63) / 64; v++) hv[i][v] = src[min(v * 64 + lane, F4 - 1)];
      }
    }
  }
  // weight rows of the first kDaFirst slots (every slot when kprime <= 12); the rows of a
  // later slot are loaded just before its dot products
  SlotRows<NT> R[kDaFirst];
  int qt[kDaSlots];
  auto load_slot = [&](SlotRows<NT> &Rs, int j) __attribute__((always_inline)) {
    const int e = sload(tok_ids + j);
    const BankArgs &B = bank_of(L, e);
    const QMat Wd = expert_mat(B, e, kDown, H, I);
#pragma unroll
    for (int g = 0; g < NT; g++)
      Rs.r[g] = B.qtype == MOE_Q_IQ2XS_LIKE ? load_row<MOE_Q_IQ2XS_LIKE>(Wd, I, r0 + g * RPP, q)
                                            : load_row<MOE_Q_IQ1M_LIKE>(Wd, I, r0 + g * RPP, q);
    return B.qtype;
  };
  static_for<kDaFirst>([&](auto ic) __attribute__((always_inline)) {
    constexpr int i = decltype(ic)::value;
    const int j = wave + kDaWaves * i;
    R[i] = SlotRows<NT>{};
    qt[i] = j < kprime ? load_slot(R[i], j) : 0;
  });
  float acc_in = 0.0f;
  if (threadIdx.x < ROWS) acc_in = acc[(size_t)t * H + tile * ROWS + threadIdx.x];
  if (threadIdx.x < kprime) {
    const int j = threadIdx.x, me = tok_ids[j];
    const float wj = w[(size_t)t * kprime + j];
    int rank = 0;
    for (int i = 0; i < kprime; i++) {
      const int o = tok_ids[i];
      rank += (o < me || (o == me && i < j)) ? 1 : 0;
    }
    order[rank] = j;
    wsorted[rank] = wj;
  }
  if constexpr (STAGE) {
#pragma unroll
    for (int i = 0; i < kDaSlots; i++) {
      const int j = wave + kDaWaves * i;
      if (j < kprime) {
#pragma unroll
        for (int v = 0; v < (F4 + 63) / 64; v++) {
          const int f = v * 64 + lane;  // float4 piece f: floats 4f..4f+3 of the row
          if (f < F4) *(u32x4 *)(hs + i * HS + (f >> 4) * kChunkPad + (f & 15) * 4) = hv[i][v];
        }
      }
    }
  }
  tables_store(tr, formats, TL, lds);  // ends with the workgroup barrier

  // a slot's dot products: its activation chunk (and group sums) read once, NT rows
  auto slot_dots = [&](const SlotRows<NT> &Rs, int qts, const float *hrow, int j) __attribute__((always_inline)) {
    XChunk X;
    if (qts == MOE_Q_IQ2XS_LIKE) {
      load_x<MOE_Q_IQ2XS_LIKE>(hrow, X);
#pragma unroll
      for (int g = 0; g < NT; g++) {
        const float v = group_sum_first<LPR>(dot_chunk<MOE_Q_IQ2XS_LIKE>(Rs.r[g], q, lds, TL, X));
        if (q == 0) ydot[j][g * RPP + sub] = v;
      }
    } else {
      load_x<MOE_Q_IQ1M_LIKE>(hrow, X);
#pragma unroll
      for (int g = 0; g < NT; g++) {
        const float v = group_sum_first<LPR>(dot_chunk<MOE_Q_IQ1M_LIKE>(Rs.r[g], q, lds, TL, X));
        if (q == 0) ydot[j][g * RPP + sub] = v;
      }
    }
  };
  static_for<kDaSlots>([&](auto ic) __attribute__((always_inline)) {
    constexpr int i = decltype(ic)::value;
    const int j = wave + kDaWaves * i;
    if (j < kprime) {
      const float *hrow = STAGE ? hs + i * HS + q * kChunkPad : h + (size_t)p[i] * I + 64 * q;
      if constexpr (i < kDaFirst) {
        slot_dots(R[i], qt[i], hrow, j);
      } else {
        SlotRows<NT> Rl;
        const int qtl = load_slot(Rl, j);
        slot_dots(Rl, qtl, hrow, j);
      }
    }
  });
  __syncthreads();
  if (threadIdx.x < ROWS) {
    float a = acc_in;
    for (int o = 0; o < kprime; o++) a = __fadd_rn(a, __fmul_rn(wsorted[o], ydot[order[o]][threadIdx.x]));
    acc[(size_t)t * H + tile * ROWS + threadIdx.x] = a;
  }
}

// ----------------------------------------------------------------------------- launch
static int lanes_per_row(int cols) { return cols / 64; }

#define MOE_LPR_DISPATCH(LPR_VAL, KERNEL, ...)                    \
  do {                                                            \
    switch (LPR_VAL) {                                            \
      case 32: hipLaunchKernelGGL(KERNEL<32>, __VA_ARGS__); break; \
      case 16: hipLaunchKernelGGL(KERNEL<16>, __VA_ARGS__); break; \
      case 8: hipLaunchKernelGGL(KERNEL<8>, __VA_ARGS__); break;   \
      default: hipLaunchKernelGGL(KERNEL<4>, __VA_ARGS__); break;  \
    }                                                             \
  } while (0)

// Workgroups for a bound on passes: one pass per wave up to the cap, then waves loop.
static unsigned grid_for_passes(long passes) {
  long wgs = (passes + 3) / 4;
  return (unsigned)(wgs < 1 ? 1 : (wgs < 2048 ? wgs : 2048));
}

hipError_t launch_gateup_gemv(const LayerArgs &L, const float *x, int T, int kprime, const int32_t *sorted_slot,
                              const WorkRec *work, int n_ids, int max_tokens, float *h, hipStream_t s) {
  const int lpr = lanes_per_row(L.hidden), rpp = 64 / lpr;
  const long max_active = n_ids < (long)T * kprime ? n_ids : (long)T * kprime;
  const size_t shmem = table_layout(layer_formats(L)).bytes;
  if (L.hidden == 2048) {
    int dev = 0, cus = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err == hipSuccess) err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess) return err;
    const long need = (max_active * (L.inter / kWideRows) + kWideWaves - 1) / kWideWaves;
    const unsigned grid = (unsigned)(need < cus ? need : cus);
    const size_t recs = kWideRecsBytes;
    const dim3 g(grid < 1 ? 1 : grid), b(64 * kWideWaves);
    for (int qt : {MOE_Q_IQ2XS_LIKE, MOE_Q_IQ1M_LIKE}) {
      if (!(L.formats & qt)) continue;
      const size_t bytes = table_layout(qt, kTabIq1Delta).bytes + wide_stage_bytes(T) + recs;
      if (T <= kXStageTokens && qt == MOE_Q_IQ2XS_LIKE)
        hipLaunchKernelGGL((k_gateup_wide<true, MOE_Q_IQ2XS_LIKE>), g, b, bytes, s, L, x, T, kprime, sorted_slot, work,
                           max_tokens, n_ids, h);
      else if (T <= kXStageTokens)
        hipLaunchKernelGGL((k_gateup_wide<true, MOE_Q_IQ1M_LIKE>), g, b, bytes, s, L, x, T, kprime, sorted_slot, work,
                           max_tokens, n_ids, h);
      else if (qt == MOE_Q_IQ2XS_LIKE)
        hipLaunchKernelGGL((k_gateup_wide<false, MOE_Q_IQ2XS_LIKE>), g, b, bytes, s, L, x, T, kprime, sorted_slot, work,
                           max_tokens, n_ids, h);
      else
        hipLaunchKernelGGL((k_gateup_wide<false, MOE_Q_IQ1M_LIKE>), g, b, bytes, s, L, x, T, kprime, sorted_slot, work,
                           max_tokens, n_ids, h);
      err = hipGetLastError();
      if (err != hipSuccess) return err;
    }
    return hipGetLastError();
  }
  MOE_LPR_DISPATCH(lpr, k_gateup, dim3(grid_for_passes(max_active * (L.inter / rpp))), dim3(256), shmem, s, L, x,
                   kprime, sorted_slot, work, max_tokens, n_ids, h);
  return hipGetLastError();
}

hipError_t launch_down_gemv(const LayerArgs &L, const float *h, int T, int kprime, const WorkRec *work, int n_ids,
                            int max_tokens, float *y, hipStream_t s) {
  const int lpr = lanes_per_row(L.inter), rpp = 64 / lpr;
  const long max_active = n_ids < (long)T * kprime ? n_ids : (long)T * kprime;
  const size_t shmem = table_layout(layer_formats(L)).bytes;
  MOE_LPR_DISPATCH(lpr, k_down, dim3(grid_for_passes(max_active * (L.hidden / rpp))), dim3(256), shmem, s, L, h,
                   work, max_tokens, y);
  return hipGetLastError();
}

// Row groups per down + accumulate workgroup: as many as keep at least two workgroups per
// compute unit in flight (fewer, larger workgroups build the LDS tables and read each
// activation chunk fewer times).
static int down_acc_groups(int T, int tiles8, int cus) {
  for (int nt : {4, 2}) {
    if (tiles8 % nt == 0 && (long)T * (tiles8 / nt) >= 2L * cus) return nt;
  }
  return 1;
}

#define MOE_DA_LAUNCH(LPR_V, STAGE_V, NT_V, SHM)                                                                \
  hipLaunchKernelGGL((k_down_acc<LPR_V, STAGE_V, NT_V>), dim3((unsigned)(T * (L.hidden / ((64 / LPR_V) * NT_V)))), \
                     dim3(64 * kDaWaves), SHM, s, L, h, kprime, ids, w, slot_pos, acc)

hipError_t launch_down_accumulate(const LayerArgs &L, const float *h, int T, int kprime, const int32_t *ids,
                                  const float *w, const int32_t *slot_pos, float *acc, hipStream_t s) {
  const int lpr = lanes_per_row(L.inter), rpp = 64 / lpr;
  const size_t tables = table_layout(layer_formats(L)).bytes;
  int dev = 0, cus = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err == hipSuccess) err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (err != hipSuccess) return err;
  const int nt = down_acc_groups(T, L.hidden / rpp, cus);
  // h is staged in LDS for inter <= 512 (at most 43.5 KB per workgroup)
  const int ns = (kprime + kDaWaves - 1) / kDaWaves;
  switch (lpr * 8 + nt) {
    case 4 * 8 + 4: MOE_DA_LAUNCH(4, true, 4, tables + down_acc_stage_bytes(4, ns)); break;
    case 4 * 8 + 2: MOE_DA_LAUNCH(4, true, 2, tables + down_acc_stage_bytes(4, ns)); break;
    case 4 * 8 + 1: MOE_DA_LAUNCH(4, true, 1, tables + down_acc_stage_bytes(4, ns)); break;
    case 8 * 8 + 4: MOE_DA_LAUNCH(8, true, 4, tables + down_acc_stage_bytes(8, ns)); break;
    case 8 * 8 + 2: MOE_DA_LAUNCH(8, true, 2, tables + down_acc_stage_bytes(8, ns)); break;
    case 8 * 8 + 1: MOE_DA_LAUNCH(8, true, 1, tables + down_acc_stage_bytes(8, ns)); break;
    case 16 * 8 + 4: MOE_DA_LAUNCH(16, false, 4, tables); break;
    case 16 * 8 + 2: MOE_DA_LAUNCH(16, false, 2, tables); break;
    case 16 * 8 + 1: MOE_DA_LAUNCH(16, false, 1, tables); break;
    case 32 * 8 + 4: MOE_DA_LAUNCH(32, false, 4, tables); break;
    case 32 * 8 + 2: MOE_DA_LAUNCH(32, false, 2, tables); break;
    default: MOE_DA_LAUNCH(32, false, 1, tables); break;
  }
  return hipGetLastError();
}

}  // namespace moe
