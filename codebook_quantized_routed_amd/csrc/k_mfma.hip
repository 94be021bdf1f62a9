// Grouped GEMM on the matrix cores for experts with many tokens (prefill).
//
// "Red Metal dev8 — resident routed top-k layer", step 4: every selected expert runs
// gate, up, SiLU(gate) * up and down.  When an expert has several tokens the rows are
// applied to a block of activation columns at once with v_mfma_f32_16x16x32_f16.
//
// Exactness of the A operand.  A weight is d/8 * (2s+1) * (+-G) (IQ2_XS-like, G in
// {8, 25, 43}) or d/8 * (2s+1) * (8G +- 1) (IQ1_M-like, G in {-1, 0, 1}).  The integer
// part (2s+1) * (+-G) <= 31 * 43 or (2s+1) * (8G +- 1) <= 15 * 9 is exact in fp16, so a
// lane decodes its 8-weight group straight into the fp16 A fragment (LDS grid row,
// sign mask, one packed multiply or fused multiply-add), and d/8 -- one value per row
// and 256-column super-block -- scales the fp32 partial of each super-block.
//
// Activations.  Each activation x is split into x_hi = fp16(x) and x_lo = fp16(x -
// x_hi); both halves run through the MFMA against the same A, so the products carry
// about 22 bits of x.  This requires |x| < 65504 (fp16 range).
//
// Layout of one MFMA (16 rows x 32 k x 16 columns): lane l holds A row l % 16, k slots
// 8 (l / 16) .. + 7 and B column l % 16, the same k slots; D row 4 (l / 16) + i,
// column l % 16.  Within a 256-column super-block the k slots of lane quarter qd at
// step ks stand for group 8 qd + ks (columns 8 (8 qd + ks) .. + 7), so a lane's eight
// groups of a super-block are contiguous in its row's code stream.
#include "matvec_common.hpp"

namespace moe {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kMfPass = 32;              // token columns per pass (two 16-column tiles)
constexpr int kMfTiles = 4;              // 16-row tiles per wave
constexpr int kXRow = 256 + 8;           // halves per staged column (16 bytes of padding)
constexpr int kXHalves = kMfPass * kXRow;  // one of hi / lo

__host__ __device__ inline size_t mfma_lds_bytes(int formats) {
  return table_layout(formats).bytes + 2 * kXHalves * sizeof(_Float16) + kMfPass * sizeof(int);
}

// The lane's codes of one tile row for one super-block.  IQ2: c = 8 codes (u16), s = the
// scale word.  IQ1: c.xy = 8 index bytes, c.z = 8 nibbles, (s:c.w) = the sd word.
struct TileCodes {
  uint4 c;
  uint32_t s;
};

template <int QT>
__device__ __forceinline__ TileCodes load_tile_codes(const QMat &m, int cols, int row, int sb, int qd) {
  const int ng = cols >> 3, nb = cols >> 8, g0 = sb * 32 + 8 * qd;
  TileCodes t;
  if constexpr (QT == MOE_Q_IQ2XS_LIKE) {
    t.c = load_stream16(m.s0 + ((size_t)row * ng + g0) * 2);
    t.s = ((const uint32_t *)m.s1)[(size_t)row * nb + sb];
  } else {
    const uint2 ql = load_stream8(m.s0 + (size_t)row * ng + g0);
    const uint32_t qh = __builtin_nontemporal_load((const uint32_t *)(m.s1 + (size_t)row * (ng / 2) + g0 / 2));
    const uint2 sd = *(const uint2 *)(m.s2 + ((size_t)row * nb + sb) * 8);
    t.c = make_uint4(ql.x, ql.y, qh, sd.x);
    t.s = sd.y;
  }
  return t;
}

// d / 8 of row `row` in super-block sb (the fp16 d is the low half of the IQ1 sd word).
template <int QT>
__device__ __forceinline__ float load_dfac(const QMat &m, int cols, int row, int sb) {
  const int nb = cols >> 8;
  const size_t stride = QT == MOE_Q_IQ2XS_LIKE ? 2 : 8;
  return half_bits_to_float(*(const uint16_t *)(m.s2 + ((size_t)row * nb + sb) * stride)) * 0.125f;
}

__device__ __forceinline__ uint32_t f16_pair(uint32_t v) {
  const uint32_t b = __builtin_bit_cast(uint16_t, (_Float16)(float)v);
  return b | (b << 16);
}

// fp16 A fragment of group 8 qd + ks of the lane's row.
template <int QT>
__device__ __forceinline__ h8 decode_a(const TileCodes &t, int ks, int qd, const uint8_t *lds, const TableLayout &TL) {
  uint4 v;
  if constexpr (QT == MOE_Q_IQ2XS_LIKE) {
    const uint32_t w = ks < 2 ? t.c.x : (ks < 4 ? t.c.y : (ks < 6 ? t.c.z : t.c.w));
    const uint32_t code = (ks & 1) ? (w >> 16) : (w & 0xFFFFu);
    v = ((const uint4 *)(lds + TL.iq2h))[code & 0x1FFu];
    const uint4 m = ((const uint4 *)(lds + TL.iq2m))[(code >> 9) & 0x7Fu];
    v.x ^= m.x;
    v.y ^= m.y;
    v.z ^= m.z;
    v.w ^= m.w;
    const uint32_t sub = (8 * qd + ks) >> 2;
    const h2 f = __builtin_bit_cast(h2, f16_pair(2 * ((t.s >> (4 * sub)) & 15u) + 1));
    h2 *p = (h2 *)&v;
#pragma unroll
    for (int i = 0; i < 4; i++) p[i] = p[i] * f;
  } else {
    const uint32_t ql8 = ((ks < 4 ? t.c.x : t.c.y) >> (8 * (ks & 3))) & 0xFFu;
    const uint32_t nib = (t.c.z >> (4 * ks)) & 15u;
    v = ((const uint4 *)(lds + TL.iq1h))[ql8 | ((nib & 7u) << 8)];
    const uint64_t sd = ((uint64_t)t.s << 32) | t.c.w;
    const uint32_t sub = (8 * qd + ks) >> 1;
    const uint32_t f = 2 * (uint32_t)((sd >> (16 + 3 * sub)) & 7u) + 1;
    const h2 f8 = __builtin_bit_cast(h2, f16_pair(8 * f));
    h2 fd = __builtin_bit_cast(h2, f16_pair(f));
    if (nib & 8u) fd = -fd;
    h2 *p = (h2 *)&v;
#pragma unroll
    for (int i = 0; i < 4; i++) p[i] = p[i] * f8 + fd;  // exact: integers <= 135
  }
  return __builtin_bit_cast(h8, v);
}

// Stages 256 columns of up to kMfPass activation rows into LDS as hi / lo fp16
// halves: thread t takes row t / 8, floats 32 (t % 8) .. + 31.  src_row[c] < 0: zeros.
__device__ __forceinline__ void stage_x(const float *base, int row_stride, const int *src_row, int col0,
                                        _Float16 *xhi, _Float16 *xlo) {
  const int c = threadIdx.x >> 3, part = threadIdx.x & 7;
  const int r = src_row[c];
  u32x4 v[8];
  if (r >= 0) {
    const u32x4 *p = (const u32x4 *)(base + (size_t)r * row_stride + col0 + 32 * part);
#pragma unroll
    for (int i = 0; i < 8; i++) v[i] = p[i];
  } else {
#pragma unroll
    for (int i = 0; i < 8; i++) v[i] = u32x4{0u, 0u, 0u, 0u};
  }
  uint32_t hi[16], lo[16];
#pragma unroll
  for (int i = 0; i < 16; i++) {
    const float a = __uint_as_float(v[i >> 1][2 * (i & 1)]), b = __uint_as_float(v[i >> 1][2 * (i & 1) + 1]);
    const _Float16 ah = (_Float16)a, bh = (_Float16)b;
    const _Float16 al = (_Float16)(a - (float)ah), bl = (_Float16)(b - (float)bh);
    hi[i] = (uint32_t)__builtin_bit_cast(uint16_t, ah) | ((uint32_t)__builtin_bit_cast(uint16_t, bh) << 16);
    lo[i] = (uint32_t)__builtin_bit_cast(uint16_t, al) | ((uint32_t)__builtin_bit_cast(uint16_t, bl) << 16);
  }
  u32x4 *dh = (u32x4 *)(xhi + c * kXRow + 32 * part), *dl = (u32x4 *)(xlo + c * kXRow + 32 * part);
#pragma unroll
  for (int i = 0; i < 4; i++) {
    dh[i] = u32x4{hi[4 * i], hi[4 * i + 1], hi[4 * i + 2], hi[4 * i + 3]};
    dl[i] = u32x4{lo[4 * i], lo[4 * i + 1], lo[4 * i + 2], lo[4 * i + 3]};
  }
}

// One pass: the wave's kMfTiles row tiles times up to kMfPass staged columns, over the
// K range [0, cols) in super-blocks.  Ct[t][n]: the fp32 result of tile t, column tile
// n.  The caller has built the grid tables.
template <int QT>
__device__ __forceinline__ void mfma_pass(const QMat (&mats)[kMfTiles], const int (&trow)[kMfTiles], int cols,
                                          const float *xbase, int x_stride, const int *src_row, int n_cols,
                                          uint8_t *lds, const TableLayout &TL, _Float16 *xhi, _Float16 *xlo,
                                          f4 (&Ct)[kMfTiles][2]) {
  const int lane = threadIdx.x & 63, qd = lane >> 4, lr = lane & 15;
  const int nsb = cols >> 8;
  const bool two = n_cols > 16;
#pragma unroll
  for (int t = 0; t < kMfTiles; t++) Ct[t][0] = Ct[t][1] = f4{0.0f, 0.0f, 0.0f, 0.0f};
  TileCodes tc[kMfTiles];
#pragma unroll
  for (int t = 0; t < kMfTiles; t++) tc[t] = load_tile_codes<QT>(mats[t], cols, trow[t] + lr, 0, qd);
  for (int sb = 0; sb < nsb; sb++) {
    float df[kMfTiles][4];
#pragma unroll
    for (int t = 0; t < kMfTiles; t++)
#pragma unroll
      for (int i = 0; i < 4; i++) df[t][i] = load_dfac<QT>(mats[t], cols, trow[t] + 4 * qd + i, sb);
    stage_x(xbase, x_stride, src_row, sb * 256, xhi, xlo);
    __syncthreads();
    TileCodes nx[kMfTiles];
    if (sb + 1 < nsb) {
#pragma unroll
      for (int t = 0; t < kMfTiles; t++) nx[t] = load_tile_codes<QT>(mats[t], cols, trow[t] + lr, sb + 1, qd);
    }
    f4 Cs[kMfTiles][2];
#pragma unroll
    for (int t = 0; t < kMfTiles; t++) Cs[t][0] = Cs[t][1] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < 8; ks++) {
      h8 A[kMfTiles];
#pragma unroll
      for (int t = 0; t < kMfTiles; t++) A[t] = decode_a<QT>(tc[t], ks, qd, lds, TL);
      const int koff = (8 * qd + ks) * 8;
      {
        const h8 bh = *(const h8 *)(xhi + lr * kXRow + koff), bl = *(const h8 *)(xlo + lr * kXRow + koff);
#pragma unroll
        for (int t = 0; t < kMfTiles; t++) {
          Cs[t][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[t], bh, Cs[t][0], 0, 0, 0);
          Cs[t][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[t], bl, Cs[t][0], 0, 0, 0);
        }
      }
      if (two) {
        const h8 bh = *(const h8 *)(xhi + (16 + lr) * kXRow + koff), bl = *(const h8 *)(xlo + (16 + lr) * kXRow + koff);
#pragma unroll
        for (int t = 0; t < kMfTiles; t++) {
          Cs[t][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[t], bh, Cs[t][1], 0, 0, 0);
          Cs[t][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[t], bl, Cs[t][1], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < kMfTiles; t++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        Ct[t][0][i] = fmaf(Cs[t][0][i], df[t][i], Ct[t][0][i]);
        Ct[t][1][i] = fmaf(Cs[t][1][i], df[t][i], Ct[t][1][i]);
      }
    if (sb + 1 < nsb) {
#pragma unroll
      for (int t = 0; t < kMfTiles; t++) tc[t] = nx[t];
    }
    __syncthreads();  // the staged columns are overwritten next
  }
}

// The i-th MFMA expert's record: they are stored from the end of the work list.
__device__ __forceinline__ WorkRec mfma_record(const WorkRec *work, int n_ids, int a) {
  return load_work(work, n_ids - a);
}

// gate + up + SiLU * up.  Workgroup = (MFMA expert, block of 128 rows of inter); wave
// w takes gate and up rows r0 .. r0 + 31, r0 = 128 * block + 32 w.  One instance per
// format: a workgroup whose expert has the other format returns at once.
template <int QT>
__global__ void __launch_bounds__(256) k_gateup_mfma(LayerArgs L, const float *__restrict__ x, int kprime,
                                                     const int32_t *__restrict__ sorted_slot,
                                                     const WorkRec *__restrict__ work, int n_ids,
                                                     float *__restrict__ h) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int H = L.hidden, I = L.inter, RB = I / 128;
  const int a = blockIdx.x / RB, rb = blockIdx.x - a * RB;
  if (a >= sload(&work[0].p1)) return;  // record 0 = (matvec experts, slots, MFMA experts, 0)
  const WorkRec W = mfma_record(work, n_ids, a);
  const BankArgs &B = bank_of(L, W.e);
  if (B.qtype != QT) return;
  const TableLayout TL = table_layout(QT);
  _Float16 *xhi = (_Float16 *)(lds + TL.bytes), *xlo = xhi + kXHalves;
  int *src_row = (int *)(xlo + kXHalves);
  build_tables(L.grids, QT, TL, lds);
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6), qd = lane >> 4, lr = lane & 15;
  const QMat Wg = expert_mat(B, W.e, kGate, I, H), Wu = expert_mat(B, W.e, kUp, I, H);
  const int r0 = rb * 128 + wave * 32;
  const QMat mats[kMfTiles] = {Wg, Wg, Wu, Wu};
  const int trow[kMfTiles] = {r0, r0 + 16, r0, r0 + 16};
  for (int pp = W.p0; pp < W.p1; pp += kMfPass) {
    const int n = min(kMfPass, W.p1 - pp);
    if (threadIdx.x < kMfPass) src_row[threadIdx.x] = threadIdx.x < n ? sorted_slot[pp + threadIdx.x] / kprime : -1;
    __syncthreads();
    f4 Ct[kMfTiles][2];
    mfma_pass<QT>(mats, trow, H, x, H, src_row, n, lds, TL, xhi, xlo, Ct);
#pragma unroll
    for (int nt = 0; nt < 2; nt++) {
      const int c = 16 * nt + lr;
      if (c < n) {
#pragma unroll
        for (int j = 0; j < 2; j++) {
          float4 o;
          o.x = silu(Ct[j][nt][0]) * Ct[2 + j][nt][0];
          o.y = silu(Ct[j][nt][1]) * Ct[2 + j][nt][1];
          o.z = silu(Ct[j][nt][2]) * Ct[2 + j][nt][2];
          o.w = silu(Ct[j][nt][3]) * Ct[2 + j][nt][3];
          *(float4 *)(h + (size_t)(pp + c) * I + r0 + 16 * j + 4 * qd) = o;
        }
      }
    }
  }
}

// down: y[p] = Wd h[p].  Workgroup = (MFMA expert, block of 256 rows of hidden); wave w
// takes rows r0 .. r0 + 63, r0 = 256 * block + 64 w.  h rows are contiguous per expert.
// One instance per format, as above.
template <int QT>
__global__ void __launch_bounds__(256) k_down_mfma(LayerArgs L, const float *__restrict__ h,
                                                   const WorkRec *__restrict__ work, int n_ids,
                                                   float *__restrict__ y) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int H = L.hidden, I = L.inter, RB = H / 256;
  const int a = blockIdx.x / RB, rb = blockIdx.x - a * RB;
  if (a >= sload(&work[0].p1)) return;
  const WorkRec W = mfma_record(work, n_ids, a);
  const BankArgs &B = bank_of(L, W.e);
  if (B.qtype != QT) return;
  const TableLayout TL = table_layout(QT);
  _Float16 *xhi = (_Float16 *)(lds + TL.bytes), *xlo = xhi + kXHalves;
  int *src_row = (int *)(xlo + kXHalves);
  build_tables(L.grids, QT, TL, lds);
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6), qd = lane >> 4, lr = lane & 15;
  const QMat Wd = expert_mat(B, W.e, kDown, H, I);
  const int r0 = rb * 256 + wave * 64;
  const QMat mats[kMfTiles] = {Wd, Wd, Wd, Wd};
  const int trow[kMfTiles] = {r0, r0 + 16, r0 + 32, r0 + 48};
  for (int pp = W.p0; pp < W.p1; pp += kMfPass) {
    const int n = min(kMfPass, W.p1 - pp);
    if (threadIdx.x < kMfPass) src_row[threadIdx.x] = threadIdx.x < n ? pp + (int)threadIdx.x : -1;
    __syncthreads();
    f4 Ct[kMfTiles][2];
    mfma_pass<QT>(mats, trow, I, h, I, src_row, n, lds, TL, xhi, xlo, Ct);
#pragma unroll
    for (int nt = 0; nt < 2; nt++) {
      const int c = 16 * nt + lr;
      if (c < n) {
#pragma unroll
        for (int t = 0; t < kMfTiles; t++)
          *(float4 *)(y + (size_t)(pp + c) * H + trow[t] + 4 * qd) =
              make_float4(Ct[t][nt][0], Ct[t][nt][1], Ct[t][nt][2], Ct[t][nt][3]);
      }
    }
  }
}

// Upper bound on the MFMA experts of a call: each has more than MOE_MATVEC_MAX_TOKENS
// of the T * kprime slots, and at most T (one slot per token).
static long max_mfma_experts(int T, int kprime, int n_ids) {
  if (T <= MOE_MATVEC_MAX_TOKENS) return 0;
  const long by_slots = (long)T * kprime / (MOE_MATVEC_MAX_TOKENS + 1);
  return by_slots < n_ids ? by_slots : n_ids;
}

hipError_t launch_gateup_mfma(const LayerArgs &L, const float *x, int T, int kprime, const int32_t *sorted_slot,
                              const WorkRec *work, int n_ids, float *h, hipStream_t s) {
  const long n = max_mfma_experts(T, kprime, n_ids);
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)(n * (L.inter / 128)));
  if (L.formats & MOE_Q_IQ2XS_LIKE) {
    hipLaunchKernelGGL(k_gateup_mfma<MOE_Q_IQ2XS_LIKE>, grid, dim3(256), mfma_lds_bytes(MOE_Q_IQ2XS_LIKE), s, L, x,
                       kprime, sorted_slot, work, n_ids, h);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (L.formats & MOE_Q_IQ1M_LIKE)
    hipLaunchKernelGGL(k_gateup_mfma<MOE_Q_IQ1M_LIKE>, grid, dim3(256), mfma_lds_bytes(MOE_Q_IQ1M_LIKE), s, L, x,
                       kprime, sorted_slot, work, n_ids, h);
  return hipGetLastError();
}

hipError_t launch_down_mfma(const LayerArgs &L, const float *h, int T, int kprime, const WorkRec *work, int n_ids,
                            float *y, hipStream_t s) {
  const long n = max_mfma_experts(T, kprime, n_ids);
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)(n * (L.hidden / 256)));
  if (L.formats & MOE_Q_IQ2XS_LIKE) {
    hipLaunchKernelGGL(k_down_mfma<MOE_Q_IQ2XS_LIKE>, grid, dim3(256), mfma_lds_bytes(MOE_Q_IQ2XS_LIKE), s, L, h,
                       work, n_ids, y);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (L.formats & MOE_Q_IQ1M_LIKE)
    hipLaunchKernelGGL(k_down_mfma<MOE_Q_IQ1M_LIKE>, grid, dim3(256), mfma_lds_bytes(MOE_Q_IQ1M_LIKE), s, L, h, work,
                       n_ids, y);
  return hipGetLastError();
}

}  // namespace moe
