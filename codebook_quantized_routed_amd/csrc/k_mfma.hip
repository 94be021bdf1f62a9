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

constexpr int kMfPass = 16;              // token columns per pass (one 16-column tile)
static_assert(kMfPass == MOE_MFMA_TILE_TOKENS, "a tile of the work list is one pass");
constexpr int kMfTiles = 4;              // 16-row tiles per wave
constexpr int kXRow = 256 + 8;           // halves per staged column (16 bytes of padding)
constexpr int kXHalves = kMfPass * kXRow;  // one of hi / lo, one buffer

// LDS: grid tables, then two buffers of staged activations (hi, lo), then the pass's
// source rows.
__host__ __device__ inline size_t mfma_lds_bytes(int formats) {
  return table_layout(formats).bytes + 4 * kXHalves * sizeof(_Float16) + kMfPass * sizeof(int);
}

// The lane's codes of one tile row for one super-block.  IQ2: c = 8 codes (u16), s = the
// scale word, d = the binary16 d.  IQ1: c.xy = 8 index bytes, c.z = 8 nibbles, (s:c.w)
// = the sd word (d in its low half).  Offsets are 32-bit from the matrix bases, so the
// loads take a scalar base and a vector offset.
struct TileCodes {
  uint4 c;
  uint32_t s, d;
};

template <int QT>
__device__ __forceinline__ TileCodes load_tile_codes(const QMat &m, int cols, int row, int sb, int qd) {
  const uint32_t ng = cols >> 3, nb = cols >> 8, g0 = sb * 32 + 8 * qd, blk = row * nb + sb;
  TileCodes t;
  if constexpr (QT == MOE_Q_IQ2XS_LIKE) {
    t.c = load_stream16(m.s0 + (uint32_t)((row * ng + g0) * 2));
    t.s = *(const uint32_t *)(m.s1 + (uint32_t)(blk * 4));
    t.d = *(const uint16_t *)(m.s2 + (uint32_t)(blk * 2));
  } else {
    const uint2 ql = load_stream8(m.s0 + (uint32_t)(row * ng + g0));
    const uint32_t qh = __builtin_nontemporal_load((const uint32_t *)(m.s1 + (uint32_t)(row * (ng / 2) + g0 / 2)));
    const uint2 sd = *(const uint2 *)(m.s2 + (uint32_t)(blk * 8));
    t.c = make_uint4(ql.x, ql.y, qh, sd.x);
    t.s = sd.y;
    t.d = sd.x & 0xFFFFu;
  }
  return t;
}

// d / 8 of the lane's four C rows 4 qd + i of a tile, taken from the lanes that hold
// those rows' codes (lane j holds row j % 16).
__device__ __forceinline__ void c_row_factors(const TileCodes &t, int qd, float (&df)[4]) {
  const float mine = half_bits_to_float(t.d) * 0.125f;
#pragma unroll
  for (int i = 0; i < 4; i++) df[i] = __shfl(mine, 4 * qd + i, 64);
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

// Staging of 256 columns of the pass's kMfPass activation rows: thread t takes row
// t / 16, floats 16 (t % 16) .. + 15.  stage_load issues the global loads (src_row[c]
// < 0: zeros), stage_store splits each value into fp16 hi / lo halves in LDS.
struct XRegs {
  u32x4 v[4];
};

__device__ __forceinline__ XRegs stage_load(const float *base, int row_stride, const int *src_row, int col0) {
  const int c = threadIdx.x >> 4, part = threadIdx.x & 15;
  const int r = src_row[c];
  XRegs x;
  const u32x4 *p = (const u32x4 *)(base + (size_t)(r < 0 ? 0 : r) * row_stride + col0 + 16 * part);
#pragma unroll
  for (int i = 0; i < 4; i++) x.v[i] = r < 0 ? u32x4{0u, 0u, 0u, 0u} : p[i];
  return x;
}

__device__ __forceinline__ void stage_store(const XRegs &x, _Float16 *xhi, _Float16 *xlo) {
  const int c = threadIdx.x >> 4, part = threadIdx.x & 15;
  uint32_t hi[8], lo[8];
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const float a = __uint_as_float(x.v[i >> 1][2 * (i & 1)]), b = __uint_as_float(x.v[i >> 1][2 * (i & 1) + 1]);
    const _Float16 ah = (_Float16)a, bh = (_Float16)b;
    const _Float16 al = (_Float16)(a - (float)ah), bl = (_Float16)(b - (float)bh);
    hi[i] = (uint32_t)__builtin_bit_cast(uint16_t, ah) | ((uint32_t)__builtin_bit_cast(uint16_t, bh) << 16);
    lo[i] = (uint32_t)__builtin_bit_cast(uint16_t, al) | ((uint32_t)__builtin_bit_cast(uint16_t, bl) << 16);
  }
  u32x4 *dh = (u32x4 *)(xhi + c * kXRow + 16 * part), *dl = (u32x4 *)(xlo + c * kXRow + 16 * part);
  dh[0] = u32x4{hi[0], hi[1], hi[2], hi[3]};
  dh[1] = u32x4{hi[4], hi[5], hi[6], hi[7]};
  dl[0] = u32x4{lo[0], lo[1], lo[2], lo[3]};
  dl[1] = u32x4{lo[4], lo[5], lo[6], lo[7]};
}

// One pass: the wave's kMfTiles row tiles times the pass's (up to) 16 staged columns,
// over the K range [0, cols) in super-blocks.  Super-block sb + 1's activations, codes
// and scales are loaded while sb is computed; the staged activations alternate
// between two LDS buffers, with one workgroup barrier per super-block.  Ct[t]: the
// fp32 result of tile t.  The caller has built the grid tables and set src_row.
template <int QT>
__device__ __forceinline__ void mfma_pass(const QMat (&mats)[kMfTiles], const int (&trow)[kMfTiles], int cols,
                                          const float *xbase, int x_stride, const int *src_row, const uint8_t *lds,
                                          const TableLayout &TL, _Float16 *xbuf, f4 (&Ct)[kMfTiles]) {
  const int lane = threadIdx.x & 63, qd = lane >> 4, lr = lane & 15;
  const int nsb = cols >> 8;
#pragma unroll
  for (int t = 0; t < kMfTiles; t++) Ct[t] = f4{0.0f, 0.0f, 0.0f, 0.0f};
  TileCodes tc[kMfTiles];
#pragma unroll
  for (int t = 0; t < kMfTiles; t++) tc[t] = load_tile_codes<QT>(mats[t], cols, trow[t] + lr, 0, qd);
  stage_store(stage_load(xbase, x_stride, src_row, 0), xbuf, xbuf + kXHalves);
  __syncthreads();
  for (int sb = 0; sb < nsb; sb++) {
    const _Float16 *xhi = xbuf + (sb & 1) * 2 * kXHalves, *xlo = xhi + kXHalves;
    const bool more = sb + 1 < nsb;
    XRegs xn;
    TileCodes nx[kMfTiles];
    if (more) {
      xn = stage_load(xbase, x_stride, src_row, (sb + 1) * 256);
#pragma unroll
      for (int t = 0; t < kMfTiles; t++) nx[t] = load_tile_codes<QT>(mats[t], cols, trow[t] + lr, sb + 1, qd);
    }
    f4 Cs[kMfTiles];
#pragma unroll
    for (int t = 0; t < kMfTiles; t++) Cs[t] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < 8; ks++) {
      const int koff = lr * kXRow + (8 * qd + ks) * 8;
      const h8 bh = *(const h8 *)(xhi + koff), bl = *(const h8 *)(xlo + koff);
#pragma unroll
      for (int t = 0; t < kMfTiles; t++) {
        const h8 A = decode_a<QT>(tc[t], ks, qd, lds, TL);
        Cs[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, bh, Cs[t], 0, 0, 0);
        Cs[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, bl, Cs[t], 0, 0, 0);
      }
    }
#pragma unroll
    for (int t = 0; t < kMfTiles; t++) {
      float df[4];
      c_row_factors(tc[t], qd, df);
#pragma unroll
      for (int i = 0; i < 4; i++) Ct[t][i] = fmaf(Cs[t][i], df[i], Ct[t][i]);
    }
    if (more) {
      _Float16 *nh = xbuf + ((sb + 1) & 1) * 2 * kXHalves;
      stage_store(xn, nh, nh + kXHalves);
#pragma unroll
      for (int t = 0; t < kMfTiles; t++) tc[t] = nx[t];
    }
    __syncthreads();
  }
}

// Tile i of the matrix-core experts: (expert, p0, p1, 0), stored after the n_ids + 1
// records of the work list.
__device__ __forceinline__ WorkRec mfma_tile(const WorkRec *work, int n_ids, int i) {
  return load_work(work, n_ids + 1 + i);
}

// gate + up + SiLU * up.  Workgroup = (tile, block of 128 rows of inter); wave
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
  if (a >= sload(&work[0].slot0)) return;  // record 0 = (matvec experts, slots, MFMA experts, tiles)
  const WorkRec W = mfma_tile(work, n_ids, a);
  const BankArgs &B = bank_of(L, W.e);
  if (B.qtype != QT) return;
  const TableLayout TL = table_layout(QT);
  _Float16 *xbuf = (_Float16 *)(lds + TL.bytes);
  int *src_row = (int *)(xbuf + 4 * kXHalves);
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
    f4 Ct[kMfTiles];
    mfma_pass<QT>(mats, trow, H, x, H, src_row, lds, TL, xbuf, Ct);
    if (lr < n) {
#pragma unroll
      for (int j = 0; j < 2; j++) {
        float4 o;
        o.x = silu(Ct[j][0]) * Ct[2 + j][0];
        o.y = silu(Ct[j][1]) * Ct[2 + j][1];
        o.z = silu(Ct[j][2]) * Ct[2 + j][2];
        o.w = silu(Ct[j][3]) * Ct[2 + j][3];
        *(float4 *)(h + (size_t)(pp + lr) * I + r0 + 16 * j + 4 * qd) = o;
      }
    }
  }
}

// down: y[p] = Wd h[p].  Workgroup = (tile, block of 256 rows of hidden); wave w
// takes rows r0 .. r0 + 63, r0 = 256 * block + 64 w.  h rows are contiguous per expert.
// One instance per format, as above.
template <int QT>
__global__ void __launch_bounds__(256) k_down_mfma(LayerArgs L, const float *__restrict__ h,
                                                   const WorkRec *__restrict__ work, int n_ids,
                                                   float *__restrict__ y) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int H = L.hidden, I = L.inter, RB = H / 256;
  const int a = blockIdx.x / RB, rb = blockIdx.x - a * RB;
  if (a >= sload(&work[0].slot0)) return;
  const WorkRec W = mfma_tile(work, n_ids, a);
  const BankArgs &B = bank_of(L, W.e);
  if (B.qtype != QT) return;
  const TableLayout TL = table_layout(QT);
  _Float16 *xbuf = (_Float16 *)(lds + TL.bytes);
  int *src_row = (int *)(xbuf + 4 * kXHalves);
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
    f4 Ct[kMfTiles];
    mfma_pass<QT>(mats, trow, I, h, I, src_row, lds, TL, xbuf, Ct);
    if (lr < n) {
#pragma unroll
      for (int t = 0; t < kMfTiles; t++)
        *(float4 *)(y + (size_t)(pp + lr) * H + trow[t] + 4 * qd) = make_float4(Ct[t][0], Ct[t][1], Ct[t][2], Ct[t][3]);
    }
  }
}

hipError_t launch_gateup_mfma(const LayerArgs &L, const float *x, int T, int kprime, const int32_t *sorted_slot,
                              const WorkRec *work, int n_ids, float *h, hipStream_t s) {
  const long n = max_mfma_tiles(T, kprime, n_ids);
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
  const long n = max_mfma_tiles(T, kprime, n_ids);
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
