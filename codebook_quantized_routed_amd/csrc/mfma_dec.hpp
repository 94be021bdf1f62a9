// Matrix-core decode of codebook-quantized rows for few tokens per expert.
//
// "Red Metal dev8 — resident routed top-k layer", step 4: every selected expert runs
// gate, up, SiLU(gate) * up and down from its resident weights; "Red Lite dev10 —
// standalone native Metal path", section "Quant grids": the IQ2_XS grid over
// 0x08 / 0x19 / 0x2b and the IQ1_M grid over -1 / 0 / +1, expanded once.
//
// The multiply-adds of a mat-vec run on v_mfma_f32_16x16x32_f16 instead of the VALU:
//  - B operand (32 k x 16 columns): column n = one weight row; lane l holds row
//    l % 16 and k slots 8 (l / 16) .. + 7, i.e. one 8-weight group of that row.  The
//    lane decodes the group straight into 8 fp16 values that are exact:
//      IQ2_XS-like: (2s + 1) * (+-G), G in {8, 25, 43}: |value| <= 31 * 43 < 2048;
//      IQ1_M-like:  (2s + 1) * (G +- 1/8), G in {-1, 0, 1}: eighths up to 135 / 8.
//    IQ2 groups read two LDS rows: the fp16 grid row, and a row of signed scales
//    +-(2s + 1) indexed by (the 7 sign bits, s) -- the 8th sign is their parity -- and
//    multiply them pairwise (4 packed fp16 multiplies).  IQ1 groups read one row of grid
//    values with the group's delta already added (index + 2048 * delta sign) and scale it.
//  - A operand (16 rows x 32 k): row m = activation vector m / 2, split into
//    x_hi = fp16(x * 2^e) (m even) and x_lo = fp16(x * 2^e - x_hi) (m odd); 2^e is a
//    power of two per vector that puts its largest magnitude in [2^13, 2^14), so both
//    halves are normal fp16 numbers for every element that matters and the products
//    carry about 22 bits of x.  Products hi * w and lo * w are exact in fp32.
//  - D (16 x 16): lane l holds D[4 (l / 16) + i][l % 16]: for column (weight row)
//    n = l % 16 the rows of vectors 2 (l / 16) and 2 (l / 16) + 1, hi and lo each.
// The k slots of lane quarter q at step s of a 256-column super-block stand for group
// 8 q + s (columns 64 q + 8 s .. + 7), so a lane's eight groups of a super-block are
// contiguous in its row's code stream.  Each super-block's D starts from zero; its
// (hi + lo) sums are scaled by the super-block factor d / 8 (IQ2) or d (IQ1) -- the
// lane's own row -- and added into the lane's partial, super-block by super-block.
// Every dequantized weight is exact (the factor products are exact in fp32); only the
// summation order differs from a sequential dot product.
#pragma once
#include "matvec_common.hpp"

namespace moe {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));

// ----------------------------------------------------------------------------- LDS tables
// Byte offsets in dynamic LDS (-1: not built).  iq2h: fp16 grid rows [512][8]; iq2ss:
// signed scales [128 sign patterns][16 scales][8]; iq1d: grid rows plus delta
// [2 (delta sign)][2048][8].
struct DecTables {
  int iq2h, iq2ss, iq1d, bytes;
};

__host__ __device__ constexpr DecTables dec_tables(int formats) {
  DecTables t{-1, -1, -1, 0};
  if (formats & MOE_Q_IQ2XS_LIKE) {
    t.iq2h = t.bytes;
    t.bytes += kIq2Rows * 16;
    t.iq2ss = t.bytes;
    t.bytes += 128 * 16 * 16;
  }
  if (formats & MOE_Q_IQ1M_LIKE) {
    t.iq1d = t.bytes;
    t.bytes += 2 * kIq1Rows * 16;
  }
  return t;
}

static_assert(kGridDecBytes == (size_t)dec_tables(MOE_Q_IQ2XS_LIKE | MOE_Q_IQ1M_LIKE).bytes,
              "the grid buffer holds the decode tables of both formats");

// Copy of the decode tables of format(s) QT from the grid buffer (written there once by
// moe_grids_expand) into LDS at dec_tables(QT): thread t of n (n >= 256) takes the
// 16-byte words t, t + n, ...  The loads are issued unconditionally (clamped) so they
// leave together; call dec_tables_copy_store after whatever else should travel with them.
struct DecTableCopy {
  uint4 w[4];
};
template <int QT>
__device__ __forceinline__ DecTableCopy dec_tables_copy_load(const uint8_t *grids, int t, int n) {
  // the IQ1 rows follow the IQ2 tables in the grid buffer
  constexpr size_t src_off = QT == MOE_Q_IQ1M_LIKE ? kIq2Rows * 16 + 128 * 16 * 16 : 0;
  constexpr int words = (int)(dec_tables(QT).bytes / 16);
  static_assert(words <= 4 * 1024, "at most four words per thread of a 1024-thread block");
  const uint4 *src = (const uint4 *)(grids + kGridDecOff + src_off);
  DecTableCopy c;
#pragma unroll
  for (int k = 0; k < 4; k++) c.w[k] = src[min(t + k * n, words - 1)];
  return c;
}
template <int QT>
__device__ __forceinline__ void dec_tables_copy_store(const DecTableCopy &c, uint8_t *lds, int t, int n) {
  constexpr int words = (int)(dec_tables(QT).bytes / 16);
  uint4 *dst = (uint4 *)lds;
#pragma unroll
  for (int k = 0; k < 4; k++)
    if (t + k * n < words) dst[t + k * n] = c.w[k];
}

// The compact rows a loader thread expands (issued early: the loads of the table build).
struct DecTableRegs {
  uint32_t c2[2], c1[8];
};

// Loader t of n (n >= 256).
__device__ __forceinline__ DecTableRegs dec_tables_load(const uint8_t *grids, int formats, int t, int n) {
  DecTableRegs r;
  const uint16_t *c2 = (const uint16_t *)(grids + kGridIq2CompactOff);
  const uint16_t *c1 = (const uint16_t *)(grids + kGridIq1CompactOff);
#pragma unroll
  for (int i = 0; i < 2; i++) {
    const int row = t + i * n;
    r.c2[i] = (formats & MOE_Q_IQ2XS_LIKE) && t >= 0 && row < kIq2Rows ? c2[row] : 0u;
  }
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const int row = t + i * n;
    r.c1[i] = (formats & MOE_Q_IQ1M_LIKE) && t >= 0 && row < kIq1Rows ? c1[row] : 0u;
  }
  return r;
}

__device__ __forceinline__ uint32_t f16x2_bits(float a, float b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) | ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
}

// Expands the tables into LDS (no barrier).
__device__ __forceinline__ void dec_tables_store(const DecTableRegs &r, int formats, const DecTables &D, uint8_t *lds,
                                                 int t, int n) {
  if (t < 0) return;
  if (formats & MOE_Q_IQ2XS_LIKE) {
    const uint32_t h0 = f16_bits((float)kIq2SymVal[0]), h1 = f16_bits((float)kIq2SymVal[1]),
                   h2_ = f16_bits((float)kIq2SymVal[2]);
    uint4 *rows = (uint4 *)(lds + D.iq2h);
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const int row = t + i * n;
      if (row < kIq2Rows) rows[row] = expand_row_f16(r.c2[i], h0, h1, h2_);
    }
    uint4 *ss = (uint4 *)(lds + D.iq2ss);
    for (int e = t; e < 128 * 16; e += n) {
      const uint32_t s7 = (uint32_t)e >> 4, sc = (uint32_t)e & 15u;
      const uint32_t S = s7 | ((__builtin_popcount(s7) & 1u) << 7);
      const float v = (float)(2 * sc + 1);
      uint32_t w[4];
#pragma unroll
      for (int p = 0; p < 4; p++)
        w[p] = f16x2_bits((S >> (2 * p)) & 1u ? -v : v, (S >> (2 * p + 1)) & 1u ? -v : v);
      ss[e] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
  if (formats & MOE_Q_IQ1M_LIKE) {
    const float d = 0.125f;
    const uint32_t p0 = f16_bits((float)kIq1SymVal[0] + d), p1 = f16_bits((float)kIq1SymVal[1] + d),
                   p2 = f16_bits((float)kIq1SymVal[2] + d);
    const uint32_t m0 = f16_bits((float)kIq1SymVal[0] - d), m1 = f16_bits((float)kIq1SymVal[1] - d),
                   m2 = f16_bits((float)kIq1SymVal[2] - d);
    uint4 *rows = (uint4 *)(lds + D.iq1d);
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const int row = t + i * n;
      if (row < kIq1Rows) {
        rows[row] = expand_row_f16(r.c1[i], p0, p1, p2);
        rows[row + kIq1Rows] = expand_row_f16(r.c1[i], m0, m1, m2);
      }
    }
  }
}

// ----------------------------------------------------------------------------- codes
// One lane's codes of one (row, 256-column super-block): its 8 groups 8 q .. 8 q + 7.
//  IQ2: c = the 8 u16 codes, w = the scale word, d = the fp16 d bits.
//  IQ1: c.xy = the 8 index bytes, c.z = the 8 nibbles, (c.w, w) = the sd word.
struct SbCodes {
  u32x4 c;  // a native vector type: keeps the struct in registers through the unit loops
  uint32_t w, d;
};

template <int QT>
__device__ __forceinline__ SbCodes load_sb(const QMat &m, int cols, int row, int sb, int q) {
  const uint32_t ng = (uint32_t)cols >> 3, nb = (uint32_t)cols >> 8, g0 = (uint32_t)sb * 32 + 8 * q;
  const uint32_t blk = (uint32_t)row * nb + sb;
  SbCodes t;
  if constexpr (QT == MOE_Q_IQ2XS_LIKE) {
    t.c = __builtin_nontemporal_load((const u32x4 *)(m.s0 + (size_t)((uint32_t)row * ng + g0) * 2));
    t.w = *(const uint32_t *)(m.s1 + (size_t)blk * 4);
    t.d = *(const uint16_t *)(m.s2 + (size_t)blk * 2);
  } else {
    // (native vector types throughout: the struct then stays in registers)
    const u32x2 ql = __builtin_nontemporal_load((const u32x2 *)(m.s0 + (size_t)((uint32_t)row * ng + g0)));
    const uint32_t qh = __builtin_nontemporal_load((const uint32_t *)(m.s1 + (size_t)((uint32_t)row * (ng / 2) + g0 / 2)));
    const u32x2 sd = *(const u32x2 *)(m.s2 + (size_t)blk * 8);
    t.c = u32x4{ql.x, ql.y, qh, sd.x};
    t.w = sd.y;
    t.d = sd.x & 0xFFFFu;
  }
  return t;
}

// The super-block factor of the lane's row: d / 8 (IQ2) or d (IQ1), exact.
template <int QT>
__device__ __forceinline__ float sb_factor(const SbCodes &t) {
  const float d = half_bits_to_float(t.d);
  return QT == MOE_Q_IQ2XS_LIKE ? d * 0.125f : d;
}

__device__ __forceinline__ h2 f16_pair_of(uint32_t v) {
  const _Float16 f = (_Float16)(float)v;
  return h2{f, f};
}

// The LDS rows of step s (group 8 q + s of the lane's row) and the A fragment, read
// ahead of their use: g = the grid row (IQ1: with the delta), m = the signed-scale row
// (IQ2) or the scale pair (IQ1, in m.x).
struct StepRaw {
  uint4 g, m;
  h8 a;
};

template <int QT>
__device__ __forceinline__ void fetch_b(const SbCodes &t, int s, int q, const uint8_t *lds, const DecTables &D,
                                        StepRaw &r) {
  if constexpr (QT == MOE_Q_IQ2XS_LIKE) {
    const uint32_t w = s < 2 ? t.c.x : (s < 4 ? t.c.y : (s < 6 ? t.c.z : t.c.w));
    const uint32_t code = (s & 1) ? (w >> 16) : (w & 0xFFFFu);
    r.g = *(const uint4 *)(lds + D.iq2h + (code & 0x1FFu) * 16);
    const uint32_t sc = (t.w >> (4 * (2 * q + (s >> 2)))) & 15u;
    r.m = *(const uint4 *)(lds + D.iq2ss + ((((code >> 9) & 0x7Fu) << 4) | sc) * 16);
  } else {
    const uint32_t ql8 = ((s < 4 ? t.c.x : t.c.y) >> (8 * (s & 3))) & 0xFFu;
    const uint32_t nib = (t.c.z >> (4 * s)) & 15u;
    r.g = *(const uint4 *)(lds + D.iq1d + (ql8 | (nib << 8)) * 16);
    const uint64_t sd = ((uint64_t)t.w << 32) | t.c.w;
    const uint32_t sub = 4 * q + (s >> 1);
    r.m.x = __builtin_bit_cast(uint32_t, f16_pair_of(2 * (uint32_t)((sd >> (16 + 3 * sub)) & 7u) + 1));
  }
}

template <int QT>
__device__ __forceinline__ h8 combine_b(const StepRaw &r) {
  uint4 v = r.g;
  h2 *pv = (h2 *)&v;
  if constexpr (QT == MOE_Q_IQ2XS_LIKE) {
    const h2 *pm = (const h2 *)&r.m;
#pragma unroll
    for (int i = 0; i < 4; i++) pv[i] = pv[i] * pm[i];
  } else {
    const h2 f = __builtin_bit_cast(h2, r.m.x);
#pragma unroll
    for (int i = 0; i < 4; i++) pv[i] = pv[i] * f;
  }
  return __builtin_bit_cast(h8, v);
}

// The B fragment of step s: group 8 q + s of the lane's row, decoded to 8 exact fp16.
template <int QT>
__device__ __forceinline__ h8 dec_b(const SbCodes &t, int s, int q, const uint8_t *lds, const DecTables &D) {
  uint4 v;
  h2 f;
  if constexpr (QT == MOE_Q_IQ2XS_LIKE) {
    const uint32_t w = s < 2 ? t.c.x : (s < 4 ? t.c.y : (s < 6 ? t.c.z : t.c.w));
    const uint32_t code = (s & 1) ? (w >> 16) : (w & 0xFFFFu);
    v = *(const uint4 *)(lds + D.iq2h + (code & 0x1FFu) * 16);
    // the signed-scale row: (7 sign bits, the 4-bit scale of sub-block 2 q + s / 4)
    const uint32_t sc = (t.w >> (4 * (2 * q + (s >> 2)))) & 15u;
    const uint4 m = *(const uint4 *)(lds + D.iq2ss + ((((code >> 9) & 0x7Fu) << 4) | sc) * 16);
    h2 *pv = (h2 *)&v;
    const h2 *pm = (const h2 *)&m;
#pragma unroll
    for (int i = 0; i < 4; i++) pv[i] = pv[i] * pm[i];
    (void)f;
  } else {
    const uint32_t ql8 = ((s < 4 ? t.c.x : t.c.y) >> (8 * (s & 3))) & 0xFFu;
    const uint32_t nib = (t.c.z >> (4 * s)) & 15u;
    v = *(const uint4 *)(lds + D.iq1d + (ql8 | (nib << 8)) * 16);
    const uint64_t sd = ((uint64_t)t.w << 32) | t.c.w;
    const uint32_t sub = 4 * q + (s >> 1);
    f = f16_pair_of(2 * (uint32_t)((sd >> (16 + 3 * sub)) & 7u) + 1);
    h2 *pv = (h2 *)&v;
#pragma unroll
    for (int i = 0; i < 4; i++) pv[i] = pv[i] * f;
  }
  return __builtin_bit_cast(h8, v);
}

// Lane-wise choice between two matrices (each computed from wave-uniform values).
__device__ __forceinline__ QMat pick_mat(bool first, const QMat &a, const QMat &b) {
  return QMat{first ? a.s0 : b.s0, first ? a.s1 : b.s1, first ? a.s2 : b.s2};
}

// Workgroup barrier that orders LDS accesses only: global stores of the threads are not
// waited for (a full __syncthreads would wait for them, and vector memory operations
// complete in order, so it would also wait for loads issued earlier for later work).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ f4 mfma16(const h8 &a, const h8 &b, const f4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// ----------------------------------------------------------------------------- activations
// Staged activation vectors: per vector, the hi and the lo row of fp16, each `row`
// halves long; column c sits at c + 8 (c / 64) (16 bytes of padding after every 64
// columns, so the four lane quarters of a fragment read hit different banks) and the
// row length is a multiple of 4 banks plus 4 (so consecutive rows do too).
__host__ __device__ inline int stage_row_halves(int cols) { return cols + cols / 8 + 8; }
__device__ __forceinline__ int stage_col(int c) { return c + ((c >> 6) << 3); }

// 2^e putting max|v| into [2^13, 2^14) (e = 0 for an all-zero vector), clamped to the
// normal range of fp32.
__device__ __forceinline__ int stage_exponent(float maxabs) {
  if (!(maxabs > 0.0f)) return 0;
  const int ex = (int)((__float_as_uint(maxabs) >> 23) & 0xFFu) - 127;
  const int e = 13 - ex;
  return e < -126 ? -126 : (e > 127 ? 127 : e);
}
__device__ __forceinline__ float pow2f(int e) { return ldexpf(1.0f, e); }

// Splits v * scale into (hi, lo) fp16 bit pairs.
__device__ __forceinline__ void split_hl(float v, float scale, uint16_t &hi, uint16_t &lo) {
  const float s = v * scale;
  const _Float16 h = (_Float16)s;
  hi = __builtin_bit_cast(uint16_t, h);
  lo = __builtin_bit_cast(uint16_t, (_Float16)(s - (float)h));
}

// Four consecutive values (columns c .. c + 3, c % 4 == 0) of a vector into its staged
// hi and lo rows.
__device__ __forceinline__ void stage4(_Float16 *hi_row, _Float16 *lo_row, int c, float4 v, float scale) {
  uint16_t h[4], l[4];
  split_hl(v.x, scale, h[0], l[0]);
  split_hl(v.y, scale, h[1], l[1]);
  split_hl(v.z, scale, h[2], l[2]);
  split_hl(v.w, scale, h[3], l[3]);
  const int o = stage_col(c);
  *(uint2 *)(hi_row + o) = make_uint2(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16));
  *(uint2 *)(lo_row + o) = make_uint2(l[0] | ((uint32_t)l[1] << 16), l[2] | ((uint32_t)l[3] << 16));
}

// The A fragment of step s of super-block sb: row m of the fragment is the staged row
// `row_of_m` (hi or lo of a vector); when row_of_m < 0 it reads the 16 zero bytes at
// `zero` instead (an address select, not a branch around the read).
__device__ __forceinline__ h8 load_a(const _Float16 *staged, int row_halves, int row_of_m, int sb, int q, int s,
                                     const _Float16 *zero) {
  const _Float16 *p = staged + (size_t)max(row_of_m, 0) * row_halves + stage_col(sb * 256 + 64 * q) + 8 * s;
  return *(const h8 *)(row_of_m < 0 ? zero : p);
}

// ----------------------------------------------------------------------------- one row block
// The partial dot products of the lane's weight row (B column n = lane % 16) with the
// vectors of the fragment (rows 2 (lane / 16), 2 (lane / 16) + 1) over super-blocks
// sb0 .. sb0 + NSB - 1: NSB independent MFMA chains (one per super-block, interleaved),
// each scaled by its factor and added in super-block order.  r0 / r1: the partials of
// vectors 2 (lane / 16) and 2 (lane / 16) + 1.
template <int QT, int NSB>
__device__ __forceinline__ void dot_sb(const SbCodes (&c)[NSB], int sb0, const _Float16 *staged, int row_halves,
                                       int row_of_m, int q, const uint8_t *lds, const DecTables &D,
                                       const _Float16 *zero, float &r0, float &r1) {
  f4 acc[NSB];
#pragma unroll
  for (int i = 0; i < NSB; i++) acc[i] = f4{0.0f, 0.0f, 0.0f, 0.0f};
  // one software pipeline over the NSB x 8 steps (super-block by super-block): the LDS
  // reads of step k + 1 are issued before the MFMA of step k
  StepRaw cur, nxt;
  fetch_b<QT>(c[0], 0, q, lds, D, cur);
  cur.a = load_a(staged, row_halves, row_of_m, sb0, q, 0, zero);
#pragma unroll
  for (int k = 0; k < 8 * NSB; k++) {
    const int i = k >> 3;
    if (k + 1 < 8 * NSB) {
      const int i1 = (k + 1) >> 3, s1 = (k + 1) & 7;
      fetch_b<QT>(c[i1], s1, q, lds, D, nxt);
      nxt.a = load_a(staged, row_halves, row_of_m, sb0 + i1, q, s1, zero);
    }
    acc[i] = mfma16(cur.a, combine_b<QT>(cur), acc[i]);
    cur = nxt;
  }
#pragma unroll
  for (int i = 0; i < NSB; i++) {
    const float f = sb_factor<QT>(c[i]);
    r0 = fmaf(acc[i][0] + acc[i][1], f, r0);
    r1 = fmaf(acc[i][2] + acc[i][3], f, r1);
  }
}

}  // namespace moe
