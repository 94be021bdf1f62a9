// Device functions of the mat-vec kernels (lane slices of quantized rows, dot products
// against fp32 activations), shared by the mat-vec kernels and the fused decode-layer
// kernel.
#pragma once
#include "matvec_common.hpp"

namespace moe {

// A lane's slice of one row.  IQ2: a = 8 codes, b = (sc word, d bits).
// IQ1: a.xy = 8 ql bytes, a.z = 4 qh bytes, b = the 64-bit sd word.
struct RowRaw {
  uint4 a;
  uint2 b;
};

// Hides a row's codes from loop-invariant code motion, which would otherwise decode
// the row once before a token loop and keep every decoded weight live.
__device__ __forceinline__ void opaque(RowRaw &R) {
  asm volatile("" : "+v"(R.a.x), "+v"(R.a.y), "+v"(R.a.z), "+v"(R.a.w), "+v"(R.b.x), "+v"(R.b.y));
}

template <int QT>
__device__ __forceinline__ RowRaw load_row(const QMat &m, int cols, int r, int q) {
  const int ng = cols >> 3, nb = cols >> 8, b = q >> 2;
  RowRaw R;
  if constexpr (QT == MOE_Q_IQ2XS_LIKE) {
    R.a = load_stream16(m.s0 + ((size_t)r * ng + 8 * q) * 2);
    R.b.x = ((const uint32_t *)m.s1)[(size_t)r * nb + b];
    R.b.y = ((const uint16_t *)m.s2)[(size_t)r * nb + b];
  } else {
    const uint2 ql = load_stream8(m.s0 + (size_t)r * ng + 8 * q);
    const uint32_t qh = __builtin_nontemporal_load((const uint32_t *)(m.s1 + (size_t)r * (ng / 2) + 4 * q));
    R.a = make_uint4(ql.x, ql.y, qh, 0u);
    R.b = *(const uint2 *)(m.s2 + ((size_t)r * nb + b) * 8);
  }
  return R;
}

// Activation slice of a lane: 64 floats, plus the 8 group sums times 1/8 (IQ1 only).
struct XChunk {
  float v[64];
  float gs8[8];
};

template <int QT>
__device__ __forceinline__ void load_x(const float *p, XChunk &X) {
  const float4 *p4 = (const float4 *)p;
#pragma unroll
  for (int i = 0; i < 16; i++) {
    const float4 f = p4[i];
    X.v[4 * i] = f.x;
    X.v[4 * i + 1] = f.y;
    X.v[4 * i + 2] = f.z;
    X.v[4 * i + 3] = f.w;
  }
  if constexpr (QT == MOE_Q_IQ1M_LIKE) {
#pragma unroll
    for (int g = 0; g < 8; g++) {
      float s = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; j++) s += X.v[8 * g + j];
      X.gs8[g] = s * 0.125f;
    }
  }
}

// ----------------------------------------------------------------------------- dot
__device__ __forceinline__ float lo16(uint32_t w) { return (float)__builtin_bit_cast(f16x2, w).x; }
__device__ __forceinline__ float hi16(uint32_t w) { return (float)__builtin_bit_cast(f16x2, w).y; }

// 8 weights (4 packed fp16 pairs) times 8 activations added into two accumulation
// chains (even and odd columns); each step is one v_fma_mix_f32.
__device__ __forceinline__ void dot8(const uint4 &w, const float *x, float &a, float &b) {
  a = fmaf(lo16(w.x), x[0], a);
  b = fmaf(hi16(w.x), x[1], b);
  a = fmaf(lo16(w.y), x[2], a);
  b = fmaf(hi16(w.y), x[3], b);
  a = fmaf(lo16(w.z), x[4], a);
  b = fmaf(hi16(w.z), x[5], b);
  a = fmaf(lo16(w.w), x[6], a);
  b = fmaf(hi16(w.w), x[7], b);
}

// Dot product of a lane's 64-column slice of one row with its activation slice.
template <int QT>
__device__ __forceinline__ float dot_chunk(const RowRaw &R, int q, const uint8_t *lds, const TableLayout &TL,
                                           const XChunk &X) {
  if constexpr (QT == MOE_Q_IQ2XS_LIKE) {
    const uint4 *rows = (const uint4 *)(lds + TL.iq2h);
    const uint4 *masks = (const uint4 *)(lds + TL.iq2m);
    float a[2] = {0.0f, 0.0f}, b[2] = {0.0f, 0.0f};
#pragma unroll
    for (int g = 0; g < 8; g++) {
      const uint32_t w32 = g < 2 ? R.a.x : (g < 4 ? R.a.y : (g < 6 ? R.a.z : R.a.w));
      const uint32_t code = (g & 1) ? (w32 >> 16) : (w32 & 0xFFFFu);
      uint4 v = rows[code & 0x1FFu];
      const uint4 m = masks[(code >> 9) & 0x7Fu];
      v.x ^= m.x;
      v.y ^= m.y;
      v.z ^= m.z;
      v.w ^= m.w;
      dot8(v, X.v + 8 * g, a[g >> 2], b[g >> 2]);
    }
    const float acc[2] = {a[0] + b[0], a[1] + b[1]};
    const int sb = 2 * (q & 3);
    return fmaf(acc[1], iq2_factor(R.b.x, R.b.y, sb + 1), acc[0] * iq2_factor(R.b.x, R.b.y, sb));
  } else {
    const uint4 *rows = (const uint4 *)(lds + TL.iq1h);
    float a[4] = {0.0f, 0.0f, 0.0f, 0.0f}, b[4] = {0.0f, 0.0f, 0.0f, 0.0f}, ds[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int g = 0; g < 8; g++) {
      const uint32_t ql8 = ((g < 4 ? R.a.x : R.a.y) >> (8 * (g & 3))) & 0xFFu;
      const uint32_t nib = (R.a.z >> (4 * g)) & 15u;
      const uint4 v = rows[ql8 | ((nib & 7u) << 8)];
      ds[g >> 1] += (nib & 8u) ? -X.gs8[g] : X.gs8[g];
      dot8(v, X.v + 8 * g, a[g >> 1], b[g >> 1]);
    }
    float acc[4];
#pragma unroll
    for (int i = 0; i < 4; i++) acc[i] = (a[i] + b[i]) + ds[i];
    const uint64_t sd = ((uint64_t)R.b.y << 32) | R.b.x;
    const int sb = 4 * (q & 3);
    float r = acc[0] * iq1_factor(sd, sb);
    r = fmaf(acc[1], iq1_factor(sd, sb + 1), r);
    r = fmaf(acc[2], iq1_factor(sd, sb + 2), r);
    return fmaf(acc[3], iq1_factor(sd, sb + 3), r);
  }
}

// ----------------------------------------------------------------------------- gate + up, hidden 2048
// Decode layout for hidden = 2048: a whole wave covers one row (32 columns per lane), so
// a lane's activation slice is 32 floats with no copy shared between lanes, loaded once
// per wave while the wave's items keep the same token.  An item is kWideRows rows of one
// expert, gate and up.  Issue order: compact-table loads, work record (scalar), row and
// activation loads, then the table build; compute waits only for what it uses.
constexpr int kWideRows = 2;

struct Row32 {  // IQ2: x = codes 0-1, y = codes 2-3, z = sc word, w = d bits.
  uint4 v;      // IQ1: x = 4 ql bytes, y = 4 qh nibbles (16 bits), z/w = the sd word.
};

__device__ __forceinline__ void opaque(Row32 &R) { asm volatile("" : "+v"(R.v.x), "+v"(R.v.y), "+v"(R.v.z), "+v"(R.v.w)); }

template <int QT>
__device__ __forceinline__ Row32 load_row32(const QMat &m, int cols, int r, int q) {
  const int ng = cols >> 3, nb = cols >> 8, b = q >> 3;
  Row32 R;
  if constexpr (QT == MOE_Q_IQ2XS_LIKE) {
    const uint2 c = load_stream8(m.s0 + ((size_t)r * ng + 4 * q) * 2);
    R.v = make_uint4(c.x, c.y, ((const uint32_t *)m.s1)[(size_t)r * nb + b], ((const uint16_t *)m.s2)[(size_t)r * nb + b]);
  } else {
    const uint32_t ql = __builtin_nontemporal_load((const uint32_t *)(m.s0 + (size_t)r * ng + 4 * q));
    const uint32_t qh = __builtin_nontemporal_load((const uint16_t *)(m.s1 + (size_t)r * (ng / 2) + 2 * q));
    const uint2 sd = *(const uint2 *)(m.s2 + ((size_t)r * nb + b) * 8);
    R.v = make_uint4(ql, qh, sd.x, sd.y);
  }
  return R;
}

struct X32 {
  float v[32];
};

template <int QT>
__device__ __forceinline__ float dot32(const Row32 &R, int q, const uint8_t *lds, const TableLayout &TL, const X32 &X) {
  if constexpr (QT == MOE_Q_IQ2XS_LIKE) {
    const uint4 *rows = (const uint4 *)(lds + TL.iq2h);
    const uint4 *masks = (const uint4 *)(lds + TL.iq2m);
    float a = 0.0f, b = 0.0f;
#pragma unroll
    for (int g = 0; g < 4; g++) {
      const uint32_t w32 = g < 2 ? R.v.x : R.v.y;
      const uint32_t code = (g & 1) ? (w32 >> 16) : (w32 & 0xFFFFu);
      uint4 v = rows[code & 0x1FFu];
      const uint4 m = masks[(code >> 9) & 0x7Fu];
      v.x ^= m.x;
      v.y ^= m.y;
      v.z ^= m.z;
      v.w ^= m.w;
      dot8(v, X.v + 8 * g, a, b);
    }
    return (a + b) * iq2_factor(R.v.z, R.v.w, q & 7);
  } else {
    // the delta rows: index bits 0-10 pick the grid row, bit 11 (the nibble's delta
    // sign) the half with -1/8 added instead of +1/8
    const uint4 *rows = (const uint4 *)(lds + TL.iq1d);
    float a[2] = {0.0f, 0.0f}, b[2] = {0.0f, 0.0f};
#pragma unroll
    for (int g = 0; g < 4; g++) {
      const uint32_t ql8 = (R.v.x >> (8 * g)) & 0xFFu;
      const uint32_t nib = (R.v.y >> (4 * g)) & 15u;
      dot8(rows[ql8 | (nib << 8)], X.v + 8 * g, a[g >> 1], b[g >> 1]);
    }
    const uint64_t sd = ((uint64_t)R.v.w << 32) | R.v.z;
    const int sb = 2 * (q & 7);
    return fmaf(a[1] + b[1], iq1_factor(sd, sb + 1), (a[0] + b[0]) * iq1_factor(sd, sb));
  }
}

__device__ __forceinline__ void load_x32(const float *p, X32 &X) {
  const float4 *p4 = (const float4 *)p;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const float4 f = p4[i];
    X.v[4 * i] = f.x;
    X.v[4 * i + 1] = f.y;
    X.v[4 * i + 2] = f.z;
    X.v[4 * i + 3] = f.w;
  }
}

struct WideItem {
  WorkRec W;
  Row32 g[kWideRows], u[kWideRows];
  int r0, qt;
};

// The loads of item rb (rows kWideRows * rb ..) of gate Wg and up Wu, format qt.
__device__ __forceinline__ void wide_issue_mats(WideItem &It, const QMat &Wg, const QMat &Wu, int qt, int H, int rb,
                                                int q) {
  It.qt = qt;
  It.r0 = rb * kWideRows;
#pragma unroll
  for (int i = 0; i < kWideRows; i++) {
    if (It.qt == MOE_Q_IQ2XS_LIKE) {
      It.g[i] = load_row32<MOE_Q_IQ2XS_LIKE>(Wg, H, It.r0 + i, q);
      It.u[i] = load_row32<MOE_Q_IQ2XS_LIKE>(Wu, H, It.r0 + i, q);
    } else {
      It.g[i] = load_row32<MOE_Q_IQ1M_LIKE>(Wg, H, It.r0 + i, q);
      It.u[i] = load_row32<MOE_Q_IQ1M_LIKE>(Wu, H, It.r0 + i, q);
    }
  }
}

// The same for an item known to have format QT: no format branch, so the compiler can
// count the item's loads exactly and wait for an older item without waiting for it.
template <int QT>
__device__ __forceinline__ void wide_issue_fmt(WideItem &It, const QMat &Wg, const QMat &Wu, int H, int rb, int q) {
  It.qt = QT;
  It.r0 = rb * kWideRows;
#pragma unroll
  for (int i = 0; i < kWideRows; i++) {
    It.g[i] = load_row32<QT>(Wg, H, It.r0 + i, q);
    It.u[i] = load_row32<QT>(Wu, H, It.r0 + i, q);
  }
}

__device__ __forceinline__ void wide_issue(const LayerArgs &L, WideItem &It, int rb, int q) {
  const int H = L.hidden, I = L.inter;
  const BankArgs &B = bank_of(L, It.W.e);
  wide_issue_mats(It, expert_mat(B, It.W.e, kGate, I, H), expert_mat(B, It.W.e, kUp, I, H), B.qtype, H, rb, q);
}

// COHERENT: h holds 64-bit (value bits, tag) pairs, each stored with one agent-scope
// relaxed atomic store (written through to the coherence point), for readers in other
// workgroups of the same launch; otherwise h holds floats.
// A token's activations: token t's slice of lane q starts at x + t * tok_stride +
// q * lane_stride (global memory: hidden and 32; LDS staging: its own padded layout).
struct XSource {
  const float *x;
  int tok_stride, lane_stride;
};

template <int QT, bool COHERENT = false>
__device__ __forceinline__ void wide_run(const LayerArgs &L, WideItem &It, X32 &X, int &cur_tok, int q, int kprime,
                                         const XSource &xsrc, const int32_t *sorted_slot,
                                         const uint8_t *lds, const TableLayout &TL, void *h, uint32_t tag = 0) {
  const int I = L.inter;
  for (int p = It.W.p0; p < It.W.p1; p++) {
    const int tok = (p == It.W.p0 ? It.W.slot0 : sload(sorted_slot + p)) / kprime;
    if (tok != cur_tok) {
      load_x32(xsrc.x + (size_t)tok * xsrc.tok_stride + q * xsrc.lane_stride, X);
      cur_tok = tok;
    }
    float vg[kWideRows], vu[kWideRows];
#pragma unroll
    for (int i = 0; i < kWideRows; i++) {
      Row32 g = It.g[i], u = It.u[i];
      opaque(g);
      opaque(u);
      // wave-uniform sums, held in scalar registers until the rows are finished
      vg[i] = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(group_sum_first<64>(dot32<QT>(g, q, lds, TL, X)))));
      vu[i] = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(group_sum_first<64>(dot32<QT>(u, q, lds, TL, X)))));
    }
    // lane i < kWideRows finishes row r0 + i: one SiLU for all the item's rows
    if (q < kWideRows) {
      float g = vg[0], u = vu[0];
#pragma unroll
      for (int i = 1; i < kWideRows; i++) {
        g = q == i ? vg[i] : g;
        u = q == i ? vu[i] : u;
      }
      const size_t at = (size_t)p * I + It.r0 + q;
      const float v = silu(g) * u;
      if constexpr (COHERENT)
        __hip_atomic_store((uint64_t *)h + at, ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      else
        ((float *)h)[at] = v;
    }
  }
}

// The same for an item of exactly one token whose activations are already in X (the
// one-token decode kernels): h holds tagged pairs, p0 is the item's sorted position.
// With no token loop there is nothing to hoist, so the rows are not made opaque: all
// products first, then all sums, so that their latencies overlap.
template <int QT>
__device__ __forceinline__ void wide_run_one(const WideItem &It, X32 &X, int q, int I, const uint8_t *lds,
                                             const TableLayout &TL, uint64_t *h, uint32_t tag) {
  float vg[kWideRows], vu[kWideRows];
#pragma unroll
  for (int i = 0; i < kWideRows; i++) {
    vg[i] = dot32<QT>(It.g[i], q, lds, TL, X);
    vu[i] = dot32<QT>(It.u[i], q, lds, TL, X);
  }
#pragma unroll
  for (int i = 0; i < kWideRows; i++) {
    vg[i] = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(group_sum_first<64>(vg[i]))));
    vu[i] = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(group_sum_first<64>(vu[i]))));
  }
  if (q < kWideRows) {  // lane i finishes row r0 + i: one SiLU for all the item's rows
    float g = vg[0], u = vu[0];
#pragma unroll
    for (int i = 1; i < kWideRows; i++) {
      g = q == i ? vg[i] : g;
      u = q == i ? vu[i] : u;
    }
    __hip_atomic_store(h + (size_t)It.W.p0 * I + It.r0 + q, ((uint64_t)tag << 32) | __float_as_uint(silu(g) * u),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ----------------------------------------------------------------------------- down + accumulate
// Shape of the fused down + accumulate workgroup (4 waves; a wave takes at most
// kDaSlots of a token's slots) and its LDS staging of h: each 64-float chunk of an h row
// padded to kChunkPad floats.
constexpr int kDaWaves = 4;
constexpr int kDaSlots = (MOE_MAX_K + 1 + kDaWaves - 1) / kDaWaves;  // slots per wave, at most
constexpr int kDaFirst = 3;  // slots per wave whose weight rows are loaded up front
constexpr int kChunkPad = 68;

__host__ __device__ inline size_t down_acc_stage_bytes(int lpr, int slots_per_wave) {
  return (size_t)kDaWaves * slots_per_wave * lpr * kChunkPad * 4;
}

template <int QT, int LPR>
__device__ __forceinline__ float down_slot_dot(const RowRaw &R, const float *hrow, int q, const uint8_t *lds,
                                               const TableLayout &TL) {
  XChunk X;
  load_x<QT>(hrow, X);
  return group_sum_first<LPR>(dot_chunk<QT>(R, q, lds, TL, X));
}

}  // namespace moe
