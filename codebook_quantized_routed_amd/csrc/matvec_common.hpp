// Device helpers shared by the mat-vec and MFMA kernels: streaming loads, the LDS
// grid tables every workgroup builds from the compact rows, SiLU, and the work list.
#pragma once
#include "decode.hpp"

namespace moe {

// ----------------------------------------------------------------------------- loads
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Streaming loads of the code streams (each byte is read once per launch).
__device__ __forceinline__ uint4 load_stream16(const uint8_t *p) {
  const u32x4 v = __builtin_nontemporal_load((const u32x4 *)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 load_stream8(const uint8_t *p) {
  const u32x2 v = __builtin_nontemporal_load((const u32x2 *)p);
  return make_uint2(v.x, v.y);
}

// ----------------------------------------------------------------------------- LDS tables
// fp16 grid rows (8 values, 16 bytes per row) and the IQ2 sign-mask rows: entry s (the
// 7 explicit sign bits) holds, per pair of weights, 0x8000 in each half whose weight is
// negative, the 8th sign being the parity of the 7.  IQ1 has two tables: the grid rows
// (kTabIq1), and the rows with the group's delta already added (kTabIq1Delta): row
// idx + 2048 s holds grid[idx][j] + 1/8 for s = 0 and grid[idx][j] - 1/8 for s = 1 (all
// exact in fp16), so a dot product reads each weight's value up to its scale directly.
constexpr int kTabIq1 = 1, kTabIq1Delta = 2;

struct TableLayout {
  int iq2h, iq2m, iq1h, iq1d, bytes;  // byte offsets in dynamic LDS (-1: not built)
};

__host__ __device__ inline TableLayout table_layout(int formats, int iq1_tables = kTabIq1) {
  TableLayout t{-1, -1, -1, -1, 0};
  if (formats & MOE_Q_IQ2XS_LIKE) {
    t.iq2h = t.bytes;
    t.bytes += kIq2Rows * 16;
    t.iq2m = t.bytes;
    t.bytes += 128 * 16;
  }
  if ((formats & MOE_Q_IQ1M_LIKE) && (iq1_tables & kTabIq1)) {
    t.iq1h = t.bytes;
    t.bytes += kIq1Rows * 16;
  }
  if ((formats & MOE_Q_IQ1M_LIKE) && (iq1_tables & kTabIq1Delta)) {
    t.iq1d = t.bytes;
    t.bytes += 2 * kIq1Rows * 16;
  }
  return t;
}

__device__ __forceinline__ uint32_t f16_bits(float v) { return __builtin_bit_cast(uint16_t, (_Float16)v); }

__device__ __forceinline__ uint4 expand_row_f16(uint32_t c, uint32_t h0, uint32_t h1, uint32_t h2) {
  uint32_t h[8];
#pragma unroll
  for (int j = 0; j < 8; j++) {
    const uint32_t s = (c >> (2 * j)) & 3u;
    h[j] = s == 0 ? h0 : (s == 1 ? h1 : h2);
  }
  return make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
}

// Builds the tables of the formats present from the compact rows (1 KB / 4 KB reads),
// in two steps: tables_load issues the global loads (call it before the loads that wait
// on HBM, so the table build does not queue behind them), tables_store expands into LDS
// and synchronizes the workgroup (unless told not to).  Loader t of n (by default every
// thread) expands rows t, t + n, ...; t < 0 loads and stores nothing.
constexpr int kTableRowsPerThread = kIq1Rows / 256;  // for n >= 256 loaders

struct TableRegs {
  uint32_t c2[kIq2Rows / 256];
  uint32_t c1[kTableRowsPerThread];
};

__device__ __forceinline__ TableRegs tables_load(const uint8_t *grids, int formats, int t = threadIdx.x,
                                                 int n = blockDim.x) {
  TableRegs tr;
  const uint16_t *c2 = (const uint16_t *)(grids + kGridIq2CompactOff);
  const uint16_t *c1 = (const uint16_t *)(grids + kGridIq1CompactOff);
#pragma unroll
  for (int i = 0; i < kIq2Rows / 256; i++) {
    const int r = t + i * n;
    tr.c2[i] = (formats & MOE_Q_IQ2XS_LIKE) && t >= 0 && r < kIq2Rows ? c2[r] : 0u;
  }
#pragma unroll
  for (int i = 0; i < kTableRowsPerThread; i++) {
    const int r = t + i * n;
    tr.c1[i] = (formats & MOE_Q_IQ1M_LIKE) && t >= 0 && r < kIq1Rows ? c1[r] : 0u;
  }
  return tr;
}

__device__ __forceinline__ void tables_store(const TableRegs &tr, int formats, const TableLayout &TL, uint8_t *lds,
                                             int t = threadIdx.x, int n = blockDim.x, bool sync = true) {
  if (formats & MOE_Q_IQ2XS_LIKE) {
    const uint32_t h0 = f16_bits((float)kIq2SymVal[0]), h1 = f16_bits((float)kIq2SymVal[1]),
                   h2 = f16_bits((float)kIq2SymVal[2]);
    uint4 *rows = (uint4 *)(lds + TL.iq2h);
#pragma unroll
    for (int i = 0; i < kIq2Rows / 256; i++) {
      const int r = t + i * n;
      if (t >= 0 && r < kIq2Rows) rows[r] = expand_row_f16(tr.c2[i], h0, h1, h2);
    }
    uint4 *masks = (uint4 *)(lds + TL.iq2m);
    for (int s = t; t >= 0 && s < 128; s += n) {
      const uint32_t S = (uint32_t)s | ((__builtin_popcount(s) & 1u) << 7);
      uint32_t m[4];
#pragma unroll
      for (int p = 0; p < 4; p++) m[p] = (((S >> (2 * p)) & 1u) << 15) | (((S >> (2 * p + 1)) & 1u) << 31);
      masks[s] = make_uint4(m[0], m[1], m[2], m[3]);
    }
  }
  if ((formats & MOE_Q_IQ1M_LIKE) && TL.iq1h >= 0) {
    const uint32_t h0 = f16_bits((float)kIq1SymVal[0]), h1 = f16_bits((float)kIq1SymVal[1]),
                   h2 = f16_bits((float)kIq1SymVal[2]);
    uint4 *rows = (uint4 *)(lds + TL.iq1h);
#pragma unroll
    for (int i = 0; i < kTableRowsPerThread; i++) {
      const int r = t + i * n;
      if (t >= 0 && r < kIq1Rows) rows[r] = expand_row_f16(tr.c1[i], h0, h1, h2);
    }
  }
  if ((formats & MOE_Q_IQ1M_LIKE) && TL.iq1d >= 0) {
    const float d = 0.125f;
    const uint32_t p0 = f16_bits((float)kIq1SymVal[0] + d), p1 = f16_bits((float)kIq1SymVal[1] + d),
                   p2 = f16_bits((float)kIq1SymVal[2] + d);
    const uint32_t m0 = f16_bits((float)kIq1SymVal[0] - d), m1 = f16_bits((float)kIq1SymVal[1] - d),
                   m2 = f16_bits((float)kIq1SymVal[2] - d);
    uint4 *rows = (uint4 *)(lds + TL.iq1d);
#pragma unroll
    for (int i = 0; i < kTableRowsPerThread; i++) {
      const int r = t + i * n;
      if (t >= 0 && r < kIq1Rows) {
        rows[r] = expand_row_f16(tr.c1[i], p0, p1, p2);
        rows[r + kIq1Rows] = expand_row_f16(tr.c1[i], m0, m1, m2);
      }
    }
  }
  if (sync) __syncthreads();
}

__device__ __forceinline__ void build_tables(const uint8_t *grids, int formats, const TableLayout &TL, uint8_t *lds) {
  const TableRegs tr = tables_load(grids, formats);
  tables_store(tr, formats, TL, lds);
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

__host__ __device__ inline int layer_formats(const LayerArgs &L) { return L.formats; }

// i must be wave-uniform.
__device__ __forceinline__ WorkRec load_work(const WorkRec *w, int i) {
  return sload(w + i);
}

// The layer's banks, copied from the kernel arguments into LDS (static indexing, so the
// copy reads scalar registers): per matrix and stream the base and the bytes of one
// expert.  Kernels that look up many experts read their matrices from this table
// instead of indexing the kernel arguments with the bank.
struct BankLds {
  const uint8_t *base[3][3];  // [gate, up, down][stream]
  uint64_t bytes[3][3];
  int32_t first, qt, pad[2];
};

// Fills the bank table (one thread).
__device__ inline void fill_banks(const LayerArgs &L, BankLds *banks) {
  const int H = L.hidden, I = L.inter;
#pragma unroll
  for (int b = 0; b < MOE_MAX_BANKS; b++) {
    if (b >= L.n_banks) break;
    const BankArgs &B = L.banks[b];
    BankLds &D = banks[b];
    D.first = B.first;
    D.qt = B.qtype;
#pragma unroll
    for (int w = 0; w < 3; w++) {
      const int rows = w == kDown ? H : I, cols = w == kDown ? I : H;
      const uint8_t *const *src = w == kGate ? B.gate : (w == kUp ? B.up : B.down);
      D.base[w][0] = src[0], D.base[w][1] = src[1], D.base[w][2] = src[2];
      D.bytes[w][0] = stream0_bytes(B.qtype, rows, cols);
      D.bytes[w][1] = stream1_bytes(B.qtype, rows, cols);
      D.bytes[w][2] = stream2_bytes(B.qtype, rows, cols);
    }
  }
}

// The bank of expert e (as bank_of).
__device__ inline int bank_index(const LayerArgs &L, int e) {
  int b = 0;
#pragma unroll
  for (int i = 1; i < MOE_MAX_BANKS; i++)
    if (i < L.n_banks && e >= L.banks[i].first) b = i;
  return b;
}

__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
  return ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32)) << 32) |
         (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
}

// The same matrix with its stream bases marked global (loads through them are global
// loads, which do not count against the LDS wait counter as flat loads would).
__device__ __forceinline__ QMat global_mat(const QMat &m) {
  typedef const __attribute__((address_space(1))) uint8_t gbyte;
  QMat g;
  g.s0 = (const uint8_t *)(gbyte *)m.s0;
  g.s1 = (const uint8_t *)(gbyte *)m.s1;
  g.s2 = (const uint8_t *)(gbyte *)m.s2;
  return g;
}

// Matrix w of expert e in bank B (the same bases and offsets as expert_mat), in scalar
// registers; the bases are marked global again (loads through them are global loads).
__device__ __forceinline__ QMat bank_mat(const BankLds &B, int e, int w) {
  const uint64_t x = (uint64_t)(e - uniform(B.first));
  QMat m;
  m.s0 = (const uint8_t *)(const __attribute__((address_space(1))) uint8_t *)(uniform64((uint64_t)B.base[w][0]) + x * uniform64(B.bytes[w][0]));
  m.s1 = (const uint8_t *)(const __attribute__((address_space(1))) uint8_t *)(uniform64((uint64_t)B.base[w][1]) + x * uniform64(B.bytes[w][1]));
  m.s2 = (const uint8_t *)(const __attribute__((address_space(1))) uint8_t *)(uniform64((uint64_t)B.base[w][2]) + x * uniform64(B.bytes[w][2]));
  return m;
}

}  // namespace moe
