// Internal header of the HIP library: kernel argument structs, format helpers and
// launcher declarations.  gfx950 only; wave64.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

constexpr int kWave = 64;
// Symbol values of the two grids ("Red Lite dev10", section "Quant grids": IQ2_XS
// symbols stand for 0x08 / 0x19 / 0x2b, IQ1_M symbols for -1 / 0 / +1).
constexpr int kIq2SymVal[3] = {0x08, 0x19, 0x2b};
constexpr int kIq1SymVal[3] = {-1, 0, 1};
constexpr int kIq2Rows = 512;
constexpr int kIq1Rows = 2048;
// Expanded grid buffer: IQ2 values u8[512][8] (8, 25, 43), IQ1 values i8[2048][8]
// (-1, 0, +1), then copies of the compact rows (u16 per grid row, 2 bits per symbol)
// from which each mat-vec workgroup builds its fp16 tables in LDS.
constexpr size_t kGridIq2Off = 0;
constexpr size_t kGridIq1Off = kIq2Rows * 8;
constexpr size_t kGridIq2CompactOff = kGridIq1Off + kIq1Rows * 8;
constexpr size_t kGridIq1CompactOff = kGridIq2CompactOff + kIq2Rows * 2;
// then the matrix-core decode tables, expanded once by moe_grids_expand in the layout the
// decode kernels keep in LDS for a layer of both formats: IQ2 fp16 grid rows [512][8],
// IQ2 signed-scale rows [128 sign patterns][16 scales][8], IQ1 rows with the delta
// added [2][2048][8] (+1/8, then -1/8)
constexpr size_t kGridDecOff = (kGridIq1CompactOff + kIq1Rows * 2 + 255) & ~(size_t)255;
constexpr size_t kGridDecBytes = kIq2Rows * 16 + 128 * 16 * 16 + 2 * kIq1Rows * 16;
constexpr size_t kGridBytes = kGridDecOff + kGridDecBytes;

// Work record of one active expert, written by the grouping: expert id, its first and
// one-past-last sorted positions, and the slot at its first position.
struct WorkRec {
  int e, p0, p1, slot0;
};

// Experts with at most this many of a call's T tokens run on the mat-vec kernels.
__host__ __device__ inline int matvec_max_tokens(int T) {
  return T <= MOE_SMALL_BATCH_TOKENS ? T : MOE_MATVEC_MAX_TOKENS;
}

// Upper bounds on the experts with more than matvec_max_tokens(T) slots (each has at
// most one slot per token) and on their tiles of MOE_MFMA_TILE_TOKENS.
__host__ __device__ inline int max_wide_experts(int T, int kprime, int n_ids) {
  const int m = matvec_max_tokens(T);
  if (T <= m) return 0;
  const long by_slots = (long)T * kprime / (m + 1);
  return (int)(by_slots < n_ids ? by_slots : n_ids);
}
__host__ __device__ inline int max_mfma_tiles(int T, int kprime, int n_ids) {
  const int w = max_wide_experts(T, kprime, n_ids);
  return w == 0 ? 0 : w + (int)(((long)T * kprime + MOE_MFMA_TILE_TOKENS - 1) / MOE_MFMA_TILE_TOKENS);
}

// Byte sizes of the three streams of one rows x cols matrix.
__host__ __device__ inline size_t stream0_bytes(int qt, int rows, int cols) {
  return qt == MOE_Q_IQ2XS_LIKE ? (size_t)rows * (cols / 8) * 2 : (size_t)rows * (cols / 8);
}
__host__ __device__ inline size_t stream1_bytes(int qt, int rows, int cols) {
  return qt == MOE_Q_IQ2XS_LIKE ? (size_t)rows * (cols / 256) * 4 : (size_t)rows * (cols / 16);
}
__host__ __device__ inline size_t stream2_bytes(int qt, int rows, int cols) {
  return qt == MOE_Q_IQ2XS_LIKE ? (size_t)rows * (cols / 256) * 2 : (size_t)rows * (cols / 256) * 8;
}
__host__ __device__ inline size_t matrix_bytes(int qt, int rows, int cols) {
  return stream0_bytes(qt, rows, cols) + stream1_bytes(qt, rows, cols) + stream2_bytes(qt, rows, cols);
}

// One matrix as seen by a kernel: stream bases of one expert.
struct QMat {
  const uint8_t *s0, *s1, *s2;
};

struct BankArgs {
  int qtype, first, n, pad;
  const uint8_t *gate[3], *up[3], *down[3];
};

// The layer, passed by value as a kernel argument (no device-side descriptor loads).
// formats = OR of the banks' qtypes, set on the host.
struct LayerArgs {
  int hidden, inter, n_banks, formats;
  BankArgs banks[MOE_MAX_BANKS];
  const uint8_t *grids;
};

enum Which { kGate = 0, kUp = 1, kDown = 2 };

// A value every lane of the wave holds: moved to a scalar register, so that what is
// computed from it (bank choice, matrix bases) stays scalar too.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Calls f(Index<0>{}), ..., f(Index<N - 1>{}): a loop whose index is a constant in the
// body, so arrays indexed by it are split into registers before any unrolling.
template <int I>
struct Index {
  static constexpr int value = I;
};
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (I < N) {
    f(Index<I>{});
    static_for<N, I + 1>(f);
  }
}

// Load of a value the whole wave shares, through the scalar cache: the address must be
// wave-uniform and the memory must not change while the kernel runs (it was written by
// an earlier launch).  Scalar loads wait on their own counter, so a wave can use the
// result without waiting for its outstanding vector loads.
template <typename T>
__device__ __forceinline__ T sload(const T *p) {
  return *(const __attribute__((address_space(4))) T *)p;
}
__device__ __forceinline__ WorkRec sload(const WorkRec *p) {
  const __attribute__((address_space(4))) int *q = (const __attribute__((address_space(4))) int *)p;
  return WorkRec{q[0], q[1], q[2], q[3]};
}

// Bank lookup for expert e (uniform across a workgroup).
__device__ inline const BankArgs &bank_of(const LayerArgs &L, int e) {
  int b = 0;
#pragma unroll
  for (int i = 1; i < MOE_MAX_BANKS; i++)
    if (i < L.n_banks && e >= L.banks[i].first) b = i;
  return L.banks[b];
}

__device__ inline QMat expert_mat(const BankArgs &B, int e, Which w, int rows, int cols) {
  const uint8_t *const *base = w == kGate ? B.gate : (w == kUp ? B.up : B.down);
  size_t i = (size_t)(e - B.first);
  QMat m;
  m.s0 = base[0] + i * stream0_bytes(B.qtype, rows, cols);
  m.s1 = base[1] + i * stream1_bytes(B.qtype, rows, cols);
  m.s2 = base[2] + i * stream2_bytes(B.qtype, rows, cols);
  return m;
}

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// Sum over each aligned group of `width` consecutive lanes (power of two <= 64); the
// result is valid in the group's first lane only.  DPP row shifts inside 16-lane rows,
// then the row sums combined as (r0 + r1) + (r2 + r3); fixed order, so deterministic.
// The whole wave (width 64) reads the four row sums with readlane instead of two LDS
// permutes, with the same additions in the same order (the same bits).
template <int width>
__device__ __forceinline__ float group_sum_first(float v) {
  if (width >= 2) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x101, 0xf, 0xf, false));
  if (width >= 4) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x102, 0xf, 0xf, false));
  if (width >= 8) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x104, 0xf, 0xf, false));
  if (width >= 16) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x108, 0xf, 0xf, false));
  if constexpr (width == 64) {
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (r0 + r1) + (r2 + r3);
  }
  if (width >= 32) v += __shfl_down(v, 16, 64);
  return v;
}

// Sum over a group of `width` consecutive lanes (power of two <= 64), fixed tree order,
// result in every lane of the group.
template <int width>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = width / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ----------------------------------------------------------------------------- launchers
hipError_t launch_grids_expand(const uint16_t *c2, const uint16_t *c1, uint8_t *grids, hipStream_t s);
hipError_t launch_dequant(int qt, int rows, int cols, QMat m, const uint8_t *grids, float *out, hipStream_t s);
hipError_t launch_route_group(const float *logits, int T, int E, int k, int add_shared, int32_t *ids, float *w,
                              int32_t *counts, int32_t *offsets, int32_t *sorted_slot, int32_t *slot_pos,
                              WorkRec *work, hipStream_t s);
hipError_t launch_group_explicit(int T, int E, int k, int add_shared, int32_t *ids, float *w, int32_t *counts,
                                 int32_t *offsets, int32_t *sorted_slot, int32_t *slot_pos, WorkRec *work,
                                 hipStream_t s);
// Mat-vec path: experts with at most max_tokens tokens (the others are skipped).
hipError_t launch_gateup_gemv(const LayerArgs &L, const float *x, int T, int kprime, const int32_t *sorted_slot,
                              const WorkRec *work, int n_ids, int max_tokens, float *h, hipStream_t s);
hipError_t launch_down_gemv(const LayerArgs &L, const float *h, int T, int kprime, const WorkRec *work, int n_ids,
                            int max_tokens, float *y, hipStream_t s);
hipError_t launch_gateup_mfma(const LayerArgs &L, const float *x, int T, int kprime, const int32_t *sorted_slot,
                              const WorkRec *work, int n_ids, float *h, hipStream_t s);
hipError_t launch_down_mfma(const LayerArgs &L, const float *h, int T, int kprime, const WorkRec *work, int n_ids,
                            float *y, hipStream_t s);
hipError_t launch_down_accumulate(const LayerArgs &L, const float *h, int T, int kprime, const int32_t *ids,
                                  const float *w, const int32_t *slot_pos, float *acc, hipStream_t s);
size_t fused_sync_bytes();
// Stack workspace: the synchronisation words, the device copy of the layer table (at a
// 256-byte boundary), then per layer the h pairs [kprime][inter] and the residual
// pairs [hidden].
inline size_t stack_pairs_offset(int n_layers) {
  return ((fused_sync_bytes() + (size_t)n_layers * sizeof(LayerArgs)) + 255) & ~(size_t)255;
}
hipError_t launch_stack_decode(const LayerArgs *d_tab, int n_layers, int formats, const uint8_t *grids, int inter,
                               const float *logits, const float *h_in, float *h_out, int E, int k, int add_shared,
                               float eps, int32_t *ids, float *w, void *ws, hipStream_t s);
hipError_t launch_layer_decode(const LayerArgs &L, const float *logits, const float *x, int E, int k, int add_shared,
                               int32_t *ids, float *w, int32_t *counts, int32_t *offsets, int32_t *sorted_slot,
                               int32_t *slot_pos, WorkRec *work, float *acc, void *ws, hipStream_t s);
// Calls of 2 .. kDecMaxTokens tokens with inter <= 512 run gate / up on the matrix-core
// decode kernel (k_dec.hip).
constexpr int kDecMaxTokens = 8;
bool dec_path_ok(const LayerArgs &L, int T);
hipError_t launch_gateup_dec(const LayerArgs &L, const float *x, int T, int kprime, const int32_t *sorted_slot,
                             const WorkRec *work, int n_ids, float *h, hipStream_t s);
hipError_t launch_accumulate(const float *y, const float *w, const int32_t *ids, const int32_t *slot_pos, int T,
                             int kprime, int H, float *acc, hipStream_t s);
hipError_t launch_rmsnorm(const float *h, int T, int H, float eps, float *x, hipStream_t s);

}  // namespace moe
