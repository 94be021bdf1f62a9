// extern "C" entry points: argument validation on the host, then kernel launches on the
// caller's stream.  No allocation, no host<->device copies, no synchronization.
#include <cstring>
#include <initializer_list>
#include <mutex>

#include "common.hpp"
#include "repack.hpp"
#include "router.hpp"

using namespace moe;

namespace {

// HIP error of this thread's last failed launch (reported by moe_last_hip_error).
thread_local hipError_t t_last_hip = hipSuccess;

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Column counts the per-lane 32-column chunking supports.
bool width_ok(int cols) { return cols == 256 || cols == 512 || cols == 1024 || cols == 2048; }

moe_status from_hip(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  t_last_hip = e;
  return MOE_E_HIP;
}

// An error left pending by earlier, unrelated runtime calls of this thread would
// otherwise be picked up by the launch check; clear it once validation has passed.
void clear_pending() { (void)hipGetLastError(); }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

moe_status check_layer(const moe_layer *layer, LayerArgs *out) {
  if (!layer || !layer->grids) return MOE_E_NULL;
  if (!aligned16(layer->grids)) return MOE_E_ALIGN;
  const int H = layer->hidden, I = layer->inter;
  if (!width_ok(H) || !width_ok(I)) return MOE_E_SHAPE;
  if (layer->n_experts < 1 || layer->has_shared < 0 || layer->has_shared > 1) return MOE_E_SHAPE;
  const int n_ids = layer->n_experts + layer->has_shared;
  if (n_ids > MOE_MAX_IDS) return MOE_E_SHAPE;
  if (layer->n_banks < 1 || layer->n_banks > MOE_MAX_BANKS) return MOE_E_SHAPE;
  out->hidden = H;
  out->inter = I;
  out->n_banks = layer->n_banks;
  out->formats = 0;
  out->grids = (const uint8_t *)layer->grids;
  int next = 0;
  for (int b = 0; b < MOE_MAX_BANKS; b++) {
    BankArgs &d = out->banks[b];
    d = BankArgs{};
    if (b >= layer->n_banks) continue;
    const moe_bank &s = layer->banks[b];
    if (s.qtype != MOE_Q_IQ2XS_LIKE && s.qtype != MOE_Q_IQ1M_LIKE) return MOE_E_QTYPE;
    if (s.first_expert != next || s.n_experts < 1) return MOE_E_SHAPE;
    next += s.n_experts;
    d.qtype = s.qtype;
    out->formats |= s.qtype;
    d.first = s.first_expert;
    d.n = s.n_experts;
    for (int i = 0; i < 3; i++) {
      if (!s.gate[i] || !s.up[i] || !s.down[i]) return MOE_E_NULL;
      if (!aligned16(s.gate[i]) || !aligned16(s.up[i]) || !aligned16(s.down[i])) return MOE_E_ALIGN;
      d.gate[i] = (const uint8_t *)s.gate[i];
      d.up[i] = (const uint8_t *)s.up[i];
      d.down[i] = (const uint8_t *)s.down[i];
    }
  }
  if (next != n_ids) return MOE_E_SHAPE;
  return MOE_OK;
}

}  // namespace

extern "C" {

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

int32_t moe_last_hip_error(void) { return (int32_t)t_last_hip; }

const char *moe_last_hip_error_string(void) { return hipGetErrorString(t_last_hip); }

const char *moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_E_NULL: return "null pointer";
    case MOE_E_SHAPE: return "size out of range or inconsistent";
    case MOE_E_QTYPE: return "unknown quantization type";
    case MOE_E_ALIGN: return "device pointer not 16-byte aligned";
    case MOE_E_WORKSPACE: return "workspace too small";
    case MOE_E_HIP: return "HIP launch error";
  }
  return "unknown status";
}

size_t moe_grids_bytes(void) { return kGridBytes; }

moe_status moe_grids_expand(const uint16_t *d_compact_iq2, const uint16_t *d_compact_iq1, void *d_grids,
                            hipStream_t stream) {
  if (!d_compact_iq2 || !d_compact_iq1 || !d_grids) return MOE_E_NULL;
  if (!aligned16(d_compact_iq2) || !aligned16(d_compact_iq1) || !aligned16(d_grids)) return MOE_E_ALIGN;
  clear_pending();
  return from_hip(launch_grids_expand(d_compact_iq2, d_compact_iq1, (uint8_t *)d_grids, stream));
}

int32_t moe_work_ints(int32_t T, int32_t kprime, int32_t n_ids) {
  if (T < 1 || kprime < 1 || n_ids < 1) return 0;
  return 4 * (n_ids + 1 + max_mfma_tiles(T, kprime, n_ids));
}

size_t moe_workspace_bytes(int32_t T, int32_t kprime, int32_t hidden, int32_t inter) {
  if (T < 1 || kprime < 1 || !width_ok(hidden) || !width_ok(inter)) return 0;
  return round_up((size_t)T * kprime * inter * sizeof(float), 256);
}

moe_status moe_route_group(const float *d_logits, int32_t T, int32_t E, int32_t k, int32_t add_shared,
                           int32_t *d_ids, float *d_w, int32_t *d_counts, int32_t *d_offsets,
                           int32_t *d_sorted_slot, int32_t *d_slot_pos, int32_t *d_work, hipStream_t stream) {
  if (!d_ids || !d_w || !d_counts || !d_offsets || !d_sorted_slot || !d_slot_pos || !d_work) return MOE_E_NULL;
  if (T < 1 || T > 65536 || E < 1 || k < 1 || k > MOE_MAX_K || k > E || add_shared < 0 || add_shared > 1)
    return MOE_E_SHAPE;
  if (E + add_shared > MOE_MAX_IDS) return MOE_E_SHAPE;
  const void *ptrs[] = {d_ids, d_w, d_counts, d_offsets, d_sorted_slot, d_slot_pos, d_work};
  for (const void *p : ptrs)
    if (!aligned16(p)) return MOE_E_ALIGN;
  if (d_logits && !aligned16(d_logits)) return MOE_E_ALIGN;
  clear_pending();
  if (d_logits)
    return from_hip(launch_route_group(d_logits, T, E, k, add_shared, d_ids, d_w, d_counts, d_offsets, d_sorted_slot,
                                       d_slot_pos, (WorkRec *)d_work, stream));
  return from_hip(launch_group_explicit(T, E, k, add_shared, d_ids, d_w, d_counts, d_offsets, d_sorted_slot,
                                        d_slot_pos, (WorkRec *)d_work, stream));
}

namespace {

moe_status check_ffn_common(const moe_layer *layer, LayerArgs *L, int32_t T, int32_t kprime,
                            std::initializer_list<const void *> ptrs) {
  moe_status st = check_layer(layer, L);
  if (st != MOE_OK) return st;
  for (const void *p : ptrs)
    if (!p) return MOE_E_NULL;
  for (const void *p : ptrs)
    if (!aligned16(p)) return MOE_E_ALIGN;
  if (T < 1 || T > 65536 || kprime < 1 || kprime > MOE_MAX_K + 1) return MOE_E_SHAPE;
  return MOE_OK;
}

// Both kernels of a projection: the mat-vec kernel takes the experts of the first work
// list, the matrix-core kernel those of the second.  Gate / up of 2 .. kDecMaxTokens
// tokens runs on one decode kernel instead (k_dec.hip).
hipError_t launch_gateup(const LayerArgs &L, const float *x, int T, int kprime, const int32_t *sorted_slot,
                         const WorkRec *work, int n_ids, float *h, hipStream_t s) {
  if (dec_path_ok(L, T)) return launch_gateup_dec(L, x, T, kprime, sorted_slot, work, n_ids, h, s);
  // m(T) = 0: the first set is empty, its kernels are not launched
  if (matvec_max_tokens(T) > 0) {
    hipError_t err = launch_gateup_gemv(L, x, T, kprime, sorted_slot, work, n_ids, matvec_max_tokens(T), h, s);
    if (err != hipSuccess) return err;
  }
  return launch_gateup_mfma(L, x, T, kprime, sorted_slot, work, n_ids, h, s);
}

hipError_t launch_down(const LayerArgs &L, const float *h, int T, int kprime, const WorkRec *work, int n_ids, float *y,
                       hipStream_t s) {
  if (matvec_max_tokens(T) > 0) {
    hipError_t err = launch_down_gemv(L, h, T, kprime, work, n_ids, matvec_max_tokens(T), y, s);
    if (err != hipSuccess) return err;
  }
  return launch_down_mfma(L, h, T, kprime, work, n_ids, y, s);
}

}  // namespace

moe_status moe_expert_gateup_q(const moe_layer *layer, const float *d_x, int32_t T, int32_t kprime,
                               const int32_t *d_sorted_slot, const int32_t *d_work, float *d_h, hipStream_t stream) {
  LayerArgs L;
  moe_status st = check_ffn_common(layer, &L, T, kprime, {d_x, d_sorted_slot, d_work, d_h});
  if (st != MOE_OK) return st;
  const int n_ids = layer->n_experts + layer->has_shared;
  clear_pending();
  return from_hip(launch_gateup(L, d_x, T, kprime, d_sorted_slot, (const WorkRec *)d_work, n_ids, d_h, stream));
}

moe_status moe_expert_down_q(const moe_layer *layer, const float *d_h, int32_t T, int32_t kprime,
                             const int32_t *d_work, float *d_y, hipStream_t stream) {
  LayerArgs L;
  moe_status st = check_ffn_common(layer, &L, T, kprime, {d_h, d_work, d_y});
  if (st != MOE_OK) return st;
  const int n_ids = layer->n_experts + layer->has_shared;
  clear_pending();
  return from_hip(launch_down(L, d_h, T, kprime, (const WorkRec *)d_work, n_ids, d_y, stream));
}

moe_status moe_expert_down_accumulate_q(const moe_layer *layer, const float *d_h, int32_t T, int32_t kprime,
                                        const int32_t *d_ids, const float *d_w, const int32_t *d_slot_pos,
                                        float *d_acc, hipStream_t stream) {
  LayerArgs L;
  moe_status st = check_ffn_common(layer, &L, T, kprime, {d_h, d_ids, d_w, d_slot_pos, d_acc});
  if (st != MOE_OK) return st;
  clear_pending();
  return from_hip(launch_down_accumulate(L, d_h, T, kprime, d_ids, d_w, d_slot_pos, d_acc, stream));
}

moe_status moe_expert_ffn_q(const moe_layer *layer, const float *d_x, int32_t T, int32_t kprime,
                            const int32_t *d_sorted_slot, const int32_t *d_work, float *d_y, void *d_ws,
                            size_t ws_bytes, hipStream_t stream) {
  LayerArgs L;
  moe_status st = check_ffn_common(layer, &L, T, kprime, {d_x, d_sorted_slot, d_work, d_y, d_ws});
  if (st != MOE_OK) return st;
  if (ws_bytes < moe_workspace_bytes(T, kprime, L.hidden, L.inter)) return MOE_E_WORKSPACE;
  const int n_ids = layer->n_experts + layer->has_shared;
  const WorkRec *work = (const WorkRec *)d_work;
  float *h = (float *)d_ws;
  clear_pending();
  hipError_t err = launch_gateup(L, d_x, T, kprime, d_sorted_slot, work, n_ids, h, stream);
  if (err != hipSuccess) return from_hip(err);
  return from_hip(launch_down(L, h, T, kprime, work, n_ids, d_y, stream));
}

size_t moe_decode_workspace_bytes(int32_t kprime, int32_t inter) {
  if (kprime < 1 || kprime > MOE_MAX_K + 1 || inter < 1) return 0;
  return fused_sync_bytes() + (size_t)kprime * inter * sizeof(uint64_t);
}

moe_status moe_layer_decode_q(const moe_layer *layer, const float *d_logits, const float *d_x, int32_t k,
                              int32_t add_shared, int32_t *d_ids, float *d_w, int32_t *d_counts, int32_t *d_offsets,
                              int32_t *d_sorted_slot, int32_t *d_slot_pos, int32_t *d_work, float *d_acc, void *d_ws,
                              size_t ws_bytes, hipStream_t stream) {
  LayerArgs L;
  moe_status st = check_ffn_common(layer, &L, 1, k + add_shared,
                                   {d_x, d_ids, d_w, d_counts, d_offsets, d_sorted_slot, d_slot_pos, d_work, d_acc, d_ws});
  if (st != MOE_OK) return st;
  if (d_logits && !aligned16(d_logits)) return MOE_E_ALIGN;
  const int E = layer->n_experts;
  if (k < 1 || k > MOE_MAX_K || k > E || add_shared != layer->has_shared || E > 512) return MOE_E_SHAPE;
  if (L.hidden != 2048 || (L.inter != 256 && L.inter != 512)) return MOE_E_SHAPE;
  if (ws_bytes < moe_decode_workspace_bytes(k + add_shared, L.inter)) return MOE_E_WORKSPACE;
  clear_pending();
  return from_hip(launch_layer_decode(L, d_logits, d_x, E, k, add_shared, d_ids, d_w, d_counts, d_offsets,
                                      d_sorted_slot, d_slot_pos, (WorkRec *)d_work, d_acc, d_ws, stream));
}

}  // extern "C"

namespace {

// The workspace of moe_layer_decode_q_static: one array per device (each device's copy
// of the code object holds its own), held until the process ends.  Host code never
// passes the array's name to a kernel: it stands for a host-side shadow, not a device
// address; the device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint8_t scratch[MOE_DECODE_STATIC_BYTES];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
uint8_t *g_scratch_ptr[kMaxScratchDevices];  // per device: the array's address, null until the first call

// With status: its word gets the decode's status word first.  Then the whole array is
// zeroed (16-byte stores; MOE_DECODE_STATIC_BYTES is a multiple of 16).
__global__ void __launch_bounds__(1024) k_scratch_reset(uint8_t *ws, uint32_t *status) {
  if (status && threadIdx.x == 0) *status = *(const volatile uint32_t *)(ws + MOE_DECODE_ERROR_OFFSET);
  __syncthreads();
  uint4 *p = (uint4 *)ws;
  for (int i = threadIdx.x; i < MOE_DECODE_STATIC_BYTES / 16; i += blockDim.x) p[i] = make_uint4(0, 0, 0, 0);
}

// The current device's array (device address), zeroed on the stream on first use.
moe_status scratch_for_current_device(hipStream_t stream, uint8_t **out) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return from_hip(err);
  if (dev < 0 || dev >= kMaxScratchDevices) return from_hip(hipErrorInvalidDevice);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return from_hip(err);
    if (!p || ((uintptr_t)p & 255)) return from_hip(hipErrorInvalidSymbol);
    hipLaunchKernelGGL(k_scratch_reset, dim3(1), dim3(1024), 0, stream, (uint8_t *)p, (uint32_t *)nullptr);
    err = hipGetLastError();
    if (err != hipSuccess) return from_hip(err);
    g_scratch_ptr[dev] = (uint8_t *)p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_layer_decode_q_static(const moe_layer *layer, const float *d_logits, const float *d_x, int32_t k,
                                     int32_t add_shared, int32_t *d_ids, float *d_w, int32_t *d_counts,
                                     int32_t *d_offsets, int32_t *d_sorted_slot, int32_t *d_slot_pos, int32_t *d_work,
                                     float *d_acc, uint32_t *d_status, hipStream_t stream) {
  LayerArgs L;
  moe_status st = check_ffn_common(layer, &L, 1, k + add_shared,
                                   {d_x, d_ids, d_w, d_counts, d_offsets, d_sorted_slot, d_slot_pos, d_work, d_acc});
  if (st != MOE_OK) return st;
  if (!d_status) return MOE_E_NULL;
  if (!aligned16(d_status) || (d_logits && !aligned16(d_logits))) return MOE_E_ALIGN;
  const int E = layer->n_experts;
  if (k < 1 || k > MOE_MAX_K || k > E || add_shared != layer->has_shared || E > 512) return MOE_E_SHAPE;
  if (L.hidden != 2048 || (L.inter != 256 && L.inter != 512)) return MOE_E_SHAPE;
  if (moe_decode_workspace_bytes(k + add_shared, L.inter) > MOE_DECODE_STATIC_BYTES) return MOE_E_WORKSPACE;
  clear_pending();
  uint8_t *ws = nullptr;
  st = scratch_for_current_device(stream, &ws);
  if (st != MOE_OK) return st;
  hipError_t err = launch_layer_decode(L, d_logits, d_x, E, k, add_shared, d_ids, d_w, d_counts, d_offsets,
                                       d_sorted_slot, d_slot_pos, (WorkRec *)d_work, d_acc, ws, stream);
  if (err != hipSuccess) return from_hip(err);
  hipLaunchKernelGGL(k_scratch_reset, dim3(1), dim3(1024), 0, stream, ws, d_status);
  return from_hip(hipGetLastError());
}

size_t moe_stack_table_bytes(int32_t n_layers) {
  if (n_layers < 1 || n_layers > MOE_MAX_STACK_LAYERS) return 0;
  return (size_t)n_layers * sizeof(LayerArgs);
}

size_t moe_stack_workspace_bytes(int32_t n_layers, int32_t kprime, int32_t hidden, int32_t inter) {
  if (n_layers < 1 || n_layers > MOE_MAX_STACK_LAYERS || kprime < 1 || kprime > MOE_MAX_K + 1 || !width_ok(hidden) ||
      !width_ok(inter))
    return 0;
  return stack_pairs_offset(n_layers) + (size_t)n_layers * ((size_t)kprime * inter + hidden) * sizeof(uint64_t);
}

}  // extern "C"

namespace {

// Every layer valid and of the one shape the stack kernel runs; each layer's kernel
// arguments into tab[l] when tab is given, the union of their formats into *formats.
moe_status check_stack(const moe_layer *layers, int n_layers, LayerArgs *tab, int *formats) {
  if (!layers) return MOE_E_NULL;
  if (n_layers < 1 || n_layers > MOE_MAX_STACK_LAYERS) return MOE_E_SHAPE;
  *formats = 0;
  for (int l = 0; l < n_layers; l++) {
    LayerArgs L;
    const moe_status st = check_layer(&layers[l], &L);
    if (st != MOE_OK) return st;
    const moe_layer &a = layers[l], &b = layers[0];
    if (a.hidden != 2048 || (a.inter != 256 && a.inter != 512) || a.n_experts > 512) return MOE_E_SHAPE;
    if (a.inter != b.inter || a.n_experts != b.n_experts || a.has_shared != b.has_shared || a.grids != b.grids)
      return MOE_E_SHAPE;
    *formats |= L.formats;
    if (tab) tab[l] = L;
  }
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_stack_table(const moe_layer *layers, int32_t n_layers, void *h_table, size_t table_bytes) {
  if (!h_table) return MOE_E_NULL;
  int formats = 0;
  moe_status st = check_stack(layers, n_layers, nullptr, &formats);
  if (st != MOE_OK) return st;
  if (table_bytes < moe_stack_table_bytes(n_layers)) return MOE_E_SHAPE;
  for (int l = 0; l < n_layers; l++) {  // through a copy: h_table need not be aligned
    LayerArgs L;
    st = check_layer(&layers[l], &L);
    if (st != MOE_OK) return st;
    memcpy((uint8_t *)h_table + (size_t)l * sizeof(LayerArgs), &L, sizeof(LayerArgs));
  }
  return MOE_OK;
}

moe_status moe_stack_decode_q(const moe_layer *layers, int32_t n_layers, const float *d_logits, const float *d_h_in,
                              float *d_h_out, int32_t k, int32_t add_shared, float eps, int32_t *d_ids, float *d_w,
                              void *d_ws, size_t ws_bytes, hipStream_t stream) {
  if (!d_logits || !d_h_in || !d_h_out || !d_ws) return MOE_E_NULL;
  if ((d_ids == nullptr) != (d_w == nullptr)) return MOE_E_NULL;
  const void *ptrs[] = {d_logits, d_h_in, d_h_out, d_ids, d_w, d_ws};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return MOE_E_ALIGN;
  int formats = 0;
  const moe_status st = check_stack(layers, n_layers, nullptr, &formats);
  if (st != MOE_OK) return st;
  const int E = layers[0].n_experts, H = layers[0].hidden, I = layers[0].inter;
  if (k < 1 || k > MOE_MAX_K || k > E || add_shared != layers[0].has_shared) return MOE_E_SHAPE;
  if (!(eps >= 0.0f)) return MOE_E_SHAPE;
  const uintptr_t a = (uintptr_t)d_h_in, b = (uintptr_t)d_h_out, n = (uintptr_t)H * sizeof(float);
  if (a < b + n && b < a + n) return MOE_E_SHAPE;
  if (ws_bytes < moe_stack_workspace_bytes(n_layers, k + add_shared, H, I)) return MOE_E_WORKSPACE;
  clear_pending();
  return from_hip(launch_stack_decode((const LayerArgs *)((const uint8_t *)d_ws + fused_sync_bytes()), n_layers,
                                      formats, (const uint8_t *)layers[0].grids, I, d_logits, d_h_in, d_h_out, E, k, add_shared, eps,
                                      d_ids, d_w, d_ws, stream));
}

moe_status moe_accumulate(const float *d_y, const float *d_w, const int32_t *d_ids, const int32_t *d_slot_pos,
                          int32_t T, int32_t kprime, int32_t hidden, float *d_acc, hipStream_t stream) {
  if (!d_y || !d_w || !d_ids || !d_slot_pos || !d_acc) return MOE_E_NULL;
  const void *ptrs[] = {d_y, d_w, d_ids, d_slot_pos, d_acc};
  for (const void *p : ptrs)
    if (!aligned16(p)) return MOE_E_ALIGN;
  if (T < 1 || T > 65536 || kprime < 1 || kprime > MOE_MAX_K + 1 || hidden < 1 || hidden % 256) return MOE_E_SHAPE;
  clear_pending();
  return from_hip(launch_accumulate(d_y, d_w, d_ids, d_slot_pos, T, kprime, hidden, d_acc, stream));
}

moe_status moe_router_logits(const float *d_x, const float *d_wr, const float *d_wsg, int32_t T, int32_t hidden,
                             int32_t E, float *d_logits, float *d_shared_w, hipStream_t stream) {
  if (!d_x || !d_wr || !d_logits) return MOE_E_NULL;
  if ((d_wsg == nullptr) != (d_shared_w == nullptr)) return MOE_E_NULL;
  const void *ptrs[] = {d_x, d_wr, d_wsg, d_logits, d_shared_w};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return MOE_E_ALIGN;
  if (T < 1 || T > 65536 || !width_ok(hidden) || E < 1 || E > MOE_MAX_IDS) return MOE_E_SHAPE;
  clear_pending();
  return from_hip(launch_router(d_x, d_wr, d_wsg, T, hidden, E, d_logits, d_shared_w, stream));
}

moe_status moe_shared_weight(const float *d_shared_w, int32_t T, int32_t kprime, float *d_w, hipStream_t stream) {
  if (!d_shared_w || !d_w) return MOE_E_NULL;
  if (!aligned16(d_shared_w) || !aligned16(d_w)) return MOE_E_ALIGN;
  if (T < 1 || T > 65536 || kprime < 2 || kprime > MOE_MAX_K + 1) return MOE_E_SHAPE;
  clear_pending();
  return from_hip(launch_shared_weight(d_shared_w, T, kprime, d_w, stream));
}

moe_status moe_repack_iq1s(const void *d_ql, const void *d_qh, const void *d_d, int32_t rows, int32_t cols,
                           void *d_ql_out, void *d_qh_out, void *d_sd_out, hipStream_t stream) {
  if (!d_ql || !d_qh || !d_d || !d_ql_out || !d_qh_out || !d_sd_out) return MOE_E_NULL;
  const void *ptrs[] = {d_ql, d_qh, d_d, d_ql_out, d_qh_out, d_sd_out};
  for (const void *p : ptrs)
    if (!aligned16(p)) return MOE_E_ALIGN;
  if (rows < 1 || cols < 256 || cols % 256) return MOE_E_SHAPE;
  const size_t n_blocks = (size_t)rows * (cols / 256);
  if (n_blocks >= ((size_t)1 << 31)) return MOE_E_SHAPE;
  clear_pending();
  return from_hip(launch_repack_iq1s((const uint8_t *)d_ql, (const uint16_t *)d_qh, (const uint16_t *)d_d, n_blocks,
                                     (uint8_t *)d_ql_out, (uint8_t *)d_qh_out, (uint64_t *)d_sd_out, stream));
}

moe_status moe_dequant_f32(int32_t qtype, int32_t rows, int32_t cols, const void *d_s0, const void *d_s1,
                           const void *d_s2, const void *d_grids, float *d_out, hipStream_t stream) {
  if (!d_s0 || !d_s1 || !d_s2 || !d_grids || !d_out) return MOE_E_NULL;
  if (qtype != MOE_Q_IQ2XS_LIKE && qtype != MOE_Q_IQ1M_LIKE) return MOE_E_QTYPE;
  if (rows < 1 || cols < 256 || cols % 256 || rows % 8) return MOE_E_SHAPE;
  const void *ptrs[] = {d_s0, d_s1, d_s2, d_grids, d_out};
  for (const void *p : ptrs)
    if (!aligned16(p)) return MOE_E_ALIGN;
  QMat m{(const uint8_t *)d_s0, (const uint8_t *)d_s1, (const uint8_t *)d_s2};
  clear_pending();
  return from_hip(launch_dequant(qtype, rows, cols, m, (const uint8_t *)d_grids, d_out, stream));
}

moe_status moe_rmsnorm(const float *d_h, int32_t T, int32_t hidden, float eps, float *d_x, hipStream_t stream) {
  if (!d_h || !d_x) return MOE_E_NULL;
  if (!aligned16(d_h) || !aligned16(d_x)) return MOE_E_ALIGN;
  if (T < 1 || hidden < 1 || !(eps >= 0.0f)) return MOE_E_SHAPE;
  clear_pending();
  return from_hip(launch_rmsnorm(d_h, T, hidden, eps, d_x, stream));
}

}  // extern "C"
