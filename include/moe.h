/* moe.h — C ABI of the routed top-k MoE expert layer on codebook-quantized experts,
 * for AMD Instinct MI355X (gfx950).
 *
 * What the layer computes ("Red Metal dev8 — resident routed top-k layer", steps 4-6;
 * "Red Lite dev10 — standalone native Metal path", sections "What is native in dev10"
 * and "Quant grids"): for each token, the router selects k experts; every selected
 * expert decodes its 2-bit-class codebook weights, runs gate and up, SiLU(gate) * up
 * and down, and its output is accumulated as acc += router_weight * expert_output.
 * Every expert stays resident in device memory; nothing is streamed from the host.
 *
 * Conventions for every entry point:
 *  - Pointers named d_* are device memory, allocated and owned by the caller.  The
 *    library never allocates, frees, copies to or from the host, or synchronizes.
 *  - Arguments are validated on the host before anything is enqueued; a rejected call
 *    enqueues nothing and returns a negative moe_status.  On MOE_OK the kernels have
 *    been enqueued on `stream` (0 = the null stream) and run asynchronously: device
 *    faults surface at the caller's next synchronization.
 *  - Every d_* pointer must be 16-byte aligned (MOE_E_ALIGN otherwise).
 *  - The library keeps no mutable global state: calls on different streams with
 *    different buffers may run concurrently.  Calls that share an output or workspace
 *    buffer must be ordered by the caller.
 *  - Results are deterministic: no floating-point atomics; a repeated call on the
 *    same inputs writes the same bits.
 *
 * Quantized matrix layouts (rows x cols, cols % 256 == 0, rows % 8 == 0; blocks run
 * along cols; NB = cols/256 super-blocks, NG = cols/8 groups of 8 weights), three
 * streams per matrix, each row-major by matrix row:
 *
 *  MOE_Q_IQ2XS_LIKE, 70 bytes / 256 weights:
 *    s0 = qs u16[rows][NG]: bits 0-8 grid index (0..511); bits 9-15 sign of weights
 *         0..6 of the group (1 = negative); weight 7 is negative iff bits 9-15 hold an
 *         odd number of ones (the group has an even number of negatives)
 *    s1 = sc u32[rows][NB]: nibble i = scale s of the 32-weight sub-block i
 *    s2 = d  u16[rows][NB]: IEEE binary16 super-block scale
 *    weight = d * (2s + 1) / 8 * (+/- iq2_grid[index][j]),  grid values 8, 25, 43
 *  MOE_Q_IQ1M_LIKE, 56 bytes / 256 weights:
 *    s0 = ql u8[rows][NG]: grid index bits 0-7
 *    s1 = qh u8[rows][NG/2]: group g uses nibble (g & 1) of byte g/2: bits 0-2 = grid
 *         index bits 8-10, bit 3 = delta sign (1 = minus)
 *    s2 = sd u64[rows][NB]: bits 0-15 binary16 d; bits 16+3i..18+3i = scale s of the
 *         16-weight sub-block i
 *    weight = d * (2s + 1) * (iq1_grid[index][j] +/- 1/8),  grid values -1, 0, +1
 *  Both products are exact in fp32.
 *
 * Compact grids ("Red Lite dev10", section "Quant grids"): one u16 per grid row,
 * symbol j in bits 2j..2j+1; IQ2_XS-like 512 rows with symbols 0,1,2 standing for
 * 0x08, 0x19, 0x2b; IQ1_M-like 2048 rows with symbols standing for -1, 0, +1.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 11
#define MOE_MAX_BANKS 4
#define MOE_MAX_K 16        /* routed experts per token */
#define MOE_MAX_IDS 1024    /* E + has_shared */
/* Which experts run where.  In a call of T tokens, experts with at most m(T) tokens
 * form the work list's first set and run on the mat-vec kernels (each weight decoded
 * once per token, the work spread over the expert's rows); experts with more run on the
 * matrix-core grouped GEMM in tiles of up to MOE_MFMA_TILE_TOKENS tokens (each weight
 * decoded once per tile).  m(T) = T for small batches, T <= MOE_SMALL_BATCH_TOKENS
 * (every expert in the first set: too few tiles would leave most of the GPU idle), else
 * MOE_MATVEC_MAX_TOKENS = 0: above it every expert with a token runs on the matrix
 * cores, and the mat-vec kernels are not launched.  For 2 to 8 tokens and inter <= 512,
 * gate / up of the first set runs instead on a matrix-core decode kernel that decodes
 * each weight once per call into fragments the expert's tokens share.  The work list
 * written by moe_route_group keeps the two sets apart. */
#define MOE_MATVEC_MAX_TOKENS 0
#define MOE_SMALL_BATCH_TOKENS 16
#define MOE_MFMA_TILE_TOKENS 16

typedef enum {
  MOE_OK = 0,
  MOE_E_NULL = -1,      /* a required pointer is NULL */
  MOE_E_SHAPE = -2,     /* a size is out of range or inconsistent */
  MOE_E_QTYPE = -3,     /* unknown quantization type */
  MOE_E_ALIGN = -4,     /* a device pointer is not 16-byte aligned */
  MOE_E_WORKSPACE = -5, /* workspace smaller than moe_workspace_bytes() */
  MOE_E_HIP = -6        /* the HIP runtime reported an error at launch */
} moe_status;

typedef enum { MOE_Q_IQ2XS_LIKE = 1, MOE_Q_IQ1M_LIKE = 2 } moe_qtype;

/* Experts [first_expert, first_expert + n_experts) of a layer, all in one format.
 * Expert i of the bank has its gate (inter x hidden), up (inter x hidden) and down
 * (hidden x inter) streams at base + i * (that stream's size for that shape). */
typedef struct {
  int32_t qtype;
  int32_t first_expert;
  int32_t n_experts;
  int32_t reserved;
  const void *gate[3];
  const void *up[3];
  const void *down[3];
} moe_bank;

/* One routed layer ("Red Lite dev16 — complete full-attention parity": top-10 routed
 * MoE plus shared expert).  Routed experts have ids 0..E-1; with has_shared the shared
 * expert has id E.  The banks must cover ids 0..E-1+has_shared without overlap.
 * hidden and inter are each one of 256, 512, 1024 or 2048 (MOE_E_SHAPE otherwise; the
 * one-launch decode calls narrow this further).  Host memory; read during the call
 * only. */
typedef struct {
  int32_t hidden;
  int32_t inter;
  int32_t n_experts;
  int32_t has_shared;
  int32_t n_banks;
  int32_t reserved;
  moe_bank banks[MOE_MAX_BANKS];
  const void *grids; /* device buffer filled by moe_grids_expand */
} moe_layer;

int32_t moe_abi_version(void);
const char *moe_status_string(moe_status s);

/* The hipError_t of the calling thread's last call that returned MOE_E_HIP, and its
 * name.  Errors left pending by the caller's own earlier runtime calls are cleared,
 * not reported, when a call passes validation. */
int32_t moe_last_hip_error(void);
const char *moe_last_hip_error_string(void);

/* Size of the expanded-grid buffer: the grid values of both formats, the compact rows,
 * and the fp16 tables the matrix-core decode kernels copy into LDS (written once here
 * instead of built by every workgroup). */
size_t moe_grids_bytes(void);

/* Expands the compact grids once ("Red Lite dev10", section "Quant grids": the runtime
 * expands the compact tables once before use).  d_compact_iq2: u16[512],
 * d_compact_iq1: u16[2048], d_grids: moe_grids_bytes() bytes.  Symbol value 3 is not
 * allowed; it expands to grid value 0 (the caller's contract). */
moe_status moe_grids_expand(const uint16_t *d_compact_iq2, const uint16_t *d_compact_iq1, void *d_grids,
                            hipStream_t stream);

/* Ints of the work list moe_route_group writes for T tokens, kprime slots per token
 * and n_ids = E + add_shared expert ids. */
int32_t moe_work_ints(int32_t T, int32_t kprime, int32_t n_ids);

/* Workspace needed by moe_expert_ffn_q for T tokens with kprime slots each. */
size_t moe_workspace_bytes(int32_t T, int32_t kprime, int32_t hidden, int32_t inter);

/* Router and grouping ("Red Metal dev8", steps 3-4: every selected expert of the layer
 * is made resident and run; default validation uses positive router weights that sum
 * to about one).  Per token t:
 *   - with d_logits ([T][E] fp32, finite): the k largest logits, ties to the lower id,
 *     in descending order, weights softmax(logits) renormalised over the selected set;
 *     logits are compared as IEEE values, so -0.0 and +0.0 tie;
 *   - with d_logits == NULL: d_ids[t][0..k-1] and d_w[t][0..k-1] are inputs (k distinct
 *     ids in [0, E) per token) and only the shared slot and the grouping are written;
 *   - with add_shared: slot k is (E, 1.0).  kprime = k + add_shared.
 * Outputs (device): d_ids, d_w [T][kprime]; d_counts [E + add_shared]; d_offsets
 * [E + add_shared + 1] (exclusive scan of counts); d_sorted_slot [T*kprime]: slots
 * s = t*kprime + j ordered by (expert id, s); d_slot_pos: its inverse; d_work
 * [moe_work_ints(T, kprime, E + add_shared)]: the work list of the FFN calls, records
 * of 4 ints.  With n_ids = E + add_shared:
 *   record 0 = (n1, T*kprime, n2, nt): n1 experts with 1..m(T) slots (see above),
 *     n2 experts with more, nt tiles;
 *   records 1..n1: (expert id, offsets[e], offsets[e+1], d_sorted_slot[offsets[e]]) of
 *     the first set, ascending id;
 *   records n_ids+1 .. n_ids+nt: the tiles of the second set, (expert id, p0, p1, 0)
 *     covering sorted positions [p0, p1) of the expert, MOE_MFMA_TILE_TOKENS at a time,
 *     ascending (id, p0).
 * Limits: 1 <= T <= 65536, 1 <= k <= min(E, MOE_MAX_K), E + add_shared <= MOE_MAX_IDS. */
moe_status moe_route_group(const float *d_logits, int32_t T, int32_t E, int32_t k, int32_t add_shared,
                           int32_t *d_ids, float *d_w, int32_t *d_counts, int32_t *d_offsets,
                           int32_t *d_sorted_slot, int32_t *d_slot_pos, int32_t *d_work,
                           hipStream_t stream);

/* Expert FFNs ("Red Metal dev8", step 4: gate, up, SiLU(gate) * up and down per
 * selected expert).  For every sorted position p (0 <= p < T*kprime) with slot
 * s = d_sorted_slot[p] of token t = s / kprime and expert e (offsets[e] <= p <
 * offsets[e+1]):  d_y[p] = Wd_e (SiLU(Wg_e x_t) * (Wu_e x_t)).
 * d_x [T][hidden] fp32; d_sorted_slot and d_work from moe_route_group;
 * d_y [T*kprime][hidden] fp32 in sorted order.  d_ws: at least
 * moe_workspace_bytes(T, kprime, hidden, inter) bytes of scratch (holds h).  Runs
 * moe_expert_gateup_q then moe_expert_down_q.  Accuracy: max |error| <= 2e-5 * ||y_p||_2
 * against an fp32 reference.  Limits: 1 <= T <= 65536, 1 <= kprime <= MOE_MAX_K + 1. */
moe_status moe_expert_ffn_q(const moe_layer *layer, const float *d_x, int32_t T, int32_t kprime,
                            const int32_t *d_sorted_slot, const int32_t *d_work, float *d_y, void *d_ws,
                            size_t ws_bytes, hipStream_t stream);

/* Gate and up with the SiLU epilogue ("Red Metal dev8", step 4, first half): for every
 * sorted position p as above, d_h[p] = SiLU(Wg_e x_t) * (Wu_e x_t), fp32
 * [T*kprime][inter].  Weights are decoded in registers: experts with at most
 * m(T) tokens on the mat-vec kernel, the others on the matrix cores
 * (fp16 weights, exact, times activations split into two fp16 halves, fp32 sums;
 * activations must lie within the fp16 range, |x| < 65504). */
moe_status moe_expert_gateup_q(const moe_layer *layer, const float *d_x, int32_t T, int32_t kprime,
                               const int32_t *d_sorted_slot, const int32_t *d_work, float *d_h, hipStream_t stream);

/* Down projection ("Red Metal dev8", step 4, second half): d_y[p] = Wd_e d_h[p], fp32
 * [T*kprime][hidden] in sorted order; experts split between the mat-vec kernel and the
 * matrix cores as in moe_expert_gateup_q (|h| < 65504 for the latter). */
moe_status moe_expert_down_q(const moe_layer *layer, const float *d_h, int32_t T, int32_t kprime,
                             const int32_t *d_work, float *d_y, hipStream_t stream);

/* Down projection fused with the weighted accumulation ("Red Metal dev8", steps 4-5):
 * d_acc[t][c] += w * (Wd_e d_h[slot_pos[s]])[c] over the slots s of token t in ascending
 * expert id, one fp32 multiply and one fp32 add per slot -- bit-identical to
 * moe_expert_down_q followed by moe_accumulate.  d_h is in sorted order (as written by
 * moe_expert_gateup_q).  Reads each selected expert's down matrix once per token, so it
 * is meant for decode (few tokens); for many tokens per expert use the separate calls. */
moe_status moe_expert_down_accumulate_q(const moe_layer *layer, const float *d_h, int32_t T, int32_t kprime,
                                        const int32_t *d_ids, const float *d_w, const int32_t *d_slot_pos,
                                        float *d_acc, hipStream_t stream);

/* Workspace of moe_layer_decode_q: MOE_DECODE_SYNC_BYTES of synchronisation words, then h
 * [kprime][inter] as 64-bit (fp32 bits, call tag) pairs. */
#define MOE_DECODE_SYNC_BYTES 4352
#define MOE_DECODE_ERROR_OFFSET 128
size_t moe_decode_workspace_bytes(int32_t kprime, int32_t inter);

/* One decode step of a layer for one token, in one launch ("Red Metal dev8", steps 3-6:
 * route, run every selected expert, accumulate; only the layer output leaves the
 * call).  Computes exactly what moe_route_group (T = 1), moe_expert_gateup_q and
 * moe_expert_down_accumulate_q compute, bit for bit, and writes the same outputs:
 * d_ids, d_w [kprime]; d_counts, d_offsets, d_sorted_slot, d_slot_pos, d_work as
 * moe_route_group; d_acc [hidden] (in/out).  d_logits [E] or NULL (explicit d_ids /
 * d_w inputs, as in moe_route_group); d_x [hidden].  kprime = k + add_shared;
 * add_shared must equal the layer's has_shared.
 * d_ws: moe_decode_workspace_bytes(kprime, inter) bytes, ALL zero before the first call
 * (not only the synchronisation words: the h pairs carry call tags that restart at 1
 * when the words are zeroed, so old pairs would read as fresh).  Each call leaves the
 * workspace ready for the next, whatever the layer (calls that share a workspace must
 * not overlap, and a workspace serves one device).  To reset a workspace, zero all of it.
 * Status word: the uint32 at byte 128 (MOE_DECODE_ERROR_OFFSET) becomes nonzero if a
 * wait of the kernel for another workgroup's h values ever timed out, which can only
 * happen when other kernels hold compute units while this one runs; the results of that
 * call are then undefined and the whole workspace must be zeroed before the next call.
 * The call cannot report this in its return value (it returns before the kernel runs):
 * read the word after the stream has finished the call.
 * Limits: hidden == 2048, inter == 256 or 512, E <= 512. */
moe_status moe_layer_decode_q(const moe_layer *layer, const float *d_logits, const float *d_x, int32_t k,
                              int32_t add_shared, int32_t *d_ids, float *d_w, int32_t *d_counts, int32_t *d_offsets,
                              int32_t *d_sorted_slot, int32_t *d_slot_pos, int32_t *d_work, float *d_acc, void *d_ws,
                              size_t ws_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, serving
 * loops that allow no hipMalloc): moe_layer_decode_q with its workspace in the library's
 * own static device array of MOE_DECODE_STATIC_BYTES per device, which each device holds
 * until the process ends.  The call allocates nothing; it computes and writes exactly
 * what moe_layer_decode_q does, with the same arguments and limits, except:
 *   d_status: one uint32 (device, output), set after the decode to its status word:
 *     nonzero if a wait for another workgroup's values timed out (the call's results
 *     are then undefined).
 * The first call on a device looks the array up and zeroes it on the stream; every call
 * zeroes it again after its decode, so each call starts from a zeroed workspace.  Every
 * call on a device shares that device's array: calls that overlap on one device (other
 * streams, other host threads) race and give undefined results.  A call whose kprime
 * and inter would need more than MOE_DECODE_STATIC_BYTES returns MOE_E_WORKSPACE (the
 * limits of moe_layer_decode_q keep every valid call within it). */
#define MOE_DECODE_STATIC_BYTES 73984 /* MOE_DECODE_SYNC_BYTES + (MOE_MAX_K + 1) * 512 * 8 */
moe_status moe_layer_decode_q_static(const moe_layer *layer, const float *d_logits, const float *d_x, int32_t k,
                                     int32_t add_shared, int32_t *d_ids, float *d_w, int32_t *d_counts,
                                     int32_t *d_offsets, int32_t *d_sorted_slot, int32_t *d_slot_pos, int32_t *d_work,
                                     float *d_acc, uint32_t *d_status, hipStream_t stream);

/* ---- Decode of a residual chain of layers in one launch ("Red Lite dev16 -- complete
 * full-attention parity", section "Pinned full-attention graph": in the field model each
 * block's routed MoE reads the post-attention RMSNorm of the hidden state and its output
 * is added back to it; section "Scope boundary": the 48-layer scheduler is the next
 * gate).  For
 * one token, l = 0 .. n_layers-1:
 *     h_{l+1} = h_l + MoE_l(RMSNorm(h_l)),
 * with MoE_l routed by its own logits row.  The attention part of the blocks is not
 * part of this call.
 *
 * Workspace, moe_stack_workspace_bytes(n_layers, kprime, hidden, inter) bytes:
 *   [0, MOE_DECODE_SYNC_BYTES)   synchronisation words;
 *   [MOE_DECODE_SYNC_BYTES, +moe_stack_table_bytes(n_layers))   the layer table, copied
 *                                there by the caller from the host buffer that
 *                                moe_stack_table filled;
 *   the rest                     per-layer exchange buffers (tagged pairs).
 * To set up: zero the WHOLE workspace (the exchange buffers too: their tags restart
 * with the synchronisation words), then copy the table in.  To reset it later, do the
 * same.  A table stays valid while the layers' device buffers do. */
#define MOE_MAX_STACK_LAYERS 256
size_t moe_stack_workspace_bytes(int32_t n_layers, int32_t kprime, int32_t hidden, int32_t inter);
size_t moe_stack_table_bytes(int32_t n_layers);

/* Host-only: validates the layers for moe_stack_decode_q and writes their table to the
 * host buffer h_table (table_bytes >= moe_stack_table_bytes(n_layers); no alignment
 * needed).  Enqueues nothing and touches no device memory. */
moe_status moe_stack_table(const moe_layer *layers, int32_t n_layers, void *h_table, size_t table_bytes);

/* One decode step of the chain for one token, in one launch.  Each layer computes,
 * bit for bit, what moe_rmsnorm followed by moe_layer_decode_q with d_acc = the
 * residual computes (so the chain's result equals that sequence of calls).
 *   layers [n_layers] (host): the layers whose table the workspace holds, in order;
 *     every layer has hidden == 2048, the same inter (256 or 512), the same n_experts
 *     (<= 512) and has_shared, and the same d_grids pointer.
 *   d_logits [n_layers][E]: router logits of each layer (the router is not part of
 *     the call).
 *   d_h_in [hidden]: h_0, read only; d_h_out [hidden]: h_{n_layers}.  The two must
 *     not overlap (a workgroup with no work in a layer may still be reading d_h_in
 *     when the last layer's rows are written).
 *   d_ids / d_w [n_layers][kprime]: each layer's selection as moe_route_group writes
 *     it, or both NULL.
 *   eps: RMSNorm epsilon (>= 0).
 * The synchronisation rules of moe_layer_decode_q apply to the workspace (the status
 * word at MOE_DECODE_ERROR_OFFSET, read after the call has run; after an error, zero
 * the whole workspace and copy the table in again).
 * Limits: 1 <= n_layers <= MOE_MAX_STACK_LAYERS. */
moe_status moe_stack_decode_q(const moe_layer *layers, int32_t n_layers, const float *d_logits, const float *d_h_in,
                              float *d_h_out, int32_t k, int32_t add_shared, float eps, int32_t *d_ids, float *d_w,
                              void *d_ws, size_t ws_bytes, hipStream_t stream);

/* Weighted accumulation ("Red Metal dev8", step 5: accumulator += router_weight *
 * expert_output after each expert).  d_acc[t][c] (in/out) gets w * y added for each
 * slot of token t, taken in ascending expert id (the shared expert, id E, last), as
 * one fp32 multiply and one fp32 add per slot.  d_y is in sorted order; d_slot_pos
 * maps a slot to its sorted position. */
moe_status moe_accumulate(const float *d_y, const float *d_w, const int32_t *d_ids, const int32_t *d_slot_pos,
                          int32_t T, int32_t kprime, int32_t hidden, float *d_acc, hipStream_t stream);

/* Router projection ("Red Lite dev9 — native runtime foundation", closing paragraph, and
 * "Red Lite dev10 — standalone native Metal path", section "What dev10 does not yet
 * claim": the router network in front of the top-k path, read as one linear map):
 *   d_logits[t][e] = sum_c d_x[t][c] * d_wr[e][c]      fp32 [T][E]
 * d_x [T][hidden] fp32; d_wr [E][hidden] fp32 row-major.  With d_wsg [hidden] (else
 * NULL), also d_shared_w[t] = 1 / (1 + exp(-sum_c d_x[t][c] * d_wsg[c])), a gate for the
 * shared expert (the pages say nothing on one; NULL keeps the weight 1.0).  Each dot is
 * fp32 with a fixed summation order that depends on hidden only, so a token's logits
 * are the same bits in any batch.  d_wsg and d_shared_w: both or neither.
 * Limits: 1 <= T <= 65536, hidden in {256, 512, 1024, 2048}, 1 <= E <= MOE_MAX_IDS. */
moe_status moe_router_logits(const float *d_x, const float *d_wr, const float *d_wsg, int32_t T, int32_t hidden,
                             int32_t E, float *d_logits, float *d_shared_w, hipStream_t stream);

/* The gated shared expert's weight: d_w[t][kprime - 1] = d_shared_w[t] for every token
 * (d_w as moe_route_group wrote it with add_shared = 1, whose last slot is the shared
 * expert with weight 1.0).  Limits: 1 <= T <= 65536, 2 <= kprime <= MOE_MAX_K + 1. */
moe_status moe_shared_weight(const float *d_shared_w, int32_t T, int32_t kprime, float *d_w, hipStream_t stream);

/* IQ1_S-like matrices (qtype 4, never passed to the other calls), 50 bytes / 256 weights,
 * the IQ1_M-like grid: s0 = ql u8[rows][NG] (index bits 0-7); s1 = qh u16[rows][NG/4],
 * one word per 32-weight sub-block: bits 3i..3i+2 = index bits 8-10 of its group i,
 * bits 12-14 = 3-bit scale s, bit 15 = delta sign (1 = minus); s2 = d u16[rows][NB].
 * weight = d * (2s + 1) * (iq1_grid[index][j] +/- 1/8).  ("Red Lite dev10 — standalone
 * native Metal path", section "Quant grids": IQ1_M reuses the IQ1_S grid; the packing
 * is a reading.) */
#define MOE_Q_IQ1S_LIKE 4

/* Repacks IQ1_S-like streams of `rows` rows of `cols` columns (any number of matrices of
 * one width back to back) into the IQ1_M-like layout, exactly: every weight keeps its
 * bits (the per-32 scale and sign are repeated per 16 and per 8).  Outputs: ql_out
 * rows*cols/8 bytes (may equal d_ql), qh_out rows*cols/16 bytes, sd_out rows*cols/256
 * u64.  Done once when a layer is loaded; the layer then uses MOE_Q_IQ1M_LIKE banks.
 * Limits: rows >= 1, cols a positive multiple of 256, rows * cols / 256 < 2^31. */
moe_status moe_repack_iq1s(const void *d_ql, const void *d_qh, const void *d_d, int32_t rows, int32_t cols,
                           void *d_ql_out, void *d_qh_out, void *d_sd_out, hipStream_t stream);

/* Bit-exact dequantization of one matrix to fp32, row-major rows x cols (debug/test). */
moe_status moe_dequant_f32(int32_t qtype, int32_t rows, int32_t cols, const void *d_s0, const void *d_s1,
                           const void *d_s2, const void *d_grids, float *d_out, hipStream_t stream);

/* Unit-weight RMSNorm, x = h / sqrt(mean(h^2) + eps) per row ("Red Lite dev16": the
 * routed MoE of a block reads the post-attention RMSNorm of the hidden state).
 * d_h, d_x: [T][hidden] fp32 (may alias). */
moe_status moe_rmsnorm(const float *d_h, int32_t T, int32_t hidden, float eps, float *d_x, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif
