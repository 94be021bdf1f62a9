/* Plain CPU oracle for the routed top-k MoE layer on codebook-quantized experts.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg load this library.  It shares no code, header, table or constant
 * with the GPU library: both sides see the same input bytes and nothing else.
 *
 * What it computes (pages: "Red Metal dev8 — resident routed top-k layer", steps 4-6;
 * "Red Lite dev10 — standalone native Metal path", sections "What is native in dev10"
 * and "Quant grids"; "Red Lite dev16 — complete full-attention parity", the block
 * composition with post-attention RMSNorm, routed MoE plus shared expert and residual):
 *
 *   route:      per token, the k largest logits (ties: lower expert id), weights are
 *               the softmax renormalised over the selected experts;
 *   group:      stable counting sort of the (token, slot) pairs by expert id;
 *   dequantize: every weight from its grid row, signs / delta and scales;
 *   FFN:        g = Wg x, u = Wu x, h = SiLU(g) * u, y = Wd h  (fp32, sequential dots);
 *   accumulate: acc += w * y over a token's experts in ascending expert id.
 *
 * Stream layouts and grid symbol encodings are those documented in the input
 * generator (synth/__init__.py).  All arrays are host memory owned by the caller.
 * Functions that can fail return 0 on success and a negative value on bad input.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_IQ2XS = 1, ORC_IQ1M = 2, ORC_IQ1S = 4 };

typedef struct {
  int32_t qtype, rows, cols, pad_;
  const void *s0, *s1, *s2; /* IQ2: qs, sc, d   IQ1: ql, qh, sd */
} orc_qmat;

typedef struct {
  orc_qmat gate, up, down; /* gate/up: inter x hidden, down: hidden x inter */
} orc_expert;

typedef struct {
  uint8_t iq2[512 * 8];  /* values 8, 25, 43 */
  int8_t iq1[2048 * 8];  /* values -1, 0, +1 */
} orc_grids;

float orc_f16_to_f32(uint16_t h);

/* Threads for the row loop of orc_matvec; every output is computed the same way. */
void orc_set_threads(int n);

/* Compact rows (symbol j in bits 2j..2j+1) -> value rows.  -1 if a symbol is 3. */
int orc_grids_expand(const uint16_t *compact_iq2, const uint16_t *compact_iq1, orc_grids *g);

/* Weight (r, c) of a matrix, in fp32 and in fp64 (identical values: the product is exact). */
float orc_weight(const orc_qmat *m, const orc_grids *g, int r, int c);
double orc_weight_f64(const orc_qmat *m, const orc_grids *g, int r, int c);
int orc_dequant(const orc_qmat *m, const orc_grids *g, float *out /* rows*cols */);

/* y = W x with fp32 products and sums, columns in order; fp64 twin. */
int orc_matvec(const orc_qmat *m, const orc_grids *g, const float *x, float *y);
int orc_matvec_f64(const orc_qmat *m, const orc_grids *g, const double *x, double *y);

float orc_silu(float g);
double orc_silu_f64(double g);

/* One expert on one token: y[hidden], optional h[inter]. */
int orc_expert_ffn(const orc_expert *e, const orc_grids *g, const float *x, float *y, float *h);
int orc_expert_ffn_f64(const orc_expert *e, const orc_grids *g, const double *x, double *y, double *h);

/* ids/w: [T][kp], kp = k + add_shared; the shared slot is (E, 1.0). */
int orc_route(const float *logits, int T, int E, int k, int add_shared, int32_t *ids, float *w);
int orc_route_f64(const float *logits, int T, int E, int k, int add_shared, int32_t *ids, double *w);

/* counts[n_ids], offsets[n_ids+1], sorted_slot / slot_pos [T*kp]. */
int orc_group(const int32_t *ids, int T, int kp, int n_ids, int32_t *counts, int32_t *offsets,
              int32_t *sorted_slot, int32_t *slot_pos);

/* acc[t] += w * y over the token's slots in ascending expert id; y is [T*kp][H] in slot order. */
int orc_accumulate(const float *y, const float *w, const int32_t *ids, int T, int kp, int H, float *acc);
int orc_accumulate_f64(const double *y, const double *w, const int32_t *ids, int T, int kp, int H, double *acc);

/* The whole layer.  experts[id] for id in [0, E + add_shared).  With logits == NULL the
 * selection is taken from ids_in / w_in ([T][k]) and only the shared slot is appended.
 * Outputs ids_out / w_out ([T][kp]) and y_out ([T*kp][H], slot order) may be NULL.
 * n_threads > 1 spreads independent output rows over OpenMP threads (same results). */
int orc_moe_layer(const orc_expert *experts, const orc_grids *g, const float *x, const float *logits,
                  const int32_t *ids_in, const float *w_in, int T, int E, int k, int add_shared, int H,
                  float *acc, int32_t *ids_out, float *w_out, float *y_out, int n_threads);
int orc_moe_layer_f64(const orc_expert *experts, const orc_grids *g, const double *x, const float *logits,
                      const int32_t *ids_in, const double *w_in, int T, int E, int k, int add_shared, int H,
                      double *acc, double *y_out);

/* x = h / sqrt(mean(h^2) + eps) per row of H values. */
int orc_rmsnorm(const float *h, int T, int H, float eps, float *x);
int orc_rmsnorm_f64(const double *h, int T, int H, double eps, double *x);

/* Router projection: logits [T][E] = x [T][H] times wr [E][H] transposed; with wsg [H]
 * (else NULL), sw [T] = sigmoid(x . wsg), the shared expert's weight.  fp32 sums in
 * column order; the _f64 variant sums in double.  orc_dot_abs: sum_c |x[t][c] w[e][c]|. */
int orc_router(const float *x, const float *wr, const float *wsg, int T, int H, int E, float *logits, float *sw);
int orc_router_f64(const float *x, const float *wr, const float *wsg, int T, int H, int E, double *logits,
                   double *sw);
int orc_dot_abs(const float *x, const float *w, int T, int H, int E, double *out);

#ifdef __cplusplus
}
#endif
#endif
