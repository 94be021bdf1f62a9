/* Plain CPU oracle for the routed top-k MoE layer on codebook-quantized experts.
 * TEST INFRASTRUCTURE ONLY: see oracle.h.  Built with -O2 -ffp-contract=off and no
 * fast-math, so every float expression rounds exactly as written.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

static int g_threads = 1;

/* Threads used by orc_matvec for independent rows (results do not depend on it). */
void orc_set_threads(int n) { g_threads = n > 1 ? n : 1; }

/* ------------------------------------------------------------------ binary16 */

float orc_f16_to_f32(uint16_t h) {
  int sign = (h >> 15) & 1, ex = (h >> 10) & 31, man = h & 1023;
  float v;
  if (ex == 0)
    v = ldexpf((float)man, -24);               /* zero / subnormal */
  else if (ex == 31)
    v = man ? NAN : INFINITY;
  else
    v = ldexpf((float)(1024 + man), ex - 25);  /* (1 + man/1024) * 2^(ex-15) */
  return sign ? -v : v;
}

/* ------------------------------------------------------------------ grids
 * "Red Lite dev10 — standalone native Metal path", section "Quant grids": the IQ2_XS
 * grid is 512 x 8 with 2-bit symbols standing for 0x08 / 0x19 / 0x2b; the IQ1_M grid
 * is 2048 x 8 with symbols standing for -1 / 0 / +1.  Expanded once, before use. */

static const uint8_t kIq2Sym[3] = {0x08, 0x19, 0x2b};
static const int8_t kIq1Sym[3] = {-1, 0, 1};

int orc_grids_expand(const uint16_t *c2, const uint16_t *c1, orc_grids *g) {
  for (int r = 0; r < 512; r++)
    for (int j = 0; j < 8; j++) {
      int s = (c2[r] >> (2 * j)) & 3;
      if (s == 3) return -1;
      g->iq2[r * 8 + j] = kIq2Sym[s];
    }
  for (int r = 0; r < 2048; r++)
    for (int j = 0; j < 8; j++) {
      int s = (c1[r] >> (2 * j)) & 3;
      if (s == 3) return -1;
      g->iq1[r * 8 + j] = kIq1Sym[s];
    }
  return 0;
}

/* ------------------------------------------------------------------ dequantization
 * One weight at a time, straight from the stream layout.
 *
 * IQ2_XS-like, per 8 weights a 9-bit grid index, 7 sign bits and a parity sign, a 4-bit
 * scale per 32 weights and an fp16 scale per 256 weights:
 *     w = d * (2s + 1) * 0.125 * (+/- grid[idx][j])
 * IQ1_M-like, per 8 weights an 11-bit grid index and a delta sign, a 3-bit scale per
 * 16 weights and an fp16 scale per 256 weights:
 *     w = d * (2s + 1) * (grid[idx][j] +/- 0.125)
 * IQ1_S-like ("Red Lite dev10", section "Quant grids": IQ1_M reuses the IQ1_S grid; the
 * packing is a reading): the same grid and formula, but one 3-bit scale and one delta
 * sign per 32 weights, packed with the four groups' index high bits in a u16. 
 * Both products have at most 22 significant bits, so they are exact in fp32. */

static int popcount7(unsigned v) {
  int n = 0;
  for (int i = 0; i < 7; i++) n += (v >> i) & 1;
  return n;
}

typedef struct {
  double d, scale, value; /* w = d * scale * value, each factor exact */
} wparts;

static wparts weight_parts(const orc_qmat *m, const orc_grids *g, int r, int c) {
  wparts p;
  int ng = m->cols / 8, nb = m->cols / 256;
  int b = c / 256, grp = c / 8, j = c % 8, inblk = c % 256;
  if (m->qtype == ORC_IQ2XS) {
    uint16_t qs = ((const uint16_t *)m->s0)[(size_t)r * ng + grp];
    uint32_t sc = ((const uint32_t *)m->s1)[(size_t)r * nb + b];
    uint16_t dh = ((const uint16_t *)m->s2)[(size_t)r * nb + b];
    unsigned idx = qs & 0x1FF, signs = qs >> 9;
    int neg = (j < 7) ? (int)((signs >> j) & 1) : (popcount7(signs) & 1);
    int s = (sc >> (4 * (inblk / 32))) & 15;
    double gv = (double)g->iq2[idx * 8 + j];
    p.d = (double)orc_f16_to_f32(dh);
    p.scale = (double)(2 * s + 1) * 0.125;
    p.value = neg ? -gv : gv;
  } else if (m->qtype == ORC_IQ1S) {
    uint8_t ql = ((const uint8_t *)m->s0)[(size_t)r * ng + grp];
    uint16_t qh = ((const uint16_t *)m->s1)[(size_t)r * (ng / 4) + grp / 4];
    uint16_t dh = ((const uint16_t *)m->s2)[(size_t)r * nb + b];
    unsigned idx = ql | (((qh >> (3 * (grp % 4))) & 7u) << 8);
    int dneg = (qh >> 15) & 1;
    int s = (qh >> 12) & 7;
    p.d = (double)orc_f16_to_f32(dh);
    p.scale = (double)(2 * s + 1);
    p.value = (double)g->iq1[idx * 8 + j] + (dneg ? -0.125 : 0.125);
  } else {
    uint8_t ql = ((const uint8_t *)m->s0)[(size_t)r * ng + grp];
    uint8_t qhb = ((const uint8_t *)m->s1)[(size_t)r * (ng / 2) + grp / 2];
    uint64_t sd = ((const uint64_t *)m->s2)[(size_t)r * nb + b];
    unsigned nib = (grp & 1) ? (qhb >> 4) : (qhb & 15);
    unsigned idx = ql | ((nib & 7u) << 8);
    int dneg = (nib >> 3) & 1;
    int s = (int)((sd >> (16 + 3 * (inblk / 16))) & 7);
    p.d = (double)orc_f16_to_f32((uint16_t)(sd & 0xFFFF));
    p.scale = (double)(2 * s + 1);
    p.value = (double)g->iq1[idx * 8 + j] + (dneg ? -0.125 : 0.125);
  }
  return p;
}

float orc_weight(const orc_qmat *m, const orc_grids *g, int r, int c) {
  wparts p = weight_parts(m, g, r, c);
  return (float)p.d * (float)p.scale * (float)p.value;
}

double orc_weight_f64(const orc_qmat *m, const orc_grids *g, int r, int c) {
  wparts p = weight_parts(m, g, r, c);
  return p.d * p.scale * p.value;
}

static int check_mat(const orc_qmat *m) {
  if (!m || !m->s0 || !m->s1 || !m->s2) return -1;
  if (m->qtype != ORC_IQ2XS && m->qtype != ORC_IQ1M && m->qtype != ORC_IQ1S) return -3;
  if (m->rows <= 0 || m->cols <= 0 || m->cols % 256) return -2;
  return 0;
}

int orc_dequant(const orc_qmat *m, const orc_grids *g, float *out) {
  int rc = check_mat(m);
  if (rc) return rc;
  for (int r = 0; r < m->rows; r++)
    for (int c = 0; c < m->cols; c++) out[(size_t)r * m->cols + c] = orc_weight(m, g, r, c);
  return 0;
}

/* ------------------------------------------------------------------ mat-vec
 * "Red Metal dev8 — resident routed top-k layer", step 4: every selected expert runs
 * gate, up, SiLU(gate) * up and down.  Each output is a plain dot product: products
 * and sums in fp32, in column order, one row at a time. */

int orc_matvec(const orc_qmat *m, const orc_grids *g, const float *x, float *y) {
  int rc = check_mat(m);
  if (rc) return rc;
#pragma omp parallel for num_threads(g_threads) if (g_threads > 1) schedule(static)
  for (int r = 0; r < m->rows; r++) {
    float acc = 0.0f;
    for (int c = 0; c < m->cols; c++) {
      float prod = orc_weight(m, g, r, c) * x[c];
      acc = acc + prod;
    }
    y[r] = acc;
  }
  return 0;
}

int orc_matvec_f64(const orc_qmat *m, const orc_grids *g, const double *x, double *y) {
  int rc = check_mat(m);
  if (rc) return rc;
  for (int r = 0; r < m->rows; r++) {
    double acc = 0.0;
    for (int c = 0; c < m->cols; c++) acc += orc_weight_f64(m, g, r, c) * x[c];
    y[r] = acc;
  }
  return 0;
}

/* SiLU(g) = g * sigmoid(g) = g / (1 + exp(-g)). */
float orc_silu(float g) { return g / (1.0f + expf(-g)); }
double orc_silu_f64(double g) { return g / (1.0 + exp(-g)); }

int orc_expert_ffn(const orc_expert *e, const orc_grids *g, const float *x, float *y, float *h_out) {
  int inter = e->gate.rows, rc;
  if (e->up.rows != inter || e->down.cols != inter || e->gate.cols != e->up.cols ||
      e->down.rows != e->gate.cols)
    return -2;
  float *gv = malloc(sizeof(float) * inter), *uv = malloc(sizeof(float) * inter),
        *h = malloc(sizeof(float) * inter);
  rc = orc_matvec(&e->gate, g, x, gv);
  if (!rc) rc = orc_matvec(&e->up, g, x, uv);
  if (!rc) {
    for (int i = 0; i < inter; i++) h[i] = orc_silu(gv[i]) * uv[i];
    rc = orc_matvec(&e->down, g, h, y);
    if (h_out) memcpy(h_out, h, sizeof(float) * inter);
  }
  free(gv);
  free(uv);
  free(h);
  return rc;
}

int orc_expert_ffn_f64(const orc_expert *e, const orc_grids *g, const double *x, double *y, double *h_out) {
  int inter = e->gate.rows, rc;
  if (e->up.rows != inter || e->down.cols != inter || e->gate.cols != e->up.cols ||
      e->down.rows != e->gate.cols)
    return -2;
  double *gv = malloc(sizeof(double) * inter), *uv = malloc(sizeof(double) * inter),
         *h = malloc(sizeof(double) * inter);
  rc = orc_matvec_f64(&e->gate, g, x, gv);
  if (!rc) rc = orc_matvec_f64(&e->up, g, x, uv);
  if (!rc) {
    for (int i = 0; i < inter; i++) h[i] = orc_silu_f64(gv[i]) * uv[i];
    rc = orc_matvec_f64(&e->down, g, h, y);
    if (h_out) memcpy(h_out, h, sizeof(double) * inter);
  }
  free(gv);
  free(uv);
  free(h);
  return rc;
}

/* ------------------------------------------------------------------ routing
 * Selection: the k largest logits, scanning experts in ascending id and keeping the
 * first of equal values, so ties go to the lower id.  Weights: softmax over all E
 * logits renormalised over the selected set, which equals exp(l_j - m) / sum over the
 * selected of exp(l_i - m) with m the largest selected logit.  The shared expert,
 * when present, is appended as (E, 1.0).  ("Red Metal dev8", positive router weights
 * normalised to about 1.0; "Red Lite dev16", routed MoE plus shared expert.) */

static int select_topk(const float *l, int E, int k, int32_t *ids) {
  char *taken = calloc((size_t)E, 1);
  if (!taken) return -1;
  for (int j = 0; j < k; j++) {
    int best = -1;
    for (int e = 0; e < E; e++)
      if (!taken[e] && (best < 0 || l[e] > l[best])) best = e;
    taken[best] = 1;
    ids[j] = best;
  }
  free(taken);
  return 0;
}

int orc_route(const float *logits, int T, int E, int k, int add_shared, int32_t *ids, float *w) {
  if (!logits || !ids || !w) return -1;
  if (T < 1 || E < 1 || k < 1 || k > E) return -2;
  int kp = k + (add_shared ? 1 : 0);
  float *ex = malloc(sizeof(float) * (size_t)k);
  for (int t = 0; t < T; t++) {
    const float *l = logits + (size_t)t * E;
    int32_t *id = ids + (size_t)t * kp;
    float *wt = w + (size_t)t * kp;
    select_topk(l, E, k, id);
    float m = l[id[0]], sum = 0.0f;
    for (int j = 0; j < k; j++) {
      ex[j] = expf(l[id[j]] - m);
      sum = sum + ex[j];
    }
    for (int j = 0; j < k; j++) wt[j] = ex[j] / sum;
    if (add_shared) {
      id[k] = E;
      wt[k] = 1.0f;
    }
  }
  free(ex);
  return 0;
}

int orc_route_f64(const float *logits, int T, int E, int k, int add_shared, int32_t *ids, double *w) {
  if (!logits || !ids || !w) return -1;
  if (T < 1 || E < 1 || k < 1 || k > E) return -2;
  int kp = k + (add_shared ? 1 : 0);
  double *ex = malloc(sizeof(double) * (size_t)k);
  for (int t = 0; t < T; t++) {
    const float *l = logits + (size_t)t * E;
    int32_t *id = ids + (size_t)t * kp;
    double *wt = w + (size_t)t * kp;
    select_topk(l, E, k, id);
    double m = l[id[0]], sum = 0.0;
    for (int j = 0; j < k; j++) {
      ex[j] = exp((double)l[id[j]] - m);
      sum += ex[j];
    }
    for (int j = 0; j < k; j++) wt[j] = ex[j] / sum;
    if (add_shared) {
      id[k] = E;
      wt[k] = 1.0;
    }
  }
  free(ex);
  return 0;
}

/* ------------------------------------------------------------------ grouping
 * "Red Metal dev8", step 3: every selected expert is made resident for one pass.  The
 * (token, slot) pairs are grouped per expert: counts, exclusive offsets, the slot list
 * ordered by (expert id, slot index), and its inverse. */

int orc_group(const int32_t *ids, int T, int kp, int n_ids, int32_t *counts, int32_t *offsets,
              int32_t *sorted_slot, int32_t *slot_pos) {
  int n = T * kp;
  for (int s = 0; s < n; s++)
    if (ids[s] < 0 || ids[s] >= n_ids) return -2;
  for (int e = 0; e < n_ids; e++) counts[e] = 0;
  for (int s = 0; s < n; s++) counts[ids[s]]++;
  offsets[0] = 0;
  for (int e = 0; e < n_ids; e++) offsets[e + 1] = offsets[e] + counts[e];
  int pos = 0;
  for (int e = 0; e < n_ids; e++)
    for (int s = 0; s < n; s++)
      if (ids[s] == e) sorted_slot[pos++] = s;
  for (int p = 0; p < n; p++) slot_pos[sorted_slot[p]] = p;
  return 0;
}

/* ------------------------------------------------------------------ accumulation
 * "Red Metal dev8", step 5: accumulator += router_weight * expert_output.  The experts
 * of a token are taken in ascending expert id (the shared expert, id E, comes last);
 * each step is one fp32 multiply and one fp32 add. */

static void ascending_order(const int32_t *id, int kp, int *order) {
  for (int j = 0; j < kp; j++) order[j] = j;
  for (int a = 0; a < kp; a++)
    for (int b = a + 1; b < kp; b++)
      if (id[order[b]] < id[order[a]]) {
        int tmp = order[a];
        order[a] = order[b];
        order[b] = tmp;
      }
}

int orc_accumulate(const float *y, const float *w, const int32_t *ids, int T, int kp, int H, float *acc) {
  int *order = malloc(sizeof(int) * (size_t)kp);
  for (int t = 0; t < T; t++) {
    ascending_order(ids + (size_t)t * kp, kp, order);
    for (int q = 0; q < kp; q++) {
      int s = t * kp + order[q];
      for (int c = 0; c < H; c++) {
        float prod = w[s] * y[(size_t)s * H + c];
        acc[(size_t)t * H + c] = acc[(size_t)t * H + c] + prod;
      }
    }
  }
  free(order);
  return 0;
}

int orc_accumulate_f64(const double *y, const double *w, const int32_t *ids, int T, int kp, int H, double *acc) {
  int *order = malloc(sizeof(int) * (size_t)kp);
  for (int t = 0; t < T; t++) {
    ascending_order(ids + (size_t)t * kp, kp, order);
    for (int q = 0; q < kp; q++) {
      int s = t * kp + order[q];
      for (int c = 0; c < H; c++) acc[(size_t)t * H + c] += w[s] * y[(size_t)s * H + c];
    }
  }
  free(order);
  return 0;
}

/* ------------------------------------------------------------------ layer */

/* Explicit selection: k distinct ids in [0, E) per token, then the shared slot. */
static int selection(const int32_t *ids_in, int T, int E, int k, int add_shared, int32_t *ids) {
  int kp = k + (add_shared ? 1 : 0);
  for (int t = 0; t < T; t++) {
    for (int j = 0; j < k; j++) {
      int32_t e = ids_in[(size_t)t * k + j];
      if (e < 0 || e >= E) return -2;
      for (int q = 0; q < j; q++)
        if (ids_in[(size_t)t * k + q] == e) return -2;
      ids[(size_t)t * kp + j] = e;
    }
    if (add_shared) ids[(size_t)t * kp + k] = E;
  }
  return 0;
}

int orc_moe_layer(const orc_expert *experts, const orc_grids *g, const float *x, const float *logits,
                  const int32_t *ids_in, const float *w_in, int T, int E, int k, int add_shared, int H,
                  float *acc, int32_t *ids_out, float *w_out, float *y_out, int n_threads) {
  if (!experts || !g || !x || !acc || (!logits && (!ids_in || !w_in))) return -1;
  if (T < 1 || E < 1 || k < 1 || k > E || H < 1) return -2;
  int kp = k + (add_shared ? 1 : 0), rc = 0;
  size_t n = (size_t)T * kp;
  int32_t *ids = malloc(sizeof(int32_t) * n);
  float *w = malloc(sizeof(float) * n);
  float *y = malloc(sizeof(float) * n * H);
  if (logits) {
    rc = orc_route(logits, T, E, k, add_shared, ids, w);
  } else {
    rc = selection(ids_in, T, E, k, add_shared, ids);
    for (int t = 0; t < T && !rc; t++) {
      for (int j = 0; j < k; j++) w[(size_t)t * kp + j] = w_in[(size_t)t * k + j];
      if (add_shared) w[(size_t)t * kp + k] = 1.0f;
    }
  }
  int saved = g_threads;
  g_threads = n_threads > 1 ? n_threads : 1;
  for (size_t s = 0; s < n && !rc; s++) {
    const float *xt = x + (s / kp) * H;
    rc = orc_expert_ffn(&experts[ids[s]], g, xt, y + s * H, NULL);
  }
  g_threads = saved;
  if (!rc) rc = orc_accumulate(y, w, ids, T, kp, H, acc);
  if (!rc && ids_out) memcpy(ids_out, ids, sizeof(int32_t) * n);
  if (!rc && w_out) memcpy(w_out, w, sizeof(float) * n);
  if (!rc && y_out) memcpy(y_out, y, sizeof(float) * n * H);
  free(ids);
  free(w);
  free(y);
  return rc;
}

int orc_moe_layer_f64(const orc_expert *experts, const orc_grids *g, const double *x, const float *logits,
                      const int32_t *ids_in, const double *w_in, int T, int E, int k, int add_shared, int H,
                      double *acc, double *y_out) {
  if (!experts || !g || !x || !acc || (!logits && (!ids_in || !w_in))) return -1;
  if (T < 1 || E < 1 || k < 1 || k > E || H < 1) return -2;
  int kp = k + (add_shared ? 1 : 0), rc = 0;
  size_t n = (size_t)T * kp;
  int32_t *ids = malloc(sizeof(int32_t) * n);
  double *w = malloc(sizeof(double) * n);
  double *y = malloc(sizeof(double) * n * H);
  if (logits) {
    rc = orc_route_f64(logits, T, E, k, add_shared, ids, w);
  } else {
    rc = selection(ids_in, T, E, k, add_shared, ids);
    for (int t = 0; t < T && !rc; t++) {
      for (int j = 0; j < k; j++) w[(size_t)t * kp + j] = w_in[(size_t)t * k + j];
      if (add_shared) w[(size_t)t * kp + k] = 1.0;
    }
  }
  for (size_t s = 0; s < n && !rc; s++) rc = orc_expert_ffn_f64(&experts[ids[s]], g, x + (s / kp) * H, y + s * H, NULL);
  if (!rc) rc = orc_accumulate_f64(y, w, ids, T, kp, H, acc);
  if (!rc && y_out) memcpy(y_out, y, sizeof(double) * n * H);
  free(ids);
  free(w);
  free(y);
  return rc;
}

/* ------------------------------------------------------------------ RMSNorm
 * "Red Lite dev16 — complete full-attention parity": the routed MoE of a block reads
 * the post-attention RMSNorm of the hidden state and its output is added back as a
 * residual.  Unit weight: x = h * (1 / sqrt(sum(h^2) / H + eps)). */

int orc_rmsnorm(const float *h, int T, int H, float eps, float *x) {
  if (!h || !x) return -1;
  for (int t = 0; t < T; t++) {
    const float *ht = h + (size_t)t * H;
    float ss = 0.0f;
    for (int c = 0; c < H; c++) {
      float sq = ht[c] * ht[c];
      ss = ss + sq;
    }
    float r = 1.0f / sqrtf(ss / (float)H + eps);
    for (int c = 0; c < H; c++) x[(size_t)t * H + c] = ht[c] * r;
  }
  return 0;
}

int orc_rmsnorm_f64(const double *h, int T, int H, double eps, double *x) {
  if (!h || !x) return -1;
  for (int t = 0; t < T; t++) {
    const double *ht = h + (size_t)t * H;
    double ss = 0.0;
    for (int c = 0; c < H; c++) ss += ht[c] * ht[c];
    double r = 1.0 / sqrt(ss / (double)H + eps);
    for (int c = 0; c < H; c++) x[(size_t)t * H + c] = ht[c] * r;
  }
  return 0;
}

/* ------------------------------------------------------------------ router projection
 * "Red Lite dev9 — native runtime foundation", closing paragraph, and "Red Lite dev10 —
 * standalone native Metal path", section "What dev10 does not yet claim": the router
 * network that feeds the top-k path is the pages' next step.  Read here as one linear
 * map, logits[t][e] = sum_c x[t][c] * wr[e][c] (wr row-major [E][H]), plus, optionally,
 * a gate on the shared expert: s[t] = 1 / (1 + exp(-sum_c x[t][c] * wsg[c])), used as
 * the shared expert's weight in place of 1.0 (the pages say nothing on such a gate).
 * fp32 sums in column order, a separate multiply and add per term. */

static float dot_f32(const float *a, const float *b, int n) {
  float s = 0.0f;
  for (int c = 0; c < n; c++) {
    float p = a[c] * b[c];
    s = s + p;
  }
  return s;
}

static double dot_f64(const float *a, const float *b, int n) {
  double s = 0.0;
  for (int c = 0; c < n; c++) s += (double)a[c] * (double)b[c];
  return s;
}

int orc_router(const float *x, const float *wr, const float *wsg, int T, int H, int E, float *logits, float *sw) {
  if (!x || !wr || !logits || T < 1 || H < 1 || E < 1 || (wsg && !sw)) return -1;
  for (int t = 0; t < T; t++) {
    const float *xt = x + (size_t)t * H;
    for (int e = 0; e < E; e++) logits[(size_t)t * E + e] = dot_f32(xt, wr + (size_t)e * H, H);
    if (wsg) sw[t] = 1.0f / (1.0f + expf(-dot_f32(xt, wsg, H)));
  }
  return 0;
}

int orc_router_f64(const float *x, const float *wr, const float *wsg, int T, int H, int E, double *logits,
                   double *sw) {
  if (!x || !wr || !logits || T < 1 || H < 1 || E < 1 || (wsg && !sw)) return -1;
  for (int t = 0; t < T; t++) {
    const float *xt = x + (size_t)t * H;
    for (int e = 0; e < E; e++) logits[(size_t)t * E + e] = dot_f64(xt, wr + (size_t)e * H, H);
    if (wsg) sw[t] = 1.0 / (1.0 + exp(-dot_f64(xt, wsg, H)));
  }
  return 0;
}

/* Sum of |x[t][c] * w[c]| over c: the scale of a dot product's rounding error. */
int orc_dot_abs(const float *x, const float *w, int T, int H, int E, double *out) {
  if (!x || !w || !out || T < 1 || H < 1 || E < 1) return -1;
  for (int t = 0; t < T; t++)
    for (int e = 0; e < E; e++) {
      double s = 0.0;
      for (int c = 0; c < H; c++) s += fabs((double)x[(size_t)t * H + c] * (double)w[(size_t)e * H + c]);
      out[(size_t)t * E + e] = s;
    }
  return 0;
}
