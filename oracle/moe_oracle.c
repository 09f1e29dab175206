/*
 * CPU oracle for the MoE layer forward -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test-suite, the smoke entry and the benchmark's CPU-baseline leg
 * may load this file's library. The GPU library never links or calls it, and
 * the two share no source. Plain C99, compiled with -ffp-contract=off so the
 * only fused multiply-adds are the explicit fmaf() of the router.
 *
 * Sources, cited by page and section:
 *  [FSM]  "FFN, SwiGLU and MoE" (bjdmk.com): sec. 2 SwiGLU formula and
 *         module; sec. 3 MoE formulas r = W_r x, p = softmax(r), TopK(p),
 *         y = sum over selected i of p_i E_i(x), and the reference module with
 *         top-k renormalisation and its per-expert masked loop.
 *  [OPS]  "ops-transformer MoE operator on Ascend NPU" (gitcode.csdn.net):
 *         MoEForward sketch (router matmul, top-k, softmax over the selected,
 *         per-expert gather / expert forward / scatter, weighted sum);
 *         Optimisation 2 (size-k heap, a new score must be strictly larger to
 *         enter, so an equal later score never displaces an earlier one);
 *         Pitfall 1 (expert capacity S*top_k/num_experts*1.2, overflow tokens
 *         dropped); Pitfall 3 (router computed in FP32).
 *  [DSV]  "DeepSeek-V4.1-Flash fine-grained MoE (5A)" (openarchlab.com):
 *         sec. 1 and 3 (select by scores + bias, weight by the raw
 *         sqrt(softplus(scores)), not normalised; SwiGLU clamped to +-10; one
 *         always-on shared expert); sec. 1 worked example; sec. 4 stable
 *         softplus for large inputs.
 *  [RTG]  "MoE routing: Top-K, Expert-Choice and Sigmoid Gating"
 *         (blogdee.com): sigmoid gating as the mixing-weight function.
 *  [ECHO] "moe f&b compute flow" (Echo's blog): the Router -> Dispatch ->
 *         FFN -> Combine stages; softmax makes weights positive, summing to 1.
 *  [OCP]  OCP Microscaling Formats (MX) v1.0: e2m1 and e4m3 element values,
 *         the e8m0 scale 2^(s-127) and the block conversion (shared
 *         exponent from the block maximum); the pages only say the experts
 *         are FP4, and the MXFP8 activation mode (OR_MXFP4_A8) is an
 *         addition that lets the products run on the scaled MFMA.
 *
 * Readings where the pages leave a step open (each is listed with its reason
 * in the design notes):
 *  - the router dot product is one fp32 fused multiply-add chain over d in
 *    ascending order (FP32 routing [OPS Pitfall 3], order fixed here);
 *  - selection key = logit + bias (one fp32 add); top-k descending by key,
 *    ties to the lower expert index [OPS Optimisation 2];
 *  - in softmax mode the bias is a logit bias (it enters the softmax); in
 *    sigmoid and sqrt-softplus modes it only steers selection [DSV sec. 3];
 *  - tokens over capacity are dropped in token order, and a dropped pair
 *    contributes zero;
 *  - H (the SwiGLU output) is stored rounded to the activation dtype (bf16),
 *    y is rounded once at the end.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* Number formats                                                      */
/* ------------------------------------------------------------------ */

/* bf16 is the upper half of an IEEE binary32 pattern. */
double oracle_bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Round a double to the nearest bf16 value, ties to even, in one step.
 * bf16 keeps 8 significant bits and binary32's exponent range: normal
 * values have quantum 2^(e-8) where v = m*2^e, 0.5 <= |m| < 1; values
 * below 2^-126 share the subnormal quantum 2^-133. */
uint16_t oracle_double_to_bf16(double v) {
  if (isnan(v)) return 0x7FC0;
  double a = fabs(v);
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  if (isinf(v)) return sign | 0x7F80;
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);                 /* a = m * 2^e, 0.5 <= m < 1 */
  int qexp = e - 8;
  if (qexp < -133) qexp = -133;
  double n = nearbyint(ldexp(a, -qexp)); /* default mode: nearest, ties even */
  double r = ldexp(n, qexp);
  if (r >= ldexp(1.0, 128)) return sign | 0x7F80;
  float f = (float)r;           /* exact: r has <= 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, 4);
  return sign | (uint16_t)((u >> 16) & 0x7FFF);
}

/* oracle_double_to_bf16 over an array (for exhaustive tests). */
void oracle_double_to_bf16_array(const double* v, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_double_to_bf16(v[i]);
}

/* e2m1: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa [OCP]. */
double oracle_e2m1(unsigned code) {
  static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  double v = mag[code & 7u];
  return (code & 8u) ? -v : v;
}

/* e8m0: 2^(s-127); 255 is NaN [OCP]. */
double oracle_e8m0(unsigned s) {
  if (s == 255u) return NAN;
  return ldexp(1.0, (int)s - 127);
}

/* e4m3 (the MX FP8 E4M3 element): bit 7 sign, bits 6..3 exponent (bias 7),
 * bits 2..0 mantissa; exponent field 0 holds the subnormals m/8 * 2^-6;
 * S.1111.111 is NaN and there is no infinity, so the largest finite
 * magnitude is 1.75 * 2^8 = 448 [OCP]. */
double oracle_e4m3(unsigned code) {
  unsigned e = (code >> 3) & 15u, m = code & 7u;
  if (e == 15u && m == 7u) return NAN;
  double v = e == 0u ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, (int)e - 7);
  return (code & 0x80u) ? -v : v;
}

/* The e4m3 code nearest to v (finite), ties to the code whose last bit is
 * 0, magnitudes beyond 448 saturated to 448. Written as a search over the
 * 127 non-negative finite codes, which are increasing in value. */
unsigned oracle_e4m3_encode(double v) {
  const double a = fabs(v);
  unsigned best = 0;
  double best_d = a;
  for (unsigned c = 1; c < 127u; ++c) {
    const double d = fabs(oracle_e4m3(c) - a);
    if (d < best_d || (d == best_d && (c & 1u) == 0u)) {
      best = c;
      best_d = d;
    }
  }
  return (signbit(v) ? 0x80u : 0u) | best;
}

/* MXFP8 quantisation of n values (n a multiple of 32), block by block of 32
 * consecutive values [OCP, the MX conversion]: the block's shared exponent
 * is floor(log2(max |V_i|)) minus 8 (the exponent of e4m3's largest
 * normal), held in e8m0, so clamped to [-127, 127] (a block of zeros gets
 * -127, scale code 0); X = 2^exponent; element i is the e4m3 code of
 * V_i / X, rounded as oracle_e4m3_encode does. */
void oracle_mxfp8_quantize(const double* v, int n, uint8_t* codes, uint8_t* scales) {
  for (int b = 0; b < n / 32; ++b) {
    double amax = 0.0;
    for (int i = 0; i < 32; ++i) amax = fmax(amax, fabs(v[32 * b + i]));
    int ex = -127;
    if (amax > 0.0) {
      int e2;
      frexp(amax, &e2);  /* amax = m 2^e2, 0.5 <= m < 1: floor(log2 amax) = e2 - 1 */
      ex = e2 - 1 - 8;
      if (ex < -127) ex = -127;
      if (ex > 127) ex = 127;
    }
    scales[b] = (uint8_t)(ex + 127);
    for (int i = 0; i < 32; ++i)
      codes[32 * b + i] = (uint8_t)oracle_e4m3_encode(ldexp(v[32 * b + i], -ex));
  }
}

/* v <- the values its MXFP8 quantisation represents. */
static void mxfp8_round_trip(double* v, int n) {
  uint8_t* codes = (uint8_t*)malloc((size_t)n);
  uint8_t* scales = (uint8_t*)malloc((size_t)n / 32);
  oracle_mxfp8_quantize(v, n, codes, scales);
  for (int i = 0; i < n; ++i) v[i] = oracle_e4m3(codes[i]) * oracle_e8m0(scales[i / 32]);
  free(codes);
  free(scales);
}

/* softplus(s) = log(1 + e^s), written in the form that cannot overflow:
 * max(s,0) + log1p(e^-|s|). For large s it returns s [DSV sec. 4]. */
double oracle_softplus(double s) {
  return fmax(s, 0.0) + log1p(exp(-fabs(s)));
}

/* SiLU(z) = z * sigmoid(z) [FSM sec. 2]. */
double oracle_silu(double z) { return z / (1.0 + exp(-z)); }

/* Capacity as the page writes it in C: integer S*top_k/num_experts, times
 * 1.2, truncated by the assignment to an int [OPS Pitfall 1]. */
int oracle_capacity_formula(int S, int top_k, int num_experts) {
  int base = S * top_k / num_experts;
  double c = base * 1.2;
  return (int)c;
}

static float act_f32(const oracle_cfg* c, const void* x, size_t i) {
  if (c->act == OR_F32) return ((const float*)x)[i];
  return (float)oracle_bf16_to_double(((const uint16_t*)x)[i]);
}

static double wt(const oracle_cfg* c, const void* W, const uint8_t* S, int e,
                 int K, int N, int kk, int n) {
  /* Logical weight element W[e][kk][n] of a [E][K][N] matrix. MXFP4 storage
   * is by 32-element K-blocks, block-major: codes [E][K/32][N][16] (byte i
   * of a block holds elements 2i, low nibble, and 2i+1), scales
   * [E][K/32][N]. */
  if (c->wdt == OR_F32) return ((const float*)W)[((size_t)e * K + kk) * N + n];
  if (c->wdt == OR_BF16)
    return oracle_bf16_to_double(((const uint16_t*)W)[((size_t)e * K + kk) * N + n]);
  const uint8_t* codes = (const uint8_t*)W;
  const size_t blk = ((size_t)e * (K / 32) + kk / 32) * N + n;
  uint8_t byte = codes[blk * 16 + (kk % 32) / 2];
  unsigned code = (kk & 1) ? (byte >> 4) : (byte & 15u);
  unsigned s = S[blk];
  return oracle_e2m1(code) * oracle_e8m0(s);
}

/* ------------------------------------------------------------------ */
/* Router                                                              */
/* ------------------------------------------------------------------ */

/* logits[t][e] = sum_d x[t][d] * W_r[d][e] with fp32 accumulation
 * [FSM sec. 3, OPS MoEForward step 1, OPS Pitfall 3]: one fused
 * multiply-add per term, d ascending, starting from +0. */
void oracle_router_logits(const oracle_cfg* c, const void* x, const float* W_r, float* logits) {
  const int T = c->T, D = c->D, E = c->E;
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    float* acc = logits + (size_t)t * E;
    for (int e = 0; e < E; ++e) acc[e] = 0.0f;
    for (int d = 0; d < D; ++d) {
      float xv = act_f32(c, x, (size_t)t * D + d);
      const float* wrow = W_r + (size_t)d * E;
      for (int e = 0; e < E; ++e) acc[e] = fmaf(xv, wrow[e], acc[e]);
    }
  }
}

static float key_of(const float* logits, const float* bias, int E, int t, int e) {
  float b = bias ? bias[e] : 0.0f;
  return logits[(size_t)t * E + e] + b;
}

/* Top-k by key = logit + bias: k rounds, each taking the largest remaining
 * key, an equal key going to the lower expert index [OPS Optimisation 2,
 * FSM sec. 3]. Slot 0 holds the largest. */
void oracle_select_topk(const oracle_cfg* c, const float* logits, const float* bias,
                        int32_t* topk_idx) {
  const int T = c->T, E = c->E, k = c->k;
  char* taken = (char*)malloc((size_t)E);
  for (int t = 0; t < T; ++t) {
    memset(taken, 0, (size_t)E);
    for (int j = 0; j < k; ++j) {
      int best = -1;
      float bk = 0.0f;
      for (int e = 0; e < E; ++e) {
        if (taken[e]) continue;
        float ke = key_of(logits, bias, E, t, e);
        if (best < 0 || ke > bk) { best = e; bk = ke; }
      }
      taken[best] = 1;
      topk_idx[(size_t)t * k + j] = best;
    }
  }
  free(taken);
}

/* Combine weights for the selected experts:
 *  softmax: p = softmax over all E of (logit + bias) [FSM sec. 3, ECHO],
 *           w_j = p of the j-th selected expert; with renorm, divided by
 *           the sum over the k selected [FSM sec. 3 module];
 *  sigmoid: w_j = 1/(1+e^-logit) of the selected expert [RTG];
 *  sqrt-softplus: w_j = sqrt(softplus(logit)), the raw score without the
 *           selection bias, not normalised [DSV sec. 1, 3].
 * Computed in double from the fp32 logits, stored as float. */
void oracle_gate_weights(const oracle_cfg* c, const float* logits, const float* bias,
                         const int32_t* topk_idx, float* topk_w) {
  const int T = c->T, E = c->E, k = c->k;
  double* w = (double*)malloc(sizeof(double) * (size_t)k);
  for (int t = 0; t < T; ++t) {
    const int32_t* idx = topk_idx + (size_t)t * k;
    if (c->gating == OR_SOFTMAX) {
      double m = -INFINITY;
      for (int e = 0; e < E; ++e) m = fmax(m, (double)key_of(logits, bias, E, t, e));
      double z = 0.0;
      for (int e = 0; e < E; ++e) z += exp((double)key_of(logits, bias, E, t, e) - m);
      for (int j = 0; j < k; ++j) w[j] = exp((double)key_of(logits, bias, E, t, idx[j]) - m) / z;
    } else {
      for (int j = 0; j < k; ++j) {
        double s = (double)logits[(size_t)t * E + idx[j]];
        if (c->gating == OR_SIGMOID) w[j] = 1.0 / (1.0 + exp(-s));
        else w[j] = sqrt(oracle_softplus(s));
      }
    }
    if (c->renorm) {
      double sum = 0.0;
      for (int j = 0; j < k; ++j) sum += w[j];
      for (int j = 0; j < k; ++j) w[j] /= sum;
    }
    for (int j = 0; j < k; ++j) topk_w[(size_t)t * k + j] = (float)w[j];
  }
  free(w);
}

/* ------------------------------------------------------------------ */
/* Dispatch                                                            */
/* ------------------------------------------------------------------ */

/* Group (token, expert) pairs by expert [ECHO Dispatch, OPS MoEForward
 * GetTokensForExpert/Gather]. Walking tokens in order, the rank of (t,e) is
 * the number of earlier tokens routed to e; a pair is kept while its rank is
 * below the capacity [OPS Pitfall 1]. Each expert's kept pairs form one
 * contiguous segment, in token order:
 *   counts[e]      all pairs routed to e (before capacity)
 *   offsets[e]     start of e's segment; offsets[E] = number kept
 *   slot_pos[t][j] row of (t, topk_idx[t][j]) in the segments, -1 if dropped
 *   perm_token[r]  token of row r (rows >= offsets[E] untouched) */
void oracle_dispatch(const oracle_cfg* c, const int32_t* topk_idx, int32_t* counts,
                     int32_t* offsets, int32_t* slot_pos, int32_t* perm_token) {
  const int T = c->T, E = c->E, k = c->k;
  int32_t* seen = (int32_t*)calloc((size_t)E, sizeof(int32_t));
  int32_t* rank = (int32_t*)malloc(sizeof(int32_t) * (size_t)T * k);
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int t = 0; t < T; ++t)
    for (int j = 0; j < k; ++j) {
      int e = topk_idx[(size_t)t * k + j];
      rank[(size_t)t * k + j] = seen[e]++;
      counts[e]++;
    }
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) {
    int kept = counts[e];
    if (c->capacity > 0 && kept > c->capacity) kept = c->capacity;
    offsets[e + 1] = offsets[e] + kept;
  }
  for (int t = 0; t < T; ++t)
    for (int j = 0; j < k; ++j) {
      int e = topk_idx[(size_t)t * k + j];
      int r = rank[(size_t)t * k + j];
      if (c->capacity > 0 && r >= c->capacity) {
        slot_pos[(size_t)t * k + j] = -1;
      } else {
        int pos = offsets[e] + r;
        slot_pos[(size_t)t * k + j] = pos;
        perm_token[pos] = t;
      }
    }
  free(seen);
  free(rank);
}

/* ------------------------------------------------------------------ */
/* Expert FFN                                                          */
/* ------------------------------------------------------------------ */

/* One SwiGLU expert on a few token rows [FSM sec. 2]:
 *   g = x W_gate, u = x W_up (clamped to [-L, L] when L > 0 [DSV sec. 1, 3]),
 *   h = SiLU(g) * u, rounded to bf16 when the activations are bf16,
 *   o = h W_down.
 * With OR_MXFP4_A8 weights, x and h are replaced by their MXFP8 values
 * (oracle_mxfp8_quantize) before the products that read them.
 * h_out [nrows][F] and o_out [nrows][D] may be NULL. */
static void swiglu_rows(const oracle_cfg* c, int F, const void* Wg, const void* Wu, const void* Wd,
                        const uint8_t* Sg, const uint8_t* Su, const uint8_t* Sd,
                        const oracle_cfg* wc, int e, int nrows, const void* x,
                        const int32_t* rows, double* h_out, double* o_out) {
  const int D = c->D;
  /* MXFP4 weights with MXFP8 activation operands: the x row and H enter
   * the products as their MXFP8 values (H quantised from its fp32 value,
   * the precision in which the GPU forms it). */
  const int a8 = wc->wdt == OR_MXFP4_A8;
#pragma omp parallel for schedule(dynamic, 1)
  for (int r = 0; r < nrows; ++r) {
    double* xr = (double*)malloc(sizeof(double) * (size_t)D);
    double* g = (double*)calloc((size_t)F, sizeof(double));
    double* u = (double*)calloc((size_t)F, sizeof(double));
    double* h = (double*)malloc(sizeof(double) * (size_t)F);
    for (int d = 0; d < D; ++d) xr[d] = act_f32(c, x, (size_t)rows[r] * D + d);
    if (a8) mxfp8_round_trip(xr, D);
    for (int d = 0; d < D; ++d) {
      for (int f = 0; f < F; ++f) {
        g[f] += xr[d] * wt(wc, Wg, Sg, e, D, F, d, f);
        u[f] += xr[d] * wt(wc, Wu, Su, e, D, F, d, f);
      }
    }
    for (int f = 0; f < F; ++f) {
      double gf = g[f], uf = u[f];
      if (c->clamp > 0.0f) {
        double L = (double)c->clamp;
        gf = fmin(fmax(gf, -L), L);
        uf = fmin(fmax(uf, -L), L);
      }
      double hv = oracle_silu(gf) * uf;
      if (a8) hv = (double)(float)hv;  /* quantised below from its fp32 value */
      else if (c->act == OR_BF16) hv = oracle_bf16_to_double(oracle_double_to_bf16(hv));
      h[f] = hv;
    }
    if (a8) mxfp8_round_trip(h, F);
    if (h_out)
      for (int f = 0; f < F; ++f) h_out[(size_t)r * F + f] = h[f];
    if (o_out) {
      double* o = o_out + (size_t)r * D;
      for (int cc = 0; cc < D; ++cc) o[cc] = 0.0;
      for (int f = 0; f < F; ++f)
        for (int cc = 0; cc < D; ++cc) o[cc] += h[f] * wt(wc, Wd, Sd, e, F, D, f, cc);
    }
    free(xr); free(g); free(u); free(h);
  }
}

void oracle_expert_rows(const oracle_cfg* c, const oracle_weights* w, int expert, int nrows,
                        const void* x, const int32_t* rows, double* h_out, double* o_out) {
  swiglu_rows(c, c->F, w->W_gate, w->W_up, w->W_down, w->S_gate, w->S_up, w->S_down, c,
              expert, nrows, x, rows, h_out, o_out);
}

/* The always-on shared expert [DSV sec. 1, 3]: a bf16 SwiGLU of width
 * shared_F, clamped like every expert. */
void oracle_shared_rows(const oracle_cfg* c, const oracle_weights* w, int nrows,
                        const void* x, const int32_t* rows, double* o_out) {
  oracle_cfg sc = *c;
  sc.wdt = OR_BF16;
  swiglu_rows(c, c->shared_F, w->Ws_gate, w->Ws_up, w->Ws_down, NULL, NULL, NULL, &sc, 0,
              nrows, x, rows, NULL, o_out);
}

/* ------------------------------------------------------------------ */
/* Combine                                                             */
/* ------------------------------------------------------------------ */

/* y[t] = sum over kept slots j (ascending) of w[t][j] * E_{idx[t][j]}(x[t])
 *        + shared(x[t]) [FSM sec. 3, OPS WeightedSum, ECHO Combine, DSV sec. 3].
 * Computed for the listed tokens only, expert by expert. y_exact (double,
 * [ntok][D]) and y_out (act dtype, [ntok][D]) may each be NULL. */
void oracle_forward_tokens(const oracle_cfg* c, const oracle_weights* w, const void* x,
                           const int32_t* topk_idx, const float* topk_w, const int32_t* slot_pos,
                           int ntok, const int32_t* tokens, double* y_exact, void* y_out) {
  const int D = c->D, k = c->k;
#pragma omp parallel for schedule(dynamic, 1)
  for (int i = 0; i < ntok; ++i) {
    int t = tokens[i];
    double* acc = (double*)calloc((size_t)D, sizeof(double));
    double* o = (double*)malloc(sizeof(double) * (size_t)D);
    for (int j = 0; j < k; ++j) {
      if (slot_pos[(size_t)t * k + j] < 0) continue;
      int e = topk_idx[(size_t)t * k + j];
      oracle_expert_rows(c, w, e, 1, x, &t, NULL, o);
      double wj = (double)topk_w[(size_t)t * k + j];
      for (int d = 0; d < D; ++d) acc[d] += wj * o[d];
    }
    if (c->shared_F > 0) {
      oracle_shared_rows(c, w, 1, x, &t, o);
      for (int d = 0; d < D; ++d) acc[d] += o[d];
    }
    for (int d = 0; d < D; ++d) {
      size_t q = (size_t)i * D + d;
      if (y_exact) y_exact[q] = acc[d];
      if (y_out) {
        if (c->act == OR_F32) ((float*)y_out)[q] = (float)acc[d];
        else ((uint16_t*)y_out)[q] = oracle_double_to_bf16(acc[d]);
      }
    }
    free(acc);
    free(o);
  }
}
