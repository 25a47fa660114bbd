/*
 * prox_oracle.c -- plain, slow, obviously-correct CPU oracle for the Prox
 * two-stage sparse SwiGLU FFN decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header, table or helper with
 * the HIP library: both sides only see the same seeded inputs.
 *
 * Source of truth: "Prox: Training-Free FFN Activation Sparsity via
 * Approximate Intermediate-Channel Salience in LLMs" (arXiv 2607.27591).
 * Every function below cites the section/equation of that paper it follows.
 *
 * Conventions (the paper's x.W layout, Sec. 2.1):
 *   W_up, W_gate : [d_model][d_ff]   (row i = input channel i)
 *   W_down       : [d_ff][d_model]   (row j = intermediate channel j)
 *   x            : [d_model]
 * Weights and activations arrive as float32 values (bf16 inputs are widened
 * exactly by the caller).  All accumulation is in double.  The quantizer is
 * the one exception: it is specified in float32 so that its integer codes are
 * fixed bit for bit (scale = absmax / 7 in IEEE float32, q = round-half-even
 * of w / scale in float32).
 *
 * Readings where the paper is silent (also listed in the design notes):
 *   - INT4 proxy: symmetric, codes in [-7, 7], scale = absmax / 7 per group of
 *     G consecutive input rows and per output column (Sec. 4.3 says
 *     "symmetric per-row INT4"; the group granularity is the workload's).
 *   - Stage 2 mask: per-token top-k of |s~| (App. A.6, top-k equation) with
 *     ties broken towards the lower channel index.
 *   - SiLU(z) = z / (1 + exp(-z)).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* SiLU, the gate nonlinearity of SwiGLU (Sec. 2.1, FFN equation).           */
static double silu(double z) { return z / (1.0 + exp(-z)); }

/* Gate activation of the gated FFN: act 0 is SiLU (SwiGLU, the pages' FFN);
 * act 1 is GELU in its tanh form, 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715
 * z^3))) (GeGLU, as in Gemma-3 style models).                                */
double prox_oracle_gate_act(double z, int act) {
  if (act == 1) {
    const double c = sqrt(2.0 / 3.14159265358979323846);
    return 0.5 * z * (1.0 + tanh(c * (z + 0.044715 * z * z * z)));
  }
  return silu(z);
}

/* ------------------------------------------------------------------------ */
/* Symmetric INT4 proxy quantization of one weight matrix (Sec. 4.3).
 *
 * W      : [d_model][d_ff] float32, paper layout.
 * q      : [d_model][d_ff] int8 codes in [-7, 7]            (output)
 * scale  : [d_model / G][d_ff] float32 scales               (output)
 *
 * For every group g of G consecutive input rows and every column j:
 *   a = max_{i in g} |W[i][j]|, scale = a / 7 (float32),
 *   q = clamp(rint(W / scale), -7, 7) (float32 divide, ties to even),
 *   a == 0  ->  scale = 0 and q = 0.
 * Returns 0, or -1 when d_model is not a multiple of G.                     */
int prox_oracle_quantize(const float *W, int d_model, int d_ff, int G,
                         int8_t *q, float *scale) {
  if (G <= 0 || d_model % G != 0) return -1;
  int ngroups = d_model / G;
  for (int g = 0; g < ngroups; ++g) {
    for (int j = 0; j < d_ff; ++j) {
      float a = 0.0f;
      for (int i = g * G; i < (g + 1) * G; ++i) {
        float w = fabsf(W[(size_t)i * d_ff + j]);
        if (w > a) a = w;
      }
      float sc = a / 7.0f;
      scale[(size_t)g * d_ff + j] = sc;
      for (int i = g * G; i < (g + 1) * G; ++i) {
        int8_t code = 0;
        if (a > 0.0f) {
          float r = rintf(W[(size_t)i * d_ff + j] / sc);
          if (r > 7.0f) r = 7.0f;
          if (r < -7.0f) r = -7.0f;
          code = (int8_t)r;
        }
        q[(size_t)i * d_ff + j] = code;
      }
    }
  }
  return 0;
}

/* Dequantized proxy weights W~[i][j] = q[i][j] * scale[i / G][j], in double
 * (the product of a small integer and a float32 is exact in double).        */
void prox_oracle_dequantize(const int8_t *q, const float *scale, int d_model,
                            int d_ff, int G, double *Wt) {
  for (int i = 0; i < d_model; ++i)
    for (int j = 0; j < d_ff; ++j)
      Wt[(size_t)i * d_ff + j] =
          (double)q[(size_t)i * d_ff + j] * (double)scale[(size_t)(i / G) * d_ff + j];
}

/* ------------------------------------------------------------------------ */
/* Stage 1 input mask (Sec. 4.1, m_x equation): input channel i survives iff
 * |x_i| >= tau (the paper's ">=").  The comparison is made in float32 on the
 * exact input values.  Writes the survivors in ascending order to idx and
 * returns their count n1.                                                   */
int prox_oracle_input_mask(const float *x, int d_model, float tau, int *idx) {
  int n1 = 0;
  for (int i = 0; i < d_model; ++i)
    if (fabsf(x[i]) >= tau) idx[n1++] = i;
  return n1;
}

/* ------------------------------------------------------------------------ */
/* Stage 1 proxy intermediate state (Sec. 4.1, u~/h~ equations):
 *   u~ = Pi_in(x, W~up, m_x),  h~ = SiLU(Pi_in(x, W~gate, m_x)),  s~ = u~ . h~
 * where Pi_in(x, W, m) = x[I(m)] W[I(m), :] (Sec. 2.2, input sparsity).
 * Wt_up / Wt_gate are the proxy weights in double, [d_model][d_ff]; passing
 * the original weights instead gives the full-precision proxy.
 * Outputs u_t, g_t (pre-activation gate) and s_t, each [d_ff].             */
void prox_oracle_proxy(const float *x, const int *idx, int n1,
                       const double *Wt_up, const double *Wt_gate, int d_ff,
                       double *u_t, double *g_t, double *s_t, int act) {
  for (int j = 0; j < d_ff; ++j) { u_t[j] = 0.0; g_t[j] = 0.0; }
  for (int n = 0; n < n1; ++n) {
    int i = idx[n];
    double xi = (double)x[i];
    const double *ru = Wt_up + (size_t)i * d_ff;
    const double *rg = Wt_gate + (size_t)i * d_ff;
    for (int j = 0; j < d_ff; ++j) {
      u_t[j] += xi * ru[j];
      g_t[j] += xi * rg[j];
    }
  }
  for (int j = 0; j < d_ff; ++j) s_t[j] = u_t[j] * prox_oracle_gate_act(g_t[j], act);
}

/* ------------------------------------------------------------------------ */
/* Per-token top-k mask (App. A.6, top-k equation): keep the k channels with
 * the largest |z_j|; among equal magnitudes the lower index wins.  The
 * ordering key is (-|z_j|, j), a total order, so the selection is unique.
 * sel receives the k chosen indices in ascending order.                     */
static const double *g_sort_keys;
static int cmp_rank(const void *a, const void *b) {
  int i = *(const int *)a, j = *(const int *)b;
  double zi = fabs(g_sort_keys[i]), zj = fabs(g_sort_keys[j]);
  if (zi > zj) return -1;
  if (zi < zj) return 1;
  return (i < j) ? -1 : (i > j);
}
static int cmp_int(const void *a, const void *b) {
  int i = *(const int *)a, j = *(const int *)b;
  return (i < j) ? -1 : (i > j);
}
int prox_oracle_topk(const double *z, int n, int k, int *sel) {
  if (k < 0 || k > n) return -1;
  int *order = (int *)malloc(sizeof(int) * (size_t)(n > 0 ? n : 1));
  if (!order) return -2;
  for (int j = 0; j < n; ++j) order[j] = j;
  g_sort_keys = z;
  qsort(order, (size_t)n, sizeof(int), cmp_rank);
  memcpy(sel, order, sizeof(int) * (size_t)k);
  qsort(sel, (size_t)k, sizeof(int), cmp_int);
  free(order);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Stage 2 threshold mask (Sec. 4.1, m_s equation): with a calibrated
 * threshold tau_s the mask keeps channel j iff |s~_j| >= tau_s.  The GPU
 * holds |s~| in float32, so the comparison is taken in float32 here too: the
 * double |s~_j| is rounded to float32 first.  Writes the kept channels in
 * ascending order to sel and returns their count.                          */
int prox_oracle_threshold_mask(const double *z, int n, float tau, int *sel) {
  int m = 0;
  for (int j = 0; j < n; ++j)
    if ((float)fabs(z[j]) >= tau) sel[m++] = j;
  return m;
}

/* ------------------------------------------------------------------------ */
/* Stage 2 exact sparse computation (Sec. 4.1, Stage 2 equations):
 *   u_sp = Pi_out(x, W_up, m_s),  h_sp = SiLU(Pi_out(x, W_gate, m_s)),
 *   s_sp = u_sp . h_sp,           y = Pi_in(s_sp, W_down, m_s)
 * with Pi_out(x, W, m) = x W[:, I(m)] (Sec. 2.2, output sparsity).  The full,
 * unthresholded x is used.  sel holds the k selected channels; s_sp[t] is the
 * exact state of channel sel[t]; y is [d_model].                            */
void prox_oracle_stage2(const float *x, int d_model, int d_ff,
                        const float *W_up, const float *W_gate,
                        const float *W_down, const int *sel, int k,
                        double *s_sp, double *y, int act) {
  double *u = (double *)calloc((size_t)(k > 0 ? k : 1), sizeof(double));
  double *g = (double *)calloc((size_t)(k > 0 ? k : 1), sizeof(double));
  for (int i = 0; i < d_model; ++i) {
    double xi = (double)x[i];
    const float *ru = W_up + (size_t)i * d_ff;
    const float *rg = W_gate + (size_t)i * d_ff;
    for (int t = 0; t < k; ++t) {
      u[t] += xi * (double)ru[sel[t]];
      g[t] += xi * (double)rg[sel[t]];
    }
  }
  for (int t = 0; t < k; ++t) s_sp[t] = u[t] * prox_oracle_gate_act(g[t], act);
  for (int c = 0; c < d_model; ++c) y[c] = 0.0;
  for (int t = 0; t < k; ++t) {
    const float *rd = W_down + (size_t)sel[t] * d_model;
    for (int c = 0; c < d_model; ++c) y[c] += s_sp[t] * (double)rd[c];
  }
  free(u);
  free(g);
}

/* ------------------------------------------------------------------------ */
/* Dense SwiGLU FFN (Sec. 2.1): u = x W_up, h = SiLU(x W_gate), s = u . h,
 * y = s W_down.  s (all d_ff channels) is returned too when s_out != NULL;
 * it is the exact intermediate state the oracle-s diagnostic ranks (Sec. 3.1). */
void prox_oracle_dense(const float *x, int d_model, int d_ff,
                       const float *W_up, const float *W_gate,
                       const float *W_down, double *s_out, double *y, int act) {
  double *u = (double *)calloc((size_t)d_ff, sizeof(double));
  double *g = (double *)calloc((size_t)d_ff, sizeof(double));
  double *s = (double *)calloc((size_t)d_ff, sizeof(double));
  for (int i = 0; i < d_model; ++i) {
    double xi = (double)x[i];
    const float *ru = W_up + (size_t)i * d_ff;
    const float *rg = W_gate + (size_t)i * d_ff;
    for (int j = 0; j < d_ff; ++j) {
      u[j] += xi * (double)ru[j];
      g[j] += xi * (double)rg[j];
    }
  }
  for (int j = 0; j < d_ff; ++j) s[j] = u[j] * prox_oracle_gate_act(g[j], act);
  for (int c = 0; c < d_model; ++c) y[c] = 0.0;
  for (int j = 0; j < d_ff; ++j) {
    const float *rd = W_down + (size_t)j * d_model;
    for (int c = 0; c < d_model; ++c) y[c] += s[j] * (double)rd[c];
  }
  if (s_out) memcpy(s_out, s, sizeof(double) * (size_t)d_ff);
  free(u);
  free(g);
  free(s);
}

/* ------------------------------------------------------------------------ */
/* Round a float32 to the nearest bfloat16 (ties to even), returned widened
 * back to float32.  bfloat16 keeps the top 16 bits of the float32 encoding;
 * NaN stays NaN.                                                             */
float prox_oracle_round_bf16(float v) {
  uint32_t b;
  memcpy(&b, &v, 4);
  if ((b & 0x7f800000u) == 0x7f800000u && (b & 0x007fffffu)) {
    b |= 0x00400000u;
  } else {
    uint32_t low = b & 0xffffu;
    uint32_t keep = b & 0xffff0000u;
    uint32_t lsb = (b >> 16) & 1u;
    if (low > 0x8000u || (low == 0x8000u && lsb)) keep += 0x10000u;
    b = keep;
  }
  b &= 0xffff0000u;
  float r;
  memcpy(&r, &b, 4);
  return r;
}

void prox_oracle_round_bf16_array(float *v, long n) {
  for (long i = 0; i < n; ++i) v[i] = prox_oracle_round_bf16(v[i]);
}

/* RMSNorm of a residual-stream vector with unit gain, then cast to the layer
 * input dtype: x = cast(r / sqrt(mean(r^2) + eps)).  The division happens in
 * double; the result is rounded to float32 and, when to_bf16 != 0, further to
 * bfloat16.                                                                  */
void prox_oracle_rmsnorm(const double *r, int n, double eps, int to_bf16,
                         float *x) {
  double ss = 0.0;
  for (int i = 0; i < n; ++i) ss += r[i] * r[i];
  double inv = 1.0 / sqrt(ss / (double)n + eps);
  for (int i = 0; i < n; ++i) {
    float v = (float)(r[i] * inv);
    x[i] = to_bf16 ? prox_oracle_round_bf16(v) : v;
  }
}
