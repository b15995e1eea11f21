/*
 * gdn_oracle.c -- plain fp64 CPU oracle for the Gated DeltaNet (GDN) layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or helper with the HIP implementation, and nothing here is on
 * the product path.
 *
 * What it computes (sources):
 *  - Layer composition and geometry: "Implement the Qwen3.8 Flash Next Rust
 *    and Metal text core" (DS4Server issue #95), section Implementation: GDN
 *    layers with 16 key / 48 value heads, convolution width 4, fp32 recurrent
 *    state, a sigmoid output gate and L2-normalised q/k; the implementation
 *    comment there adds a BF16 width-4 convolution history.
 *  - "Add a performance-parity Qwen3.8-27B Q4 and Q8 text backend on Metal"
 *    (DS4Server issue #88), section Scope: causal depthwise Conv1D, Gated
 *    DeltaNet recurrence and a recurrent-state cache kept apart from the KV
 *    cache.
 *  - The recurrence itself is the gated delta rule of Yang, Kautz and
 *    Hatamizadeh, "Gated Delta Networks: Improving Mamba2 with Delta Rule"
 *    (ICLR 2025):  S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,
 *    o_t = S_t q_t.  The pages name the recurrence but print no formula.
 *
 * Readings taken where the pages are silent (each is listed in the design
 * notes of the repository):
 *  - conv: xi[t,c] = sum_{j=0..W-1} w[c,j] * x[t-(W-1)+j, c]; tap W-1 is the
 *    current token; rows before t=0 come from the conv history, stored oldest
 *    first as [B][W-1][C_ch]; no bias.  SiLU u = xi / (1 + exp(-xi)) on every
 *    channel.
 *  - channel order of the concatenated projections: [q | k | v], head-major,
 *    dimension fastest; value head h reads key head h / (H_v/H_k).
 *  - L2 norm with the epsilon inside the root: x / sqrt(sum x^2 + eps); q is
 *    further multiplied by q_scale.
 *  - decay a = exp(g) with g <= 0 and beta are given per (b, t, value head).
 *  - the readout uses the updated state; y = o * sigmoid(z).
 *
 * Arithmetic: every value is widened to double on load and all arithmetic is
 * double.  None of the pages prints a worked example or a test vector, so
 * no stored value comes from them.  Every function here is pinned instead by
 * the CPU test suite: the conv against numpy.convolve and identity/shift
 * taps, the history roll against the last rows, the norm against
 * numpy.linalg.norm and the epsilon placement, the recurrence against closed
 * forms (beta = 0 with a = 1 keeps the state, one-hot and orthonormal keys
 * overwrite, full decay forgets, the per-step retrieval identity) and dense
 * brute-force products, the layer against its composed stages.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1

/* Widen element i of an fp32 or bf16 array to double (exact). */
static double widen(const void *p, size_t i, int dtype) {
  if (dtype == ORACLE_F32) return (double)((const float *)p)[i];
  uint32_t bits = ((uint32_t)((const uint16_t *)p)[i]) << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static double silu(double xi) { return xi / (1.0 + exp(-xi)); }
static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

/* Input row tau of channel c for sequence b: x for tau >= 0, else the conv
 * history row (W-1)+tau. */
static double conv_input(const void *x, const void *hist, int dtype, int64_t T,
                         int C_ch, int W, int b, int64_t tau, int c) {
  if (tau >= 0) return widen(x, ((size_t)b * T + tau) * C_ch + c, dtype);
  return widen(hist, ((size_t)b * (W - 1) + (W - 1) + tau) * C_ch + c, dtype);
}

/* Causal depthwise convolution of channel c at token t, before SiLU. */
static double conv_at(const void *x, const void *w, const void *hist, int dtype,
                      int64_t T, int C_ch, int W, int b, int64_t t, int c) {
  double acc = 0.0;
  for (int j = 0; j < W; ++j)
    acc += widen(w, (size_t)c * W + j, dtype) *
           conv_input(x, hist, dtype, T, C_ch, W, b, t - (W - 1) + j, c);
  return acc;
}

/* Stage a1: conv + SiLU for every channel.  out: double [B,T,C_ch]. */
int oracle_conv_silu(int B, int64_t T, int C_ch, int W, int dtype,
                     const void *x, const void *w, const void *hist,
                     double *out) {
  if (B < 0 || T < 0 || C_ch <= 0 || W < 1) return -1;
  for (int b = 0; b < B; ++b)
    for (int64_t t = 0; t < T; ++t)
      for (int c = 0; c < C_ch; ++c)
        out[((size_t)b * T + t) * C_ch + c] =
            silu(conv_at(x, w, hist, dtype, T, C_ch, W, b, t, c));
  return 0;
}

/* The conv history after the call: the last W-1 rows of concat(hist, x),
 * copied bit for bit in the input dtype. */
int oracle_conv_history_next(int B, int64_t T, int C_ch, int W, int dtype,
                             const void *x, const void *hist, void *hist_out) {
  if (B < 0 || T < 0 || C_ch <= 0 || W < 1) return -1;
  size_t es = dtype == ORACLE_F32 ? 4 : 2;
  for (int b = 0; b < B; ++b)
    for (int r = 0; r < W - 1; ++r) {
      int64_t tau = T - (W - 1) + r; /* source row in concat coordinates */
      const char *src;
      if (tau >= 0)
        src = (const char *)x + (((size_t)b * T + tau) * C_ch) * es;
      else
        src = (const char *)hist + (((size_t)b * (W - 1) + (W - 1) + tau) * C_ch) * es;
      memcpy((char *)hist_out + (((size_t)b * (W - 1) + r) * C_ch) * es, src,
             (size_t)C_ch * es);
    }
  return 0;
}

/* Stage a2: n vectors of length d, each divided by sqrt(sum x^2 + eps) and
 * multiplied by scale. */
int oracle_l2norm(int64_t n, int d, const double *in, double eps, double scale,
                  double *out) {
  if (n < 0 || d <= 0) return -1;
  for (int64_t i = 0; i < n; ++i) {
    double ss = 0.0;
    for (int j = 0; j < d; ++j) ss += in[i * d + j] * in[i * d + j];
    double inv = 1.0 / sqrt(ss + eps);
    for (int j = 0; j < d; ++j) out[i * d + j] = in[i * d + j] * inv * scale;
  }
  return 0;
}

/* One token of the gated delta rule for one value head, in place on S
 * (d_v x d_k, row-major).  p receives S_{t-1} k (scratch of length d_v).
 *   S <- a S (I - beta k k^T) + beta v k^T
 *      = a S - a beta (S k) k^T + beta v k^T
 * then o = S q with the updated S. */
static void delta_step(int d_v, int d_k, double *S, const double *k,
                       const double *v, const double *q, double a, double beta,
                       double *p, double *o) {
  for (int i = 0; i < d_v; ++i) {
    double s = 0.0;
    for (int j = 0; j < d_k; ++j) s += S[(size_t)i * d_k + j] * k[j];
    p[i] = s;
  }
  for (int i = 0; i < d_v; ++i)
    for (int j = 0; j < d_k; ++j)
      S[(size_t)i * d_k + j] = a * S[(size_t)i * d_k + j] - a * beta * p[i] * k[j] +
                               beta * v[i] * k[j];
  for (int i = 0; i < d_v; ++i) {
    double s = 0.0;
    for (int j = 0; j < d_k; ++j) s += S[(size_t)i * d_k + j] * q[j];
    o[i] = s;
  }
}

/* Stages a3..a7 on already convolved and normalised inputs, token by token.
 *   q, k: [B,T,H_k,d_k]; v, z: [B,T,H_v,d_v]; g, beta: [B,T,H_v]
 *   S: [B,H_v,d_v,d_k] in/out; y: [B,T,H_v,d_v] out; o (may be NULL): the
 *   ungated readout, same shape as y. */
int oracle_recurrence(int B, int64_t T, int H_k, int H_v, int d_k, int d_v,
                      const double *q, const double *k, const double *v,
                      const double *g, const double *beta, const double *z,
                      double *S, double *y, double *o) {
  if (B < 0 || T < 0 || H_k <= 0 || H_v <= 0 || H_v % H_k || d_k <= 0 || d_v <= 0)
    return -1;
  int G = H_v / H_k;
  double *p = (double *)malloc(sizeof(double) * (size_t)d_v);
  double *ot = (double *)malloc(sizeof(double) * (size_t)d_v);
  if (!p || !ot) { free(p); free(ot); return -2; }
  for (int b = 0; b < B; ++b)
    for (int64_t t = 0; t < T; ++t)
      for (int h = 0; h < H_v; ++h) {
        int kh = h / G;
        size_t bt = (size_t)b * T + t;
        const double *qt = q + (bt * H_k + kh) * d_k;
        const double *kt = k + (bt * H_k + kh) * d_k;
        const double *vt = v + (bt * H_v + h) * d_v;
        double a = exp(g[bt * H_v + h]);
        double *Sh = S + ((size_t)b * H_v + h) * d_v * d_k;
        delta_step(d_v, d_k, Sh, kt, vt, qt, a, beta[bt * H_v + h], p, ot);
        for (int i = 0; i < d_v; ++i) {
          size_t yi = (bt * H_v + h) * d_v + i;
          if (o) o[yi] = ot[i];
          y[yi] = ot[i] * sigmoid(z[yi]);
        }
      }
  free(p);
  free(ot);
  return 0;
}

/* ---------------------------------------------------------------------------
 * Whole layer from raw inputs, streaming one token at a time.  Work is split
 * into independent (b, value head) tasks; each task convolves the channels it
 * reads (q and k of its key head, v of its value head) straight from x and the
 * initial conv history, so tasks share nothing mutable.
 * ------------------------------------------------------------------------- */
typedef struct {
  int B, H_k, H_v, d_k, d_v, W, dtype;
  int64_t T;
  double eps, q_scale;
  const void *x, *z, *w, *hist;
  const float *g, *beta;
  double *S, *y;
  const int32_t *tasks; /* pairs (b, h) */
  int n_tasks;
  int next;             /* next task index, guarded by mu */
  pthread_mutex_t mu;
  int failed;
} layer_job;

static void layer_task(layer_job *J, int b, int h) {
  int d_k = J->d_k, d_v = J->d_v, W = J->W, G = J->H_v / J->H_k, kh = h / G;
  int C_ch = 2 * J->H_k * d_k + J->H_v * d_v;
  double *buf = (double *)malloc(sizeof(double) * (size_t)(3 * d_k + 3 * d_v));
  if (!buf) { J->failed = 1; return; }
  double *q = buf, *k = q + d_k, *v = k + d_k, *p = v + d_v, *o = p + d_v;
  double *tmp = o + d_v; /* d_k scratch for the norm */
  double *Sh = J->S + ((size_t)b * J->H_v + h) * d_v * d_k;
  for (int64_t t = 0; t < J->T; ++t) {
    for (int j = 0; j < d_k; ++j)
      tmp[j] = silu(conv_at(J->x, J->w, J->hist, J->dtype, J->T, C_ch, W, b, t,
                            kh * d_k + j));
    oracle_l2norm(1, d_k, tmp, J->eps, J->q_scale, q);
    for (int j = 0; j < d_k; ++j)
      tmp[j] = silu(conv_at(J->x, J->w, J->hist, J->dtype, J->T, C_ch, W, b, t,
                            J->H_k * d_k + kh * d_k + j));
    oracle_l2norm(1, d_k, tmp, J->eps, 1.0, k);
    for (int i = 0; i < d_v; ++i)
      v[i] = silu(conv_at(J->x, J->w, J->hist, J->dtype, J->T, C_ch, W, b, t,
                          2 * J->H_k * d_k + h * d_v + i));
    size_t bth = ((size_t)b * J->T + t) * J->H_v + h;
    double a = exp((double)J->g[bth]);
    delta_step(d_v, d_k, Sh, k, v, q, a, (double)J->beta[bth], p, o);
    for (int i = 0; i < d_v; ++i)
      J->y[bth * d_v + i] =
          J->z ? o[i] * sigmoid(widen(J->z, bth * d_v + i, J->dtype)) : o[i];
  }
  free(buf);
}

static void *layer_worker(void *arg) {
  layer_job *J = (layer_job *)arg;
  for (;;) {
    pthread_mutex_lock(&J->mu);
    int i = J->next++;
    pthread_mutex_unlock(&J->mu);
    if (i >= J->n_tasks) break;
    layer_task(J, J->tasks[2 * i], J->tasks[2 * i + 1]);
  }
  return NULL;
}

/* Full layer.
 *   x: [B,T,C_ch] dtype; z: [B,T,H_v,d_v] dtype, or NULL for the ungated
 *   readout y = o = S_t q_t (the recurrence's output before the sigmoid
 *   gate); g, beta: [B,T,H_v] fp32;
 *   w: [C_ch,W] dtype; hist: [B,W-1,C_ch] dtype, read only (use
 *   oracle_conv_history_next for the updated history);
 *   S: [B,H_v,d_v,d_k] double in/out; y: [B,T,H_v,d_v] double out.
 *   tasks/n_tasks: the (b, h) pairs to compute (NULL = all); y and S of other
 *   heads are left untouched.  nthreads >= 1. */
int oracle_layer(int B, int64_t T, int H_k, int H_v, int d_k, int d_v, int W,
                 int dtype, double eps, double q_scale, const void *x,
                 const void *z, const float *g, const float *beta, const void *w,
                 const void *hist, double *S, double *y, const int32_t *tasks,
                 int n_tasks, int nthreads) {
  if (B < 0 || T < 0 || H_k <= 0 || H_v <= 0 || H_v % H_k || d_k <= 0 ||
      d_v <= 0 || W < 1 || nthreads < 1)
    return -1;
  if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
  int32_t *all = NULL;
  if (!tasks) {
    n_tasks = B * H_v;
    all = (int32_t *)malloc(sizeof(int32_t) * 2 * (size_t)(n_tasks > 0 ? n_tasks : 1));
    if (!all) return -2;
    for (int b = 0; b < B; ++b)
      for (int h = 0; h < H_v; ++h) {
        all[2 * (b * H_v + h)] = b;
        all[2 * (b * H_v + h) + 1] = h;
      }
    tasks = all;
  }
  layer_job J;
  memset(&J, 0, sizeof J);
  J.B = B; J.H_k = H_k; J.H_v = H_v; J.d_k = d_k; J.d_v = d_v; J.W = W;
  J.dtype = dtype; J.T = T; J.eps = eps; J.q_scale = q_scale;
  J.x = x; J.z = z; J.w = w; J.hist = hist; J.g = g; J.beta = beta;
  J.S = S; J.y = y; J.tasks = tasks; J.n_tasks = n_tasks;
  pthread_mutex_init(&J.mu, NULL);
  if (nthreads > n_tasks) nthreads = n_tasks > 0 ? n_tasks : 1;
  pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
  int started = 0;
  if (th)
    for (; started < nthreads - 1; ++started)
      if (pthread_create(&th[started], NULL, layer_worker, &J)) break;
  layer_worker(&J);
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
  free(th);
  pthread_mutex_destroy(&J.mu);
  free(all);
  return J.failed ? -2 : 0;
}

/* Zero-centred grouped RMS norm, then the sigmoid output gate ("Implement the
 * Qwen3.8 Flash Next Rust and Metal text core", section Implementation:
 * zero-centred norms; its implementation comment: zero-centred grouped RMS
 * and the sigmoid output gate).  Reading taken: a group is the d values of
 * one value head of one token; each is divided by the square root of the
 * group's mean square plus eps and multiplied by (1 + w[i]) (a zero-centred
 * weight: w = 0 is the identity scale), then by sigmoid(z[i]) when z is
 * given.  groups x d values in o, z and y; w has d entries (NULL: all 0). */
int oracle_gated_rmsnorm(int64_t groups, int d, const double *o, const double *z,
                         const double *w, double eps, double *y) {
  if (groups < 0 || d <= 0 || eps < 0) return -1;
  for (int64_t gi = 0; gi < groups; ++gi) {
    const double *og = o + gi * d;
    double ss = 0.0;
    for (int i = 0; i < d; ++i) ss += og[i] * og[i];
    double inv = 1.0 / sqrt(ss / d + eps);
    for (int i = 0; i < d; ++i) {
      double v = og[i] * inv * (1.0 + (w ? w[i] : 0.0));
      y[gi * d + i] = z ? v * sigmoid(z[gi * d + i]) : v;
    }
  }
  return 0;
}
