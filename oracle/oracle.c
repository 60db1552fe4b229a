/*
 * oracle.c -- plain fp64 CPU reference for YOCO's cross-decoder hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library; it includes only the C
 * standard library and OpenMP.
 *
 * Pages followed (cited by title and section; no line numbers):
 *   [Notes]  "YOCO：You Only Cache Once 中文精读笔记" (reading notes of
 *            arXiv:2405.05254v2), section 2.1, Eq. 2 (shared K/V projected once
 *            from the self-decoder output) and Eq. 3 (per-layer query, causal
 *            GQA attention, position n reads cache rows m <= n).
 *   [Blog]   "NeurIPS'24 | YOCO: 长上下文 LLM 为什么不必每层都存一份 KV Cache?",
 *            section 2 (single-head attention softmax(q K_{<=t}^T / sqrt(d_h))
 *            V_{<=t}), section 3 (Norm(M) W_K, Norm(M) W_V; Norm_l(X) W_Q),
 *            section 7 (shapes: K, V [B,S,8,128] from [B,S,1024]; Q
 *            [B,T,24,128]).
 *   [Deep]   "You Only Cache Once: Decoder-Decoder Architectures for Language
 *            Models" (papercache deep notes), section 2.2 Cross-Decoder (LN is
 *            RMSNorm; K/V reused by all L/2 cross layers; GQA-compatible).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - RMSNorm: y = x * g / sqrt(mean(x^2) + eps), eps inside the root, no
 *     centring, no bias (the pages only name RMSNorm).
 *   - One norm (one gain vector) is shared by K and V; Eq. 2 applies a single
 *     LN(M) to both projections.
 *   - W_K, W_V are [d_model, H_kv*d_h]; output column j = g*d_h + e becomes
 *     head g, element e (the reshape in the blog's section 7 table).
 *   - GQA: query head h reads KV head floor(h / G), G = H_q / H_kv.
 *   - Causal boundary is inclusive: a query at absolute position p reads rows
 *     0..p.
 *   - Softmax scale is passed in (1/sqrt(d_h) in every workload, [Blog] s.2).
 *
 * The method reaches the plain softmax-attention definition exactly (tiling,
 * split-N and online softmax are exact rewrites), so this file writes that
 * definition out: max, exp, sum, weighted sum, divide.  Sums are naive
 * left-to-right fp64 loops.  OpenMP only distributes independent
 * (query row, head) tasks; it changes no arithmetic.
 *
 * Input storage codes: 0 = float32, 1 = bf16 (raw uint16 bits, widened
 * exactly).  Every element is converted to double when read.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_F32 0
#define ORACLE_BF16 1

static double read_elem(const void *p, int dtype, int64_t i) {
  if (dtype == ORACLE_F32) {
    return (double)((const float *)p)[i];
  }
  uint32_t bits = ((uint32_t)((const uint16_t *)p)[i]) << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* RMSNorm ([Notes] s.2.1: "LN" is RMSNorm; [Deep] s.2.1).
 * x: [n, d] stored values; gain: [d] float32 or NULL for all ones.
 * y[r, c] = x[r, c] * gain[c] / sqrt((1/d) * sum_c x[r, c]^2 + eps). */
void oracle_rmsnorm(const void *x, int x_dtype, int64_t n, int64_t d,
                    const float *gain, double eps, double *y) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r) {
    double sum_sq = 0.0;
    for (int64_t c = 0; c < d; ++c) {
      double v = read_elem(x, x_dtype, r * d + c);
      sum_sq += v * v;
    }
    double rms = sqrt(sum_sq / (double)d + eps);
    for (int64_t c = 0; c < d; ++c) {
      double g = gain ? (double)gain[c] : 1.0;
      y[r * d + c] = read_elem(x, x_dtype, r * d + c) * g / rms;
    }
  }
}

/* Row-vector times matrix: out[r, j] = sum_c y[r, c] * w[c, j].
 * y: [n, d] double; w: [d, ncols] stored values; out: [n, ncols] double.
 * This is the "LN(M) W" product of [Notes] Eq. 2-3. */
void oracle_matmul(const double *y, int64_t n, int64_t d, const void *w,
                   int w_dtype, int64_t ncols, double *out) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r) {
    for (int64_t j = 0; j < ncols; ++j) {
      double acc = 0.0;
      for (int64_t c = 0; c < d; ++c) {
        acc += y[r * d + c] * read_elem(w, w_dtype, c * ncols + j);
      }
      out[r * ncols + j] = acc;
    }
  }
}

/* Normalise, then project: out = RMSNorm(x; gain, eps) @ w.
 * [Notes] Eq. 2 (K^ = LN(M) W_K, V^ = LN(M) W_V) and Eq. 3 (Q^l = LN(X^l) W_Q^l).
 * Returns 0, or -1 if scratch memory cannot be obtained. */
int oracle_project(const void *x, int x_dtype, int64_t n, int64_t d,
                   const float *gain, double eps, const void *w, int w_dtype,
                   int64_t ncols, double *out) {
  double *y = (double *)malloc((size_t)(n * d) * sizeof(double));
  if (!y) return -1;
  oracle_rmsnorm(x, x_dtype, n, d, gain, eps, y);
  oracle_matmul(y, n, d, w, w_dtype, ncols, out);
  free(y);
  return 0;
}

/* Rotary position embedding (RoPE) of every head of every row, in place.
 *
 * [Blog] s.7: the shared projection rotates K^ by position and each cross
 * layer rotates its own Q likewise; V is not rotated.  [Notes] s.4.3,
 * Table 7: the base theta of each training stage (640K for 64K tokens, 5M
 * for 256K, 80M for 1M).
 *
 * Readings where the pages are silent: pair i (0 <= i < dh/2) of a head
 * turns by the angle pos * theta^(-2i/dh).  interleaved = 1: the pair is
 * elements (2i, 2i+1), read as the complex number x_2i + j*x_2i+1 times
 * exp(j*angle) -- the complex notation Theta_n = exp(i*n*theta) the pages use
 * for the retention of the self-decoder; interleaved = 0: the pair is
 * (i, i + dh/2).
 *
 * x: [n][heads][dh] double, rotated in place; pos: [n] absolute positions.
 */
void oracle_rope(double *x, int64_t n, int heads, int dh, const int64_t *pos,
                 double theta, int interleaved) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r) {
    for (int h = 0; h < heads; ++h) {
      double *xh = x + (r * heads + h) * dh;
      for (int i = 0; i < dh / 2; ++i) {
        const double freq = pow(theta, -2.0 * (double)i / (double)dh);
        const double angle = (double)pos[r] * freq;
        const double c = cos(angle);
        const double s = sin(angle);
        const int j0 = interleaved ? 2 * i : i;
        const int j1 = interleaved ? 2 * i + 1 : i + dh / 2;
        const double a = xh[j0];
        const double b = xh[j1];
        xh[j0] = a * c - b * s;
        xh[j1] = a * s + b * c;
      }
    }
  }
}

/* Causal GQA softmax attention over one shared K/V slab.
 *
 * [Notes] s.2.1, Eq. 3: Attention(Q^l, K^, V^) with a causal mask -- the
 * query at position n reads only cache rows m <= n; GQA supported.
 * [Blog] s.2: o_t = softmax(q_t K_{<=t}^T / sqrt(d_h)) V_{<=t}.
 *
 * q:   [n_q, hq, dh] stored values; query row i sits at absolute position
 *      pos[i] and reads cache rows 0..pos[i] inclusive.
 * k,v: [kv_rows, hkv, dh] stored values (one sequence's shared slab).
 * o:   [n_q, hq, dh] double.  lse: [n_q, hq] double or NULL;
 *      lse = m + ln(l) is the log of the softmax denominator.
 * Query head h reads KV head h / (hq / hkv).
 *
 * Returns 0; -1 on bad arguments (hq % hkv != 0, or pos[i] outside
 * [0, kv_rows)); -2 if scratch memory cannot be obtained.
 */
int oracle_attention(const void *q, int q_dtype, int64_t n_q, const int64_t *pos,
                     int hq, const void *k, const void *v, int kv_dtype,
                     int64_t kv_rows, int hkv, int dh, double scale, double *o,
                     double *lse) {
  if (hq <= 0 || hkv <= 0 || dh <= 0 || hq % hkv != 0) return -1;
  for (int64_t i = 0; i < n_q; ++i) {
    if (pos[i] < 0 || pos[i] >= kv_rows) return -1;
  }
  const int group = hq / hkv;
  const int64_t n_tasks = n_q * (int64_t)hq;
  int failed = 0;

#pragma omp parallel
  {
    int64_t cap = 0;
    double *logits = NULL;
    double *acc = (double *)malloc((size_t)dh * sizeof(double));
#pragma omp for schedule(dynamic, 1)
    for (int64_t task = 0; task < n_tasks; ++task) {
      const int64_t i = task / hq;
      const int h = (int)(task % hq);
      const int g = h / group;
      const int64_t n_keys = pos[i] + 1;
      if (n_keys > cap) {
        free(logits);
        cap = n_keys;
        logits = (double *)malloc((size_t)cap * sizeof(double));
      }
      if (!logits || !acc) {
        cap = 0;
#pragma omp atomic write
        failed = 1;
        continue;
      }
      const int64_t q_base = (i * hq + h) * (int64_t)dh;

      /* x_j = scale * <q, k_j> for every visible row j. */
      for (int64_t j = 0; j < n_keys; ++j) {
        const int64_t k_base = (j * hkv + g) * (int64_t)dh;
        double dot = 0.0;
        for (int e = 0; e < dh; ++e) {
          dot += read_elem(q, q_dtype, q_base + e) * read_elem(k, kv_dtype, k_base + e);
        }
        logits[j] = scale * dot;
      }

      /* softmax: m = max_j x_j, p_j = exp(x_j - m), l = sum_j p_j. */
      double m = logits[0];
      for (int64_t j = 1; j < n_keys; ++j) {
        if (logits[j] > m) m = logits[j];
      }
      double l = 0.0;
      for (int64_t j = 0; j < n_keys; ++j) {
        logits[j] = exp(logits[j] - m);
        l += logits[j];
      }

      /* o_e = (sum_j p_j v_{j,e}) / l; each sum runs j = 0, 1, ... in order. */
      for (int e = 0; e < dh; ++e) acc[e] = 0.0;
      for (int64_t j = 0; j < n_keys; ++j) {
        const int64_t v_base = (j * hkv + g) * (int64_t)dh;
        for (int e = 0; e < dh; ++e) {
          acc[e] += logits[j] * read_elem(v, kv_dtype, v_base + e);
        }
      }
      for (int e = 0; e < dh; ++e) o[q_base + e] = acc[e] / l;
      if (lse) lse[i * hq + h] = m + log(l);
    }
    free(logits);
    free(acc);
  }
  return failed ? -2 : 0;
}
