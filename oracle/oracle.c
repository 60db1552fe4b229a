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
 * exactly), 2 = float64.  Every element is converted to double when read.
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
#define ORACLE_F64 2

static double read_elem(const void *p, int dtype, int64_t i) {
  if (dtype == ORACLE_F32) {
    return (double)((const float *)p)[i];
  }
  if (dtype == ORACLE_F64) {
    return ((const double *)p)[i];
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

/* Backward of causal GQA attention (the gradient of [Notes] Eq. 3 with
 * respect to the query, K^ and V^; [Deep] s.2.2: every cross layer reads the
 * same K^/V^, so by the chain rule their gradients are the sums of each
 * layer's contribution).
 *
 * For query row i at position pos[i], head h (KV head g = h / (hq / hkv)),
 * logits x_j = scale * <q, k_j> over the visible rows j = 0..pos[i], and
 * upstream gradient dO of the output o = sum_j p_j v_j:
 *   p_j  = softmax(x)_j                      (max, exp, sum, divide)
 *   dp_j = <dO, v_j>                          (gradient of o wrt p_j)
 *   D    = sum_j p_j dp_j                     (softmax Jacobian term)
 *   ds_j = p_j (dp_j - D)                     (gradient wrt x_j)
 *   dq   = scale * sum_j ds_j k_j
 *   dk_j += scale * ds_j q,   dv_j += p_j dO.
 *
 * q, dout: [n_q][hq][dh]; k, v: [kv_rows][hkv][dh]; dq: [n_q][hq][dh]
 * (written); dk, dv: [kv_rows][hkv][dh] (ADDED to, so that calls for several
 * layers, or for disjoint sets of query rows, sum).  Only rows j <= pos[i]
 * of the given query rows contribute to dk, dv.
 *
 * The work is split in two passes that do not change the arithmetic of a
 * term: pass 1 (independent (row, head) tasks) forms the softmax statistics
 * m, l, D and dq; pass 2 (independent (KV head, block of 64 cache rows)
 * tasks) adds every (row, head) contribution to its cache rows, in order of
 * ascending query row, then query head.
 *
 * Returns 0; -1 on bad arguments; -2 if scratch memory cannot be obtained.
 */
int oracle_attention_bwd(const void *q, int q_dtype, int64_t n_q, const int64_t *pos, int hq,
                         const void *k, const void *v, int kv_dtype, int64_t kv_rows, int hkv,
                         int dh, const void *dout, int do_dtype, double scale, double *dq,
                         double *dk, double *dv) {
  if (hq <= 0 || hkv <= 0 || dh <= 0 || hq % hkv != 0) return -1;
  for (int64_t i = 0; i < n_q; ++i) {
    if (pos[i] < 0 || pos[i] >= kv_rows) return -1;
  }
  const int group = hq / hkv;
  const int64_t n_tasks = n_q * (int64_t)hq;
  double *stat_m = (double *)malloc((size_t)(n_tasks > 0 ? n_tasks : 1) * sizeof(double));
  double *stat_l = (double *)malloc((size_t)(n_tasks > 0 ? n_tasks : 1) * sizeof(double));
  double *stat_d = (double *)malloc((size_t)(n_tasks > 0 ? n_tasks : 1) * sizeof(double));
  if (!stat_m || !stat_l || !stat_d) {
    free(stat_m);
    free(stat_l);
    free(stat_d);
    return -2;
  }
  int failed = 0;

  /* Pass 1: per (row, head), the logits, softmax, D and dq. */
#pragma omp parallel
  {
    int64_t cap = 0;
    double *x = NULL, *dp = NULL;
#pragma omp for schedule(dynamic, 1)
    for (int64_t task = 0; task < n_tasks; ++task) {
      const int64_t i = task / hq;
      const int h = (int)(task % hq);
      const int kvh = h / group;
      const int64_t n_vis = pos[i] + 1;
      if (n_vis > cap) {
        free(x);
        free(dp);
        cap = n_vis;
        x = (double *)malloc((size_t)cap * sizeof(double));
        dp = (double *)malloc((size_t)cap * sizeof(double));
      }
      if (!x || !dp) {
        cap = 0;
#pragma omp atomic write
        failed = 1;
        continue;
      }
      const int64_t q_base = (i * hq + h) * (int64_t)dh;
      for (int64_t j = 0; j < n_vis; ++j) {
        const int64_t kv_base = (j * hkv + kvh) * (int64_t)dh;
        double qk = 0.0, dpj = 0.0;
        for (int e = 0; e < dh; ++e) {
          qk += read_elem(q, q_dtype, q_base + e) * read_elem(k, kv_dtype, kv_base + e);
          dpj += read_elem(dout, do_dtype, q_base + e) * read_elem(v, kv_dtype, kv_base + e);
        }
        x[j] = scale * qk;
        dp[j] = dpj;
      }
      double m = x[0];
      for (int64_t j = 1; j < n_vis; ++j) {
        if (x[j] > m) m = x[j];
      }
      double l = 0.0;
      for (int64_t j = 0; j < n_vis; ++j) l += exp(x[j] - m);
      double d_term = 0.0;
      for (int64_t j = 0; j < n_vis; ++j) d_term += (exp(x[j] - m) / l) * dp[j];
      for (int e = 0; e < dh; ++e) dq[q_base + e] = 0.0;
      for (int64_t j = 0; j < n_vis; ++j) {
        const double ds = (exp(x[j] - m) / l) * (dp[j] - d_term);
        const int64_t kv_base = (j * hkv + kvh) * (int64_t)dh;
        for (int e = 0; e < dh; ++e) dq[q_base + e] += ds * read_elem(k, kv_dtype, kv_base + e);
      }
      for (int e = 0; e < dh; ++e) dq[q_base + e] *= scale;
      stat_m[task] = m;
      stat_l[task] = l;
      stat_d[task] = d_term;
    }
    free(x);
    free(dp);
  }

  /* Pass 2: per (KV head, block of cache rows), every contribution to dk, dv. */
  const int64_t kBlock = 64;
  const int64_t n_blocks = (kv_rows + kBlock - 1) / kBlock;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t task = 0; task < n_blocks * hkv; ++task) {
    const int g = (int)(task % hkv);
    const int64_t j0 = (task / hkv) * kBlock;
    const int64_t j1 = j0 + kBlock < kv_rows ? j0 + kBlock : kv_rows;
    for (int64_t i = 0; i < n_q; ++i) {
      if (pos[i] < j0) continue;
      const int64_t j_end = pos[i] + 1 < j1 ? pos[i] + 1 : j1;
      for (int h = g * group; h < (g + 1) * group; ++h) {
        const int64_t t = i * hq + h;
        const int64_t q_base = t * (int64_t)dh;
        for (int64_t j = j0; j < j_end; ++j) {
          const int64_t kv_base = (j * hkv + g) * (int64_t)dh;
          double qk = 0.0, dpj = 0.0;
          for (int e = 0; e < dh; ++e) {
            qk += read_elem(q, q_dtype, q_base + e) * read_elem(k, kv_dtype, kv_base + e);
            dpj += read_elem(dout, do_dtype, q_base + e) * read_elem(v, kv_dtype, kv_base + e);
          }
          const double p = exp(scale * qk - stat_m[t]) / stat_l[t];
          const double ds = p * (dpj - stat_d[t]);
          for (int e = 0; e < dh; ++e) {
            dv[kv_base + e] += p * read_elem(dout, do_dtype, q_base + e);
            dk[kv_base + e] += scale * ds * read_elem(q, q_dtype, q_base + e);
          }
        }
      }
    }
  }
  free(stat_m);
  free(stat_l);
  free(stat_d);
  return failed ? -2 : 0;
}

/* Backward of the shared projection K^ = RMSNorm(x) W_K, V^ = RMSNorm(x) W_V
 * ([Notes] Eq. 2; the norm's formula is the reading stated at the top).
 *
 * With y = RMSNorm(x; g, eps), r = sqrt(mean_c x_c^2 + eps) per row, and the
 * upstream gradients dz_k, dz_v of the two outputs:
 *   dW_t[c][j] = sum_rows y[c] dz_t[j]                  (t = K, V)
 *   dy[c]      = sum_j dz_k[j] W_K[c][j] + sum_j dz_v[j] W_V[c][j]
 *   dgain[c]   = sum_rows dy[c] x[c] / r
 *   dx[c]      = g[c] dy[c] / r - x[c] / (d r^3) * sum_c' g[c'] dy[c'] x[c']
 * (the last from dr/dx_c = x_c / (d r)).
 *
 * x: [n][d] stored; gain: [d] float32 or NULL (all ones); w_k, w_v:
 * [d][ncols] stored; dz_k, dz_v: [n][ncols] stored; outputs double: dx
 * [n][d], dw_k, dw_v [d][ncols], dgain [d] (skipped when NULL).
 * Returns 0, or -2 if scratch memory cannot be obtained.
 */
int oracle_project_bwd(const void *x, int x_dtype, int64_t n, int64_t d, const float *gain,
                       double eps, const void *w_k, const void *w_v, int w_dtype, int64_t ncols,
                       const void *dz_k, const void *dz_v, int dz_dtype, double *dx,
                       double *dw_k, double *dw_v, double *dgain) {
  double *y = (double *)malloc((size_t)(n * d > 0 ? n * d : 1) * sizeof(double));
  double *dy = (double *)malloc((size_t)(n * d > 0 ? n * d : 1) * sizeof(double));
  double *rr = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
  if (!y || !dy || !rr) {
    free(y);
    free(dy);
    free(rr);
    return -2;
  }
  oracle_rmsnorm(x, x_dtype, n, d, gain, eps, y);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r) {
    double ss = 0.0;
    for (int64_t c = 0; c < d; ++c) {
      const double xv = read_elem(x, x_dtype, r * d + c);
      ss += xv * xv;
    }
    rr[r] = sqrt(ss / (double)d + eps);
    for (int64_t c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int64_t j = 0; j < ncols; ++j) {
        acc += read_elem(dz_k, dz_dtype, r * ncols + j) * read_elem(w_k, w_dtype, c * ncols + j);
      }
      for (int64_t j = 0; j < ncols; ++j) {
        acc += read_elem(dz_v, dz_dtype, r * ncols + j) * read_elem(w_v, w_dtype, c * ncols + j);
      }
      dy[r * d + c] = acc;
    }
    double proj = 0.0;
    for (int64_t c = 0; c < d; ++c) {
      const double g = gain ? (double)gain[c] : 1.0;
      proj += g * dy[r * d + c] * read_elem(x, x_dtype, r * d + c);
    }
    const double r3 = rr[r] * rr[r] * rr[r];
    for (int64_t c = 0; c < d; ++c) {
      const double g = gain ? (double)gain[c] : 1.0;
      const double xv = read_elem(x, x_dtype, r * d + c);
      dx[r * d + c] = g * dy[r * d + c] / rr[r] - xv / ((double)d * r3) * proj;
    }
  }
#pragma omp parallel for schedule(static)
  for (int64_t c = 0; c < d; ++c) {
    for (int64_t j = 0; j < ncols; ++j) {
      double ak = 0.0, av = 0.0;
      for (int64_t r = 0; r < n; ++r) {
        ak += y[r * d + c] * read_elem(dz_k, dz_dtype, r * ncols + j);
        av += y[r * d + c] * read_elem(dz_v, dz_dtype, r * ncols + j);
      }
      dw_k[c * ncols + j] = ak;
      dw_v[c * ncols + j] = av;
    }
    if (dgain) {
      double ag = 0.0;
      for (int64_t r = 0; r < n; ++r) ag += dy[r * d + c] * read_elem(x, x_dtype, r * d + c) / rr[r];
      dgain[c] = ag;
    }
  }
  free(y);
  free(dy);
  free(rr);
  return 0;
}

/* ---- Gated retention (gRet), the self-decoder's token mixer --------------
 * [Notes] section 2.2, Eq. 4 (parallel form) and Eq. 5 (recurrent form);
 * [Deep] section 3.1 (gated retention: head-wise data-controlled decay);
 * [Blog] section 4 (the 2x2 state example).  Per head, with q_n, k_n of
 * length dk, v_n of length dv and a scalar gate gamma_n:
 *   gamma_n = sigmoid(g_n)^(1/tau)                              (Eq. 4)
 *   D[n][m] = prod_{i=m+1..n} gamma_i  for m <= n, 0 otherwise
 *   O       = (Q K^T (.) D) V                                    (Eq. 4)
 *   S_n     = gamma_n S_{n-1} + k_n^T v_n,   O_n = q_n S_n      (Eq. 5)
 * Positions count from 0 here (the pages count from 1).  The rotation of
 * Q and K (Theta) is applied before these functions: they take q and k as
 * they enter the products. */

/* gamma[i] = sigmoid(g[i])^(1/tau), i < count. */
void oracle_gret_gate(const float *g, int64_t count, double tau, double *gamma) {
  for (int64_t i = 0; i < count; ++i) {
    const double sig = 1.0 / (1.0 + exp(-(double)g[i]));
    gamma[i] = pow(sig, 1.0 / tau);
  }
}

/* Parallel form (Eq. 4) over a block of n positions of every head, starting
 * from the state s_in that the recurrence (Eq. 5) held before the block
 * (NULL: zero, a fresh sequence).  Unrolling Eq. 5 from that state gives
 *   O_t = sum_{m<=t} D[t][m] (q_t . k_m) v_m + (prod_{i<=t} gamma_i) q_t s_in.
 * D[t][m] is formed as a running product while m walks down from t.
 * q, k: [n][heads][dk]; v: [n][heads][dv] (stored values, one dtype);
 * gamma: [n][heads]; s_in: [heads][dk][dv] or NULL; rows: the positions to
 * evaluate (NULL: all n), o: [n_rows][heads][dv].  s_out (NULL: skipped):
 * [heads][dk][dv], the state after the block,
 *   S = (prod_all gamma) s_in + sum_m D[n-1][m] k_m^T v_m.
 * Returns 0, or -1 for a row outside [0, n). */
int oracle_gret(const void *q, const void *k, const void *v, int dtype, const double *gamma, int64_t n,
                int heads, int dk, int dv, const double *s_in, const int64_t *rows, int64_t n_rows,
                double *o, double *s_out) {
  if (rows == NULL) n_rows = n;
  for (int64_t i = 0; i < n_rows; ++i) {
    if (rows != NULL && (rows[i] < 0 || rows[i] >= n)) return -1;
  }
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int64_t i = 0; i < n_rows; ++i) {
    for (int h = 0; h < heads; ++h) {
      const int64_t t = rows ? rows[i] : i;
      double *out = o + (i * heads + h) * dv;
      for (int e = 0; e < dv; ++e) out[e] = 0.0;
      double decay = 1.0; /* D[t][m] for the current m */
      for (int64_t m = t; m >= 0; --m) {
        double dot = 0.0;
        for (int c = 0; c < dk; ++c) {
          dot += read_elem(q, dtype, (t * heads + h) * dk + c) * read_elem(k, dtype, (m * heads + h) * dk + c);
        }
        for (int e = 0; e < dv; ++e) out[e] += decay * dot * read_elem(v, dtype, (m * heads + h) * dv + e);
        decay *= gamma[m * heads + h];
      }
      if (s_in != NULL) {
        /* decay is now prod_{i=0..t} gamma_i */
        const double *s = s_in + (int64_t)h * dk * dv;
        for (int e = 0; e < dv; ++e) {
          double acc = 0.0;
          for (int c = 0; c < dk; ++c) acc += read_elem(q, dtype, (t * heads + h) * dk + c) * s[c * dv + e];
          out[e] += decay * acc;
        }
      }
    }
  }
  if (s_out != NULL) {
#pragma omp parallel for schedule(static)
    for (int h = 0; h < heads; ++h) {
      double *s = s_out + (int64_t)h * dk * dv;
      for (int64_t x = 0; x < (int64_t)dk * dv; ++x) s[x] = 0.0;
      double decay = 1.0; /* D[n-1][m] */
      for (int64_t m = n - 1; m >= 0; --m) {
        for (int c = 0; c < dk; ++c) {
          const double kc = decay * read_elem(k, dtype, (m * heads + h) * dk + c);
          for (int e = 0; e < dv; ++e) s[c * dv + e] += kc * read_elem(v, dtype, (m * heads + h) * dv + e);
        }
        decay *= gamma[m * heads + h];
      }
      if (s_in != NULL) {
        const double *si = s_in + (int64_t)h * dk * dv;
        for (int64_t x = 0; x < (int64_t)dk * dv; ++x) s[x] += decay * si[x];
      }
    }
  }
  return 0;
}

/* One step of the recurrent form (Eq. 5) for n_seq sequences: per sequence b
 * and head h, S <- gamma S + k^T v, then o = q S with the updated S.
 * q, k: [n_seq][heads][dk]; v: [n_seq][heads][dv]; gamma: [n_seq][heads];
 * state: [n_seq][heads][dk][dv], updated in place; o: [n_seq][heads][dv]. */
void oracle_gret_step(const void *q, const void *k, const void *v, int dtype, const double *gamma,
                      int64_t n_seq, int heads, int dk, int dv, double *state, double *o) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t b = 0; b < n_seq; ++b) {
    for (int h = 0; h < heads; ++h) {
      const int64_t bh = b * heads + h;
      double *s = state + bh * dk * dv;
      const double gm = gamma[bh];
      for (int c = 0; c < dk; ++c) {
        const double kc = read_elem(k, dtype, bh * dk + c);
        for (int e = 0; e < dv; ++e) s[c * dv + e] = gm * s[c * dv + e] + kc * read_elem(v, dtype, bh * dv + e);
      }
      for (int e = 0; e < dv; ++e) {
        double acc = 0.0;
        for (int c = 0; c < dk; ++c) acc += read_elem(q, dtype, bh * dk + c) * s[c * dv + e];
        o[bh * dv + e] = acc;
      }
    }
  }
}
