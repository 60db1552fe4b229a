/* Drives every function of oracle/oracle.c on tiny inputs, for a host
 * AddressSanitizer / UndefinedBehaviorSanitizer build (tests/test_host_sanitizers.py).
 * Exits non-zero on a failed check; the sanitizers abort on any memory or
 * undefined-behaviour error. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_num_threads(void);
void oracle_set_num_threads(int n);
void oracle_rmsnorm(const void *x, int x_dtype, int64_t n, int64_t d, const float *gain, double eps, double *y);
void oracle_matmul(const double *y, int64_t n, int64_t d, const void *w, int w_dtype, int64_t ncols, double *out);
int oracle_project(const void *x, int x_dtype, int64_t n, int64_t d, const float *gain, double eps, const void *w,
                   int w_dtype, int64_t ncols, double *out);
void oracle_rope(double *x, int64_t n, int heads, int dh, const int64_t *pos, double theta, int interleaved);
int oracle_attention(const void *q, int q_dtype, int64_t n_q, const int64_t *pos, int hq, const void *k,
                     const void *v, int kv_dtype, int64_t kv_rows, int hkv, int dh, double scale, double *o,
                     double *lse);
int oracle_attention_bwd(const void *q, int q_dtype, int64_t n_q, const int64_t *pos, int hq, const void *k,
                         const void *v, int kv_dtype, int64_t kv_rows, int hkv, int dh, const void *dout,
                         int do_dtype, double scale, double *dq, double *dk, double *dv);
int oracle_project_bwd(const void *x, int x_dtype, int64_t n, int64_t d, const float *gain, double eps,
                       const void *w_k, const void *w_v, int w_dtype, int64_t ncols, const void *dz_k,
                       const void *dz_v, int dz_dtype, double *dx, double *dw_k, double *dw_v, double *dgain);
void oracle_gret_gate(const float *g, int64_t count, double tau, double *gamma);
int oracle_gret(const void *q, const void *k, const void *v, int dtype, const double *gamma, int64_t n, int heads,
                int dk, int dv, const double *s_in, const int64_t *rows, int64_t n_rows, double *o, double *s_out);
void oracle_gret_step(const void *q, const void *k, const void *v, int dtype, const double *gamma, int64_t n_seq,
                      int heads, int dk, int dv, double *state, double *o);

enum { F32 = 0, BF16 = 1, F64 = 2 };
static int failures = 0;
#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); ++failures; } } while (0)

static uint32_t state = 12345u;
static float rnd(void) { state = state * 1664525u + 1013904223u; return ((state >> 8) / 16777216.0f) * 2.f - 1.f; }
static uint16_t to_bf16(float f) { uint32_t u; memcpy(&u, &f, 4); return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16); }

int main(void) {
  oracle_set_num_threads(2);
  CHECK(oracle_num_threads() >= 1);
  enum { N = 7, D = 16, HQ = 4, HKV = 2, DH = 8, NC = HKV * DH };
  float x[N * D], gain[D], w[D * NC], wv[D * NC], q[N * HQ * DH], k[N * HKV * DH], v[N * HKV * DH], dout[N * HQ * DH];
  uint16_t xb[N * D], kb[N * HKV * DH], vb[N * HKV * DH], qb[N * HQ * DH];
  for (int i = 0; i < N * D; ++i) { x[i] = rnd(); xb[i] = to_bf16(x[i]); }
  for (int i = 0; i < D; ++i) gain[i] = 1.f + 0.1f * rnd();
  for (int i = 0; i < D * NC; ++i) { w[i] = rnd(); wv[i] = rnd(); }
  for (int i = 0; i < N * HQ * DH; ++i) { q[i] = rnd(); qb[i] = to_bf16(q[i]); dout[i] = rnd(); }
  for (int i = 0; i < N * HKV * DH; ++i) { k[i] = rnd(); v[i] = rnd(); kb[i] = to_bf16(k[i]); vb[i] = to_bf16(v[i]); }

  double y[N * D], z[N * NC], z2[N * NC];
  oracle_rmsnorm(x, F32, N, D, gain, 1e-6, y);
  oracle_rmsnorm(xb, BF16, N, D, NULL, 1e-6, y);
  oracle_matmul(y, N, D, w, F32, NC, z);
  CHECK(oracle_project(x, F32, N, D, gain, 1e-6, w, F32, NC, z) == 0);
  CHECK(oracle_project(xb, BF16, N, D, NULL, 1e-6, w, F32, NC, z2) == 0);
  int64_t pos[N];
  for (int i = 0; i < N; ++i) pos[i] = i;
  oracle_rope(z, N, HKV, DH, pos, 640000.0, 1);
  oracle_rope(z2, N, HKV, DH, pos, 640000.0, 0);

  double o[N * HQ * DH], lse[N * HQ];
  CHECK(oracle_attention(q, F32, N, pos, HQ, k, v, F32, N, HKV, DH, 0.35, o, lse) == 0);
  /* row 0 sees one key: its output is V row 0 of its KV head exactly */
  for (int h = 0; h < HQ; ++h)
    for (int e = 0; e < DH; ++e) CHECK(o[h * DH + e] == (double)v[(h / (HQ / HKV)) * DH + e]);
  CHECK(oracle_attention(qb, BF16, N, pos, HQ, kb, vb, BF16, N, HKV, DH, 0.35, o, NULL) == 0);
  int64_t bad[1] = {N};
  CHECK(oracle_attention(q, F32, 1, bad, HQ, k, v, F32, N, HKV, DH, 0.35, o, lse) == -1);
  CHECK(oracle_attention(q, F32, 1, pos, 3, k, v, F32, N, HKV, DH, 0.35, o, lse) == -1);

  double dq[N * HQ * DH], dk[N * HKV * DH], dv[N * HKV * DH];
  memset(dk, 0, sizeof dk);
  memset(dv, 0, sizeof dv);
  CHECK(oracle_attention_bwd(q, F32, N, pos, HQ, k, v, F32, N, HKV, DH, dout, F32, 0.35, dq, dk, dv) == 0);
  double s = 0.0;  /* sum_j dV_j equals the sum of dO over the group's rows and heads */
  for (int j = 0; j < N; ++j) s += dv[(j * HKV + 0) * DH + 3];
  double want = 0.0;
  for (int i = 0; i < N; ++i)
    for (int h = 0; h < HQ / HKV; ++h) want += dout[(i * HQ + h) * DH + 3];
  CHECK(fabs(s - want) < 1e-9);

  double dx[N * D], dwk[D * NC], dwv[D * NC], dg[D];
  float dzk[N * NC], dzv[N * NC];
  for (int i = 0; i < N * NC; ++i) { dzk[i] = rnd(); dzv[i] = rnd(); }
  CHECK(oracle_project_bwd(x, F32, N, D, gain, 1e-6, w, wv, F32, NC, dzk, dzv, F32, dx, dwk, dwv, dg) == 0);
  CHECK(oracle_project_bwd(xb, BF16, N, D, NULL, 1e-6, w, wv, F32, NC, dzk, dzv, F32, dx, dwk, dwv, NULL) == 0);

  float g[N * HKV];
  double gamma[N * HKV], go[N * HKV * DH], st[HKV * DH * DH], st2[HKV * DH * DH];
  for (int i = 0; i < N * HKV; ++i) g[i] = 2.f * rnd();
  oracle_gret_gate(g, N * HKV, 16.0, gamma);
  for (int i = 0; i < N * HKV; ++i) CHECK(gamma[i] > 0.0 && gamma[i] < 1.0);
  CHECK(oracle_gret(k, k, v, F32, gamma, N, HKV, DH, DH, NULL, NULL, 0, go, st) == 0);
  int64_t rows[2] = {0, N - 1};
  CHECK(oracle_gret(kb, kb, vb, BF16, gamma, N, HKV, DH, DH, st, rows, 2, go, st2) == 0);
  int64_t badrow[1] = {N};
  CHECK(oracle_gret(k, k, v, F32, gamma, N, HKV, DH, DH, NULL, badrow, 1, go, NULL) != 0);
  memset(st, 0, sizeof st);
  oracle_gret_step(k, k, v, F32, gamma, 1, HKV, DH, DH, st, go);

  if (failures) fprintf(stderr, "%d checks failed\n", failures);
  else printf("oracle driver: all functions ran clean\n");
  return failures ? 1 : 0;
}
