/*
 * yoco.h -- C ABI of the MI355X (gfx950) shared-KV cross-decoder library.
 *
 * YOCO ("You Only Cache Once") splits a decoder into a self-decoder and a
 * cross-decoder.  The self-decoder output M is projected ONCE into a global
 * K^/V^ cache, and every one of the L/2 cross-decoder layers brings its own
 * query Q^l = RMSNorm_l(X^l) W_Q^l to that single cache through causal GQA
 * softmax attention.  Sources (page title, section, equation):
 *   [Notes] "YOCO：You Only Cache Once 中文精读笔记", section 2.1, Eq. 2
 *           (K^ = LN(M) W_K, V^ = LN(M) W_V, projected once at the boundary)
 *           and Eq. 3 (Q^l = LN(X^l) W_Q^l; Attention(Q^l, K^, V^) with a
 *           causal mask, position n reads rows m <= n; GQA).
 *   [Blog]  "NeurIPS'24 | YOCO: 长上下文 LLM 为什么不必每层都存一份 KV Cache?",
 *           section 2 (o_t = softmax(q_t K_{<=t}^T / sqrt(d_h)) V_{<=t}),
 *           section 6 (prefill skips history cross outputs; the last prompt
 *           token still runs every cross layer), section 7 (CrossDecoder
 *           projects the shared K/V once and writes the cache before the
 *           skip branch; each CrossAttention projects only its own Q and
 *           calls causal attention on the K/V passed to it; shapes K, V
 *           [B,S,8,128], Q [B,T,24,128]).
 *   [Deep]  "You Only Cache Once: Decoder-Decoder Architectures for Language
 *           Models" (papercache deep notes), section 2.2 Cross-Decoder.
 *
 * Conventions for every function:
 *   - Data pointers are DEVICE pointers unless marked HOST.  The caller owns
 *     all memory; the library allocates, frees and retains nothing.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and the library never synchronizes.  Buffers must stay alive until the
 *     stream work completes.
 *   - All validation happens on the host before anything is enqueued.  On any
 *     status other than YOCO_OK nothing was enqueued and every host-side
 *     length is unchanged; yoco_last_error() gives the reason.
 *   - Row-major layouts; element [a][b][c] of an [A][B][C] array sits at
 *     offset (a*B + b)*C + c.
 *   - Alignment: every device array is 16-byte aligned (hipMalloc and torch
 *     allocations are 256-byte aligned; row slices keep it when a row is a
 *     multiple of 16 bytes), except the per-row or per-head scalar arrays
 *     (lse, gate_logits), which need 4 bytes.  Any other pointer is rejected
 *     with YOCO_ERR_ALIGNMENT before anything is enqueued.
 *   - head_dim is 64 or 128; H_q must be a multiple of H_kv with group size
 *     G = H_q / H_kv in {1, 2, 3, 4, 6, 8}.  Query head h reads KV head
 *     floor(h / G).
 *   - RMSNorm is y = x * g / sqrt(mean(x^2) + eps) per row, statistics in
 *     fp32; the projections accumulate in fp32 and store with
 *     round-to-nearest-even when the destination is bf16.
 *   - Functions are re-entrant.  The only library state is the per-thread
 *     error text and a per-device record that the device is gfx950.
 */
#ifndef YOCO_H
#define YOCO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define YOCO_ABI_VERSION 9
#define YOCO_MAX_SEQ 256

/* Storage types. */
typedef enum yoco_dtype {
  YOCO_DT_F32 = 0,  /* IEEE binary32 */
  YOCO_DT_BF16 = 1  /* bfloat16: the upper 16 bits of a binary32 */
} yoco_dtype;

typedef enum yoco_status {
  YOCO_OK = 0,
  YOCO_ERR_NULL_POINTER = 1, /* a required pointer is NULL */
  YOCO_ERR_BAD_SHAPE = 2,    /* unsupported head_dim / group size / counts */
  YOCO_ERR_BAD_DTYPE = 3,    /* unsupported or mismatched storage type */
  YOCO_ERR_OUT_OF_RANGE = 4, /* rows or positions outside the cache */
  YOCO_ERR_WORKSPACE = 5,    /* workspace too small */
  YOCO_ERR_HIP = 6,          /* HIP runtime error, or the device is not gfx950 */
  YOCO_ERR_BAD_VALUE = 7,    /* bad scalar argument (eps, scale, split rows) */
  YOCO_ERR_ALIGNMENT = 8     /* a device pointer breaks the alignment rule below */
} yoco_status;

/* The shared global K^/V^ cache ([Notes] Eq. 2; [Blog] section 7): ONE copy,
 * read by every cross layer.  k and v are each
 * [n_seq][seq_capacity][n_kv_heads][head_dim] in `dtype`, rows possibly
 * padded to row_stride elements (layout below).  len_host[b]
 * (HOST memory) is the number of valid rows of sequence b; the project and
 * append calls advance it when they enqueue their writes.  Lowering
 * len_host[b] truncates a sequence (e.g. to roll back speculative tokens). */
typedef struct yoco_kv_cache {
  void *k;
  void *v;
  int64_t *len_host;    /* HOST [n_seq] */
  int64_t seq_capacity; /* rows per sequence slab, >= 1 */
  int32_t n_seq;        /* 1 .. YOCO_MAX_SEQ */
  int32_t n_kv_heads;   /* >= 1 */
  int32_t head_dim;     /* 64 or 128 */
  int32_t dtype;        /* yoco_dtype of k and v */
  int64_t row_stride;   /* elements from one cache row to the next (see below) */
} yoco_kv_cache;

/* Cache layout.  Element e of KV head g at row r of sequence b sits at
 *   ((b * seq_capacity + r) * row_stride + g * head_dim + e)
 * of k (and of v).  row_stride 0 means dense rows (n_kv_heads * head_dim);
 * otherwise row_stride >= n_kv_heads * head_dim, a multiple of 16 bytes and
 * at most 2^20 elements, and the elements past n_kv_heads * head_dim are
 * never read or written.  The logical cache is [n_seq][capacity][H_kv][d_h]
 * either way; padding only moves each row in memory.
 * yoco_kv_cache_row_stride gives the stride the kernels stream fastest. */

/* Returns YOCO_ABI_VERSION of the built library. */
int yoco_abi_version(void);

/* Text describing the last non-OK status returned on the calling thread
 * ("" if none).  The pointer stays valid until the next call on the thread. */
const char *yoco_last_error(void);

/* Host-only helper: bytes of ONE of the k / v tensors of a cache with these
 * dimensions and row stride (0: dense rows; 2 * this value for the whole
 * cache).  Dense, 131072 rows, 8 KV heads, head dim 128 in bf16 give the
 * pair 2*131072*8*128*2 B = 0.5 GiB, the size [Blog] section 7 prints for the
 * shared cache.  Errors: NULL bytes -> NULL_POINTER; non-positive sizes or a
 * row stride outside the rule above -> BAD_SHAPE; unknown dtype ->
 * BAD_DTYPE. */
yoco_status yoco_kv_cache_bytes(int32_t n_seq, int64_t seq_capacity, int32_t n_kv_heads,
                                int32_t head_dim, int32_t dtype, int64_t row_stride, size_t *bytes);

/* Host-only helper: the row stride (elements) the kernels stream fastest.
 * Rows of 1 KiB or more whose size is a multiple of 512 bytes get 128 bytes
 * of padding: with dense rows every KV head's block sits at the same offset
 * in every row, and under a full decode some of those offsets stream 20-30%
 * slower than others (measured on MI355X); the padding walks each head's
 * block through the offsets from row to row.  Other rows stay dense.  At 8
 * KV heads x 128 in bf16 the rows grow from 2048 to 2176 bytes (6.25%).
 * Errors: NULL row_stride -> NULL_POINTER; non-positive sizes -> BAD_SHAPE;
 * unknown dtype -> BAD_DTYPE. */
yoco_status yoco_kv_cache_row_stride(int32_t n_kv_heads, int32_t head_dim, int32_t dtype,
                                     int64_t *row_stride);

/* Shared K^/V^ projection with one cache write ([Notes] Eq. 2; [Blog]
 * section 7: computed once in the cross-decoder front and written before the
 * early-exit return, so prefill of history tokens needs only this call).
 *
 *   r_n       = sqrt(mean_c m[n][c]^2 + eps)                  (fp32)
 *   K^[n][j]  = sum_c (m[n][c] * gain[c] / r_n) * w_k[c][j]   (fp32 accumulate)
 *   V^[n][j]  = likewise with w_v; one norm is shared by K and V.
 *   column j = g*head_dim + e is stored at cache row (row_start + n), head g,
 *   element e of sequence `seq`.
 *
 * m:     [n][d_model], m_dtype (f32 or bf16).
 * gain:  [d_model] fp32, or NULL for unit gain.
 * w_k, w_v: [d_model][n_kv_heads*head_dim], w_dtype (f32 or bf16).
 * Writes k/v rows row_start .. row_start+n-1 of `seq` in the cache dtype,
 * then sets len_host[seq] = max(len_host[seq], row_start + n).
 * n == 0 is a successful no-op.
 * workspace / workspace_bytes: see "Few-row projections" below (NULL, 0
 * is always valid).
 * Errors: NULL m/w_k/w_v/cache/cache->k/v/len_host -> NULL_POINTER;
 * d_model < 1, bad cache dims, seq outside [0, n_seq) -> BAD_SHAPE;
 * dtype codes -> BAD_DTYPE; row_start < 0 or row_start + n > seq_capacity ->
 * OUT_OF_RANGE; eps < 0 or not finite -> BAD_VALUE; WORKSPACE (given but
 * too small for a call that uses it). */
yoco_status yoco_kv_project(const void *m, int32_t m_dtype, int64_t n, int32_t d_model,
                            const float *gain, float eps, const void *w_k, const void *w_v,
                            int32_t w_dtype, yoco_kv_cache *cache, int32_t seq,
                            int64_t row_start, void *workspace, size_t workspace_bytes,
                            void *stream);

/* Generation-time append ([Notes] section 2.1 and section 2.5: each new token
 * goes through the self-decoder and its K/V row is appended to the shared
 * cache; then every cross layer reads the whole cache).
 * m_new: [n_seq][d_model], one new self-decoder output row per sequence.
 * Projects each row exactly as yoco_kv_project does and writes it at row
 * len_host[b] of sequence b, then increments every len_host[b].
 * Errors as yoco_kv_project; any len_host[b] + 1 > seq_capacity or
 * len_host[b] < 0 -> OUT_OF_RANGE (and nothing is written). */
yoco_status yoco_kv_append(const void *m_new, int32_t m_dtype, int32_t d_model,
                           const float *gain, float eps, const void *w_k, const void *w_v,
                           int32_t w_dtype, yoco_kv_cache *cache, void *workspace,
                           size_t workspace_bytes, void *stream);

/* Per-layer query projection ([Notes] Eq. 3: Q^l = LN(X^l) W_Q^l with the
 * layer's own norm; [Blog] section 7: each cross layer projects only its Q).
 * x: [n][d_model] (f32 or bf16); gain: [d_model] fp32 or NULL;
 * w_q: [d_model][n_q_heads*head_dim]; q_out: [n][n_q_heads][head_dim] in
 * q_dtype (f32 or bf16).  n == 0 is a no-op.
 * Errors: NULL_POINTER, BAD_SHAPE (head_dim not 64/128, counts < 1),
 * BAD_DTYPE, BAD_VALUE (eps), WORKSPACE. */
yoco_status yoco_q_project(const void *x, int32_t x_dtype, int64_t n, int32_t d_model,
                           const float *gain, float eps, const void *w_q, int32_t w_dtype,
                           int32_t n_q_heads, int32_t head_dim, void *q_out, int32_t q_dtype,
                           void *workspace, size_t workspace_bytes, void *stream);

/* Few-row projections (generation: one appended row per sequence, one query
 * row per layer).  With at most 8 input rows the projection is a
 * matrix-vector product bound by reading W once.  Given a workspace, the
 * calls above (and their _rope forms) with 1..32 input rows split W's
 * d_model rows over about 512 workgroups that each stream whole 256-byte
 * row segments, and the last workgroup of each column block adds the
 * partials in a fixed order (bitwise reproducible); without one (NULL, 0)
 * the same rows run on a kernel that needs no workspace and streams W
 * several times slower.  The workspace is device memory of at least the
 * size yoco_project_workspace reports for the call's shapes; its first
 * YOCO_PROJECT_COUNTER_BYTES bytes are arrival counters that must be zero
 * before the first call, and every completed call leaves them zero (so
 * zero-filling it once at allocation is enough).  Calls that share a
 * workspace must not overlap in time (same stream, or synchronized).  Calls
 * whose shapes do not use the path ignore the workspace. */
#define YOCO_PROJECT_COUNTER_BYTES 16384

/* Bytes of workspace a projection of n input rows of width d_model to
 * n_out weights of n_cols columns (K^ and V^: n_out 2, n_cols
 * n_kv_heads*head_dim; Q^: n_out 1, n_cols n_q_heads*head_dim) in w_dtype
 * uses; 0 when those shapes do not use the few-row path (n outside
 * [1, 32], n_cols not a multiple of 128 bf16 / 64 fp32 columns, or more
 * than 128 such column blocks over the n_out weights).
 * Host-only.  Errors: NULL_POINTER; BAD_SHAPE (n < 0, d_model < 1,
 * n_cols < 1, n_out not 1 or 2); BAD_DTYPE. */
yoco_status yoco_project_workspace(int64_t n, int32_t d_model, int32_t n_cols, int32_t n_out,
                                   int32_t w_dtype, size_t *bytes);

/* Rotary position embedding on the projections ([Blog] "NeurIPS'24 | YOCO:
 * 长上下文 LLM 为什么不必每层都存一份 KV Cache?" section 7: the shared projection
 * rotates K^ by position and each cross layer rotates its own Q; V is not
 * rotated.  [Notes] section 4.3, Table 7: the base theta of each training
 * stage -- 640K for 64K tokens, 5M for 256K, 80M for 1M).
 *
 * Pair i (0 <= i < head_dim/2) of every head, elements (2i, 2i+1), turns by
 * pos * rope_theta^(-2i/head_dim) radians:
 *   x'_2i = x_2i cos - x_2i+1 sin,   x'_2i+1 = x_2i sin + x_2i+1 cos.
 * (The pages do not fix which elements pair up; a model trained with the
 * pairs (i, i + head_dim/2) uses these calls after the same permutation of
 * the columns of its W_K and W_Q, which leaves every score unchanged.)
 * The angle is formed in double precision and reduced mod 2*pi there, sine
 * and cosine are taken in single precision, and the rotation is applied to
 * the fp32 projection before its one rounding to the output type.
 * rope_theta must be finite and > 1, else BAD_VALUE; everything else is as
 * in the call without _rope. */

/* yoco_kv_project with K^ row row_start + r rotated at position
 * row_start + r (its cache row); V^ is not rotated. */
yoco_status yoco_kv_project_rope(const void *m, int32_t m_dtype, int64_t n, int32_t d_model,
                                 const float *gain, float eps, const void *w_k, const void *w_v,
                                 int32_t w_dtype, yoco_kv_cache *cache, int32_t seq,
                                 int64_t row_start, double rope_theta, void *workspace,
                                 size_t workspace_bytes, void *stream);

/* yoco_kv_append with the new K^ row of sequence b rotated at position
 * len_host[b] (its cache row). */
yoco_status yoco_kv_append_rope(const void *m_new, int32_t m_dtype, int32_t d_model,
                                const float *gain, float eps, const void *w_k, const void *w_v,
                                int32_t w_dtype, yoco_kv_cache *cache, double rope_theta,
                                void *workspace, size_t workspace_bytes, void *stream);

/* yoco_q_project with query row r rotated at position pos_host[r] (a HOST
 * array of n >= 0 positions, n <= YOCO_MAX_SEQ, else BAD_SHAPE; decode: the
 * query of sequence b sits at len_host[b] - 1) or, when pos_host is NULL, at
 * pos0 + r (prefill: pos0 = q_start).  A negative position is OUT_OF_RANGE. */
yoco_status yoco_q_project_rope(const void *x, int32_t x_dtype, int64_t n, int32_t d_model,
                                const float *gain, float eps, const void *w_q, int32_t w_dtype,
                                int32_t n_q_heads, int32_t head_dim, void *q_out,
                                int32_t q_dtype, const int64_t *pos_host, int64_t pos0,
                                double rope_theta, void *workspace, size_t workspace_bytes,
                                void *stream);

/* Weight preparation, run once per model (not per token): the RMSNorm gain
 * of [Notes] Eq. 2 / Eq. 3 folded into the weights of the projection that
 * follows it.  LN(x) W = (x * gain / r) W = (x / r) (diag(gain) W), so
 *   w_out[c][j] = RNE_bf16(fp32(w[c][j]) * gain[c])   (fp32 product)
 * given to yoco_kv_project / yoco_kv_append / yoco_q_project (and their
 * _rope forms) with a NULL gain computes LN(x) W with the gain rounded into
 * each weight once, instead of applied to every activation.  Prompt-sized
 * calls then take the unit-gain matrix-core path (one bf16 product per
 * fragment; an fp32 gain on the activations takes two, x*gain entering as a
 * bf16 hi + lo pair); the price is one bf16 rounding of gain*w per weight.
 * w: [d_model][n_cols] in w_dtype (f32 or bf16); gain: [d_model] fp32;
 * w_out: [d_model][n_cols] bf16, written.  w_out may be w itself when
 * w_dtype is bf16; any other overlap of the two is BAD_VALUE.
 * Errors: NULL w/gain/w_out -> NULL_POINTER; d_model < 1 or n_cols < 1 ->
 * BAD_SHAPE; dtype code -> BAD_DTYPE; ALIGNMENT; BAD_VALUE; HIP. */
yoco_status yoco_fold_norm_gain(const void *w, int32_t w_dtype, const float *gain, int32_t d_model,
                                int32_t n_cols, void *w_out, void *stream);

/* Host-only helper: the softmax scale 1/sqrt(head_dim) of [Blog] section 2
 * (o_t = softmax(q_t K^T / sqrt(d_h)) V), the scale the attention calls below
 * use in the pages' method; the calls take the scale explicitly.  Errors:
 * NULL scale -> NULL_POINTER; head_dim < 1 -> BAD_SHAPE. */
yoco_status yoco_default_softmax_scale(int32_t head_dim, float *scale);

/* Causal cross-attention over the shared cache for a block of query rows
 * (prefill / training forward: [Notes] Eq. 3 with the causal mask; [Blog]
 * section 2 formula; [Notes] Table 2: the quadratic term the early exit
 * skips at inference but training still pays).
 *
 * Query row i sits at absolute position p = q_start + i and reads cache rows
 * 0..p of sequence `seq` (inclusive).  For head h with KV head g = h / G:
 *   x_j = softmax_scale * <q[i][h], K^[j][g]>,  j = 0..p
 *   o[i][h] = sum_j softmax(x)_j V^[j][g];   lse[i][h] = ln sum_j exp(x_j)
 * q:   [t][n_q_heads][head_dim] in the cache dtype.
 * o:   [t][n_q_heads][head_dim] in o_dtype (f32 or bf16).
 * lse: [t][n_q_heads] fp32, or NULL.
 * No W_O and no residual: the output is the concatenated heads.
 * The bf16 path runs both contractions on bf16 MFMA with fp32 accumulation
 * (probabilities are rounded to bf16 for the second); the f32 path uses
 * fp32 arithmetic throughout.  t == 0 is a no-op.
 * Errors: NULL_POINTER; BAD_SHAPE (head/group/head_dim, seq); BAD_DTYPE
 * (q dtype != cache dtype, o dtype); OUT_OF_RANGE (q_start < 0, t < 0,
 * q_start + t > len_host[seq]); BAD_VALUE (scale not finite or <= 0). */
yoco_status yoco_cross_attn_prefill(const void *q, int32_t q_dtype, int64_t q_start, int64_t t,
                                    int32_t n_q_heads, const yoco_kv_cache *cache, int32_t seq,
                                    float softmax_scale, void *o, int32_t o_dtype, float *lse,
                                    void *stream);

/* Bytes of device workspace yoco_cross_attn_prefill_bwd needs for t query
 * rows of n_q_heads heads: 2 * t * n_q_heads floats.  Errors: NULL_POINTER,
 * BAD_SHAPE (t < 0, n_q_heads <= 0). */
yoco_status yoco_cross_attn_prefill_bwd_workspace(int64_t t, int32_t n_q_heads, size_t *bytes);

/* Backward of yoco_cross_attn_prefill for one cross layer (training): the
 * gradient of [Notes] Eq. 3 with respect to the query and the shared K^/V^.
 * [Deep] s.2.2: all cross layers read the same K^/V^, so their gradients
 * sum over the layers; this call ADDS its layer's share to d_k and d_v
 * (clear them before the first layer).
 *
 * For query row i at position p = q_start + i, head h, KV head g = h / G,
 * with P_j = exp(softmax_scale <q, k_j> - lse) over rows j = 0..p and the
 * upstream gradient dO of o:
 *   dP_j = <dO, v_j>,  D = <dO, o>,  dS_j = P_j (dP_j - D)
 *   d_q[i][h] = softmax_scale * sum_j dS_j k_j
 *   d_k[j][g] += softmax_scale * dS_j q,   d_v[j][g] += P_j dO.
 * q, d_o: [t][n_q_heads][head_dim] bf16; o: the forward's output, o_dtype
 * (f32 or bf16); lse: [t][n_q_heads] fp32, the forward's lse (natural log);
 * the cache must be bf16 and hold rows 0..q_start+t-1 of `seq`.
 * d_q: [t][n_q_heads][head_dim] fp32, written.  d_k, d_v: [q_start+t][H_kv]
 * [head_dim] fp32 (device), added to.  workspace: device memory of at least
 * yoco_cross_attn_prefill_bwd_workspace bytes (per-row statistics; its
 * contents on entry do not matter).
 * P and dS are rounded to bf16 for the MFMA products, with fp32
 * accumulation.  The result is bitwise reproducible (no atomics).  Calls on
 * one stream that share d_k/d_v run in order; t == 0 is a no-op.
 * Errors: NULL_POINTER; BAD_SHAPE (heads, seq); BAD_DTYPE (cache not bf16,
 * o dtype); OUT_OF_RANGE (q_start < 0, t < 0, q_start + t > len_host[seq]);
 * BAD_VALUE (scale); WORKSPACE (too small). */
yoco_status yoco_cross_attn_prefill_bwd(const void *q, const void *o, int32_t o_dtype, const void *d_o,
                                        const float *lse, int64_t q_start, int64_t t, int32_t n_q_heads,
                                        const yoco_kv_cache *cache, int32_t seq, float softmax_scale,
                                        float *d_q, float *d_k, float *d_v, void *workspace,
                                        size_t workspace_bytes, void *stream);

/* Bytes of device workspace yoco_kv_project_bwd (n_out = 2, n_cols =
 * n_kv_heads * head_dim) or yoco_q_project_bwd (n_out = 1, n_cols =
 * n_q_heads * head_dim) needs for n input rows of width d_model.  The size
 * depends on the shapes only.  Errors: NULL_POINTER; BAD_SHAPE (n < 0,
 * d_model outside [1, 4096], n_cols < 1, n_out not 1 or 2). */
yoco_status yoco_project_bwd_workspace(int64_t n, int32_t d_model, int32_t n_cols, int32_t n_out,
                                       size_t *bytes);

/* Backward of yoco_kv_project (training): the gradient of [Notes] Eq. 2,
 * K^ = RMSNorm(M) W_K and V^ = RMSNorm(M) W_V with one norm shared by both.
 * With y = m g / r, r = sqrt(mean_c m_c^2 + eps) per row, and the upstream
 * gradients dz_k, dz_v of the row's K^ and V^ columns (for a shared cache:
 * the sums over the cross layers that yoco_cross_attn_prefill_bwd adds up):
 *   dy[c]     = sum_j dz_k[j] W_K[c][j] + sum_j dz_v[j] W_V[c][j]
 *   d_m[c]    = g[c] dy[c] / r - m[c] / (d_model r^3) sum_c' g[c'] dy[c'] m[c']
 *   d_w_k    += sum over rows of y^T dz_k   (likewise d_w_v)
 *   d_gain[c] += sum over rows of dy[c] m[c] / r
 * m: [n][d_model], m_dtype; gain: [d_model] fp32 or NULL (unit gain; then
 * d_gain may still be requested); w_k, w_v: [d_model][n_kv_heads*head_dim],
 * w_dtype; dz_k, dz_v: [n][n_kv_heads*head_dim] in dz_dtype (f32 or bf16;
 * the [rows][H_kv][d_h] layout of the cache and of the attention backward's
 * d_k, d_v).  d_m: [n][d_model] fp32, written.  d_w_k, d_w_v:
 * [d_model][n_kv_heads*head_dim] fp32 and d_gain: [d_model] fp32 (or NULL to
 * skip it) are ADDED to, so calls over several row blocks accumulate.
 * With bf16 m and w, d_model % 256 == 0 and n_kv_heads*head_dim % 256 == 0
 * the two products run on bf16 MFMA with fp32 accumulation, y and fp32 dz
 * rounded to bf16 first; otherwise in fp32 arithmetic.  Results are bitwise
 * reproducible (fixed reduction orders, no atomics).  The rows must not
 * carry a rotary embedding (for a *_rope forward the caller passes dz_k
 * turned back to the unrotated frame).  n == 0 is a no-op.
 * workspace: device memory of at least yoco_project_bwd_workspace bytes
 * (contents on entry do not matter).
 * Errors: NULL_POINTER; BAD_SHAPE (n < 0, d_model outside [1, 4096],
 * n_kv_heads outside [1, 64], head_dim); BAD_DTYPE; BAD_VALUE (eps);
 * WORKSPACE (too small). */
yoco_status yoco_kv_project_bwd(const void *m, int32_t m_dtype, int64_t n, int32_t d_model,
                                const float *gain, float eps, const void *w_k, const void *w_v,
                                int32_t w_dtype, int32_t n_kv_heads, int32_t head_dim,
                                const void *dz_k, const void *dz_v, int32_t dz_dtype, float *d_m,
                                float *d_w_k, float *d_w_v, float *d_gain, void *workspace,
                                size_t workspace_bytes, void *stream);

/* Backward of yoco_q_project ([Notes] Eq. 3, Q^l = RMSNorm_l(X^l) W_Q^l):
 * the same formulas with one weight.  x: [n][d_model]; w_q:
 * [d_model][n_q_heads*head_dim]; dz_q: [n][n_q_heads][head_dim] (the
 * attention backward's d_q); d_x written, d_w_q and d_gain added to.
 * Errors as yoco_kv_project_bwd; n_q_heads outside [1, 4096] -> BAD_SHAPE. */
yoco_status yoco_q_project_bwd(const void *x, int32_t x_dtype, int64_t n, int32_t d_model,
                               const float *gain, float eps, const void *w_q, int32_t w_dtype,
                               int32_t n_q_heads, int32_t head_dim, const void *dz_q,
                               int32_t dz_dtype, float *d_x, float *d_w_q, float *d_gain,
                               void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of device workspace yoco_cross_attn_decode needs for this cache,
 * query head count and split size, valid for any len_host up to
 * seq_capacity.  rows_per_split: 0 selects the library's split size;
 * otherwise a positive multiple of 256.  Errors: NULL_POINTER, BAD_SHAPE,
 * BAD_DTYPE, BAD_VALUE (rows_per_split). */
yoco_status yoco_cross_attn_decode_workspace(const yoco_kv_cache *cache, int32_t n_q_heads,
                                             int64_t rows_per_split, size_t *bytes);

/* One generation step of one cross layer over the shared cache: split-N
 * flash decoding ([Notes] section 2.5 and [Blog] section 7: every cross layer
 * re-reads the whole global cache; sharing storage does not merge the
 * layers' queries, so each layer is its own call).
 *
 * For every sequence b (with len_host[b] >= 1) the single query row sits at
 * position len_host[b] - 1 and reads rows 0..len_host[b]-1 (the appended
 * row included).  q: [n_seq][n_q_heads][head_dim] in the cache dtype;
 * o: [n_seq][n_q_heads][head_dim] fp32; lse: [n_seq][n_q_heads] fp32 or NULL.
 *
 * The rows of each (sequence, KV head) are cut into splits of
 * rows_per_split rows (0 = library choice from the current lengths); one
 * workgroup streams one split with 128-bit loads, all G query heads of the
 * group sharing each row it reads, and keeps a running (max, sum, weighted
 * V) per head; the last workgroup of each (sequence, KV head) to finish
 * merges the splits in a fixed order, so results are bitwise reproducible
 * for a fixed split size.
 *
 * workspace: device memory of at least the size yoco_cross_attn_decode_workspace
 * reports for the same cache, n_q_heads and rows_per_split.  Its first
 * YOCO_DECODE_COUNTER_BYTES bytes are arrival counters that must be zero
 * before the first call; every completed call leaves them zero again, so
 * zero-filling a workspace once at allocation is enough.  Calls that share a
 * workspace must not overlap in time (same stream, or synchronized).
 * Errors: NULL_POINTER; BAD_SHAPE; BAD_DTYPE (q dtype != cache dtype);
 * OUT_OF_RANGE (some len_host[b] < 1 or > seq_capacity); WORKSPACE (too
 * small); BAD_VALUE (scale, rows_per_split). */
#define YOCO_DECODE_COUNTER_BYTES (YOCO_MAX_SEQ * 64 * 4)
yoco_status yoco_cross_attn_decode(const void *q, int32_t q_dtype, int32_t n_q_heads,
                                   const yoco_kv_cache *cache, float softmax_scale, float *o,
                                   float *lse, void *workspace, size_t workspace_bytes,
                                   int64_t rows_per_split, void *stream);

/* yoco_cross_attn_decode for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  It takes no workspace: the counters and partials live in a
 * library array of YOCO_DECODE_NOALLOC_SCRATCH_BYTES in device memory (laid
 * out as the workspace above), one per device, which each device holds until
 * the process ends.  The call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine); the caller still passes q, o and lse.  The
 * first call on a device looks the array up and clears its counters with a
 * kernel on `stream`; every completed call leaves them zero.  Every call on
 * a device shares that device's array, so calls that overlap in time on one
 * device (different streams, or threads without synchronization) race.
 * Results are the bits yoco_cross_attn_decode gives for the same cache,
 * query, scale and rows_per_split.  Errors as yoco_cross_attn_decode, and
 * WORKSPACE when this call's split plan needs more than the array holds:
 * it has room for 15,763 partial rows of head_dim 128 (one per split, KV
 * head and query head), e.g. 656 splits at 8 KV heads x 3 query heads; the
 * library's split size (rows_per_split 0) plans at most
 * (CUs x resident workgroups) / n_kv_heads + n_seq splits, and a caller's
 * larger rows_per_split needs fewer. */
#define YOCO_DECODE_NOALLOC_SCRATCH_BYTES (8 * 1024 * 1024)
yoco_status yoco_cross_attn_decode_noalloc(const void *q, int32_t q_dtype, int32_t n_q_heads,
                                           const yoco_kv_cache *cache, float softmax_scale,
                                           float *o, float *lse, int64_t rows_per_split,
                                           void *stream);

/* ---- Gated retention (gRet), the self-decoder's token mixer -------------
 * [Notes] "YOCO：You Only Cache Once 中文精读笔记" section 2.2, Eq. 4-5 and
 * section 2.3 (chunkwise form); [Deep] section 3.1.  The self-decoder output
 * M that yoco_kv_project turns into the shared cache comes from layers built
 * around this mixer.  Per head, with q_t, k_t, v_t of length head_dim and
 * the head-wise gate gamma_t = sigmoid(g_t)^(1/tau):
 *   S_t = gamma_t S_{t-1} + k_t^T v_t,   o_t = q_t S_t             (Eq. 5)
 * equal to O = (Q K^T (.) D) V, D[t][m] = prod_{i=m+1..t} gamma_i (Eq. 4).
 * q and k enter as given (a position rotation, if any, is applied by the
 * caller); the output is before the per-head normalisation, gate and W_O of
 * the full layer.  States are fp32 [heads][head_dim][head_dim] per sequence
 * (row index: key element, column: value element), outputs fp32.
 * tau must be finite and > 0 (BAD_VALUE otherwise). */

/* Bytes of device workspace yoco_gret_prefill needs: nonzero only for the
 * chunkwise matrix-core path (bf16, head_dim 128).  Errors: NULL_POINTER,
 * BAD_SHAPE, BAD_DTYPE. */
yoco_status yoco_gret_prefill_workspace(int64_t n, int32_t n_heads, int32_t head_dim, int32_t dtype,
                                        size_t *bytes);

/* A block of n positions of one sequence (prefill, or the training forward
 * of the mixer).  q, k, v: [n][n_heads][head_dim] in dtype; gate_logits:
 * [n][n_heads] fp32 (g = x W_gamma); state_in: [n_heads][D][D] fp32, the
 * state before the block, or NULL for a fresh sequence; o: [n][n_heads][D]
 * fp32, written; state_out: [n_heads][D][D] fp32 (the state after the
 * block, which yoco_gret_decode continues from), or NULL.  state_in and
 * state_out must not overlap o.  bf16 with head_dim 128 runs the chunkwise
 * form on MFMA (chunks of 128 positions; q.k scores and the carried state
 * rounded to bf16 for the products, fp32 accumulation); other inputs run the
 * recurrent form in fp32 (one workgroup per head, sequential over the
 * positions).  n == 0 is a no-op.  Errors: NULL_POINTER; BAD_SHAPE; BAD_DTYPE;
 * BAD_VALUE (tau); WORKSPACE. */
yoco_status yoco_gret_prefill(const void *q, const void *k, const void *v, int32_t dtype,
                              const float *gate_logits, float tau, int64_t n, int32_t n_heads,
                              int32_t head_dim, const float *state_in, float *o, float *state_out,
                              void *workspace, size_t workspace_bytes, void *stream);

/* One generation step of every sequence: q, k, v: [n_seq][n_heads][D] in
 * dtype, gate_logits: [n_seq][n_heads] fp32; state: [n_seq][n_heads][D][D]
 * fp32, updated in place (S <- gamma S + k^T v); o: [n_seq][n_heads][D] fp32
 * = q times the updated state.  n_seq == 0 is a no-op.  Errors as
 * yoco_gret_prefill (state NULL -> NULL_POINTER). */
yoco_status yoco_gret_decode(const void *q, const void *k, const void *v, int32_t dtype,
                             const float *gate_logits, float tau, int32_t n_seq, int32_t n_heads,
                             int32_t head_dim, float *state, float *o, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* YOCO_H */
