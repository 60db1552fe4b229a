// Internal interface between the host API (api.cpp) and the kernel files.
// Launchers validate nothing: api.cpp has checked every argument before any
// of these is called.  Each launcher returns the hipError_t of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/yoco.h"
#include "decode_args.h"

namespace yoco {


// ---------------------------------------------------------------------------
// Fused RMSNorm + projection (shared K/V, per-layer Q, append).
// Output row r of the input goes to destination row dst_row(r):
//   contiguous: dst_row_base + r;   indexed: dst_rows[r] (r < YOCO_MAX_SEQ).
// Destination element (row, col) is out[p][row * out_stride + col] for
// weight p (out_stride >= ncols: padded cache rows).
// ---------------------------------------------------------------------------
struct ProjArgs {
  const void *x;
  const float *gain;         // may be null (unit gain)
  const void *w[2];          // [d][ncols] each; w[1] unused when n_out == 1
  void *out[2];
  int64_t n;                 // input rows
  int64_t dst_row_base;      // contiguous mode
  int32_t d;                 // d_model
  int32_t ncols;             // columns per weight (H*d_h)
  int64_t out_stride;        // elements between destination rows
  int32_t n_out;             // 1 (Q) or 2 (K and V)
  int32_t indexed;           // 1: use dst_rows
  float eps;
  // Rotary position embedding of output rope_out (-1: none), pairs
  // (2i, 2i+1) of each head_dim-wide head.  Input row r sits at position
  //   pos_indexed ? dst_rows[r] - r * pos_stride : pos_base + r.
  double rope_log2_theta = 0.0;
  int32_t rope_out = -1;
  int32_t head_dim = 0;
  int32_t pos_indexed;
  int64_t pos_base;
  int64_t pos_stride;
  int64_t dst_rows[YOCO_MAX_SEQ];
};

__device__ __forceinline__ int64_t proj_row_pos(const ProjArgs &a, int64_t r) {
  return a.pos_indexed ? a.dst_rows[r] - r * a.pos_stride : a.pos_base + r;
}

hipError_t launch_project(const ProjArgs &a, int x_dt, int w_dt, int o_dt, hipStream_t s);

// w_out[c][j] = bf16(w[c][j] * gain[c]) over d x n_cols (fold_gain.hip).
hipError_t launch_fold_gain(const void *w, int w_dt, const float *gain, int32_t d, int32_t n_cols, void *out,
                            hipStream_t s);

// Few-row projection split over W's reduction rows (project_rows.hip).  The
// caller's workspace holds kProjRowsCounterBytes of arrival counters (zero
// between calls) and then the partials of one launch of up to 8 input rows.
constexpr int kProjRowsCounterBytes = YOCO_PROJECT_COUNTER_BYTES;
constexpr int kProjRowsCounterStride = 32;  // words between counters: one 128-byte line each
constexpr int kProjRowsMaxBlocks = kProjRowsCounterBytes / (4 * kProjRowsCounterStride);  // column blocks
constexpr int kProjRowsMaxRows = 32;                           // input rows per call on this path
struct ProjRowsPlan {
  int32_t n_cb;          // column blocks over all outputs
  int32_t splits;        // S: splits of W's d rows
  int32_t split_rows;    // R: rows per split (multiple of 16, <= 256)
  int32_t block_cols;    // CB: 128 (bf16 W) or 64 (fp32 W)
  int64_t part_floats;   // partial storage for one launch
};
// Plan for these shapes; false when the path does not apply (columns not a
// multiple of the block width, or more blocks than counters).
bool project_rows_plan(int32_t d, int32_t ncols, int32_t n_out, int w_dt, ProjRowsPlan *p);
size_t project_rows_workspace_bytes(const ProjRowsPlan &p);
hipError_t launch_project_rows(const ProjArgs &a, const ProjRowsPlan &p, int x_dt, int w_dt, int o_dt,
                               void *workspace, hipStream_t s);
// Matrix-core path for prompt-sized bf16 projections (d_model % 64 == 0,
// columns % 256 == 0, contiguous destination rows).
bool project_mfma_applies(const ProjArgs &a, int x_dt, int w_dt, int o_dt);
hipError_t launch_project_mfma(const ProjArgs &a, hipStream_t s);

// ---------------------------------------------------------------------------
// Causal prefill over the shared cache.
// ---------------------------------------------------------------------------
struct PrefillArgs {
  const void *q;      // [t][n_q_heads][head_dim]
  const void *k;      // sequence slab base: [capacity][H_kv][d_h]
  const void *v;
  void *o;            // [t][n_q_heads][head_dim]
  float *lse;         // [t][n_q_heads] or null
  int64_t q_start;
  int64_t t;
  int64_t kv_len;     // rows of the slab that hold data (len_host[seq])
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t kv_row_stride;  // elements between cache rows
  float scale_log2;
  int32_t o_bf16;
};

hipError_t launch_prefill(const PrefillArgs &a, int dtype, int head_dim, hipStream_t s);

// Backward of the prefill (bf16 operands, fp32 gradients).
struct BwdArgs {
  const void *q;      // [t][n_q_heads][head_dim] bf16
  const void *o;      // [t][n_q_heads][head_dim] forward output, fp32 or bf16
  const void *d_o;    // [t][n_q_heads][head_dim] bf16
  const float *lse;   // [t][n_q_heads] natural log, from the forward
  const void *k;      // sequence slab base: [capacity][H_kv][d_h] bf16
  const void *v;
  float *d_q;         // [t][n_q_heads][head_dim], written
  float *d_k;         // [kv_len][H_kv][d_h] (dense rows), added to
  float *d_v;
  float *ws_d;        // [n_q_heads][t] workspace: <dO, o>
  float *ws_lse2;     // [n_q_heads][t] workspace: lse * log2(e)
  int64_t q_start;
  int64_t t;
  int64_t kv_len;     // q_start + t: the cache rows the block's rows see
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t kv_row_stride;  // elements between cache rows (k, v)
  float scale;
  float scale_log2;
  int32_t o_bf16;
};

hipError_t launch_prefill_bwd(const BwdArgs &a, int head_dim, hipStream_t s);

// Backward of the fused RMSNorm + projection (training).  x, gain, W_p and
// dz_p as in the forward; dx written, dW_p and dgain added to.  Workspace
// regions (device): inv_r [n]; matrix-core path: ybf [n][d], dzb_p [n][ncols]
// (or the caller's bf16 dz), dw_part [splits][n_out][d][ncols]; dgain_part
// [ceil(n / kProjBwdFinRows)][d].
constexpr int kProjBwdFinRows = 64;     // input rows per block of the dx kernel
constexpr int kProjBwdMaxD = 4096;      // d_model bound: the dx kernel keeps 4 x d floats in LDS (64 KiB)
struct ProjBwdArgs {
  const void *x;             // [n][d]
  const float *gain;         // [d] or null
  const void *w[2];          // [d][ncols]
  const void *dz[2];         // [n][ncols]
  float *dx;                 // [n][d], written
  float *dw[2];              // [d][ncols], added to
  float *dgain;              // [d], added to, or null
  float *inv_r;              // workspace [n]
  uint16_t *ybf;             // workspace [n][d] bf16 (matrix-core path)
  uint16_t *dzb[2];          // bf16 dz (matrix-core path)
  float *dw_part;            // workspace (matrix-core path)
  float *dgain_part;         // workspace
  int64_t n;
  int32_t d;
  int32_t ncols;
  int32_t n_out;
  int32_t x_bf16, w_bf16, dz_bf16;
  int32_t mfma;
  int32_t splits;            // matrix-core dW: row splits
  int32_t split_rows;        // rows per split (multiple of 64)
  float eps;
};

bool project_bwd_mfma_applies(int64_t n, int32_t d, int32_t ncols, int x_dt, int w_dt);
void project_bwd_split_plan(int64_t n, int32_t d, int32_t ncols, int32_t n_out, int32_t *splits, int32_t *rows);
hipError_t launch_project_bwd(const ProjBwdArgs &a, hipStream_t s);

// Gated retention (self-decoder token mixer).  Token t of sequence b is
// element (b * n_tokens + t) of q, k, v ([..][heads][D]), gate ([..][heads])
// and o; one of n_seq and n_tokens is 1.  States are [n_seq][heads][D][D]
// fp32 (state_in may be null: zero; state_out may be null; they may alias).
// Chunkwise path workspace: lcum [n_tokens][heads], gdec [groups][heads],
// tg and sg [groups][heads][D][D], all fp32.
struct GretArgs {
  const void *q;
  const void *k;
  const void *v;
  const float *gate;
  const float *state_in;
  float *state_out;
  float *o;
  float *lcum;      // [n][heads] inclusive cumulative log gates inside each chunk
  float *gdec;      // [groups][heads] log decay over each group
  float *tg;        // [groups][heads][D][D] group-local state after each group (transposed)
  float *sg;        // [groups][heads][D][D] state entering each group (transposed)
  int64_t n_tokens;
  int32_t heads;
  float inv_tau;
};

bool gret_chunked_applies(int dtype, int head_dim);
int64_t gret_n_chunks(int64_t n);
int64_t gret_n_groups(int64_t n);
hipError_t launch_gret_recurrent(const GretArgs &a, int dtype, int head_dim, int n_seq, hipStream_t s);
hipError_t launch_gret_chunked(const GretArgs &a, hipStream_t s);

}  // namespace yoco
