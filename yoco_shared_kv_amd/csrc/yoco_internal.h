// Internal interface between the host API (api.cpp) and the kernel files.
// Launchers validate nothing: api.cpp has checked every argument before any
// of these is called.  Each launcher returns the hipError_t of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/yoco.h"

namespace yoco {

constexpr int kMaxKvHeads = 64;        // counters are laid out [YOCO_MAX_SEQ][kMaxKvHeads]
constexpr int kDecodeSplitQuantum = 256;   // caller-chosen split sizes are multiples of this
constexpr int kDecodeAutoQuantum = 64;     // library-chosen split sizes are multiples of this
constexpr int kDecodeMinSplitRows = 256;   // library-chosen split sizes are at least this
constexpr int kDecodeMaxTargetBlocks = 4096;  // cap on the library's workgroup target

// ---------------------------------------------------------------------------
// Fused RMSNorm + projection (shared K/V, per-layer Q, append).
// Output row r of the input goes to destination row dst_row(r):
//   contiguous: dst_row_base + r;   indexed: dst_rows[r] (r < YOCO_MAX_SEQ).
// Destination element (row, col) is out[p][row * ncols + col] for weight p.
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
  int32_t n_out;             // 1 (Q) or 2 (K and V)
  int32_t indexed;           // 1: use dst_rows
  float eps;
  int64_t dst_rows[YOCO_MAX_SEQ];
};

hipError_t launch_project(const ProjArgs &a, int x_dt, int w_dt, int o_dt, hipStream_t s);

// ---------------------------------------------------------------------------
// Split-N decode with last-arriver merge.
// ---------------------------------------------------------------------------
struct DecodeArgs {
  const void *k;
  const void *v;
  const void *q;          // [n_seq][n_q_heads][head_dim]
  float *o;               // [n_seq][n_q_heads][head_dim]
  float *lse;             // [n_seq][n_q_heads] or null
  unsigned int *counters; // [YOCO_MAX_SEQ][kMaxKvHeads]
  float *part_ml;         // [total_splits][n_kv_heads][G][2]
  float *part_acc;        // [total_splits][n_kv_heads][G][head_dim]
  int64_t seq_stride;     // elements between sequence slabs (capacity*H_kv*d_h)
  int32_t n_seq;
  int32_t n_kv_heads;
  int32_t n_q_heads;
  int32_t split_rows;
  float scale_log2;       // softmax_scale * log2(e)
  int32_t total_splits;
  int32_t len[YOCO_MAX_SEQ];
  int32_t split_begin[YOCO_MAX_SEQ + 1];  // prefix sums of splits per sequence
};

hipError_t launch_decode(const DecodeArgs &a, int dtype, int head_dim, int group, hipStream_t s);
// Resident workgroups per CU of the decode kernel for this shape (0 on error).
int decode_blocks_per_cu(int dtype, int head_dim, int group);

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
  float scale_log2;
  int32_t o_bf16;
};

hipError_t launch_prefill(const PrefillArgs &a, int dtype, int head_dim, hipStream_t s);

}  // namespace yoco
