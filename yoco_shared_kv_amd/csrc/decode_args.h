// Arguments and constants of the split-N decode kernel (its own header, so
// the decode kernel's sources are exactly decode.hip, decode_kernel.h, this
// file and device_common.h, plus the public constants of yoco.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/yoco.h"

namespace yoco {

constexpr int kMaxKvHeads = 64;        // counters are laid out [kMaxKvHeads][YOCO_MAX_SEQ]
constexpr int kDecodeSplitQuantum = 256;   // caller-chosen split sizes are multiples of this
constexpr int kDecodeAutoQuantum = 64;     // library-chosen split sizes are multiples of this
constexpr int kDecodeMinSplitRows = 256;   // library-chosen split sizes are at least this
constexpr int kDecodeMaxTargetBlocks = 4096;  // cap on the library's workgroup target

// ---------------------------------------------------------------------------
// Split-N decode with last-arriver merge.
// ---------------------------------------------------------------------------
struct DecodeArgs {
  const void *k;
  const void *v;
  const void *q;          // [n_seq][n_q_heads][head_dim]
  float *o;               // [n_seq][n_q_heads][head_dim]
  float *lse;             // [n_seq][n_q_heads] or null
  unsigned int *counters; // [kMaxKvHeads][YOCO_MAX_SEQ]
  float *part_ml;         // [total_splits][n_kv_heads][G][2]
  float *part_acc;        // [total_splits][n_kv_heads][G][head_dim]
  int64_t seq_stride;     // elements between sequence slabs (capacity * row_stride)
  int64_t row_stride;     // elements between cache rows (>= H_kv * d_h)
  int32_t n_seq;
  int32_t n_kv_heads;
  int32_t n_q_heads;
  float scale_log2;       // softmax_scale * log2(e)
  int32_t total_splits;
  int32_t len[YOCO_MAX_SEQ];
  int32_t split_begin[YOCO_MAX_SEQ + 1];  // prefix sums of splits per sequence
  int32_t split_rows[YOCO_MAX_SEQ];       // rows per split of each sequence (its last split may be shorter)
};

hipError_t launch_decode(const DecodeArgs &a, int dtype, int head_dim, int group, hipStream_t s);
// Device address of this device's no-allocation decode scratch
// (YOCO_DECODE_NOALLOC_SCRATCH_BYTES), set up on the first call on a device.
hipError_t decode_noalloc_scratch(void **ptr, hipStream_t s);
// Resident workgroups per CU of the decode kernel for this shape (0 on error).
int decode_blocks_per_cu(int dtype, int head_dim, int group);

}  // namespace yoco
