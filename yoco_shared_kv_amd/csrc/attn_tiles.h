// Tile helpers shared by the attention kernels on MFMA (forward prefill and
// backward): fragment types, the XOR swizzle of head rows in LDS and the
// 16-byte buffer loads that stage 64-row tiles of a head into LDS.
#pragma once

#include <type_traits>

#include "device_common.h"
#include "yoco_internal.h"

namespace yoco {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float floatx2_t __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef short shortx4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4_t lds_shortx4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

namespace pf {
constexpr int kWaves = 8;
constexpr int kRowsPerWave = 32;
constexpr int kBlockRows = kWaves * kRowsPerWave;  // 256 query rows
constexpr int kKeyTile = 64;
constexpr int kThreads = kWaves * 64;
constexpr int kXcds = 8;
constexpr float kSumLimit = 1.152921504606846976e18f;  // 2^60: a row sum at or above it is recomputed
}  // namespace pf

union Frag8 {
  bf16x8_t v;
  uint4 u;
  uint32_t w[4];
  shortx4_t s4[2];
};

// Two fp32 values -> packed bf16 pair (round to nearest even, v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  const floatx2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

__device__ __forceinline__ float dot2_bf16_f32(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

template <int DH>
struct PrefillShape {
  static constexpr int kChunks = DH / 8;                    // 16-byte chunks per row
  static constexpr int kRowBytes = DH * 2;
  static constexpr int kTileBytes = pf::kKeyTile * kRowBytes;
  static constexpr int kRowsPerLoad = 64 / kChunks;         // rows per wave-wide 1 KiB load
  static constexpr int kLoadsPerTile = pf::kKeyTile / kRowsPerLoad;    // per K (or V) tile
  static constexpr int KSTEPS = DH / 16;                    // S^T k-steps over head_dim
  static constexpr int DSUB = DH / 32;                      // O^T 32-row tiles over head_dim
};

// Row-dependent XOR applied to the 16-byte chunk index of a tile row.
// Mode 0: row % chunks.  Mode 1 (head_dim 128): bits (r1 r0 r2) in the low
// three bits plus r3, so that 8 consecutive rows hit 8 distinct chunk slots
// mod 8 (16-byte K reads) and rows 4k..4k+3 with chunks c, c^1 hit 8
// distinct slots mod 8 (the 8-byte transposed V reads of one 16-lane group).
// Mode 2 (head_dim 128): (r1 r0) in bits 3..2 and (r3 r2) in bits 1..0.
template <int DH, int SWZ>
__device__ __forceinline__ int row_xor(int row) {
  using S = PrefillShape<DH>;
  if constexpr (SWZ == 1 && S::kChunks == 16) {
    return ((row & 3) << 1) | ((row >> 2) & 1) | (row & 8);
  } else if constexpr (SWZ == 2 && S::kChunks == 16) {
    return ((row & 3) << 2) | ((row >> 2) & 3);
  } else {
    return row & (S::kChunks - 1);
  }
}

// LDS byte offset of element `dim` (multiple of 4 for 8-byte reads, of 8 for
// 16-byte reads) of tile row `row`, with the XOR-swizzled chunk layout.
template <int DH, int SWZ>
__device__ __forceinline__ int swz(int row, int dim) {
  using S = PrefillShape<DH>;
  const int chunk = dim >> 3;
  const int slot = chunk ^ row_xor<DH, SWZ>(row);
  return row * S::kRowBytes + slot * 16 + (dim & 7) * 2;
}

// Per-lane byte offsets (within a tile) of this wave's direct-to-LDS loads:
// load i of the wave fills 1 KiB block blk = wave * kLoadsPerWave + i, lane
// L writes LDS bytes blk*1024 + L*16 = (row, slot) and so reads global chunk
// slot ^ row_xor(row) of that row.
// NW: waves of the workgroup that share the staging of a tile.
template <int DH, int SWZ, int NW = pf::kWaves>
struct StageOffsets {
  using S = PrefillShape<DH>;
  static constexpr int kLoadsPerWave = S::kLoadsPerTile / NW;
  uint32_t boff[kLoadsPerWave];  // (row * row_stride + chunk * 8) * 2
  __device__ __forceinline__ void init(int wave, int lane, int row_stride) {
#pragma unroll
    for (int i = 0; i < kLoadsPerWave; ++i) {
      const int row = (wave * kLoadsPerWave + i) * S::kRowsPerLoad + lane / S::kChunks;
      const int chunk = (lane % S::kChunks) ^ row_xor<DH, SWZ>(row);
      boff[i] = static_cast<uint32_t>(row * row_stride + chunk * 8) * 2u;
    }
  }
};

// Issue this wave's share of the direct-to-LDS buffer loads of one 64-row K
// or V tile (rows key0 .. key0+63 of one KV head).  The buffer descriptor
// covers only the rows that hold data (< kv_len): the hardware range check
// turns the bytes of rows past it into zeros in LDS, so no lane reads
// outside the cache.  `wave` is wave-uniform (an SGPR), so the LDS address
// in M0 is scalar arithmetic.
constexpr int32_t kBufferFlags = 0x00020000;  // raw buffer, 32-bit data format
template <int DH, int SWZ, int NW>
__device__ __forceinline__ void stage_tile(char *lds_dst, const bf16_t *src, int row_stride, int key0, int kv_len,
                                           int wave, const StageOffsets<DH, SWZ, NW> &so) {
  constexpr int kLoadsPerWave = StageOffsets<DH, SWZ, NW>::kLoadsPerWave;
  // Bytes from the tile start to the end of row kv_len-1 of this head; a
  // staged tile always starts at or before that row.
  // (64-bit: the distance to the last row can pass 2 GiB in long slabs.)
  const int64_t tile_bytes = static_cast<int64_t>(pf::kKeyTile) * row_stride * 2;
  const int64_t valid = (static_cast<int64_t>(kv_len - 1 - key0) * row_stride + DH) * 2;
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t *>(src + (int64_t)key0 * row_stride), 0, static_cast<int>(min(valid, tile_bytes)),
      kBufferFlags);
#pragma unroll
  for (int i = 0; i < kLoadsPerWave; ++i) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t *)(lds_dst + (wave * kLoadsPerWave + i) * 1024), 16,
                                             so.boff[i], 0, 0, 0);
  }
}

}  // namespace yoco
