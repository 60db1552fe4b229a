// Backward of the fused RMSNorm + projection (training).
//
// What it computes: the gradient of [Notes] "YOCO：You Only Cache Once 中文精读
// 笔记" s.2.1 Eq. 2 (K^ = LN(M) W_K, V^ = LN(M) W_V, one norm shared by both
// outputs) and of Eq. 3's query projection Q^l = LN(X^l) W_Q^l, with LN the
// RMSNorm y = x g / r, r = sqrt(mean_c x_c^2 + eps).  For the upstream
// gradients dz_p of the outputs z_p = y W_p (p < n_out) of one input row:
//   dy[c]     = sum_p sum_j dz_p[j] W_p[c][j]
//   dW_p     += sum_rows y^T dz_p
//   dgain[c] += sum_rows dy[c] x[c] / r
//   dx[c]     = g[c] dy[c] / r - x[c] / (d r^3) * sum_c' g[c'] dy[c'] x[c']
// (the last term from dr/dx_c = x_c / (d r)).
//
// Kernels, all without atomics (results are bitwise reproducible):
//   * pbwd_prep_kernel: 1/r per row; on the matrix-core path also y rounded
//     to bf16 and, for fp32 dz, dz rounded to bf16 (the operands of both
//     products, like P and dS in the attention backward).
//   * pbwd_dy_kernel (matrix cores): dy^T = W dz^T per 256 x 256 tile with
//     v_mfma_f32_32x32x16_bf16; both operands are read along the reduction
//     index, so both tiles are row-major [256][64] in LDS with 16-byte reads.
//     The epilogue stores dy / r (fp32) into dx, which the row kernel below
//     finishes in place.
//   * pbwd_dw_kernel (matrix cores): dW_p = y^T dz_p, the reduction runs over
//     input rows, split into a fixed number of row ranges; each split writes
//     its partial product, and pbwd_dw_reduce_kernel adds the partials into
//     dW_p in split order.  Both operands run along their rows in memory, so
//     their tiles are staged [64 rows][256] and read with ds_read_b64_tr_b16.
//   * pbwd_dy_valu_kernel / pbwd_dw_valu_kernel: the same two products in
//     fp32 arithmetic for fp32 inputs and for shapes the tiles do not cover.
//   * pbwd_dx_kernel: per row, s = sum_c g dy/r x (one wave reduction),
//     then dx = g dy/r - x s / (d r^2) and the row block's share of dgain.
//   * pbwd_dgain_reduce_kernel: adds the row blocks' dgain shares in a fixed
//     order.
#include "device_common.h"
#include "yoco_internal.h"

namespace yoco {
namespace pb {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float floatx2_t __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef short shortx4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4_t lds_shortx4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kTile = 256;                          // M and N of a workgroup tile
constexpr int kK = 64;                              // reduction slice per stage
constexpr int kTileBytes = kTile * kK * 2;          // 32 KiB per operand tile
constexpr int kLoads = kTileBytes / 1024 / kWaves;  // 1 KiB loads per wave per tile
constexpr int kHalfBytes = kTileBytes / 2;          // [64][128] half of a row-run tile
constexpr int kXcds = 8;
constexpr int32_t kBufferFlags = 0x00020000;        // raw buffer, 32-bit data format

union Frag8 {
  bf16x8_t v;
  uint4 u;
  uint32_t w[4];
  shortx4_t s4[2];
};

__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  const floatx2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, static_cast<int>(bytes > 0 ? bytes : 0),
                                           kBufferFlags);
}

// --- Operands read along the reduction index ("k-contiguous") --------------
// Tile: 256 rows (the M or N index) x 64 k, 128-byte rows in LDS, the 16-byte
// chunk index of row i XOR (i % 8).  Load i of a wave fills 1 KiB block
// b = wave * kLoads + i = rows 8b .. 8b+7: lane L writes LDS bytes
// b*1024 + L*16 = (row 8b + L/8, slot L%8) and so reads chunk slot ^ (row%8).
struct KcStage {
  uint32_t off[kLoads];
  __device__ __forceinline__ void init(int wave, int lane, int ld) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int row = (wave * kLoads + i) * 8 + (lane >> 3);
      const int chunk = (lane & 7) ^ (row & 7);
      off[i] = static_cast<uint32_t>(row * ld * 2 + chunk * 16);
    }
  }
  // rows 0..255 of the tile start at `base`; k0 selects the slice.
  __device__ __forceinline__ void load(char *dst, __amdgpu_buffer_rsrc_t r, int k0, int wave) const {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)(dst + (wave * kLoads + i) * 1024), 16, off[i],
                                               k0 * 2, 0, 0);
    }
  }
};
// Fragment (tile row rb + lane%32, k = ks*16 + (lane/32)*8 .. +8): rb is a
// multiple of 32, so the row's XOR is lane%8.
__device__ __forceinline__ int kc_off(int col, int half, int ks) {
  return col * 128 + (((2 * ks + half) ^ (col & 7)) << 4);
}

// --- Operands whose rows run along the reduction index ("row-run") --------
// Tile: 64 k rows x 256 (M or N), stored as two [64][128] halves with
// 256-byte rows, the 16-byte chunk index of row k XOR rr_xor(k).  Block
// b = wave * kLoads + i is half b/16, rows (b%16)*4 .. +3: lane L writes
// (row (b%16)*4 + L/16, slot L%16) and reads chunk slot ^ rr_xor(row).
__device__ __forceinline__ int rr_xor(int k) { return ((k & 3) << 2) | ((k >> 2) & 3); }
__device__ __forceinline__ int rr_off(int k, int idx) {
  return k * 256 + (((idx >> 3) ^ rr_xor(k)) << 4) + (idx & 7) * 2;
}
struct RrStage {
  uint32_t off[kLoads];
  __device__ __forceinline__ void init(int wave, int lane, int ld) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int blk = wave * kLoads + i;
      const int k = (blk & 15) * 4 + (lane >> 4);
      const int chunk = (lane & 15) ^ rr_xor(k);
      off[i] = static_cast<uint32_t>((k * ld + (blk >> 4) * 128) * 2 + chunk * 16);
    }
  }
  // `r` starts at element (k0, idx0) of the operand.
  __device__ __forceinline__ void load(char *dst, __amdgpu_buffer_rsrc_t r, int wave) const {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)(dst + (wave * kLoads + i) * 1024), 16, off[i], 0,
                                               0, 0);
    }
  }
};
// Transposed fragment reads: in each 16-lane group, source lane a + 4j points
// at k row kb + j, columns cb + 4a .. +3, and lane i of the group receives k
// rows kb..kb+3 of column cb + i.  Lanes 0..31 take k rows 0..7 of the step
// (reads at kb = 0 and 4), lanes 32..63 rows 8..15.  off[r] is the byte
// offset of read r for the 32 columns starting at idx_base (a multiple of 32
// within one half); k step ks adds ks * 16 rows.
struct RrFrag {
  int off[2];
  __device__ __forceinline__ void init(int lane, int idx_base) {
    const int grp = lane >> 4;
    const int src_a = lane & 3;
    const int src_j = (lane >> 2) & 3;
    const int krow = (grp >> 1) * 8 + src_j;
    const int ccol = (grp & 1) * 16 + src_a * 4;
    const int half = idx_base >> 7;
#pragma unroll
    for (int r = 0; r < 2; ++r) off[r] = half * kHalfBytes + rr_off(krow + 4 * r, (idx_base & 127) + ccol);
  }
  __device__ __forceinline__ bf16x8_t read(const char *tile, int ks) const {
    Frag8 f;
    f.s4[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4_t *)(tile + off[0] + ks * 16 * 256));
    f.s4[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4_t *)(tile + off[1] + ks * 16 * 256));
    return f.v;
  }
};

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) x += __shfl_xor(x, s, 64);
  return x;
}

}  // namespace pb

// ---------------------------------------------------------------------------
// 1/r per row; matrix-core path: y = x g / r and dz in bf16.  One wave per row.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void pbwd_prep_kernel(const ProjBwdArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= a.n) return;
  const int d = a.d;
  const bool vec = a.x_bf16 && (d % 8 == 0);
  float ss = 0.f;
  if (vec) {
    const bf16_t *xr = static_cast<const bf16_t *>(a.x) + row * d;
    for (int c = lane * 8; c < d; c += 512) {
      const uint4 w = ld16(xr + c);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ss = fmaf(bf16_lo(ww[j]), bf16_lo(ww[j]), ss);
        ss = fmaf(bf16_hi(ww[j]), bf16_hi(ww[j]), ss);
      }
    }
  } else {
    for (int c = lane; c < d; c += 64) {
      const float v = a.x_bf16 ? load_elem(static_cast<const bf16_t *>(a.x) + row * d + c)
                               : load_elem(static_cast<const float *>(a.x) + row * d + c);
      ss = fmaf(v, v, ss);
    }
  }
  ss = pb::wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / static_cast<float>(d) + a.eps);
  if (lane == 0) a.inv_r[row] = inv;
  if (!a.mfma) return;
  // y = x g / r in bf16 (the matrix-core path has bf16 x and d % 256 == 0).
  const bf16_t *xr = static_cast<const bf16_t *>(a.x) + row * d;
  bf16_t *yr = a.ybf + row * d;
  for (int c = lane * 8; c < d; c += 512) {
    const uint4 w = ld16(xr + c);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
    float g[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) g[j] = a.gain ? a.gain[c + j] : 1.f;
    uint4 o;
    uint32_t *ow = reinterpret_cast<uint32_t *>(&o);
#pragma unroll
    for (int j = 0; j < 4; ++j) ow[j] = pb::cvt_pk_bf16(bf16_lo(ww[j]) * g[2 * j] * inv, bf16_hi(ww[j]) * g[2 * j + 1] * inv);
    *reinterpret_cast<uint4 *>(yr + c) = o;
  }
  if (a.dz_bf16) return;
  for (int p = 0; p < a.n_out; ++p) {
    const float *zr = static_cast<const float *>(a.dz[p]) + row * a.ncols;
    bf16_t *zb = a.dzb[p] + row * a.ncols;
    for (int c = lane * 8; c < a.ncols; c += 512) {
      const uint4 u0 = ld16(zr + c), u1 = ld16(zr + c + 4);
      uint4 o;
      o.x = pb::cvt_pk_bf16(__uint_as_float(u0.x), __uint_as_float(u0.y));
      o.y = pb::cvt_pk_bf16(__uint_as_float(u0.z), __uint_as_float(u0.w));
      o.z = pb::cvt_pk_bf16(__uint_as_float(u1.x), __uint_as_float(u1.y));
      o.w = pb::cvt_pk_bf16(__uint_as_float(u1.z), __uint_as_float(u1.w));
      *reinterpret_cast<uint4 *>(zb + c) = o;
    }
  }
}

// The same on the matrix-core path (bf16 x, d % 256 == 0, d <= 512 GX):
// every load of a row is issued before the first is used, x stays in
// registers between the sum of squares and y, and dz is converted four
// 8-column groups per batch.  Same arithmetic, in the same order.
template <int GX>
__global__ __launch_bounds__(256) void pbwd_prep_rows_kernel(const ProjBwdArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= a.n) return;
  const int d = a.d;
  const bf16_t *xr = static_cast<const bf16_t *>(a.x) + row * d;
  uint4 xw[GX];
#pragma unroll
  for (int i = 0; i < GX; ++i) {
    const int c = lane * 8 + 512 * i;
    xw[i] = c < d ? ld16(xr + c) : make_uint4(0, 0, 0, 0);
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < GX; ++i) {
    const uint32_t ww[4] = {xw[i].x, xw[i].y, xw[i].z, xw[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ss = fmaf(bf16_lo(ww[j]), bf16_lo(ww[j]), ss);
      ss = fmaf(bf16_hi(ww[j]), bf16_hi(ww[j]), ss);
    }
  }
  ss = pb::wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / static_cast<float>(d) + a.eps);
  if (lane == 0) a.inv_r[row] = inv;
  bf16_t *yr = a.ybf + row * d;
#pragma unroll
  for (int i = 0; i < GX; ++i) {
    const int c = lane * 8 + 512 * i;
    if (c >= d) continue;
    const uint32_t ww[4] = {xw[i].x, xw[i].y, xw[i].z, xw[i].w};
    float g[8];
    if (a.gain) {
      const float4 g0 = *reinterpret_cast<const float4 *>(a.gain + c);
      const float4 g1 = *reinterpret_cast<const float4 *>(a.gain + c + 4);
      g[0] = g0.x, g[1] = g0.y, g[2] = g0.z, g[3] = g0.w, g[4] = g1.x, g[5] = g1.y, g[6] = g1.z, g[7] = g1.w;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) g[j] = 1.f;
    }
    uint4 o;
    uint32_t *ow = reinterpret_cast<uint32_t *>(&o);
#pragma unroll
    for (int j = 0; j < 4; ++j) ow[j] = pb::cvt_pk_bf16(bf16_lo(ww[j]) * g[2 * j] * inv, bf16_hi(ww[j]) * g[2 * j + 1] * inv);
    *reinterpret_cast<uint4 *>(yr + c) = o;
  }
  if (a.dz_bf16) return;
  constexpr int kBatch = 4;
  for (int p = 0; p < a.n_out; ++p) {
    const float *zr = static_cast<const float *>(a.dz[p]) + row * a.ncols;
    bf16_t *zb = a.dzb[p] + row * a.ncols;
    for (int c0 = lane * 8; c0 < a.ncols; c0 += 512 * kBatch) {
      uint4 u[kBatch][2];
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int c = c0 + 512 * b;
        if (c < a.ncols) {
          u[b][0] = ld16(zr + c);
          u[b][1] = ld16(zr + c + 4);
        }
      }
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int c = c0 + 512 * b;
        if (c >= a.ncols) continue;
        uint4 o;
        o.x = pb::cvt_pk_bf16(__uint_as_float(u[b][0].x), __uint_as_float(u[b][0].y));
        o.y = pb::cvt_pk_bf16(__uint_as_float(u[b][0].z), __uint_as_float(u[b][0].w));
        o.z = pb::cvt_pk_bf16(__uint_as_float(u[b][1].x), __uint_as_float(u[b][1].y));
        o.w = pb::cvt_pk_bf16(__uint_as_float(u[b][1].z), __uint_as_float(u[b][1].w));
        *reinterpret_cast<uint4 *>(zb + c) = o;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dy^T = W dz^T on the matrix cores; stores dy / r into dx.
// Tile: 256 model columns c (A = W_p rows) x 256 input rows r (B = dz_p
// rows); the reduction runs over the n_out * ncols columns of dz in slices of
// 64.  Wave (wm, wn) owns c in wm*128 + [0,128) and r in wn*64 + [0,64).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(pb::kThreads, 1) void pbwd_dy_kernel(const ProjBwdArgs a) {
  using namespace pb;
  __shared__ __attribute__((aligned(1024))) char lds_a0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char lds_a1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char lds_b0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char lds_b1[kTileBytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5;
  const int col = lane & 31;

  // The column tiles of one row tile run on consecutive slots of one XCD, so
  // the row tile's dz rows are shared in its L2.
  const int ctiles = a.d / kTile;
  const int rtiles = static_cast<int>((a.n + kTile - 1) / kTile);
  const int xcd = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int rtile = (slot / ctiles) * kXcds + xcd;
  if (rtile >= rtiles) return;
  const int c0 = (slot % ctiles) * kTile;
  const int64_t r0 = static_cast<int64_t>(rtile) * kTile;
  const int rows_here = a.n - r0 < kTile ? static_cast<int>(a.n - r0) : kTile;
  const int nc = a.ncols;
  const int per_out = nc / kK;
  const int n_slices = a.n_out * per_out;  // even: ncols % 256 == 0

  __amdgpu_buffer_rsrc_t ra[2], rb[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int pp = p < a.n_out ? p : 0;
    ra[p] = rsrc(static_cast<const bf16_t *>(a.w[pp]) + static_cast<int64_t>(c0) * nc, int64_t(kTile) * nc * 2);
    rb[p] = rsrc(a.dzb[pp] + r0 * nc, int64_t(rows_here) * nc * 2);
  }
  KcStage st;
  st.init(wave, lane, nc);
  auto stage = [&](char *adst, char *bdst, int s) __attribute__((always_inline)) {
    const int p = s >= per_out ? 1 : 0;
    const int k0 = (s - p * per_out) * kK;
    st.load(adst, p ? ra[1] : ra[0], k0, wave);
    st.load(bdst, p ? rb[1] : rb[0], k0, wave);
  };

  const int wm = wave >> 2;
  const int wn = wave & 3;
  int koff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) koff[ks] = kc_off(col, half, ks);

  floatx16 acc[4][2];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[t][s2][i] = 0.f;
    }
  }
  auto compute = [&](const char *at, const char *bt) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      Frag8 af[4], bf[2];
#pragma unroll
      for (int t = 0; t < 4; ++t) af[t].u = *reinterpret_cast<const uint4 *>(at + (wm * 128 + t * 32) * 128 + koff[ks]);
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) bf[s2].u = *reinterpret_cast<const uint4 *>(bt + (wn * 64 + s2 * 32) * 128 + koff[ks]);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) acc[t][s2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[t].v, bf[s2].v, acc[t][s2], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  stage(lds_a0, lds_b0, 0);
  for (int s = 0; s < n_slices; s += 2) {
    // Slice s has landed for every wave, and every wave is done with slice
    // s-1, whose buffers the next loads overwrite.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    stage(lds_a1, lds_b1, s + 1);
    compute(lds_a0, lds_b0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (s + 2 < n_slices) stage(lds_a0, lds_b0, s + 2);
    compute(lds_a1, lds_b1);
  }

  // acc[t][s2] element i: c = c0 + wm*128 + t*32 + (i/4)*8 + half*4 + i%4,
  // r = r0 + wn*64 + s2*32 + col.
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    const int rl = wn * 64 + s2 * 32 + col;
    if (rl >= rows_here) continue;
    const int64_t r = r0 + rl;
    const float inv = a.inv_r[r];
    float *dxr = a.dx + r * a.d + c0 + wm * 128;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const float4 v = make_float4(acc[t][s2][i4 * 4 + 0] * inv, acc[t][s2][i4 * 4 + 1] * inv,
                                     acc[t][s2][i4 * 4 + 2] * inv, acc[t][s2][i4 * 4 + 3] * inv);
        *reinterpret_cast<float4 *>(dxr + t * 32 + i4 * 8 + half * 4) = v;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Partial dW_p = y^T dz_p over one split of the input rows, on the matrix
// cores.  Tile: 256 model columns c (A = y^T) x 256 output columns j (B =
// dz_p); the reduction runs over the split's rows in slices of 64, padded to
// an even count (rows past the split load as zeros).  Wave (wm, wn) owns c in
// wm*128 + [0,128) and j in wn*64 + [0,64).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(pb::kThreads, 1) void pbwd_dw_kernel(const ProjBwdArgs a) {
  using namespace pb;
  __shared__ __attribute__((aligned(1024))) char lds_a0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char lds_a1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char lds_b0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char lds_b1[kTileBytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5;
  const int col = lane & 31;

  // Every tile of one split runs on one XCD, so the split's rows of y and dz
  // are shared in its L2.
  const int d = a.d;
  const int nc = a.ncols;
  const int ctiles = d / kTile;
  const int jtiles = nc / kTile;
  const int per_split = ctiles * jtiles * a.n_out;
  const int xcd = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int split = (slot / per_split) * kXcds + xcd;
  if (split >= a.splits) return;
  const int rem = slot % per_split;
  const int p = rem / (ctiles * jtiles);
  const int c0 = ((rem / jtiles) % ctiles) * kTile;
  const int j0 = (rem % jtiles) * kTile;
  const int64_t k_begin = static_cast<int64_t>(split) * a.split_rows;
  const int64_t k_end = k_begin + a.split_rows < a.n ? k_begin + a.split_rows : a.n;
  const int n_slices = ((static_cast<int>((k_end - k_begin + kK - 1) / kK)) + 1) & ~1;

  const bf16_t *ybase = a.ybf;
  const bf16_t *zbase = a.dzb[p];
  RrStage sa, sb;
  sa.init(wave, lane, d);
  sb.init(wave, lane, nc);
  // The descriptor of a slice starts at its first row and ends with the
  // tile's columns of the split's last row, so rows past the split load as
  // zeros.
  auto stage = [&](char *adst, char *bdst, int s) __attribute__((always_inline)) {
    const int64_t k0 = k_begin + static_cast<int64_t>(s) * kK;
    const int64_t rows = k_end - k0 < kK ? k_end - k0 : kK;  // rows of this slice inside the split
    const int64_t abytes = rows > 0 ? ((rows - 1) * d + kTile) * 2 : 0;
    const int64_t bbytes = rows > 0 ? ((rows - 1) * nc + kTile) * 2 : 0;
    const int64_t kk = rows > 0 ? k0 : 0;
    sa.load(adst, rsrc(ybase + kk * d + c0, abytes), wave);
    sb.load(bdst, rsrc(zbase + kk * nc + j0, bbytes), wave);
  };

  const int wm = wave >> 2;
  const int wn = wave & 3;
  RrFrag fa[4], fb[2];
#pragma unroll
  for (int t = 0; t < 4; ++t) fa[t].init(lane, wm * 128 + t * 32);
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) fb[s2].init(lane, wn * 64 + s2 * 32);

  floatx16 acc[4][2];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[t][s2][i] = 0.f;
    }
  }
  auto compute = [&](const char *at, const char *bt) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8_t af[4], bf[2];
#pragma unroll
      for (int t = 0; t < 4; ++t) af[t] = fa[t].read(at, ks);
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) bf[s2] = fb[s2].read(bt, ks);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) acc[t][s2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[t], bf[s2], acc[t][s2], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  stage(lds_a0, lds_b0, 0);
  for (int s = 0; s < n_slices; s += 2) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    stage(lds_a1, lds_b1, s + 1);
    compute(lds_a0, lds_b0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (s + 2 < n_slices) stage(lds_a0, lds_b0, s + 2);
    compute(lds_a1, lds_b1);
  }

  // acc[t][s2] element i: c = c0 + wm*128 + t*32 + (i/4)*8 + half*4 + i%4,
  // j = j0 + wn*64 + s2*32 + col.
  float *part = a.dw_part + ((static_cast<int64_t>(split) * a.n_out + p) * d + c0 + wm * 128) * nc + j0 + wn * 64;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int cl = t * 32 + (i >> 2) * 8 + half * 4 + (i & 3);
        part[static_cast<int64_t>(cl) * nc + s2 * 32 + col] = acc[t][s2][i];
      }
    }
  }
}

// dW_p += sum over splits of the partials, in split order.  Four elements per
// thread (ncols % 256 == 0 on this path).
__global__ __launch_bounds__(256) void pbwd_dw_reduce_kernel(const ProjBwdArgs a) {
  const int64_t per_out = static_cast<int64_t>(a.d) * a.ncols;
  const int64_t idx4 = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (idx4 >= per_out * a.n_out) return;
  const int p = static_cast<int>(idx4 / per_out);
  const int64_t e = idx4 - p * per_out;
  float4 s = *reinterpret_cast<const float4 *>(a.dw[p] + e);
  for (int sp = 0; sp < a.splits; ++sp) {
    const float4 v = *reinterpret_cast<const float4 *>(a.dw_part + (static_cast<int64_t>(sp) * a.n_out + p) * per_out + e);
    s.x += v.x;
    s.y += v.y;
    s.z += v.z;
    s.w += v.w;
  }
  *reinterpret_cast<float4 *>(a.dw[p] + e) = s;
}

// ---------------------------------------------------------------------------
// fp32 products for fp32 inputs and shapes the tiles do not cover.
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ float elem(const void *p, int64_t i) {
  return load_elem(static_cast<const T *>(p) + i);
}

// dx[r][c] = (1/r) sum_p sum_j dz_p[r][j] W_p[c][j]; the 64 lanes of a wave
// take 64 consecutive rows of one column c, so W_p[c][j] is one address per
// wave.  Block: 64 rows x 4 columns.
template <typename TX, typename TW, typename TZ>
__global__ __launch_bounds__(256) void pbwd_dy_valu_kernel(const ProjBwdArgs a) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 64 + (threadIdx.x & 63);
  const int c = blockIdx.y * 4 + (threadIdx.x >> 6);
  if (r >= a.n || c >= a.d) return;
  float acc = 0.f;
  for (int p = 0; p < a.n_out; ++p) {
    const int64_t zb = r * a.ncols;
    const int64_t wb = static_cast<int64_t>(c) * a.ncols;
    for (int j = 0; j < a.ncols; ++j) acc = fmaf(elem<TZ>(a.dz[p], zb + j), elem<TW>(a.w[p], wb + j), acc);
  }
  a.dx[r * a.d + c] = acc * a.inv_r[r];
}

// dW_p[c][j] += sum_r (x[r][c] g[c] / r_r) dz_p[r][j]; lanes take consecutive
// columns j.  Block: 256 columns j of one (p, c).
template <typename TX, typename TW, typename TZ>
__global__ __launch_bounds__(256) void pbwd_dw_valu_kernel(const ProjBwdArgs a) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  const int c = blockIdx.y;
  const int p = blockIdx.z;
  if (j >= a.ncols) return;
  const float g = a.gain ? a.gain[c] : 1.f;
  float acc = 0.f;
  for (int64_t r = 0; r < a.n; ++r) {
    const float y = elem<TX>(a.x, r * a.d + c) * g * a.inv_r[r];
    acc = fmaf(y, elem<TZ>(a.dz[p], r * a.ncols + j), acc);
  }
  float *w = a.dw[p] + static_cast<int64_t>(c) * a.ncols + j;
  *w += acc;
}

// ---------------------------------------------------------------------------
// Rows: dx = g dy/r - x s / (d r^2) with s = sum_c g dy/r x, and the row
// block's share of dgain (sum over its rows of dy/r x).  dx holds dy/r on
// entry.  A block of 4 waves takes kProjBwdFinRows rows; wave w handles rows
// w, w+4, ... of the block, lane l owns the column groups l*4 + 256 i (four
// consecutive columns each, when d % 4 == 0) or, for other widths, single
// columns l + 64 (4 i + e).  The row sum is a wave reduction.  Each wave
// keeps its dgain share in its own [d] slice of LDS (dynamic, 4 d floats);
// the slices are added in wave order at the end.
// ---------------------------------------------------------------------------
template <typename TX>
__global__ __launch_bounds__(256) void pbwd_dx_kernel(const ProjBwdArgs a) {
  extern __shared__ float s_dg[];  // [4][d]
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int d = a.d;
  const bool vec = d % 4 == 0;
  const int groups = (d + 255) / 256;
  float *my_dg = s_dg + wave * d;
  for (int c = lane; c < d; c += 64) my_dg[c] = 0.f;
  // Column of element (i, e) of this lane.
  auto column = [&](int i, int e) __attribute__((always_inline)) {
    return vec ? lane * 4 + 256 * i + e : lane + 64 * (4 * i + e);
  };
  // dy/r, x and g of element group i of row r (zeros past the row's end).
  auto load = [&](int64_t r, int i, float (&dv)[4], float (&xv)[4], float (&g)[4]) __attribute__((always_inline)) {
    const float *dxr = a.dx + r * d;
    if (vec) {
      const int c = column(i, 0);
      if (c < d) {
        const float4 t = *reinterpret_cast<const float4 *>(dxr + c);
        dv[0] = t.x, dv[1] = t.y, dv[2] = t.z, dv[3] = t.w;
#pragma unroll
        for (int e = 0; e < 4; ++e) xv[e] = elem<TX>(a.x, r * d + c + e);
        if (a.gain) {
          const float4 gg = *reinterpret_cast<const float4 *>(a.gain + c);
          g[0] = gg.x, g[1] = gg.y, g[2] = gg.z, g[3] = gg.w;
        } else {
          g[0] = g[1] = g[2] = g[3] = 1.f;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) dv[e] = xv[e] = g[e] = 0.f;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = column(i, e);
        dv[e] = (c < d) ? dxr[c] : 0.f;
        xv[e] = (c < d) ? elem<TX>(a.x, r * d + c) : 0.f;
        g[e] = (c < d) ? (a.gain ? a.gain[c] : 1.f) : 0.f;
      }
    }
  };
  const int64_t r_begin = static_cast<int64_t>(blockIdx.x) * kProjBwdFinRows;
  const int64_t r_end = r_begin + kProjBwdFinRows < a.n ? r_begin + kProjBwdFinRows : a.n;
  for (int64_t r = r_begin + wave; r < r_end; r += 4) {
    float s = 0.f;
#pragma unroll 2
    for (int i = 0; i < groups; ++i) {
      float dv[4], xv[4], g[4];
      load(r, i, dv, xv, g);
#pragma unroll
      for (int e = 0; e < 4; ++e) s = fmaf(g[e] * dv[e], xv[e], s);
    }
    s = pb::wave_sum(s);
    const float inv = a.inv_r[r];
    const float coef = inv * inv * s / static_cast<float>(d);
    float *dxr = a.dx + r * d;
    // Second sweep over the row (in cache): every lane has read all of its
    // elements above, so the in-place stores cannot overtake a read.
#pragma unroll 2
    for (int i = 0; i < groups; ++i) {
      float dv[4], xv[4], g[4], o[4];
      load(r, i, dv, xv, g);
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = g[e] * dv[e] - xv[e] * coef;
      if (vec) {
        const int c = column(i, 0);
        if (c < d) {
          *reinterpret_cast<float4 *>(dxr + c) = make_float4(o[0], o[1], o[2], o[3]);
          float4 t = *reinterpret_cast<float4 *>(my_dg + c);
          t.x = fmaf(dv[0], xv[0], t.x);
          t.y = fmaf(dv[1], xv[1], t.y);
          t.z = fmaf(dv[2], xv[2], t.z);
          t.w = fmaf(dv[3], xv[3], t.w);
          *reinterpret_cast<float4 *>(my_dg + c) = t;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c = column(i, e);
          if (c < d) {
            dxr[c] = o[e];
            my_dg[c] = fmaf(dv[e], xv[e], my_dg[c]);
          }
        }
      }
    }
  }
  if (a.dgain == nullptr) return;
  __syncthreads();
  for (int c = threadIdx.x; c < d; c += 256) {
    const float v = ((s_dg[c] + s_dg[d + c]) + s_dg[2 * d + c]) + s_dg[3 * d + c];
    a.dgain_part[static_cast<int64_t>(blockIdx.x) * d + c] = v;
  }
}

// The same for d % 256 == 0 with G = d / 256 <= 12 column groups per lane: a row's
// loads are all issued before the first is used and both sweeps run from
// registers; the gain and the wave's dgain share stay in registers across
// its rows.  Same arithmetic, in the same order.
template <typename TX, int G>
__global__ __launch_bounds__(256) void pbwd_dx_rows_kernel(const ProjBwdArgs a) {
  extern __shared__ float s_dg[];  // [4][d]
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int d = a.d;
  float g[G][4], dg[G][4];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    if (a.gain) {
      const float4 gg = *reinterpret_cast<const float4 *>(a.gain + lane * 4 + 256 * i);
      g[i][0] = gg.x, g[i][1] = gg.y, g[i][2] = gg.z, g[i][3] = gg.w;
    } else {
      g[i][0] = g[i][1] = g[i][2] = g[i][3] = 1.f;
    }
    dg[i][0] = dg[i][1] = dg[i][2] = dg[i][3] = 0.f;
  }
  const int64_t r_begin = static_cast<int64_t>(blockIdx.x) * kProjBwdFinRows;
  const int64_t r_end = r_begin + kProjBwdFinRows < a.n ? r_begin + kProjBwdFinRows : a.n;
  for (int64_t r = r_begin + wave; r < r_end; r += 4) {
    float *dxr = a.dx + r * d;
    float4 dv[G];
    float xv[G][4];
    if constexpr (sizeof(TX) == 2) {
      uint2 xw[G];
      const bf16_t *xr = static_cast<const bf16_t *>(a.x) + r * d;
#pragma unroll
      for (int i = 0; i < G; ++i) {
        dv[i] = *reinterpret_cast<const float4 *>(dxr + lane * 4 + 256 * i);
        xw[i] = *reinterpret_cast<const uint2 *>(xr + lane * 4 + 256 * i);
      }
#pragma unroll
      for (int i = 0; i < G; ++i) {
        xv[i][0] = bf16_lo(xw[i].x), xv[i][1] = bf16_hi(xw[i].x);
        xv[i][2] = bf16_lo(xw[i].y), xv[i][3] = bf16_hi(xw[i].y);
      }
    } else {
      float4 xw[G];
      const float *xr = static_cast<const float *>(a.x) + r * d;
#pragma unroll
      for (int i = 0; i < G; ++i) {
        dv[i] = *reinterpret_cast<const float4 *>(dxr + lane * 4 + 256 * i);
        xw[i] = *reinterpret_cast<const float4 *>(xr + lane * 4 + 256 * i);
      }
#pragma unroll
      for (int i = 0; i < G; ++i) xv[i][0] = xw[i].x, xv[i][1] = xw[i].y, xv[i][2] = xw[i].z, xv[i][3] = xw[i].w;
    }
    float s = 0.f;
    float gd[G][4];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const float dvv[4] = {dv[i].x, dv[i].y, dv[i].z, dv[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        gd[i][e] = g[i][e] * dvv[e];
        s = fmaf(gd[i][e], xv[i][e], s);
        dg[i][e] = fmaf(dvv[e], xv[i][e], dg[i][e]);
      }
    }
    s = pb::wave_sum(s);
    const float inv = a.inv_r[r];
    const float coef = inv * inv * s / static_cast<float>(d);
#pragma unroll
    for (int i = 0; i < G; ++i) {
      *reinterpret_cast<float4 *>(dxr + lane * 4 + 256 * i) =
          make_float4(gd[i][0] - xv[i][0] * coef, gd[i][1] - xv[i][1] * coef, gd[i][2] - xv[i][2] * coef,
                      gd[i][3] - xv[i][3] * coef);
    }
  }
  if (a.dgain == nullptr) return;
  float *my_dg = s_dg + wave * d;
#pragma unroll
  for (int i = 0; i < G; ++i)
    *reinterpret_cast<float4 *>(my_dg + lane * 4 + 256 * i) = make_float4(dg[i][0], dg[i][1], dg[i][2], dg[i][3]);
  __syncthreads();
  for (int c = threadIdx.x; c < d; c += 256) {
    const float v = ((s_dg[c] + s_dg[d + c]) + s_dg[2 * d + c]) + s_dg[3 * d + c];
    a.dgain_part[static_cast<int64_t>(blockIdx.x) * d + c] = v;
  }
}

// dgain[c] += sum over row blocks of their shares.  A block takes 16
// columns; thread (slice, column) sums a contiguous run of row blocks, and
// the 16 runs are added in order.
__global__ __launch_bounds__(256) void pbwd_dgain_reduce_kernel(const ProjBwdArgs a, int n_blocks) {
  __shared__ float s_part[16][16];
  const int cl = threadIdx.x & 15;
  const int slice = threadIdx.x >> 4;
  const int c = blockIdx.x * 16 + cl;
  const int per = (n_blocks + 15) / 16;
  const int b0 = slice * per;
  const int b1 = b0 + per < n_blocks ? b0 + per : n_blocks;
  float s = 0.f;
  if (c < a.d) {
    for (int b = b0; b < b1; ++b) s += a.dgain_part[static_cast<int64_t>(b) * a.d + c];
  }
  s_part[slice][cl] = s;
  __syncthreads();
  if (slice == 0 && c < a.d) {
    float t = a.dgain[c];
    for (int k = 0; k < 16; ++k) t += s_part[k][cl];
    a.dgain[c] = t;
  }
}

// ---------------------------------------------------------------------------
bool project_bwd_mfma_applies(int64_t n, int32_t d, int32_t ncols, int x_dt, int w_dt) {
  return x_dt == YOCO_DT_BF16 && w_dt == YOCO_DT_BF16 && n > 0 && d % pb::kTile == 0 && ncols % pb::kTile == 0 &&
         static_cast<int64_t>(pb::kTile) * d * 2 < (int64_t(1) << 31) &&
         static_cast<int64_t>(pb::kTile) * ncols * 2 < (int64_t(1) << 31);
}

// Split plan of the matrix-core dW product: enough splits for about three
// workgroups per CU of a 256-CU device, each at least 512 rows, rows per
// split a multiple of 64.  A function of the shapes only, so results do not
// depend on the device.
void project_bwd_split_plan(int64_t n, int32_t d, int32_t ncols, int32_t n_out, int32_t *splits, int32_t *rows) {
  const int64_t tiles = static_cast<int64_t>(d / pb::kTile) * (ncols / pb::kTile) * n_out;
  int64_t s = tiles > 0 ? (768 + tiles - 1) / tiles : 1;
  const int64_t by_rows = (n + 511) / 512;
  if (s > by_rows) s = by_rows;
  if (s < 1) s = 1;
  int64_t r = (n + s - 1) / s;
  r = (r + pb::kK - 1) / pb::kK * pb::kK;
  if (r < pb::kK) r = pb::kK;
  *rows = static_cast<int32_t>(r);
  *splits = static_cast<int32_t>((n + r - 1) / r);
}

template <typename TX, int G>
static void launch_dx_rows(const ProjBwdArgs &a, unsigned blocks, size_t lds, hipStream_t s) {
  hipLaunchKernelGGL((pbwd_dx_rows_kernel<TX, G>), dim3(blocks), dim3(256), lds, s, a);
}

template <typename TX>
hipError_t launch_dx(const ProjBwdArgs &a, hipStream_t s) {
  const unsigned blocks = static_cast<unsigned>((a.n + kProjBwdFinRows - 1) / kProjBwdFinRows);
  const size_t lds = static_cast<size_t>(4) * a.d * sizeof(float);  // <= 64 KiB for d <= kProjBwdMaxD
  // Past 12 column groups the row kernel's registers allow one wave per SIMD.
  if (a.d % 256 != 0 || a.d > 12 * 256) {
    hipLaunchKernelGGL((pbwd_dx_kernel<TX>), dim3(blocks), dim3(256), lds, s, a);
    return hipGetLastError();
  }
  switch (a.d / 256) {
    case 1: launch_dx_rows<TX, 1>(a, blocks, lds, s); break;
    case 2: launch_dx_rows<TX, 2>(a, blocks, lds, s); break;
    case 3: launch_dx_rows<TX, 3>(a, blocks, lds, s); break;
    case 4: launch_dx_rows<TX, 4>(a, blocks, lds, s); break;
    case 5: launch_dx_rows<TX, 5>(a, blocks, lds, s); break;
    case 6: launch_dx_rows<TX, 6>(a, blocks, lds, s); break;
    case 7: launch_dx_rows<TX, 7>(a, blocks, lds, s); break;
    case 8: launch_dx_rows<TX, 8>(a, blocks, lds, s); break;
    case 9: launch_dx_rows<TX, 9>(a, blocks, lds, s); break;
    case 10: launch_dx_rows<TX, 10>(a, blocks, lds, s); break;
    case 11: launch_dx_rows<TX, 11>(a, blocks, lds, s); break;
    default: launch_dx_rows<TX, 12>(a, blocks, lds, s); break;
  }
  return hipGetLastError();
}

static hipError_t launch_prep(const ProjBwdArgs &a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((a.n + 3) / 4));
  if (!a.mfma) {
    hipLaunchKernelGGL(pbwd_prep_kernel, grid, dim3(256), 0, s, a);
    return hipGetLastError();
  }
  // the matrix-core path has d % 256 == 0 and d <= kProjBwdMaxD
  switch ((a.d + 511) / 512) {
    case 1: hipLaunchKernelGGL((pbwd_prep_rows_kernel<1>), grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((pbwd_prep_rows_kernel<2>), grid, dim3(256), 0, s, a); break;
    case 3: hipLaunchKernelGGL((pbwd_prep_rows_kernel<3>), grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL((pbwd_prep_rows_kernel<4>), grid, dim3(256), 0, s, a); break;
    case 5: hipLaunchKernelGGL((pbwd_prep_rows_kernel<5>), grid, dim3(256), 0, s, a); break;
    case 6: hipLaunchKernelGGL((pbwd_prep_rows_kernel<6>), grid, dim3(256), 0, s, a); break;
    case 7: hipLaunchKernelGGL((pbwd_prep_rows_kernel<7>), grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((pbwd_prep_rows_kernel<8>), grid, dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

template <typename TX, typename TW, typename TZ>
hipError_t launch_valu_products(const ProjBwdArgs &a, hipStream_t s) {
  hipLaunchKernelGGL((pbwd_dy_valu_kernel<TX, TW, TZ>), dim3(static_cast<unsigned>((a.n + 63) / 64), (a.d + 3) / 4),
                     dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((pbwd_dw_valu_kernel<TX, TW, TZ>), dim3((a.ncols + 255) / 256, a.d, a.n_out), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename TX, typename TW>
hipError_t launch_valu_products_z(const ProjBwdArgs &a, hipStream_t s) {
  return a.dz_bf16 ? launch_valu_products<TX, TW, bf16_t>(a, s) : launch_valu_products<TX, TW, float>(a, s);
}

hipError_t launch_project_bwd(const ProjBwdArgs &a, hipStream_t s) {
  hipError_t e = launch_prep(a, s);
  if (e != hipSuccess) return e;
  if (a.mfma) {
    const int64_t rtiles = (a.n + pb::kTile - 1) / pb::kTile;
    const int64_t ctiles = a.d / pb::kTile;
    const int64_t dy_blocks = (rtiles + pb::kXcds - 1) / pb::kXcds * pb::kXcds * ctiles;
    const int64_t per_split = ctiles * (a.ncols / pb::kTile) * a.n_out;
    const int64_t dw_blocks = (a.splits + pb::kXcds - 1) / pb::kXcds * pb::kXcds * per_split;
    if (dy_blocks > 0x7fffffff || dw_blocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(pbwd_dy_kernel, dim3(static_cast<unsigned>(dy_blocks)), dim3(pb::kThreads), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(pbwd_dw_kernel, dim3(static_cast<unsigned>(dw_blocks)), dim3(pb::kThreads), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t elems4 = static_cast<int64_t>(a.d) * a.ncols * a.n_out / 4;
    hipLaunchKernelGGL(pbwd_dw_reduce_kernel, dim3(static_cast<unsigned>((elems4 + 255) / 256)), dim3(256), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    e = launch_dx<bf16_t>(a, s);
  } else {
    if (a.x_bf16) {
      e = a.w_bf16 ? launch_valu_products_z<bf16_t, bf16_t>(a, s) : launch_valu_products_z<bf16_t, float>(a, s);
    } else {
      e = a.w_bf16 ? launch_valu_products_z<float, bf16_t>(a, s) : launch_valu_products_z<float, float>(a, s);
    }
    if (e != hipSuccess) return e;
    e = a.x_bf16 ? launch_dx<bf16_t>(a, s) : launch_dx<float>(a, s);
  }
  if (e != hipSuccess || a.dgain == nullptr) return e;
  const int n_blocks = static_cast<int>((a.n + kProjBwdFinRows - 1) / kProjBwdFinRows);
  hipLaunchKernelGGL(pbwd_dgain_reduce_kernel, dim3((a.d + 15) / 16), dim3(256), 0, s, a, n_blocks);
  return hipGetLastError();
}

}  // namespace yoco
