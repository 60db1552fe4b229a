// Prompt-sized fused RMSNorm + projection on the matrix cores (bf16 in, bf16
// out), written straight to its destination rows.
//
// What it computes ([Notes] "YOCO：You Only Cache Once 中文精读笔记" s.2.1
// Eq. 2: K^ = LN(M) W_K, V^ = LN(M) W_V with LN = RMSNorm, projected once at
// the self/cross boundary; Eq. 3: Q^l = LN(X^l) W_Q^l):
//   out_p[row][j] = (sum_c x[row][c] * gain[c] * W_p[c][j]) / rms_row,
//   rms_row = sqrt(mean_c x[row][c]^2 + eps).
// The row factor 1/rms is applied after the sum (the same value).
//
// Layout of the work: the product is computed transposed, out^T = W^T x^T,
// with v_mfma_f32_32x32x16_bf16:
//   * A = W^T: lane l holds output column l%32 and 8 consecutive k; read
//     from the row-major W tile in LDS with ds_read_b64_tr_b16 (4 k rows of
//     one column per read, two reads per fragment);
//   * B = x^T: lane l holds input row l%32 and 8 consecutive k, one 16-byte
//     LDS read from the row-major x tile;
//   * C: each lane owns ONE input row and 16 output columns, so the 1/rms
//     factor is lane-local and the bf16 stores are 8 bytes wide.
// The sum of squares of each row comes from the same x fragments (bf16 dot2
// of a fragment with itself, exact products, fp32 sums).  With a gain, x*g is
// formed in fp32 and split into bf16 hi + lo (hi = RNE(x*g), lo = RNE(x*g -
// hi)), two MFMAs per fragment: the split leaves about 2^-17 of the term,
// far below the fp32 accumulation error; without a gain x enters as stored.
//
// A workgroup is 8 waves and computes 256 input rows x 256 output columns of
// one weight, in wave tiles of 64 x 128 (32 x 256 with a gain).  The
// reduction runs in slices of 32, staged global -> LDS with 16-byte buffer
// loads to LDS through a ring of four slots, three slices in flight while
// the fourth is read: x slice [256][32] (64-byte rows, chunk index XOR
// (row/4)%4), W slice [32][256] as two [32][128] halves (256-byte rows,
// chunk index XOR a 4-bit function of the row).  The x descriptor ends at
// the last input row, so rows past it load as zeros and are not stored.
#include <type_traits>

#include "device_common.h"
#include "rope.h"
#include "yoco_internal.h"

namespace yoco {
namespace pm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float floatx2_t __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef short shortx4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4_t lds_shortx4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kRows = 256;                      // input rows per workgroup
constexpr int kCols = 256;                      // output columns per workgroup
constexpr int kK = 32;                          // reduction slice per stage
constexpr int kStages = 4;                      // LDS ring slots (three slices in flight)
constexpr int kXRowBytes = kK * 2;              // 64
constexpr int kXTileBytes = kRows * kXRowBytes;  // 16 KiB
constexpr int kWRowBytes = 128 * 2;             // one half: 128 columns
constexpr int kWHalfBytes = kK * kWRowBytes;    // 8 KiB
constexpr int kWHalfBlocks = kWHalfBytes / 1024;         // 1 KiB load blocks per W half
constexpr int kXLoads = kXTileBytes / 1024 / kWaves;     // 1 KiB loads per wave per stage
constexpr int kXcds = 8;
constexpr int64_t kNarrowBelowTiles = 256;      // 256-column tiles fill the device from this many
constexpr int32_t kBufferFlags = 0x00020000;    // raw buffer, 32-bit data format

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

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Chunk-index XOR of an x tile row (4 chunks of 16 bytes): 16 consecutive
// rows read at one chunk index fall on 16 different 16-byte bank groups.
__device__ __forceinline__ int x_xor(int row) { return (row >> 2) & 3; }

// s_waitcnt immediate that waits for vector memory only, down to n
// outstanding operations (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// in 6:4, lgkmcnt in 11:8).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Chunk-index XOR of a W half-tile row (16 chunks of 16 bytes).
__device__ __forceinline__ int w_xor(int k) { return ((k & 3) << 2) | ((k >> 2) & 3); }

// LDS byte offset of column `col` (multiple of 4) in row k of a W half tile.
__device__ __forceinline__ int w_off(int k, int col) {
  return k * kWRowBytes + (((col >> 3) ^ w_xor(k)) << 4) + (col & 7) * 2;
}

}  // namespace pm

// NCOLS: output columns per workgroup, 256 or 128 (twice the workgroups for
// short inputs, at more LDS reads per MFMA).
// Wave tiles: without a gain each wave owns 64 rows x NCOLS/2 columns (4 x 2
// waves); with a gain each wave owns 32 rows x NCOLS columns (8 x 1 waves),
// so every x fragment is split into hi + lo by one wave only, for twice the
// W reads per MFMA.  The MFMAs of an output element are the same in both.
template <int NCOLS, bool kGain>
struct PmShape {
  static constexpr int kColsT = NCOLS;
  static constexpr int kHalves = NCOLS / 128;                           // [64][128] W half tiles per stage
  static constexpr int kWLoadsT = kHalves * pm::kWHalfBytes / 1024 / pm::kWaves;
  static constexpr int kRB = kGain ? 1 : 2;                             // 32-row blocks per wave
  static constexpr int kWavesR = pm::kWaves / kRB;                      // waves along the rows
  static constexpr int kWaveRows = 32 * kRB;
  static constexpr int kWaveCols = NCOLS / kRB;                         // columns of one wave
  static constexpr int NT = kWaveCols / 32;                             // 32-column accumulator tiles per wave
};

template <bool kGain, int NCOLS>
__global__ __launch_bounds__(pm::kThreads, 1) void project_mfma_kernel(const ProjArgs a) {
  using namespace pm;
  using Sh = PmShape<NCOLS, kGain>;
  constexpr int kColsT = Sh::kColsT;
  constexpr int kHalves = Sh::kHalves;
  constexpr int kWaveCols = Sh::kWaveCols;
  constexpr int NT = Sh::NT;
  constexpr int kRB = Sh::kRB;
  // One array per ring slot, selected at compile time: the compiler can then
  // tell that reads of one slot do not alias the direct-to-LDS loads still
  // landing in the others, and waits only as the counted waits below say.
  __shared__ __attribute__((aligned(1024))) char lds_x0[kXTileBytes];
  __shared__ __attribute__((aligned(1024))) char lds_x1[kXTileBytes];
  __shared__ __attribute__((aligned(1024))) char lds_x2[kXTileBytes];
  __shared__ __attribute__((aligned(1024))) char lds_x3[kXTileBytes];
  __shared__ __attribute__((aligned(1024))) char lds_w0[kHalves * kWHalfBytes];
  __shared__ __attribute__((aligned(1024))) char lds_w1[kHalves * kWHalfBytes];
  __shared__ __attribute__((aligned(1024))) char lds_w2[kHalves * kWHalfBytes];
  __shared__ __attribute__((aligned(1024))) char lds_w3[kHalves * kWHalfBytes];
  // Gains of a slice: each wave stages its own copy (64 floats, of which the
  // slice's 32 are read), so every wave issues the same loads.
  __shared__ __attribute__((aligned(1024))) float lds_g0[kWaves * 64];
  __shared__ __attribute__((aligned(1024))) float lds_g1[kWaves * 64];
  __shared__ __attribute__((aligned(1024))) float lds_g2[kWaves * 64];
  __shared__ __attribute__((aligned(1024))) float lds_g3[kWaves * 64];
  __shared__ double lds_rev[64];  // RoPE turns per position, per pair of a head
  auto xslot = [&](auto b_c) __attribute__((always_inline)) -> char * {
    constexpr int B = decltype(b_c)::value;
    if constexpr (B == 0) return lds_x0;
    else if constexpr (B == 1) return lds_x1;
    else if constexpr (B == 2) return lds_x2;
    else return lds_x3;
  };
  auto wslot = [&](auto b_c) __attribute__((always_inline)) -> char * {
    constexpr int B = decltype(b_c)::value;
    if constexpr (B == 0) return lds_w0;
    else if constexpr (B == 1) return lds_w1;
    else if constexpr (B == 2) return lds_w2;
    else return lds_w3;
  };
  auto gslot = [&](auto b_c) __attribute__((always_inline)) -> float * {
    constexpr int B = decltype(b_c)::value;
    if constexpr (B == 0) return lds_g0;
    else if constexpr (B == 1) return lds_g1;
    else if constexpr (B == 2) return lds_g2;
    else return lds_g3;
  };

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5;
  const int col = lane & 31;

  // Block -> (row tile, column tile): the column tiles of one row tile run
  // on consecutive slots of one XCD, so their x rows are shared in its L2.
  const int col_tiles_per_out = a.ncols / kColsT;
  const int col_tiles = col_tiles_per_out * a.n_out;
  const int row_tiles = static_cast<int>((a.n + kRows - 1) / kRows);
  const int xcd = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int row_tile = (slot / col_tiles) * kXcds + xcd;
  if (row_tile >= row_tiles) return;
  const int ct = slot % col_tiles;
  const int p = ct / col_tiles_per_out;
  const int col0 = (ct % col_tiles_per_out) * kColsT;
  const int64_t row0 = static_cast<int64_t>(row_tile) * kRows;
  const int rows_here = a.n - row0 < kRows ? static_cast<int>(a.n - row0) : kRows;
  const int d = a.d;
  const int n_stages = d / kK;

  const bf16_t *xg = static_cast<const bf16_t *>(a.x) + row0 * d;
  const bf16_t *wg = static_cast<const bf16_t *>(a.w[p]);
  const __amdgpu_buffer_rsrc_t x_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t *>(xg), 0, rows_here * d * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t w_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t *>(wg), 0, d * a.ncols * 2, kBufferFlags);
  __amdgpu_buffer_rsrc_t g_rsrc;
  if constexpr (kGain) g_rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(a.gain), 0, d * 4, kBufferFlags);
  // Descriptors of zero size for the slices past the last one: every lane is
  // out of range, so those loads touch no memory (they land zeros in a slot
  // nobody reads).  Issuing them keeps the staging unconditional, and with it
  // the count of loads in flight the same at every step.
  const __amdgpu_buffer_rsrc_t x_none = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t *>(xg), 0, 0, kBufferFlags);
  const __amdgpu_buffer_rsrc_t w_none = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t *>(wg), 0, 0, kBufferFlags);

  // Per-lane byte offsets of this wave's staging loads.  x block b (16
  // rows): lane L -> row b*16 + L/4, LDS slot L%4 holding global chunk
  // slot^x_xor(row).  W block b (4 rows of half b/8): lane L -> row
  // (b%8)*4 + L/16, slot L%16 holding global chunk slot^w_xor(row).
  // (wsoff has its 256-column size for both widths: host compilation drops
  // the kernel's instantiation when the buffer-load builtins below see an
  // operand whose type depends on NCOLS.)
  constexpr int kWLoadsMax = 2 * kWHalfBytes / 1024 / kWaves;
  uint32_t xsoff[kXLoads], wsoff[kWLoadsMax];
#pragma unroll
  for (int i = 0; i < kXLoads; ++i) {
    const int row = (wave * kXLoads + i) * 16 + (lane >> 2);
    const int chunk = (lane & 3) ^ x_xor(row);
    xsoff[i] = static_cast<uint32_t>(row * d * 2 + chunk * 16);
  }
#pragma unroll
  for (int i = 0; i < kWLoadsMax; ++i) {
    const int blk = wave * Sh::kWLoadsT + (i < Sh::kWLoadsT ? i : 0);
    const int k = (blk % kWHalfBlocks) * 4 + (lane >> 4);
    const int chunk = (lane & 15) ^ w_xor(k);
    wsoff[i] = static_cast<uint32_t>((k * a.ncols + (blk / kWHalfBlocks) * 128) * 2 + chunk * 16);
  }
  auto stage = [&](auto b_c, int s) __attribute__((always_inline)) {
    char *xdst = xslot(b_c);
    char *wdst = wslot(b_c);
    float *gdst = gslot(b_c);
    const bool live = s < n_stages;  // block-uniform
    const int sl = live ? s : 0;
    const uint32_t k0 = static_cast<uint32_t>(sl * kK);
    const __amdgpu_buffer_rsrc_t xr = live ? x_rsrc : x_none;
    const __amdgpu_buffer_rsrc_t wr_ = live ? w_rsrc : w_none;
#pragma unroll
    for (int i = 0; i < kXLoads; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void_t *)(xdst + (wave * kXLoads + i) * 1024), 16, xsoff[i],
                                               k0 * 2, 0, 0);
    }
    const uint32_t wbase = (k0 * a.ncols + col0) * 2;
#pragma unroll
    for (int i = 0; i < kWLoadsMax; ++i) {
      if (i >= Sh::kWLoadsT) break;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wr_, (lds_void_t *)(wdst + (wave * Sh::kWLoadsT + i) * 1024), 16, wsoff[i],
                                               wbase, 0, 0);
    }
    if constexpr (kGain) {
      // The 32 gains of this slice, 4 bytes per lane (lanes 32..63 fetch the
      // next ones, unused).  The slice offset goes into the per-lane offset,
      // not the scalar one: the range check of a raw buffer load sees only
      // the per-lane offset, so past the last slice those lanes read zeros,
      // never past the gains.
      __builtin_amdgcn_raw_ptr_buffer_load_lds(g_rsrc, (lds_void_t *)(gdst + wave * 64), 4, lane * 4u + k0 * 4, 0, 0, 0);
    }
  };

  // Wave tile: rows wr*kWaveRows + s*32 (s < kRB), columns wc*kWaveCols + t*32 (t < NT).
  const int wr = wave % Sh::kWavesR;
  const int wc = wave / Sh::kWavesR;
  // B (x^T) read: row wr*kWaveRows + s*32 + col, chunk 2*ks + half;
  // x_xor(row) = x_xor(col) (wave rows start at multiples of 32).
  constexpr int kKSteps = kK / 16;
  int xoff[kKSteps];
#pragma unroll
  for (int ks = 0; ks < kKSteps; ++ks) xoff[ks] = (wr * Sh::kWaveRows + col) * kXRowBytes + (((2 * ks + half) ^ x_xor(col)) << 4);
  // A (W^T) reads: in each 16-lane group, source lane a + 4j points at k row
  // kb + j, columns cb + 4a .. +3, and lane i of the group receives k rows
  // kb..kb+3 of column cb + i.  Lanes 0..31 take k rows 0..7 of the step (two
  // reads: kb = 0 and 4), lanes 32..63 rows 8..15, matching the B operand.
  const int grp = lane >> 4;
  const int src_a = lane & 3;
  const int src_j = (lane >> 2) & 3;
  const int krow = (grp >> 1) * 8 + src_j;
  const int ccol = (grp & 1) * 16 + src_a * 4;
  // Column tile t of the wave (32 columns from cw = wc*kWaveCols + t*32)
  // sits in W half tile cw/128 at column cw%128 of that half.
  int woff[2][NT];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
      woff[r][t] = ((wc * kWaveCols + t * 32) / 128) * kWHalfBytes +
                   w_off(krow + 4 * r, (wc * kWaveCols + t * 32) % 128 + ccol);
  }

  floatx16 acc[NT][kRB];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int s2 = 0; s2 < kRB; ++s2) {
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[t][s2][i] = 0.f;
    }
  }
  float sumsq[kRB];
#pragma unroll
  for (int s2 = 0; s2 < kRB; ++s2) sumsq[s2] = 0.f;

  auto compute = [&](const char *xt, const char *wt, const float *gt) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      Frag8 b[kRB];
#pragma unroll
      for (int s2 = 0; s2 < kRB; ++s2) b[s2].u = *reinterpret_cast<const uint4 *>(xt + xoff[ks] + s2 * 32 * kXRowBytes);
      Frag8 af[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        af[t].s4[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4_t *)(wt + woff[0][t] + ks * 16 * kWRowBytes));
        af[t].s4[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4_t *)(wt + woff[1][t] + ks * 16 * kWRowBytes));
      }
#pragma unroll
      for (int s2 = 0; s2 < kRB; ++s2) {
#pragma unroll
        for (int j = 0; j < 4; ++j) sumsq[s2] = dot2_bf16(b[s2].w[j], b[s2].w[j], sumsq[s2]);
      }
      if constexpr (kGain) {
        const float4 g0 = *reinterpret_cast<const float4 *>(gt + wave * 64 + ks * 16 + half * 8);
        const float4 g1 = *reinterpret_cast<const float4 *>(gt + wave * 64 + ks * 16 + half * 8 + 4);
        const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
        for (int s2 = 0; s2 < kRB; ++s2) {
          Frag8 hi, lo;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float x0 = __uint_as_float(b[s2].w[j] << 16) * g[2 * j];
            const float x1 = __uint_as_float(b[s2].w[j] & 0xffff0000u) * g[2 * j + 1];
            hi.w[j] = cvt_pk_bf16(x0, x1);
            lo.w[j] = cvt_pk_bf16(x0 - __uint_as_float(hi.w[j] << 16), x1 - __uint_as_float(hi.w[j] & 0xffff0000u));
          }
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            acc[t][s2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[t].v, hi.v, acc[t][s2], 0, 0, 0);
            acc[t][s2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[t].v, lo.v, acc[t][s2], 0, 0, 0);
          }
        }
      } else {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
#pragma unroll
          for (int s2 = 0; s2 < kRB; ++s2) {
            acc[t][s2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[t].v, b[s2].v, acc[t][s2], 0, 0, 0);
          }
        }
      }
      // One k-step's operands in flight at a time (the accumulators take
      // half the registers).  The 128-column tiles (half the accumulators)
      // leave the compiler free to read ahead across k-steps, which measured
      // faster there and slower for the 256-column tiles.
      if constexpr (NCOLS == 256) __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Vector memory operations per wave per slice, for the counted waits.
  constexpr int kLoads = kXLoads + Sh::kWLoadsT + (kGain ? 1 : 0);
  // Slice s sits in ring slot s % 4; n_stages is a multiple of 4 (d_model %
  // 128 == 0), so the loop runs four slices per pass and every slot is a
  // compile-time choice.  Every step stages a slice (the last three steps
  // stage empty ones), so the compiler's own wait tracking sees the same
  // loads in flight on every path and needs no wait of its own.
  auto step = [&](auto b_c, int s) __attribute__((always_inline)) {
    constexpr int B = decltype(b_c)::value;
    // Slice s has landed for every wave: this wave waits until only the
    // loads of the two later slices it has issued are outstanding, then the
    // barrier.  Every wave is then also done with slice s-1, whose slot
    // slice s+3 takes.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kLoads));
    // A plain barrier: __syncthreads() adds a workgroup release fence, which
    // would wait for every load still landing in LDS.  LDS is one memory for
    // the workgroup, so the counted wait above is what orders this wave's
    // landed slice before the others' reads; the empty asm statements keep
    // the compiler from moving memory accesses across the barrier.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    stage(std::integral_constant<int, (B + kStages - 1) % kStages>(), s + kStages - 1);
    compute(xslot(b_c), wslot(b_c), gslot(b_c));
  };
  stage(std::integral_constant<int, 0>(), 0);
  stage(std::integral_constant<int, 1>(), 1);
  stage(std::integral_constant<int, 2>(), 2);
  for (int s = 0; s < n_stages; s += kStages) {
    step(std::integral_constant<int, 0>(), s);
    step(std::integral_constant<int, 1>(), s + 1);
    step(std::integral_constant<int, 2>(), s + 2);
    step(std::integral_constant<int, 3>(), s + 3);
  }
  // The empty slices' loads land before the workgroup's LDS is released.
  __builtin_amdgcn_s_waitcnt(0);

  // Epilogue: acc[t][s2] element i is output column
  //   col0 + wc*kWaveCols + t*32 + (i/4)*8 + half*4 + (i%4)
  // of input row row0 + wr*kWaveRows + s2*32 + col.  With RoPE, columns (2i, 2i+1)
  // of a head sit in elements (i4*4 + 2j, i4*4 + 2j + 1) of the same lane.
  const bool rope = a.rope_out == p;  // block-uniform
  if (rope) {
    if (threadIdx.x < a.head_dim / 2) lds_rev[threadIdx.x] = rope_rev(threadIdx.x, a.head_dim, a.rope_log2_theta);
    __syncthreads();
  }
  bf16_t *out = static_cast<bf16_t *>(a.out[p]);
#pragma unroll
  for (int s2 = 0; s2 < kRB; ++s2) {
    const float ss = sumsq[s2] + shfl_xor_f(sumsq[s2], 32);
    const int r = wr * Sh::kWaveRows + s2 * 32 + col;
    if (r >= rows_here) continue;
    const float inv = 1.0f / sqrtf(ss / static_cast<float>(d) + a.eps);
    bf16_t *orow = out + (a.dst_row_base + row0 + r) * a.out_stride + col0 + wc * kWaveCols;
    const int64_t pos = rope ? proj_row_pos(a, row0 + r) : 0;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        float v0 = acc[t][s2][i4 * 4 + 0] * inv, v1 = acc[t][s2][i4 * 4 + 1] * inv;
        float v2 = acc[t][s2][i4 * 4 + 2] * inv, v3 = acc[t][s2][i4 * 4 + 3] * inv;
        if (rope) {
          const int pair = ((col0 + wc * kWaveCols + t * 32 + i4 * 8 + half * 4) % a.head_dim) >> 1;
          rope_turn(v0, v1, pos, lds_rev[pair]);
          rope_turn(v2, v3, pos, lds_rev[pair + 1]);
        }
        uint2 v;
        v.x = cvt_pk_bf16(v0, v1);
        v.y = cvt_pk_bf16(v2, v3);
        *reinterpret_cast<uint2 *>(orow + t * 32 + i4 * 8 + half * 4) = v;
      }
    }
  }
}

bool project_mfma_applies(const ProjArgs &a, int x_dt, int w_dt, int o_dt) {
  return x_dt == YOCO_DT_BF16 && w_dt == YOCO_DT_BF16 && o_dt == YOCO_DT_BF16 && !a.indexed && a.n > 0 &&
         a.d % (pm::kStages * pm::kK) == 0 && a.ncols % pm::kCols == 0 &&
         static_cast<int64_t>(a.d) * a.ncols * 2 < (int64_t(1) << 31) &&
         static_cast<int64_t>(pm::kRows) * a.d * 2 < (int64_t(1) << 31);
}

template <int NCOLS>
static hipError_t launch_project_mfma_t(const ProjArgs &a, int64_t row_tiles, hipStream_t s) {
  const int64_t col_tiles = static_cast<int64_t>(a.ncols / NCOLS) * a.n_out;
  const int64_t blocks = (row_tiles + pm::kXcds - 1) / pm::kXcds * pm::kXcds * col_tiles;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (a.gain != nullptr) {
    hipLaunchKernelGGL((project_mfma_kernel<true, NCOLS>), dim3(static_cast<unsigned>(blocks)), dim3(pm::kThreads), 0,
                       s, a);
  } else {
    hipLaunchKernelGGL((project_mfma_kernel<false, NCOLS>), dim3(static_cast<unsigned>(blocks)), dim3(pm::kThreads), 0,
                       s, a);
  }
  return hipGetLastError();
}

// 256-column tiles unless they leave CUs idle (fewer tiles than the 256 CUs
// of the device, e.g. 4096 rows at 2 x 1024 columns): then 128-column tiles.
hipError_t launch_project_mfma(const ProjArgs &a, hipStream_t s) {
  const int64_t row_tiles = (a.n + pm::kRows - 1) / pm::kRows;
  const int64_t tiles256 = row_tiles * (a.ncols / pm::kCols) * a.n_out;
  if (tiles256 < pm::kNarrowBelowTiles) return launch_project_mfma_t<128>(a, row_tiles, s);
  return launch_project_mfma_t<256>(a, row_tiles, s);
}

}  // namespace yoco
