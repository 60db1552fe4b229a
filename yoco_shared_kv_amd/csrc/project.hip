// Fused RMSNorm + projection, written straight to its destination rows.
//
// What it computes ([Notes] "YOCO：You Only Cache Once 中文精读笔记" s.2.1
// Eq. 2: K^ = LN(M) W_K, V^ = LN(M) W_V with LN = RMSNorm, projected once at
// the self/cross boundary; Eq. 3: Q^l = LN(X^l) W_Q^l):
//   out_p[dst(r)][j] = (sum_c x[r][c] * gain[c] * W_p[c][j]) / rms_r,
//   rms_r = sqrt(mean_c x[r][c]^2 + eps).
// Dividing after the sum is the same value as normalising first, since the
// row factor 1/rms_r is common to every term.
//
// Two kernels share this arithmetic:
//  * prompt projections in bf16 with d_model % 64 == 0 and a multiple of 256
//    columns run on the matrix cores (project_mfma.hip); the others here:
//  * rows >= 9 (prompt projection): one workgroup computes a 64-row x
//    64-column tile of one output (K or V, or Q): it first reduces the 64 row
//    norms (fp32), then streams [64 x 32] slices of x (times gain) and
//    [32 x 64] slices of W through LDS and accumulates a 4x4 block per thread
//    with fp32 FMA.
//  * rows <= 8 (generation-time append, per-token Q): the work is a
//    matrix-vector product bound by reading W once, so one 1024-thread
//    workgroup (512 for 8 rows) owns a 16-column strip of one weight for all
//    d_model rows (128 workgroups for a 3072 x 1024 pair of weights).
//    Each 2-lane pair reads 32 bytes of a W row per load (a wave covers 32
//    rows, the workgroup 512 rows per pass, so a 3072-row weight is one pass
//    of loads in flight), multiplies them by the LDS-resident x*gain of every
//    input row, and the per-lane partial sums are reduced across lanes
//    (shuffles) and waves (LDS) in a fixed order.
//    Rows run in launches of up to 8 (fewer when d_model is large, since a
//    launch stages x*gain in at most 48 KiB of LDS).
// Destination rows are either contiguous (a cache slab or a Q buffer) or, for
// the generation-time append, one indexed row per sequence.
#include "device_common.h"
#include "rope.h"
#include "yoco_internal.h"

namespace yoco {

namespace pj {
constexpr int BM = 64;
constexpr int BN = 64;
constexpr int BK = 32;
constexpr int kThreads = 256;
}  // namespace pj

template <typename TX, typename TW, typename TO>
__global__ __launch_bounds__(pj::kThreads) void project_kernel(const ProjArgs a) {
  using namespace pj;
  __shared__ float s_x[BK][BM + 4];   // x * gain, transposed: [k][row]
  __shared__ float s_w[BK][BN + 4];
  __shared__ float s_inv_rms[BM];

  const int tid = threadIdx.x;
  const int n_col_tiles = a.ncols / BN;
  const int col_tile = blockIdx.x % n_col_tiles;
  const int out_id = (blockIdx.x / n_col_tiles) % a.n_out;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x / (n_col_tiles * a.n_out)) * BM;
  const TX *x = static_cast<const TX *>(a.x);
  const TW *w = static_cast<const TW *>(a.w[out_id]);
  const int d = a.d;

  // Row norms: 4 threads per row, then a 4-lane DPP sum.
  {
    const int rr = tid >> 2;
    const int part = tid & 3;
    const int64_t row = row0 + rr;
    float ss = 0.f;
    if (row < a.n) {
      const TX *xr = x + row * d;
      for (int c = part; c < d; c += 4) {
        const float v = load_elem<TX>(xr + c);
        ss = fmaf(v, v, ss);
      }
    }
    ss = group_sum<4>(ss);
    if (part == 0) s_inv_rms[rr] = 1.0f / sqrtf(ss / static_cast<float>(d) + a.eps);
  }

  // 16 x 16 threads, each a 4 x 4 block: rows ty*4.., cols tx*4..
  const int tx = tid & 15;
  const int ty = tid >> 4;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

  for (int k0 = 0; k0 < d; k0 += BK) {
    __syncthreads();
    // x slice [BM][BK]: 2048 elements, 8 per thread.
#pragma unroll
    for (int it = 0; it < (BM * BK) / kThreads; ++it) {
      const int idx = tid + it * kThreads;
      const int rr = idx / BK;
      const int kk = idx - rr * BK;
      const int64_t row = row0 + rr;
      const int c = k0 + kk;
      float v = 0.f;
      if (row < a.n && c < d) {
        v = load_elem<TX>(x + row * d + c);
        if (a.gain != nullptr) v *= a.gain[c];
      }
      s_x[kk][rr] = v;
    }
    // W slice [BK][BN].
#pragma unroll
    for (int it = 0; it < (BK * BN) / kThreads; ++it) {
      const int idx = tid + it * kThreads;
      const int kk = idx / BN;
      const int cc = idx - kk * BN;
      const int c = k0 + kk;
      s_w[kk][cc] = (c < d) ? load_elem<TW>(w + static_cast<int64_t>(c) * a.ncols + col_tile * BN + cc) : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < BK; ++kk) {
      float xv[4], wv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) xv[i] = s_x[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) wv[j] = s_w[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(xv[i], wv[j], acc[i][j]);
    }
  }

  TO *out = static_cast<TO *>(a.out[out_id]);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = ty * 4 + i;
    const int64_t row = row0 + rr;
    if (row >= a.n) continue;
    const int64_t dst = a.indexed ? a.dst_rows[row] : a.dst_row_base + row;
    const float inv = s_inv_rms[rr];
    TO *orow = out + dst * a.out_stride + col_tile * BN + tx * 4;
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = acc[i][j] * inv;
    if (a.rope_out == out_id) {
      // columns tx*4 .. +3 are pairs (2i, 2i+1) and (2i+2, 2i+3) of a head
      const int pair = ((col_tile * BN + tx * 4) % a.head_dim) >> 1;
      const int64_t pos = proj_row_pos(a, row);
      rope_turn(v[0], v[1], pos, rope_rev(pair, a.head_dim, a.rope_log2_theta));
      rope_turn(v[2], v[3], pos, rope_rev(pair + 1, a.head_dim, a.rope_log2_theta));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) store_elem<TO>(orow + j, v[j]);
  }
}


namespace pg {
// 16 waves (8 for 8 input rows, whose accumulators need the larger
// per-lane register budget of a 512-thread workgroup).
constexpr int kCols = 16;            // columns per workgroup: 2 lanes x 8 columns per W row
constexpr int kLanesPerRow = kCols / 8;
constexpr int kRowSlots = 64 / kLanesPerRow;  // W rows one wave reads per load
template <int NR>
struct Shape {
  static constexpr int kWaves = (NR == 8) ? 8 : 16;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kRowsPerPass = kWaves * kRowSlots;
};
constexpr int kMaxRows = 8;
constexpr int kMaxXBytes = 48 * 1024;  // dynamic LDS for x * gain (within the default 64 KiB)
constexpr int kMaxChunks = 4;          // launches per call before the tiled kernel takes over
constexpr int kXcds = 8;               // workgroups are dealt to the XCDs round-robin
}  // namespace pg

// W loads of 8 consecutive columns as fp32.
template <typename TW>
__device__ __forceinline__ void load_w8(const TW *p, float (&w)[8]);
template <>
__device__ __forceinline__ void load_w8<bf16_t>(const bf16_t *p, float (&w)[8]) {
  const uint4 v = ld16_stream(p);
  w[0] = bf16_lo(v.x); w[1] = bf16_hi(v.x); w[2] = bf16_lo(v.y); w[3] = bf16_hi(v.y);
  w[4] = bf16_lo(v.z); w[5] = bf16_hi(v.z); w[6] = bf16_lo(v.w); w[7] = bf16_hi(v.w);
}
template <>
__device__ __forceinline__ void load_w8<float>(const float *p, float (&w)[8]) {
  const uint4 a = ld16_stream(p), b = ld16_stream(p + 4);
  w[0] = __uint_as_float(a.x); w[1] = __uint_as_float(a.y); w[2] = __uint_as_float(a.z); w[3] = __uint_as_float(a.w);
  w[4] = __uint_as_float(b.x); w[5] = __uint_as_float(b.y); w[6] = __uint_as_float(b.z); w[7] = __uint_as_float(b.w);
}

// Rows [row_base, row_base + nr) of the input, nr <= NR <= 8.
template <typename TX, typename TW, typename TO, int NR>
__global__ __launch_bounds__(pg::Shape<NR>::kThreads) void project_small_kernel(const ProjArgs a, int64_t row_base,
                                                                               int nr) {
  using namespace pg;
  constexpr int kWaves = Shape<NR>::kWaves;
  constexpr int kThreads = Shape<NR>::kThreads;
  constexpr int kRowsPerPass = Shape<NR>::kRowsPerPass;
  extern __shared__ float s_dyn[];
  float *s_x = s_dyn;                          // [NR][d]
  __shared__ float s_red[kWaves][NR][kCols];
  __shared__ float s_inv_rms[NR];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // Consecutive workgroups go to consecutive XCDs, and each XCD has its own
  // L2: XCD x takes a contiguous run of strips, so the 128-byte lines of a W
  // row that several strips share are fetched into one L2, not into four.
  const int n_strips = a.ncols / kCols;
  const int per_xcd = (n_strips * a.n_out + kXcds - 1) / kXcds;
  const int linear = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (linear >= n_strips * a.n_out) return;
  const int strip = linear % n_strips;
  const int out_id = linear / n_strips;
  const int d = a.d;
  const TX *x = static_cast<const TX *>(a.x);
  const TW *w = static_cast<const TW *>(a.w[out_id]);
  const int c8 = lane % kLanesPerRow;     // 8-column chunk of the strip
  const int rslot = lane / kLanesPerRow;  // row within the wave's kRowSlots rows
  constexpr int kUnroll = (NR <= 2) ? 8 : 4;
  const TW *wcol = w + strip * kCols + c8 * 8;
  float wv[kUnroll][8];
  auto load_batch = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int k = k0 + u * kRowsPerPass + wave * kRowSlots + rslot;
      load_w8<TW>(wcol + static_cast<int64_t>(k < d ? k : d - 1) * a.ncols, wv[u]);
    }
  };
  load_batch(0);

  // Stage x * gain (fp32); the same loads give each thread's share of the
  // row sums of squares, which reduce over lanes (shuffles) and then waves
  // (LDS, in wave order).
  __shared__ float s_ss[kWaves][NR];
  float ssp[NR];
#pragma unroll
  for (int rr = 0; rr < NR; ++rr) ssp[rr] = 0.f;
  // Four elements per thread per round: the loads of a round are issued
  // before any of them is used (addresses clamped into the input, values
  // past it replaced by zero), so a round costs one memory round trip.
  constexpr int kStage = 4;
  for (int base = tid; base < NR * d; base += kStage * kThreads) {
    float v[kStage], g[kStage];
#pragma unroll
    for (int j = 0; j < kStage; ++j) {
      const int idx = base + j * kThreads;
      const int r = idx / d;
      const int c = idx - r * d;
      const int rc = r < nr ? r : 0;
      const int cc = idx < NR * d ? c : 0;
      v[j] = load_elem<TX>(x + (row_base + rc) * d + cc);
      g[j] = a.gain != nullptr ? a.gain[cc] : 1.f;
    }
#pragma unroll
    for (int j = 0; j < kStage; ++j) {
      const int idx = base + j * kThreads;
      const int r = idx / d;
      const float vj = (idx < NR * d && r < nr) ? v[j] : 0.f;
#pragma unroll
      for (int rr = 0; rr < NR; ++rr) ssp[rr] = (r == rr) ? fmaf(vj, vj, ssp[rr]) : ssp[rr];
      if (idx < NR * d) s_x[idx] = vj * g[j];
    }
  }
#pragma unroll
  for (int rr = 0; rr < NR; ++rr) {
    float t = ssp[rr];
#pragma unroll
    for (int sft = 32; sft >= 1; sft >>= 1) t += shfl_xor_f(t, sft);
    if (lane == 0) s_ss[wave][rr] = t;
  }
  __syncthreads();
  if (tid < NR) {
    float ss = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < kWaves; ++w2) ss += s_ss[w2][tid];
    s_inv_rms[tid] = 1.0f / sqrtf(ss / static_cast<float>(d) + a.eps);
  }
  __syncthreads();

  float acc[NR][8];
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[r][e] = 0.f;

  // W rows in flight per lane; fewer for more input rows (more accumulators).
  // All kUnroll loads of a batch are issued before the first is used: rows
  // past d read row d-1 and are zeroed afterwards (no branch around a load).
  // The first batch is issued before x is staged (one batch covers
  // d <= 4096 for up to two input rows); later batches at the top of their
  // iteration.
  for (int k0 = 0; k0 < d; k0 += kRowsPerPass * kUnroll) {
    if (k0 > 0) load_batch(k0);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int k = k0 + u * kRowsPerPass + wave * kRowSlots + rslot;
      const bool in = k < d;
      const int kc = in ? k : d - 1;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const float xv = in ? s_x[r * d + kc] : 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][e] = fmaf(xv, wv[u][e], acc[r][e]);
      }
    }
  }

  // Reduce over the row slots of the wave (the lane bits above the chunk),
  // then over the waves.
#pragma unroll
  for (int sft = kLanesPerRow; sft < 64; sft <<= 1) {
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[r][e] += shfl_xor_f(acc[r][e], sft);
  }
  if (rslot == 0) {
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int e = 0; e < 8; ++e) s_red[wave][r][c8 * 8 + e] = acc[r][e];
  }
  __syncthreads();
  // One thread per column pair (2c, 2c+1), so the RoPE rotation has both.
  TO *out = static_cast<TO *>(a.out[out_id]);
  const bool rope = a.rope_out == out_id;
  for (int idx = tid; idx < NR * (kCols / 2); idx += kThreads) {
    const int r = idx / (kCols / 2);
    const int col = 2 * (idx - r * (kCols / 2));
    if (r >= nr) continue;
    float v0 = 0.f, v1 = 0.f;
#pragma unroll
    for (int wv2 = 0; wv2 < kWaves; ++wv2) {
      v0 += s_red[wv2][r][col];
      v1 += s_red[wv2][r][col + 1];
    }
    v0 *= s_inv_rms[r];
    v1 *= s_inv_rms[r];
    const int64_t row = row_base + r;
    if (rope) {
      const int pair = ((strip * kCols + col) % a.head_dim) >> 1;
      rope_turn(v0, v1, proj_row_pos(a, row), rope_rev(pair, a.head_dim, a.rope_log2_theta));
    }
    const int64_t dst = a.indexed ? a.dst_rows[row] : a.dst_row_base + row;
    store_elem<TO>(out + dst * a.out_stride + strip * kCols + col, v0);
    store_elem<TO>(out + dst * a.out_stride + strip * kCols + col + 1, v1);
  }
}

// Input rows per launch of the small-row kernel: the largest power of two
// <= 8 whose x*gain fits kMaxXBytes (0 if not even one row fits).
static int small_chunk_rows(int d) {
  int nr = pg::kMaxRows;
  while (nr > 0 && static_cast<int64_t>(nr) * d * 4 > pg::kMaxXBytes) nr >>= 1;
  return nr;
}

// Whether the small-row kernel takes this projection.
static bool use_small(const ProjArgs &a) {
  const int chunk = small_chunk_rows(a.d);
  return chunk > 0 && a.n <= static_cast<int64_t>(chunk) * pg::kMaxChunks;
}

template <typename TX, typename TW, typename TO>
static hipError_t launch_project_small(const ProjArgs &a, hipStream_t s) {
  const unsigned int per_xcd = static_cast<unsigned int>(((a.ncols / pg::kCols) * a.n_out + pg::kXcds - 1) / pg::kXcds);
  const unsigned int blocks = per_xcd * pg::kXcds;
  const int chunk = small_chunk_rows(a.d);
  for (int64_t base = 0; base < a.n; base += chunk) {
    const int nr = static_cast<int>(a.n - base < chunk ? a.n - base : chunk);
    const int nr_pow2 = nr <= 1 ? 1 : nr <= 2 ? 2 : nr <= 4 ? 4 : 8;
    const size_t lds = static_cast<size_t>(nr_pow2) * a.d * sizeof(float);
    switch (nr_pow2) {
      case 1: hipLaunchKernelGGL((project_small_kernel<TX, TW, TO, 1>), dim3(blocks), dim3(pg::Shape<1>::kThreads), lds, s, a, base, nr); break;
      case 2: hipLaunchKernelGGL((project_small_kernel<TX, TW, TO, 2>), dim3(blocks), dim3(pg::Shape<2>::kThreads), lds, s, a, base, nr); break;
      case 4: hipLaunchKernelGGL((project_small_kernel<TX, TW, TO, 4>), dim3(blocks), dim3(pg::Shape<4>::kThreads), lds, s, a, base, nr); break;
      default: hipLaunchKernelGGL((project_small_kernel<TX, TW, TO, 8>), dim3(blocks), dim3(pg::Shape<8>::kThreads), lds, s, a, base, nr); break;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename TX, typename TW>
static hipError_t launch_project_o(const ProjArgs &a, int o_dt, hipStream_t s) {
  const int64_t row_tiles = (a.n + pj::BM - 1) / pj::BM;
  const unsigned int blocks = static_cast<unsigned int>(row_tiles * (a.ncols / pj::BN) * a.n_out);
  if (use_small(a)) {
    if (o_dt == YOCO_DT_F32) return launch_project_small<TX, TW, float>(a, s);
    if (o_dt == YOCO_DT_BF16) return launch_project_small<TX, TW, bf16_t>(a, s);
    return hipErrorInvalidValue;
  }
  if (o_dt == YOCO_DT_F32) {
    hipLaunchKernelGGL((project_kernel<TX, TW, float>), dim3(blocks), dim3(pj::kThreads), 0, s, a);
  } else if (o_dt == YOCO_DT_BF16) {
    hipLaunchKernelGGL((project_kernel<TX, TW, bf16_t>), dim3(blocks), dim3(pj::kThreads), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename TX>
static hipError_t launch_project_w(const ProjArgs &a, int w_dt, int o_dt, hipStream_t s) {
  if (w_dt == YOCO_DT_F32) return launch_project_o<TX, float>(a, o_dt, s);
  if (w_dt == YOCO_DT_BF16) return launch_project_o<TX, bf16_t>(a, o_dt, s);
  return hipErrorInvalidValue;
}

hipError_t launch_project(const ProjArgs &a, int x_dt, int w_dt, int o_dt, hipStream_t s) {
  if (!use_small(a) && project_mfma_applies(a, x_dt, w_dt, o_dt)) return launch_project_mfma(a, s);
  if (x_dt == YOCO_DT_F32) return launch_project_w<float>(a, w_dt, o_dt, s);
  if (x_dt == YOCO_DT_BF16) return launch_project_w<bf16_t>(a, w_dt, o_dt, s);
  return hipErrorInvalidValue;
}

}  // namespace yoco
