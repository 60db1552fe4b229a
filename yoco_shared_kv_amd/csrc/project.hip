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
// One workgroup computes a 64-row x 64-column tile of one output (K or V, or
// Q): it first reduces the 64 row norms (fp32), then streams [64 x 32] slices
// of x (times gain) and [32 x 64] slices of W through LDS and accumulates a
// 4x4 block per thread with fp32 FMA.  Destination rows are either
// contiguous (a cache slab or a Q buffer) or, for the generation-time
// append, one indexed row per sequence.
#include "device_common.h"
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
    TO *orow = out + dst * a.ncols + col_tile * BN + tx * 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) store_elem<TO>(orow + j, acc[i][j] * inv);
  }
}

template <typename TX, typename TW>
static hipError_t launch_project_o(const ProjArgs &a, int o_dt, hipStream_t s) {
  const int64_t row_tiles = (a.n + pj::BM - 1) / pj::BM;
  const unsigned int blocks = static_cast<unsigned int>(row_tiles * (a.ncols / pj::BN) * a.n_out);
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
  if (x_dt == YOCO_DT_F32) return launch_project_w<float>(a, w_dt, o_dt, s);
  if (x_dt == YOCO_DT_BF16) return launch_project_w<bf16_t>(a, w_dt, o_dt, s);
  return hipErrorInvalidValue;
}

}  // namespace yoco
