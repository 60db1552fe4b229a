// RMSNorm gain folded into the projection weights (a weight preparation,
// run once per model, not per token).
//
// [Notes] "YOCO：You Only Cache Once 中文精读笔记" s.2.1 Eq. 2 and Eq. 3 put
// an RMSNorm with a per-channel gain in front of every projection:
//   LN(x) W = (x * g / r) W = (x / r) (diag(g) W),  r = sqrt(mean x^2 + eps).
// With W' = diag(g) W the projection kernels run with unit gain: prompt-sized
// projections then take one bf16 product per fragment on the matrix cores,
// where an fp32 gain applied to the activations takes two (x*g entered as a
// bf16 hi + lo pair so that it is not rounded).  The gain's rounding moves to
// the weights, once per element:
//   w_out[c][j] = RNE_bf16(fp32(w[c][j]) * g[c])   (fp32 product, IEEE).
//
// An elementwise pass over d x n_cols weights, bound by HBM: each lane reads
// 8 consecutive elements of one row (16 or 32 bytes) and writes 16 bytes;
// rows whose length is not a multiple of 8 take one element per lane.  Each
// lane writes only what it has read, so w and out may be the same bf16 array.
#include "device_common.h"
#include "yoco_internal.h"

namespace yoco {

namespace {

constexpr int kFoldThreads = 256;
constexpr int64_t kFoldMaxBlocks = 256 * 16;  // 16 workgroups per CU; the loop covers the rest

template <typename TW>
__global__ __launch_bounds__(kFoldThreads) void fold_gain8_kernel(const TW *w,
                                                                  const float *__restrict__ gain,
                                                                  bf16_t *out, int64_t n_groups,
                                                                  int32_t groups_per_row) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kFoldThreads;
  for (int64_t gi = static_cast<int64_t>(blockIdx.x) * kFoldThreads + threadIdx.x; gi < n_groups; gi += stride) {
    const float g = gain[gi / groups_per_row];
    Vec8<TW> v;
    v.load(w + gi * 8);
    uint4 o;
    o.x = pack_bf16x2(v[0] * g, v[1] * g);
    o.y = pack_bf16x2(v[2] * g, v[3] * g);
    o.z = pack_bf16x2(v[4] * g, v[5] * g);
    o.w = pack_bf16x2(v[6] * g, v[7] * g);
    *reinterpret_cast<uint4 *>(out + gi * 8) = o;
  }
}

template <typename TW>
__global__ __launch_bounds__(kFoldThreads) void fold_gain1_kernel(const TW *w,
                                                                  const float *__restrict__ gain,
                                                                  bf16_t *out, int64_t n_elems,
                                                                  int32_t n_cols) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kFoldThreads;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kFoldThreads + threadIdx.x; i < n_elems; i += stride)
    out[i] = f32_to_bf16(load_elem<TW>(w + i) * gain[i / n_cols]);
}

template <typename TW>
hipError_t launch_fold_t(const void *w, const float *gain, int32_t d, int32_t n_cols, void *out, hipStream_t s) {
  const int64_t n_elems = static_cast<int64_t>(d) * n_cols;
  const bool vec = n_cols % 8 == 0;
  const int64_t items = vec ? n_elems / 8 : n_elems;
  int64_t blocks = (items + kFoldThreads - 1) / kFoldThreads;
  if (blocks > kFoldMaxBlocks) blocks = kFoldMaxBlocks;
  if (vec) {
    hipLaunchKernelGGL(fold_gain8_kernel<TW>, dim3(static_cast<unsigned>(blocks)), dim3(kFoldThreads), 0, s,
                       static_cast<const TW *>(w), gain, static_cast<bf16_t *>(out), items, n_cols / 8);
  } else {
    hipLaunchKernelGGL(fold_gain1_kernel<TW>, dim3(static_cast<unsigned>(blocks)), dim3(kFoldThreads), 0, s,
                       static_cast<const TW *>(w), gain, static_cast<bf16_t *>(out), items, n_cols);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fold_gain(const void *w, int w_dt, const float *gain, int32_t d, int32_t n_cols, void *out,
                            hipStream_t s) {
  if (w_dt == YOCO_DT_BF16) return launch_fold_t<bf16_t>(w, gain, d, n_cols, out, s);
  if (w_dt == YOCO_DT_F32) return launch_fold_t<float>(w, gain, d, n_cols, out, s);
  return hipErrorInvalidValue;
}

}  // namespace yoco
