// Few-row fused RMSNorm + projection, split over the reduction rows of W.
//
// What it computes is the projection of project.hip ([Notes] "YOCO：You Only
// Cache Once 中文精读笔记" s.2.1 Eq. 2: K^ = LN(M) W_K, V^ = LN(M) W_V, and
// Eq. 3: Q^l = LN(X^l) W_Q^l, LN = RMSNorm):
//   out_p[dst(r)][j] = (sum_c x[r][c] * gain[c] * W_p[c][j]) / rms_r,
//   rms_r = sqrt(mean_c x[r][c]^2 + eps).
// At generation time ([Notes] s.2.5: each new token's K/V row is appended;
// [Blog] "NeurIPS'24 | YOCO: 长上下文 LLM 为什么不必每层都存一份 KV Cache?"
// s.7: each cross layer projects its own Q) there are at most a few input
// rows, so the work is a matrix-vector product bound by reading W once.
//
// Decomposition (gfx950: 256 CUs, 64-wide waves):
//   * A column block is CB = 16 lanes x 16 bytes of a W row (128 bf16 or 64
//     fp32 columns of one weight); a wave's load instruction covers 4 W rows
//     x 256 contiguous bytes, so every 128-byte line it touches is used
//     whole.
//   * The d rows of W are cut into S splits of R rows (a multiple of 16);
//     workgroup (split, column block) streams its R x CB slice with every
//     load issued before the first is used, so the grid of S x blocks
//     (about 256 workgroups) keeps all CUs streaming.
//   * Each workgroup reduces its lanes (shuffles) and its 4 waves (LDS, in
//     wave order) into one partial row [NR][CB] plus the partial sums of
//     x^2 over its R input columns, and writes it with agent-scope stores.
//   * Arrival counters (one per column block and 128-byte line, in the
//     caller's workspace) find the last workgroup of each column block; it
//     adds the S partials
//     in split order (a fixed subset per task, the subsets combined in a
//     fixed order through LDS), so results are bitwise reproducible, then
//     applies 1/rms, the optional rotary embedding and the one rounding to
//     the output type, and resets its counter to zero.
#include "device_common.h"
#include "rope.h"
#include "yoco_internal.h"

namespace yoco {

namespace pr {
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kLanesPerSeg = 16;                  // lanes covering one W row segment
constexpr int kRowSlots = 64 / kLanesPerSeg;      // W rows per wave load instruction
constexpr int kRowsPerRound = kWaves * kRowSlots;  // W rows per workgroup load round
constexpr int kMaxLoads = 16;                     // W loads in flight per lane
constexpr int kMaxSplitRows = kMaxLoads * kRowsPerRound;  // 256
constexpr int kTargetBlocks = 256;                // one workgroup per CU
constexpr int kMaxInRows = 8;                     // input rows per launch
constexpr int kMergeSubs = 8;                     // split subsets the merge adds separately
constexpr int32_t kRowsBufferFlags = 0x00020000;  // raw buffer, 32-bit data format
}  // namespace pr

// Columns per block for a weight type: 16 lanes x 16 bytes.
static inline int rows_block_cols(int w_dt) { return w_dt == YOCO_DT_BF16 ? 128 : 64; }

bool project_rows_plan(int32_t d, int32_t ncols, int32_t n_out, int w_dt, ProjRowsPlan *p) {
  const int cb = rows_block_cols(w_dt);
  if (d < 1 || ncols < cb || ncols % cb != 0 || (n_out != 1 && n_out != 2)) return false;
  const int n_cb = n_out * (ncols / cb);
  if (n_cb > kProjRowsMaxBlocks) return false;
  int s = (pr::kTargetBlocks + n_cb - 1) / n_cb;
  int r = (d + s - 1) / s;
  r = ((r + pr::kRowsPerRound - 1) / pr::kRowsPerRound) * pr::kRowsPerRound;
  if (r > pr::kMaxSplitRows) r = pr::kMaxSplitRows;
  s = (d + r - 1) / r;
  p->n_cb = n_cb;
  p->splits = s;
  p->split_rows = r;
  p->block_cols = cb;
  p->part_floats = static_cast<int64_t>(n_cb) * s * pr::kMaxInRows * (cb + 4);
  return true;
}

size_t project_rows_workspace_bytes(const ProjRowsPlan &p) {
  return kProjRowsCounterBytes + static_cast<size_t>(p.part_floats) * sizeof(float);
}

namespace {

// Agent-scope (device-coherent) relaxed store / 16-byte load: partials are
// written on one XCD and read on another, and these bypass the per-XCD
// caches without a write-back or invalidate.
__device__ __forceinline__ void rows_store_agent(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float4 rows_load_agent4(const float4 *p) {
  const uint64_t *q = reinterpret_cast<const uint64_t *>(p);
  const uint64_t lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_float4(__uint_as_float(static_cast<uint32_t>(lo)), __uint_as_float(static_cast<uint32_t>(lo >> 32)),
                     __uint_as_float(static_cast<uint32_t>(hi)), __uint_as_float(static_cast<uint32_t>(hi >> 32)));
}

// The VE columns of one 16-byte W piece as fp32.
template <typename TW>
struct WPiece;
template <>
struct WPiece<bf16_t> {
  static constexpr int VE = 8;
  static __device__ __forceinline__ void unpack(const uint4 &v, float (&w)[8]) {
    w[0] = bf16_lo(v.x); w[1] = bf16_hi(v.x); w[2] = bf16_lo(v.y); w[3] = bf16_hi(v.y);
    w[4] = bf16_lo(v.z); w[5] = bf16_hi(v.z); w[6] = bf16_lo(v.w); w[7] = bf16_hi(v.w);
  }
};
template <>
struct WPiece<float> {
  static constexpr int VE = 4;
  static __device__ __forceinline__ void unpack(const uint4 &v, float (&w)[4]) {
    w[0] = __uint_as_float(v.x); w[1] = __uint_as_float(v.y); w[2] = __uint_as_float(v.z); w[3] = __uint_as_float(v.w);
  }
};

template <typename TO>
__device__ __forceinline__ void store4(TO *p, float4 v);
template <>
__device__ __forceinline__ void store4<float>(float *p, float4 v) {
  *reinterpret_cast<float4 *>(p) = v;
}
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t *p, float4 v) {
  *reinterpret_cast<uint2 *>(p) = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
}

}  // namespace

// Input rows [row_base, row_base + nr), nr <= NR <= 8.
template <typename TX, typename TW, typename TO, int NR>
__global__ __launch_bounds__(pr::kThreads) void project_rows_kernel(const ProjArgs a, const ProjRowsPlan p,
                                                                    int64_t row_base, int nr,
                                                                    unsigned int *__restrict__ counters,
                                                                    float *__restrict__ part) {
  using namespace pr;
  constexpr int VE = WPiece<TW>::VE;
  constexpr int CB = kLanesPerSeg * VE;
  constexpr int PROW = CB + 4;       // partial row: CB sums | sum of x^2 | 0 0 0
  constexpr int NC4 = CB / 4 + 1;    // float4 chunks per partial row
  constexpr int NCH = NR * NC4;      // float4 chunks per partial
  // The merge's sums reuse the staging memory, dead by then.
  union Lds {
    struct {
      float x[NR][kMaxSplitRows];    // x * gain of this split's columns
      float sq[NR][kMaxSplitRows];   // x^2
      float red[kWaves][NR][CB];     // per-wave column sums
    } s;
    float4 sum[kMergeSubs][NCH];
  };
  __shared__ Lds lds;
  auto &s_x = lds.s.x;
  auto &s_sq = lds.s.sq;
  auto &s_red = lds.s.red;
  __shared__ float s_ss[NR];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int cb = static_cast<int>(blockIdx.x % static_cast<unsigned>(p.n_cb));
  const int split = static_cast<int>(blockIdx.x / static_cast<unsigned>(p.n_cb));
  const int cb_per_out = a.ncols / CB;
  const int out_id = cb / cb_per_out;
  const int col0 = (cb - out_id * cb_per_out) * CB;
  const int d = a.d;
  const int k_begin = split * p.split_rows;
  const int nk = min(p.split_rows, d - k_begin);  // >= 1 by the plan
  const int n_loads = (nk + kRowsPerRound - 1) / kRowsPerRound;  // workgroup-uniform

  // W loads first, all kMaxLoads of them and none under a branch (a load
  // under a branch makes the compiler wait for it before the branch joins,
  // one round trip per load): load i of this lane reads row
  // i*16 + wave*4 + lane/16 of the split, 16 bytes at column
  // col0 + (lane%16)*VE, through a buffer descriptor that ends at the
  // split's last row, so the range check returns zeros for rows past it
  // without a memory access.
  const int seg = lane % kLanesPerSeg;
  const int rslot = lane / kLanesPerSeg;
  const __amdgpu_buffer_rsrc_t w_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<TW *>(static_cast<const TW *>(a.w[out_id]) + static_cast<int64_t>(k_begin) * a.ncols), 0,
      nk * a.ncols * static_cast<int>(sizeof(TW)), kRowsBufferFlags);
  const int w_lane_off = (col0 + seg * VE) * static_cast<int>(sizeof(TW));
  uint4 wraw[kMaxLoads];
#pragma unroll
  for (int i = 0; i < kMaxLoads; ++i) {
    const int kk = i * kRowsPerRound + wave * kRowSlots + rslot;
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, kk * a.ncols * static_cast<int>(sizeof(TW)) + w_lane_off,
                                                         0, 0);
    wraw[i] = make_uint4(v[0], v[1], v[2], v[3]);
  }

  // Stage x * gain and x^2 of this split's columns; every load of a round is
  // issued before any is used, at a clamped address (no load under a branch).
  const TX *x = static_cast<const TX *>(a.x);
  constexpr int kStage = (NR * kMaxSplitRows) / kThreads;  // rounds cover NR x 256
  const float *gain = a.gain;
#pragma unroll
  for (int j0 = 0; j0 < kStage; j0 += 4) {
    float v[4], g[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int idx = tid + (j0 + j) * kThreads;
      const int r = idx / kMaxSplitRows;
      const int kk = idx - r * kMaxSplitRows;
      const bool ok = (j0 + j) < kStage && r < nr && kk < nk;
      const int64_t off = ok ? (row_base + r) * d + k_begin + kk : 0;  // in bounds either way
      const int gk = ok ? k_begin + kk : 0;
      v[j] = load_elem<TX>(x + off);
      g[j] = gain != nullptr ? gain[gk] : 1.f;
      v[j] = ok ? v[j] : 0.f;
      g[j] = ok ? g[j] : 1.f;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if ((j0 + j) < kStage) {
        const int idx = tid + (j0 + j) * kThreads;
        const int r = idx / kMaxSplitRows;
        const int kk = idx - r * kMaxSplitRows;
        s_x[r][kk] = v[j] * g[j];
        s_sq[r][kk] = v[j] * v[j];
      }
    }
  }
  __syncthreads();

  // Partial sums of x^2 over the split's columns: wave w takes input rows
  // w, w + 4 (lane-strided sums, then a wave reduction).
#pragma unroll
  for (int r = wave; r < NR; r += kWaves) {
    float t = 0.f;
#pragma unroll
    for (int kk = lane; kk < kMaxSplitRows; kk += 64) t += s_sq[r][kk];
#pragma unroll
    for (int sft = 32; sft >= 1; sft >>= 1) t += shfl_xor_f(t, sft);
    if (lane == 0) s_ss[r] = t;
  }

  // Rows past the split hold zeros in wraw and in s_x (staged as 0), so they
  // add nothing; loads past the split's last round are skipped whole.
  float acc[NR][VE];
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int e = 0; e < VE; ++e) acc[r][e] = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxLoads; ++i) {
    if (i < n_loads) {
      const int kk = i * kRowsPerRound + wave * kRowSlots + rslot;
      float w[VE];
      WPiece<TW>::unpack(wraw[i], w);
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const float xv = s_x[r][kk];
#pragma unroll
        for (int e = 0; e < VE; ++e) acc[r][e] = fmaf(xv, w[e], acc[r][e]);
      }
    }
  }
  // Lanes of one column segment (lane bits 4 and 5), then the waves.
#pragma unroll
  for (int sft = kLanesPerSeg; sft < 64; sft <<= 1) {
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int e = 0; e < VE; ++e) acc[r][e] += shfl_xor_f(acc[r][e], sft);
  }
  if (rslot == 0) {
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int e = 0; e < VE; ++e) s_red[wave][r][seg * VE + e] = acc[r][e];
  }
  __syncthreads();

  // This workgroup's partial: [NR][PROW] at (column block, split).
  float *mine = part + (static_cast<int64_t>(cb) * p.splits + split) * (NR * PROW);
  for (int idx = tid; idx < NR * CB; idx += kThreads) {
    const int r = idx / CB;
    const int c = idx - r * CB;
    float v = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < kWaves; ++w2) v += s_red[w2][r][c];
    rows_store_agent(mine + r * PROW + c, v);
  }
  if (tid < NR * 4) {
    const int r = tid >> 2;
    rows_store_agent(mine + r * PROW + CB + (tid & 3), (tid & 3) == 0 ? s_ss[r] : 0.f);
  }

  // Every wave waits until its partial stores are performed at agent scope,
  // then thread 0 counts this workgroup's arrival at its column block.  The
  // partials travel only through agent-scope atomic stores and loads, which
  // the per-XCD caches do not hold, so the counter needs no release or
  // acquire fence (each would write back or invalidate this XCD's L2, once
  // per workgroup); the wait orders the stores before the count, and the
  // last arriver's loads are issued after its count has returned.  Counters
  // sit kProjRowsCounterStride words apart, one 128-byte line each, so the
  // column blocks' arrivals do not queue on one line.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  __shared__ int s_is_last;
  unsigned int *counter = counters + cb * kProjRowsCounterStride;
  if (tid == 0) {
    const unsigned int prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_is_last = (prev == static_cast<unsigned int>(p.splits - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (!s_is_last) return;

  // ---- Last arriver: add the S partials of this column block.  Task
  // (sub, ch) adds float4 chunk ch of splits sub, sub + NSUB, ... in order,
  // kBatch loads in flight; the NSUB task sums are then added in sub order.
  // The order depends on neither the launch's row count nor its other rows.
  constexpr int NSUB = kMergeSubs;
  constexpr int kBatch = 8;
  auto &s_sum = lds.sum;
  const float4 *parts = reinterpret_cast<const float4 *>(part + static_cast<int64_t>(cb) * p.splits * (NR * PROW));
  constexpr int kSplitStride4 = NR * PROW / 4;
  for (int task = tid; task < NSUB * NCH; task += kThreads) {
    const int sub = task / NCH;
    const int ch = task - sub * NCH;
    float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s0 = sub; s0 < p.splits; s0 += NSUB * kBatch) {
      // All kBatch loads at clamped splits, then the sums of the real ones.
      float4 vv[kBatch];
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int s = min(s0 + b * NSUB, p.splits - 1);
        vv[b] = rows_load_agent4(parts + static_cast<int64_t>(s) * kSplitStride4 + ch);
      }
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        if (s0 + b * NSUB < p.splits) {
          t.x += vv[b].x;
          t.y += vv[b].y;
          t.z += vv[b].z;
          t.w += vv[b].w;
        }
      }
    }
    s_sum[sub][ch] = t;
  }
  __syncthreads();
  __shared__ float s_inv_rms[NR];
  if (tid < NR) {
    float ss = 0.f;
    for (int sb = 0; sb < NSUB; ++sb) ss += s_sum[sb][tid * NC4 + CB / 4].x;
    s_inv_rms[tid] = 1.0f / sqrtf(ss / static_cast<float>(d) + a.eps);
  }
  __syncthreads();
  TO *out = static_cast<TO *>(a.out[out_id]);
  const bool rope = a.rope_out == out_id;
  for (int idx = tid; idx < NR * (CB / 4); idx += kThreads) {
    const int r = idx / (CB / 4);
    const int c4 = idx - r * (CB / 4);
    if (r >= nr) continue;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int sb = 0; sb < NSUB; ++sb) {
      const float4 u = s_sum[sb][r * NC4 + c4];
      v.x += u.x;
      v.y += u.y;
      v.z += u.z;
      v.w += u.w;
    }
    const float inv = s_inv_rms[r];
    v.x *= inv;
    v.y *= inv;
    v.z *= inv;
    v.w *= inv;
    const int64_t row = row_base + r;
    const int col = col0 + 4 * c4;
    if (rope) {
      // columns col .. col+3 are pairs (2i, 2i+1) and (2i+2, 2i+3) of a head
      const int pair = (col % a.head_dim) >> 1;
      const int64_t pos = proj_row_pos(a, row);
      rope_turn(v.x, v.y, pos, rope_rev(pair, a.head_dim, a.rope_log2_theta));
      rope_turn(v.z, v.w, pos, rope_rev(pair + 1, a.head_dim, a.rope_log2_theta));
    }
    const int64_t dst = a.indexed ? a.dst_rows[row] : a.dst_row_base + row;
    store4<TO>(out + dst * a.out_stride + col, v);
  }
  if (tid == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename TX, typename TW, typename TO>
static hipError_t launch_rows_t(const ProjArgs &a, const ProjRowsPlan &p, unsigned int *counters, float *part,
                                hipStream_t s) {
  const unsigned int blocks = static_cast<unsigned int>(p.n_cb) * static_cast<unsigned int>(p.splits);
  for (int64_t base = 0; base < a.n; base += pr::kMaxInRows) {
    const int nr = static_cast<int>(a.n - base < pr::kMaxInRows ? a.n - base : pr::kMaxInRows);
    const int nr_pow2 = nr <= 1 ? 1 : nr <= 2 ? 2 : nr <= 4 ? 4 : 8;
    switch (nr_pow2) {
      case 1: hipLaunchKernelGGL((project_rows_kernel<TX, TW, TO, 1>), dim3(blocks), dim3(pr::kThreads), 0, s, a, p, base, nr, counters, part); break;
      case 2: hipLaunchKernelGGL((project_rows_kernel<TX, TW, TO, 2>), dim3(blocks), dim3(pr::kThreads), 0, s, a, p, base, nr, counters, part); break;
      case 4: hipLaunchKernelGGL((project_rows_kernel<TX, TW, TO, 4>), dim3(blocks), dim3(pr::kThreads), 0, s, a, p, base, nr, counters, part); break;
      default: hipLaunchKernelGGL((project_rows_kernel<TX, TW, TO, 8>), dim3(blocks), dim3(pr::kThreads), 0, s, a, p, base, nr, counters, part); break;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename TX, typename TW>
static hipError_t launch_rows_o(const ProjArgs &a, const ProjRowsPlan &p, int o_dt, unsigned int *c, float *part,
                                hipStream_t s) {
  if (o_dt == YOCO_DT_F32) return launch_rows_t<TX, TW, float>(a, p, c, part, s);
  if (o_dt == YOCO_DT_BF16) return launch_rows_t<TX, TW, bf16_t>(a, p, c, part, s);
  return hipErrorInvalidValue;
}

template <typename TX>
static hipError_t launch_rows_w(const ProjArgs &a, const ProjRowsPlan &p, int w_dt, int o_dt, unsigned int *c,
                                float *part, hipStream_t s) {
  if (w_dt == YOCO_DT_F32) return launch_rows_o<TX, float>(a, p, o_dt, c, part, s);
  if (w_dt == YOCO_DT_BF16) return launch_rows_o<TX, bf16_t>(a, p, o_dt, c, part, s);
  return hipErrorInvalidValue;
}

hipError_t launch_project_rows(const ProjArgs &a, const ProjRowsPlan &p, int x_dt, int w_dt, int o_dt,
                               void *workspace, hipStream_t s) {
  unsigned int *counters = static_cast<unsigned int *>(workspace);
  float *part = reinterpret_cast<float *>(static_cast<char *>(workspace) + kProjRowsCounterBytes);
  if (x_dt == YOCO_DT_F32) return launch_rows_w<float>(a, p, w_dt, o_dt, counters, part, s);
  if (x_dt == YOCO_DT_BF16) return launch_rows_w<bf16_t>(a, p, w_dt, o_dt, counters, part, s);
  return hipErrorInvalidValue;
}

}  // namespace yoco
