// Split-N flash decoding over the shared K^/V^ cache, one launch per call.
//
// What it computes ([Notes] "YOCO：You Only Cache Once 中文精读笔记" s.2.1
// Eq. 3; [Blog] "NeurIPS'24 | YOCO: 长上下文 LLM 为什么不必每层都存一份 KV
// Cache?" s.2 and s.7): for each sequence b and query head h, the query at
// position len_b - 1 attends causally to every cache row 0..len_b-1 of KV head
// g = h / G, o = softmax(scale * q K^T) V.  Every cross layer re-reads the
// whole cache ([Blog] s.7), so this kernel is bound by HBM bandwidth.
//
// Work decomposition (gfx950: 64-wide waves, 8 XCDs, 256 CUs):
//   blockIdx.x = split_index * H_kv + g.  Consecutive blocks go to
//   consecutive XCDs, so with H_kv = 8 every split of KV head g lands on the
//   same XCD and the merge reads partials from that XCD's L2.
//   A workgroup of NW waves streams rows [split*split_rows, +split_rows) of
//   (b, g).  A row of one head is head_dim elements; each lane owns 8
//   consecutive elements (one 16-byte load for bf16), so LPR = head_dim/8
//   lanes cover a row and a wave covers 64/LPR rows per load instruction.
//   Each K/V row is read once and used by all G query heads of the group.
//   <q, k> partials reduce across the LPR lanes with DPP (no LDS).
//   Each lane keeps its own running softmax state (reference max m, sum l,
//   weighted V) per head over the rows it saw, rescaling only when a logit
//   exceeds the reference by more than kRescaleSlack (in log2 units), which
//   keeps every exp2 argument <= kRescaleSlack.  The states of the lanes and
//   waves are merged with the usual log-sum-exp rule, giving one partial
//   (acc[head_dim] | m | l) per (split, g, head).
//   The workgroup that finishes last for (b, g) (device-scope arrival
//   counter) merges that group's partials in split order and writes o and
//   lse, then resets the counter to zero.
#include "device_common.h"
#include "yoco_internal.h"

namespace yoco {

constexpr float kRescaleSlack = 8.0f;  // log2 units: exp2 arguments stay <= 8

template <typename T, int DH, int G>
struct DecodeCfg {
  static constexpr int NW = 8;                        // waves per workgroup
  static constexpr int NT = NW * 64;
  static constexpr int LPR = DH / 8;                  // lanes per row
  static constexpr int RPP = 64 / LPR;                // rows per load pass
  static constexpr int U = (G <= 4) ? 8 : 4;          // passes per tile
  static constexpr int TILE = U * RPP;                // rows per wave tile
  static constexpr int PROW = DH + 4;                 // partial row: acc | m | l | 0 | 0
  static constexpr int NCH = G * PROW / 4;            // float4 chunks per (split, g)
};

// One wave tile: rows [row0, row0 + TILE) of this split, rows >= nrows masked.
template <typename T, int DH, int G, bool MASKED>
__device__ __forceinline__ void decode_tile(const T *__restrict__ kbase, const T *__restrict__ vbase,
                                            int64_t row_stride, int row0, int nrows, int r, int c,
                                            float scale_log2, const float (&q)[G][8], float (&m)[G],
                                            float (&l)[G], float (&acc)[G][8]) {
  using C = DecodeCfg<T, DH, G>;
  Vec8<T> kv[C::U], vv[C::U];
#pragma unroll
  for (int u = 0; u < C::U; ++u) {
    const int row = row0 + u * C::RPP + r;
    if (!MASKED || row < nrows) {
      kv[u].load(kbase + row * row_stride + c * 8);
    } else {
      kv[u].zero();
    }
  }
#pragma unroll
  for (int u = 0; u < C::U; ++u) {
    const int row = row0 + u * C::RPP + r;
    if (!MASKED || row < nrows) {
      vv[u].load(vbase + row * row_stride + c * 8);
    } else {
      vv[u].zero();
    }
  }

  float x[C::U][G];
#pragma unroll
  for (int u = 0; u < C::U; ++u) {
#pragma unroll
    for (int i = 0; i < G; ++i) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) d = fmaf(q[i][e], kv[u][e], d);
      x[u][i] = group_sum<C::LPR>(d) * scale_log2;
    }
    if (MASKED && row0 + u * C::RPP + r >= nrows) {
#pragma unroll
      for (int i = 0; i < G; ++i) x[u][i] = -INFINITY;
    }
  }

  // Lazy rescale: move the reference max only when a logit passes it by more
  // than the slack.  The condition is evaluated per lane; the branch is taken
  // by the whole wave when any lane needs it.
  float mt[G];
  bool need = false;
#pragma unroll
  for (int i = 0; i < G; ++i) {
    mt[i] = x[0][i];
#pragma unroll
    for (int u = 1; u < C::U; ++u) mt[i] = fmaxf(mt[i], x[u][i]);
    need |= mt[i] > m[i] + kRescaleSlack;
  }
  if (__any(need)) {
#pragma unroll
    for (int i = 0; i < G; ++i) {
      if (mt[i] > m[i] + kRescaleSlack) {
        const float alpha = fast_exp2(m[i] - mt[i]);  // m = -inf gives 0
        l[i] *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[i][e] *= alpha;
        m[i] = mt[i];
      }
    }
  }

#pragma unroll
  for (int u = 0; u < C::U; ++u) {
    const bool valid = !MASKED || (row0 + u * C::RPP + r < nrows);
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const float p = valid ? fast_exp2(x[u][i] - m[i]) : 0.f;
      l[i] += p;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[i][e] = fmaf(p, vv[u][e], acc[i][e]);
    }
  }
}

// Log-sum-exp merge weight of a state with reference max `ms` into `mnew`.
__device__ __forceinline__ float merge_weight(float ms, float mnew) {
  return (ms == -INFINITY) ? 0.f : fast_exp2(ms - mnew);
}

template <typename T, int DH, int G>
__global__ __launch_bounds__(512) void decode_kernel(const DecodeArgs a) {
  using C = DecodeCfg<T, DH, G>;
  static_assert(C::NT == 512, "launch bounds assume 8 waves");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int H = a.n_kv_heads;
  const int ws = blockIdx.x / H;
  const int g = blockIdx.x - ws * H;

  // Sequence that owns split ws: the last b with split_begin[b] <= ws.
  int lo = 0, hi = a.n_seq - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.split_begin[mid] <= ws) lo = mid; else hi = mid - 1;
  }
  const int b = lo;
  const int first_split = a.split_begin[b];
  const int n_splits = a.split_begin[b + 1] - first_split;
  const int row_begin = (ws - first_split) * a.split_rows;
  const int nrows = min(a.split_rows, a.len[b] - row_begin);

  const int64_t row_stride = (int64_t)H * DH;
  const T *kbase = static_cast<const T *>(a.k) + b * a.seq_stride + row_begin * row_stride + g * DH;
  const T *vbase = static_cast<const T *>(a.v) + b * a.seq_stride + row_begin * row_stride + g * DH;

  const int r = lane / C::LPR;
  const int c = lane % C::LPR;

  float q[G][8];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const T *qp = static_cast<const T *>(a.q) + ((int64_t)b * a.n_q_heads + g * G + i) * DH + c * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) q[i][e] = load_elem<T>(qp + e);
  }

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[i][e] = 0.f;
  }

  for (int t = wave; t * C::TILE < nrows; t += C::NW) {
    const int row0 = t * C::TILE;
    if (row0 + C::TILE <= nrows) {
      decode_tile<T, DH, G, false>(kbase, vbase, row_stride, row0, nrows, r, c, a.scale_log2, q, m, l, acc);
    } else {
      decode_tile<T, DH, G, true>(kbase, vbase, row_stride, row0, nrows, r, c, a.scale_log2, q, m, l, acc);
    }
  }

  // Merge the RPP row slots of the wave (lanes that differ in the row bits).
#pragma unroll
  for (int s = C::LPR; s < 64; s <<= 1) {
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const float mo = shfl_xor_f(m[i], s);
      const float lo2 = shfl_xor_f(l[i], s);
      const float mn = fmaxf(m[i], mo);
      const float wa = merge_weight(m[i], mn);
      const float wb = merge_weight(mo, mn);
      l[i] = l[i] * wa + lo2 * wb;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float ao = shfl_xor_f(acc[i][e], s);
        acc[i][e] = acc[i][e] * wa + ao * wb;
      }
      m[i] = mn;
    }
  }

  // Merge the NW waves through LDS into this workgroup's partial.
  __shared__ float s_m[C::NW][G];
  __shared__ float s_l[C::NW][G];
  __shared__ float s_acc[C::NW][G][DH];
  if (lane < C::LPR) {
#pragma unroll
    for (int i = 0; i < G; ++i) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s_acc[wave][i][c * 8 + e] = acc[i][e];
      if (lane == 0) {
        s_m[wave][i] = m[i];
        s_l[wave][i] = l[i];
      }
    }
  }
  __syncthreads();

  float *part = a.part_acc + ((int64_t)ws * H + g) * G * C::PROW;
  for (int idx = tid; idx < G * DH; idx += C::NT) {
    const int i = idx / DH;
    const int e = idx - i * DH;
    float mw = -INFINITY;
#pragma unroll
    for (int w = 0; w < C::NW; ++w) mw = fmaxf(mw, s_m[w][i]);
    float av = 0.f, lv = 0.f;
#pragma unroll
    for (int w = 0; w < C::NW; ++w) {
      const float wt = merge_weight(s_m[w][i], mw);
      av = fmaf(s_acc[w][i][e], wt, av);
      lv = fmaf(s_l[w][i], wt, lv);
    }
    part[i * C::PROW + e] = av;
    if (e == 0) {
      part[i * C::PROW + DH + 0] = mw;
      part[i * C::PROW + DH + 1] = lv;
      part[i * C::PROW + DH + 2] = 0.f;
      part[i * C::PROW + DH + 3] = 0.f;
    }
  }

  // Publish this workgroup's partial, then count arrivals for (b, g).
  __threadfence();
  __syncthreads();
  __shared__ int s_is_last;
  unsigned int *counter = a.counters + b * kMaxKvHeads + g;
  if (tid == 0) {
    const unsigned int prev = atomicAdd(counter, 1u);
    s_is_last = (prev == static_cast<unsigned int>(n_splits - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (!s_is_last) return;
  __threadfence();  // acquire: observe every other split's partial

  // ---- Last arriver: merge the n_splits partials of (b, g) in split order.
  const float4 *parts =
      reinterpret_cast<const float4 *>(a.part_acc + ((int64_t)first_split * H + g) * G * C::PROW);
  const int64_t split_stride4 = (int64_t)H * G * C::PROW / 4;  // float4s between splits

  // Per-head maximum of the split reference maxima.
  __shared__ float s_wmax[C::NW][G];
  float mloc[G];
#pragma unroll
  for (int i = 0; i < G; ++i) mloc[i] = -INFINITY;
  for (int s = tid; s < n_splits; s += C::NT) {
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const float4 ml = parts[s * split_stride4 + (i * C::PROW + DH) / 4];
      mloc[i] = fmaxf(mloc[i], ml.x);
    }
  }
#pragma unroll
  for (int i = 0; i < G; ++i) {
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) mloc[i] = fmaxf(mloc[i], shfl_xor_f(mloc[i], s));
  }
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < G; ++i) s_wmax[wave][i] = mloc[i];
  }
  __syncthreads();
  float mall[G];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    mall[i] = s_wmax[0][i];
#pragma unroll
    for (int w = 1; w < C::NW; ++w) mall[i] = fmaxf(mall[i], s_wmax[w][i]);
  }

  // Weighted sums over splits.  Thread -> (subset, chunk): subset `sub`
  // handles splits sub, sub + nsub, ... of each chunk of kChunk splits.
  constexpr int kChunk = C::NT;
  constexpr int NSUB = C::NT / C::NCH;
  __shared__ float s_w[kChunk][G];
  __shared__ float4 s_red[NSUB > 0 ? NSUB : 1][C::NCH];
  const int sub = tid / C::NCH;
  const int oc = tid - sub * C::NCH;
  const int oc_head = (oc * 4) / C::PROW;
  float4 part_sum = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int cs = 0; cs < n_splits; cs += kChunk) {
    const int clen = min(kChunk, n_splits - cs);
    __syncthreads();
    if (tid < clen) {
#pragma unroll
      for (int i = 0; i < G; ++i) {
        const float4 ml = parts[(cs + tid) * split_stride4 + (i * C::PROW + DH) / 4];
        s_w[tid][i] = merge_weight(ml.x, mall[i]);
      }
    }
    __syncthreads();
    if (sub < NSUB) {
#pragma unroll 4
      for (int s = sub; s < clen; s += NSUB) {
        const float wt = s_w[s][oc_head];
        const float4 v = parts[(cs + s) * split_stride4 + oc];
        part_sum.x = fmaf(wt, v.x, part_sum.x);
        part_sum.y = fmaf(wt, v.y, part_sum.y);
        part_sum.z = fmaf(wt, v.z, part_sum.z);
        part_sum.w = fmaf(wt, v.w, part_sum.w);
      }
    }
  }
  if (sub < NSUB) s_red[sub][oc] = part_sum;
  __syncthreads();
  if (tid < C::NCH) {
    float4 tot = s_red[0][tid];
    for (int s2 = 1; s2 < NSUB; ++s2) {
      const float4 v = s_red[s2][tid];
      tot.x += v.x; tot.y += v.y; tot.z += v.z; tot.w += v.w;
    }
    s_red[0][tid] = tot;
  }
  __syncthreads();
  const int h0 = g * G;
  for (int idx = tid; idx < G * DH / 4; idx += C::NT) {
    const int i = (idx * 4) / DH;
    const int e4 = idx - i * (DH / 4);
    const float L = s_red[0][(i * C::PROW + DH) / 4].y;
    const float inv = 1.0f / L;
    float4 v = s_red[0][(i * C::PROW) / 4 + e4];
    v.x *= inv; v.y *= inv; v.z *= inv; v.w *= inv;
    reinterpret_cast<float4 *>(a.o + ((int64_t)b * a.n_q_heads + h0 + i) * DH)[e4] = v;
  }
  if (a.lse != nullptr && tid < G) {
    const float L = s_red[0][(tid * C::PROW + DH) / 4].y;
    a.lse[(int64_t)b * a.n_q_heads + h0 + tid] = (mall[tid] + __log2f(L)) * kLn2;
  }
  if (tid == 0) *counter = 0u;
}

template <typename T, int DH, int G>
static hipError_t launch_decode_t(const DecodeArgs &a, hipStream_t s) {
  using C = DecodeCfg<T, DH, G>;
  const unsigned int blocks = static_cast<unsigned int>(a.total_splits) * a.n_kv_heads;
  hipLaunchKernelGGL((decode_kernel<T, DH, G>), dim3(blocks), dim3(C::NT), 0, s, a);
  return hipGetLastError();
}

template <typename T, int DH>
static hipError_t launch_decode_g(const DecodeArgs &a, int group, hipStream_t s) {
  switch (group) {
    case 1: return launch_decode_t<T, DH, 1>(a, s);
    case 2: return launch_decode_t<T, DH, 2>(a, s);
    case 3: return launch_decode_t<T, DH, 3>(a, s);
    case 4: return launch_decode_t<T, DH, 4>(a, s);
    case 6: return launch_decode_t<T, DH, 6>(a, s);
    case 8: return launch_decode_t<T, DH, 8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const DecodeArgs &a, int dtype, int head_dim, int group, hipStream_t s) {
  if (dtype == YOCO_DT_BF16) {
    if (head_dim == 128) return launch_decode_g<bf16_t, 128>(a, group, s);
    if (head_dim == 64) return launch_decode_g<bf16_t, 64>(a, group, s);
  } else if (dtype == YOCO_DT_F32) {
    if (head_dim == 128) return launch_decode_g<float, 128>(a, group, s);
    if (head_dim == 64) return launch_decode_g<float, 64>(a, group, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace yoco
