// Split-N flash decoding over the shared K^/V^ cache: kernel template.
//
// What it computes ([Notes] "YOCO：You Only Cache Once 中文精读笔记" s.2.1
// Eq. 3; [Blog] "NeurIPS'24 | YOCO: 长上下文 LLM 为什么不必每层都存一份 KV
// Cache?" s.2 and s.7): for each sequence b and query head h, the query at
// position len_b - 1 attends causally to every cache row 0..len_b-1 of KV head
// g = h / G, o = softmax(scale * q K^T) V.  Every cross layer re-reads the
// whole cache ([Blog] s.7), so the kernel is bound by HBM bandwidth and is
// written around the stream, not around a matrix core.
//
// Work decomposition (gfx950: 64-wide waves, 8 XCDs, 256 CUs):
//   blockIdx.x = split_index * H_kv + g.  Consecutive blocks go to
//   consecutive XCDs, so with H_kv = 8 every split of KV head g runs on one
//   XCD and the merge reads partials from that XCD's L2.
//   A workgroup of NW waves streams rows [split*split_rows_b, +split_rows_b)
//   of (b, g), with a split size per sequence.  Each lane owns EPL elements of a head row in 16-byte pieces;
//   LPR = head_dim / EPL lanes cover a row, and piece j of lane c holds
//   elements j*LPR*VE + c*VE .. +VE (VE elements per 16 bytes), so each load
//   instruction reads whole contiguous segments of the rows.  A wave covers
//   RPP = 64 / LPR rows per pass and U passes per tile; with PF the next
//   tile's loads are issued before the current tile is computed (register
//   double buffering).
//   Each K/V row is read once and used by all G query heads of the group.
//   <q, k> partials reduce across the LPR lanes with DPP.  For bf16 the
//   partial dot products use v_dot2_f32_bf16 on packed pairs (exact products,
//   fp32 accumulation); the weighted V sum always runs in fp32 FMA.
//   Each lane keeps its own running softmax state (reference max m, sum l,
//   weighted V) per head over the rows it saw, and moves the reference only
//   when a logit passes it by more than kRescaleSlack (log2 units), so every
//   exp2 argument stays <= kRescaleSlack.  Lane and wave states merge with
//   the log-sum-exp rule into one partial (acc[head_dim] | m | l) per
//   (split, g, head).
//   Cross-workgroup merge: partials are written with agent-scope atomic
//   stores and read with agent-scope atomic loads (they bypass the
//   per-XCD caches, so no cache write-back or invalidate is needed); every
//   wave waits for its stores, then thread 0 increments the (b, g) arrival
//   counter with an agent-scope RMW.  The workgroup that
//   arrives last merges the group's partials: each task combines a fixed
//   subset of the splits in one round trip, and the subsets are combined in a
//   fixed order through LDS, so results are bitwise reproducible.  It writes
//   o and lse and resets the counter to zero.
#pragma once

#include "device_common.h"
#include "decode_args.h"

namespace yoco {

constexpr float kRescaleSlack = 8.0f;  // log2 units: exp2 arguments stay <= 8

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

template <int NW_, int EPL_, int U_, bool PF_>
struct DecodeTune {
  static constexpr int NW = NW_;    // waves per workgroup
  static constexpr int EPL = EPL_;  // elements per lane per row
  static constexpr int U = U_;      // passes per tile
  static constexpr bool PF = PF_;   // prefetch next tile
};

template <typename T, int DH, int G, class TUNE>
struct DecodeCfg {
  static constexpr int NW = TUNE::NW;
  static constexpr int NT = NW * 64;
  static constexpr int EPL = TUNE::EPL;
  static constexpr int VE = 16 / sizeof(T);           // elements per 16-byte piece
  static constexpr int NL = EPL / VE;                 // pieces per lane per row
  static constexpr int LPR = DH / EPL;                // lanes per row
  static constexpr int RPP = 64 / LPR;                // rows per pass
  static constexpr int U = TUNE::U;
  static constexpr int TILE = U * RPP;                // rows per wave tile
  static constexpr bool PF = TUNE::PF;
  static constexpr int PROW = DH + 4;                 // partial row: acc | m | l | 0 | 0
  static constexpr int NCH = G * PROW / 4;            // float4 chunks per (split, g)
  static constexpr bool DOT2 = (sizeof(T) == 2);
  static_assert(LPR == 4 || LPR == 8 || LPR == 16, "lanes per row");
  static_assert(NL * VE == EPL, "pieces");
};

// Registers of one wave tile: NL 16-byte pieces for U rows, K and V.
template <class C>
struct TileRegs {
  uint4 k[C::U][C::NL];
  uint4 v[C::U][C::NL];
};

template <class C, bool MASKED, typename T>
__device__ __forceinline__ void load_tile(TileRegs<C> &t, const T *__restrict__ kbase,
                                          const T *__restrict__ vbase, int64_t row_stride, int row0,
                                          int nrows, int r, int c) {
#pragma unroll
  for (int u = 0; u < C::U; ++u) {
    const int row = row0 + u * C::RPP + r;
    const bool ok = !MASKED || row < nrows;
#pragma unroll
    for (int j = 0; j < C::NL; ++j) {
      const int64_t off = row * row_stride + j * (C::LPR * C::VE) + c * C::VE;
      t.k[u][j] = ok ? ld16_stream(kbase + off) : make_uint4(0, 0, 0, 0);
    }
  }
#pragma unroll
  for (int u = 0; u < C::U; ++u) {
    const int row = row0 + u * C::RPP + r;
    const bool ok = !MASKED || row < nrows;
#pragma unroll
    for (int j = 0; j < C::NL; ++j) {
      const int64_t off = row * row_stride + j * (C::LPR * C::VE) + c * C::VE;
      t.v[u][j] = ok ? ld16_stream(vbase + off) : make_uint4(0, 0, 0, 0);
    }
  }
}

__device__ __forceinline__ float word_elem(const uint4 &w, int i, bool bf16) {
  if (bf16) {
    const uint32_t d = (i < 2) ? w.x : (i < 4) ? w.y : (i < 6) ? w.z : w.w;
    return (i & 1) ? bf16_hi(d) : bf16_lo(d);
  }
  const uint32_t d = (i == 0) ? w.x : (i == 1) ? w.y : (i == 2) ? w.z : w.w;
  return __uint_as_float(d);
}

// Query registers: packed bf16 pairs (dot2) or fp32 values, in the lane's
// element order (piece j, element e).
template <class C>
struct QRegs {
  uint32_t packed[C::DOT2 ? C::NL * 4 : 1];
  float f[C::DOT2 ? 1 : C::EPL];
};

template <class C, int G, bool MASKED>
__device__ __forceinline__ void compute_tile(const TileRegs<C> &t, int row0, int nrows, int r,
                                             float scale_log2, const QRegs<C> (&q)[G], float (&m)[G],
                                             float (&l)[G], float (&acc)[G][C::EPL]) {
  float x[C::U][G];
#pragma unroll
  for (int u = 0; u < C::U; ++u) {
#pragma unroll
    for (int i = 0; i < G; ++i) {
      float d = 0.f;
      if constexpr (C::DOT2) {
#pragma unroll
        for (int j = 0; j < C::NL; ++j) {
          d = dot2_bf16(t.k[u][j].x, q[i].packed[j * 4 + 0], d);
          d = dot2_bf16(t.k[u][j].y, q[i].packed[j * 4 + 1], d);
          d = dot2_bf16(t.k[u][j].z, q[i].packed[j * 4 + 2], d);
          d = dot2_bf16(t.k[u][j].w, q[i].packed[j * 4 + 3], d);
        }
      } else {
#pragma unroll
        for (int j = 0; j < C::NL; ++j) {
#pragma unroll
          for (int e = 0; e < C::VE; ++e) d = fmaf(q[i].f[j * C::VE + e], word_elem(t.k[u][j], e, false), d);
        }
      }
      x[u][i] = group_sum<C::LPR>(d) * scale_log2;
    }
    if (MASKED && row0 + u * C::RPP + r >= nrows) {
#pragma unroll
      for (int i = 0; i < G; ++i) x[u][i] = -INFINITY;
    }
  }

  // Lazy rescale: move the reference max only when a logit passes it by more
  // than the slack.  Evaluated per lane; taken by the wave when any lane needs it.
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
        for (int e = 0; e < C::EPL; ++e) acc[i][e] *= alpha;
        m[i] = mt[i];
      }
    }
  }

#pragma unroll
  for (int u = 0; u < C::U; ++u) {
    const bool valid = !MASKED || (row0 + u * C::RPP + r < nrows);
    float p[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      p[i] = valid ? fast_exp2(x[u][i] - m[i]) : 0.f;
      l[i] += p[i];
    }
#pragma unroll
    for (int j = 0; j < C::NL; ++j) {
#pragma unroll
      for (int e = 0; e < C::VE; ++e) {
        const float vv = word_elem(t.v[u][j], e, C::DOT2);
#pragma unroll
        for (int i = 0; i < G; ++i) acc[i][j * C::VE + e] = fmaf(p[i], vv, acc[i][j * C::VE + e]);
      }
    }
  }
}

// Agent-scope (device-coherent) relaxed atomic store / load of partials.
__device__ __forceinline__ void store_agent(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float4 load_agent4(const float4 *p) {
  const uint64_t *q = reinterpret_cast<const uint64_t *>(p);
  const uint64_t lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_float4(__uint_as_float(static_cast<uint32_t>(lo)), __uint_as_float(static_cast<uint32_t>(lo >> 32)),
                     __uint_as_float(static_cast<uint32_t>(hi)), __uint_as_float(static_cast<uint32_t>(hi >> 32)));
}

// The (m, l) pair of a partial row (its first 8 bytes), agent scope.
__device__ __forceinline__ float2 load_agent2(const float *p) {
  const uint64_t v = __hip_atomic_load(reinterpret_cast<const uint64_t *>(p), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float(static_cast<uint32_t>(v)), __uint_as_float(static_cast<uint32_t>(v >> 32)));
}

// Log-sum-exp merge weight of a state with reference max `ms` into `mnew`.
__device__ __forceinline__ float merge_weight(float ms, float mnew) {
  return (ms == -INFINITY) ? 0.f : fast_exp2(ms - mnew);
}

template <typename T, int DH, int G, class TUNE>
__global__ __launch_bounds__(TUNE::NW * 64) void decode_kernel(const DecodeArgs a) {
  using C = DecodeCfg<T, DH, G, TUNE>;
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
  const int split_rows = a.split_rows[b];
  const int row_begin = (ws - first_split) * split_rows;
  const int nrows = min(split_rows, a.len[b] - row_begin);

  const int64_t row_stride = a.row_stride;
  const T *kbase = static_cast<const T *>(a.k) + b * a.seq_stride + row_begin * row_stride + g * DH;
  const T *vbase = static_cast<const T *>(a.v) + b * a.seq_stride + row_begin * row_stride + g * DH;

  const int r = lane / C::LPR;
  const int c = lane % C::LPR;

  QRegs<C> q[G];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const T *qp = static_cast<const T *>(a.q) + ((int64_t)b * a.n_q_heads + g * G + i) * DH;
#pragma unroll
    for (int j = 0; j < C::NL; ++j) {
      const uint4 w = ld16(qp + j * (C::LPR * C::VE) + c * C::VE);
      if constexpr (C::DOT2) {
        q[i].packed[j * 4 + 0] = w.x;
        q[i].packed[j * 4 + 1] = w.y;
        q[i].packed[j * 4 + 2] = w.z;
        q[i].packed[j * 4 + 3] = w.w;
      } else {
#pragma unroll
        for (int e = 0; e < C::VE; ++e) q[i].f[j * C::VE + e] = word_elem(w, e, false);
      }
    }
  }

  float m[G], l[G], acc[G][C::EPL];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
#pragma unroll
    for (int e = 0; e < C::EPL; ++e) acc[i][e] = 0.f;
  }

  // Wave tiles t = wave, wave + NW, ...; tiles before n_full are whole.
  const int n_full = nrows / C::TILE;
  const int n_tiles = (nrows + C::TILE - 1) / C::TILE;
  if constexpr (C::PF) {
    TileRegs<C> ta, tb;
    int t = wave;
    if (t < n_tiles) {
      if (t < n_full) load_tile<C, false>(ta, kbase, vbase, row_stride, t * C::TILE, nrows, r, c);
      else load_tile<C, true>(ta, kbase, vbase, row_stride, t * C::TILE, nrows, r, c);
    }
    while (t < n_tiles) {
      int tn = t + C::NW;
      if (tn < n_tiles) {
        if (tn < n_full) load_tile<C, false>(tb, kbase, vbase, row_stride, tn * C::TILE, nrows, r, c);
        else load_tile<C, true>(tb, kbase, vbase, row_stride, tn * C::TILE, nrows, r, c);
      }
      if (t < n_full) compute_tile<C, G, false>(ta, t * C::TILE, nrows, r, a.scale_log2, q, m, l, acc);
      else compute_tile<C, G, true>(ta, t * C::TILE, nrows, r, a.scale_log2, q, m, l, acc);
      t = tn;
      if (t >= n_tiles) break;
      tn = t + C::NW;
      if (tn < n_tiles) {
        if (tn < n_full) load_tile<C, false>(ta, kbase, vbase, row_stride, tn * C::TILE, nrows, r, c);
        else load_tile<C, true>(ta, kbase, vbase, row_stride, tn * C::TILE, nrows, r, c);
      }
      if (t < n_full) compute_tile<C, G, false>(tb, t * C::TILE, nrows, r, a.scale_log2, q, m, l, acc);
      else compute_tile<C, G, true>(tb, t * C::TILE, nrows, r, a.scale_log2, q, m, l, acc);
      t = tn;
    }
  } else {
    TileRegs<C> ta;
    int t = wave;
    for (; t < n_full; t += C::NW) {
      load_tile<C, false>(ta, kbase, vbase, row_stride, t * C::TILE, nrows, r, c);
      compute_tile<C, G, false>(ta, t * C::TILE, nrows, r, a.scale_log2, q, m, l, acc);
    }
    if (t < n_tiles) {
      load_tile<C, true>(ta, kbase, vbase, row_stride, t * C::TILE, nrows, r, c);
      compute_tile<C, G, true>(ta, t * C::TILE, nrows, r, a.scale_log2, q, m, l, acc);
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
      for (int e = 0; e < C::EPL; ++e) {
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
      for (int j = 0; j < C::NL; ++j) {
#pragma unroll
        for (int e = 0; e < C::VE; ++e) s_acc[wave][i][j * (C::LPR * C::VE) + c * C::VE + e] = acc[i][j * C::VE + e];
      }
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
    store_agent(&part[i * C::PROW + e], av);
    if (e == 0) {
      store_agent(&part[i * C::PROW + DH + 0], mw);
      store_agent(&part[i * C::PROW + DH + 1], lv);
      store_agent(&part[i * C::PROW + DH + 2], 0.f);
      store_agent(&part[i * C::PROW + DH + 3], 0.f);
    }
  }

  // Every wave waits until its partial stores are performed at agent scope,
  // then thread 0 counts this workgroup's arrival for (b, g).  The partials
  // travel only through agent-scope atomic stores and loads, which the
  // per-XCD caches do not hold, so the count needs no release or acquire
  // fence (each would write back or invalidate this XCD's L2, once per
  // workgroup): the wait orders the stores before the count, and the last
  // arriver's loads are issued after its count has returned.  The counters
  // of one sequence's KV heads are YOCO_MAX_SEQ words apart, on separate
  // 128-byte lines, so the heads' arrivals do not queue on one line.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  __shared__ int s_is_last;
  unsigned int *counter = a.counters + g * YOCO_MAX_SEQ + b;
  if (tid == 0) {
    const unsigned int prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_is_last = (prev == static_cast<unsigned int>(n_splits - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (!s_is_last) return;

  // ---- Last arriver: merge the n_splits partials of (b, g).
  // Task (sub, oc) combines float4 chunk oc of splits sub, sub + NSUB, ...
  // with its own running reference; the (m, l) of chunk oc's head come from
  // the same splits, so each task's (m, l, acc) triple is self-consistent.
  const float4 *parts =
      reinterpret_cast<const float4 *>(a.part_acc + ((int64_t)first_split * H + g) * G * C::PROW);
  const int64_t split_stride4 = (int64_t)H * G * C::PROW / 4;  // float4s between splits
  constexpr int NSUB = (C::NT / C::NCH) > 0 ? (C::NT / C::NCH) : 1;
  constexpr int MAXS = 8;  // splits per task in flight per batch
  __shared__ float4 s_pacc[NSUB][C::NCH];
  __shared__ float s_pm[NSUB][C::NCH];
  __shared__ float s_pl[NSUB][C::NCH];
  for (int task = tid; task < NSUB * C::NCH; task += C::NT) {
    const int sub = task / C::NCH;
    const int oc = task - sub * C::NCH;
    const int ml_chunk = (((oc * 4) / C::PROW) * C::PROW + DH) / 4;
    float mr = -INFINITY, lr = 0.f;
    float4 ar = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s0 = sub; s0 < n_splits; s0 += NSUB * MAXS) {
      // Every load of the batch is issued at a clamped split (a load under a
      // branch would be waited for before the branch joins: one round trip
      // per split), then the splits past the last are replaced by the
      // empty state.
      // (Only the 8 bytes of (m, l) are loaded: a loaded value left unused
      // would also force a wait, since its register is then reused while
      // the load is still in flight.)
      float4 vv[MAXS];
      float2 mm[MAXS];
#pragma unroll
      for (int k = 0; k < MAXS; ++k) {
        const int s = min(s0 + k * NSUB, n_splits - 1);
        vv[k] = load_agent4(parts + s * split_stride4 + oc);
        mm[k] = load_agent2(reinterpret_cast<const float *>(parts + s * split_stride4 + ml_chunk));
      }
#pragma unroll
      for (int k = 0; k < MAXS; ++k) {
        if (s0 + k * NSUB >= n_splits) {
          vv[k] = make_float4(0.f, 0.f, 0.f, 0.f);
          mm[k] = make_float2(-INFINITY, 0.f);
        }
      }
      float mb = mr;
#pragma unroll
      for (int k = 0; k < MAXS; ++k) mb = fmaxf(mb, mm[k].x);
      const float wr = merge_weight(mr, mb);
      lr *= wr;
      ar.x *= wr; ar.y *= wr; ar.z *= wr; ar.w *= wr;
#pragma unroll
      for (int k = 0; k < MAXS; ++k) {
        const float w = merge_weight(mm[k].x, mb);
        lr = fmaf(w, mm[k].y, lr);
        ar.x = fmaf(w, vv[k].x, ar.x);
        ar.y = fmaf(w, vv[k].y, ar.y);
        ar.z = fmaf(w, vv[k].z, ar.z);
        ar.w = fmaf(w, vv[k].w, ar.w);
      }
      mr = mb;
    }
    s_pacc[sub][oc] = ar;
    s_pm[sub][oc] = mr;
    s_pl[sub][oc] = lr;
  }
  __syncthreads();
  const int h0 = g * G;
  for (int idx = tid; idx < G * DH / 4; idx += C::NT) {
    const int i = (idx * 4) / DH;
    const int e4 = idx - i * (DH / 4);
    const int oc = (i * C::PROW) / 4 + e4;
    float mt = -INFINITY;
    for (int sb = 0; sb < NSUB; ++sb) mt = fmaxf(mt, s_pm[sb][oc]);
    float L = 0.f;
    float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int sb = 0; sb < NSUB; ++sb) {
      const float w = merge_weight(s_pm[sb][oc], mt);
      L = fmaf(w, s_pl[sb][oc], L);
      const float4 v = s_pacc[sb][oc];
      A.x = fmaf(w, v.x, A.x);
      A.y = fmaf(w, v.y, A.y);
      A.z = fmaf(w, v.z, A.z);
      A.w = fmaf(w, v.w, A.w);
    }
    const float inv = 1.0f / L;
    A.x *= inv; A.y *= inv; A.z *= inv; A.w *= inv;
    reinterpret_cast<float4 *>(a.o + ((int64_t)b * a.n_q_heads + h0 + i) * DH)[e4] = A;
    if (e4 == 0 && a.lse != nullptr) a.lse[(int64_t)b * a.n_q_heads + h0 + i] = (mt + log2f(L)) * kLn2;
  }
  if (tid == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace yoco
