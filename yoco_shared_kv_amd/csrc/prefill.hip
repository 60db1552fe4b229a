// Causal cross-attention of a block of query rows over the shared cache
// (prefill / training forward).
//
// What it computes ([Notes] "YOCO：You Only Cache Once 中文精读笔记" s.2.1
// Eq. 3, causal mask m <= n, GQA; [Blog] "NeurIPS'24 | YOCO: 长上下文 LLM
// 为什么不必每层都存一份 KV Cache?" s.2): query row i at absolute position
// p = q_start + i, head h, reads cache rows 0..p of KV head g = h / G:
//   o = softmax(scale * q K^T) V,  lse = ln sum exp(scale * q K^T).
//
// bf16 path (a dense contraction, so it runs on MFMA):
//   A workgroup is 4 waves = 128 query rows of one query head; each wave owns
//   32 rows.  Keys are processed in tiles of 64 rows.
//   * Staging: each K or V tile (64 rows x head_dim bf16) is copied straight
//     from global memory into LDS with 16-byte direct-to-LDS loads (no
//     registers), two buffers deep: the loads of tile kt+1 are in flight
//     while tile kt is computed.  Rows are stored unpadded with the 16-byte
//     chunk index XOR-swizzled by the row (slot = chunk ^ (row % chunks)), so
//     the operand reads below hit distinct LDS banks.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16 (A = K rows read from LDS, B = Q^T kept in
//     registers).  In the 32x32 accumulator layout each lane holds ONE query
//     row (its column) and 16 of the 32 keys; the other 16 keys of the row
//     sit in lane l ^ 32.  Row maxima need one cross-lane exchange per tile
//     and the running sum stays lane-local.
//   * The output is accumulated transposed too, O^T += V^T P^T.  P^T comes
//     straight from the score accumulators (rounded to bf16) as the B
//     operand; the MFMA's k order is free as long as A and B agree, so the
//     keys each lane already holds define it.  The A operand V^T is read from
//     the row-major V tile with ds_read_b64_tr_b16, which hands each lane 4
//     consecutive keys of one head-dim column (two reads per MFMA).
//   * Softmax: the scale is folded into one FMA per score before exp2, and
//     the reference maximum moves only when a tile's maximum passes it by
//     more than 8 (log2 units), so the O^T rescale is rare and every
//     probability is <= 2^8.
//   * Causality: a workgroup visits key tiles 0..(last position it needs)/64;
//     a wave skips tiles wholly above its rows, and the diagonal tile masks
//     keys > p.  Workgroups run longest first, and the G query heads of a KV
//     group for the same query tile are placed on the same XCD so their K/V
//     tiles are shared in that XCD's L2.
// fp32 path: plain fp32 VALU kernel (one lane per query row, exact online
// softmax) for fp32 caches.
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
constexpr int kWaves = 4;
constexpr int kRowsPerWave = 32;
constexpr int kBlockRows = kWaves * kRowsPerWave;  // 128 query rows
constexpr int kKeyTile = 64;
constexpr int kThreads = kWaves * 64;
constexpr int kXcds = 8;
constexpr float kRescaleSlack = 8.0f;
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

template <int DH>
struct PrefillShape {
  static constexpr int kChunks = DH / 8;                    // 16-byte chunks per row
  static constexpr int kRowBytes = DH * 2;
  static constexpr int kTileBytes = pf::kKeyTile * kRowBytes;
  static constexpr int kRowsPerLoad = 64 / kChunks;         // rows per wave-wide 1 KiB load
  static constexpr int kLoadsPerTile = pf::kKeyTile / kRowsPerLoad;    // per K (or V) tile
  static constexpr int kLoadsPerWave = kLoadsPerTile / pf::kWaves;
  static constexpr int KSTEPS = DH / 16;                    // S^T k-steps over head_dim
  static constexpr int DSUB = DH / 32;                      // O^T 32-row tiles over head_dim
};

// LDS byte offset of element `dim` (multiple of 4 for 8-byte reads, of 8 for
// 16-byte reads) of tile row `row`, with the XOR-swizzled chunk layout.
template <int DH>
__device__ __forceinline__ int swz(int row, int dim) {
  using S = PrefillShape<DH>;
  const int chunk = dim >> 3;
  const int slot = chunk ^ (row & (S::kChunks - 1));
  return row * S::kRowBytes + slot * 16 + (dim & 7) * 2;
}

// Issue this wave's share of the direct-to-LDS loads of one K/V tile pair.
template <int DH>
__device__ __forceinline__ void stage_tile(char *lds_k, char *lds_v, const bf16_t *kg, const bf16_t *vg,
                                           int64_t row_stride, int64_t key0, int64_t kv_len, int wave,
                                           int lane) {
  using S = PrefillShape<DH>;
#pragma unroll
  for (int i = 0; i < S::kLoadsPerWave; ++i) {
    const int blk = wave * S::kLoadsPerWave + i;        // which 1 KiB block of the tile
    const int row = blk * S::kRowsPerLoad + lane / S::kChunks;
    const int slot = lane % S::kChunks;
    const int chunk = slot ^ (row & (S::kChunks - 1));
    int64_t key = key0 + row;
    key = key < kv_len ? key : kv_len - 1;              // rows past the data are masked later
    const int64_t goff = key * row_stride + chunk * 8;
    __builtin_amdgcn_global_load_lds(static_cast<const void *>(kg + goff),
                                     (lds_void_t *)(lds_k + blk * 1024), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(static_cast<const void *>(vg + goff),
                                     (lds_void_t *)(lds_v + blk * 1024), 16, 0, 0);
  }
}

template <int DH>
__global__ __launch_bounds__(pf::kThreads, 2) void prefill_bf16_kernel(const PrefillArgs a) {
  using S = PrefillShape<DH>;
  __shared__ __attribute__((aligned(1024))) char lds_k[2][S::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char lds_v[2][S::kTileBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;       // 0 or 1
  const int col = lane & 31;        // the query row this lane owns (within the wave)

  // Block -> (query tile, query head): units (qtile, g) longest first; the G
  // heads of a unit get consecutive slots on the same XCD.
  const int group = a.n_q_heads / a.n_kv_heads;
  const int n_qtiles = static_cast<int>((a.t + pf::kBlockRows - 1) / pf::kBlockRows);
  const int n_units = n_qtiles * a.n_kv_heads;
  const int xcd = blockIdx.x % pf::kXcds;
  const int slot_on_xcd = blockIdx.x / pf::kXcds;
  const int unit = (slot_on_xcd / group) * pf::kXcds + xcd;
  if (unit >= n_units) return;
  const int qtile = n_qtiles - 1 - unit / a.n_kv_heads;
  const int g = unit % a.n_kv_heads;
  const int h = g * group + slot_on_xcd % group;

  const int64_t row_stride_q = (int64_t)a.n_q_heads * DH;
  const int64_t row_stride_kv = (int64_t)a.n_kv_heads * DH;
  const bf16_t *qg = static_cast<const bf16_t *>(a.q);
  const bf16_t *kg = static_cast<const bf16_t *>(a.k) + g * DH;
  const bf16_t *vg = static_cast<const bf16_t *>(a.v) + g * DH;

  const int64_t blk_row0 = (int64_t)qtile * pf::kBlockRows;
  const int64_t wave_row_first = blk_row0 + wave * pf::kRowsPerWave;
  const int64_t my_row = wave_row_first + col;
  const bool row_valid = my_row < a.t;
  const int64_t my_pos = a.q_start + (row_valid ? my_row : (a.t - 1));
  const int64_t wave_last_row = min(wave_row_first + pf::kRowsPerWave, a.t) - 1;
  const int64_t wave_pos_last = a.q_start + wave_last_row;
  const int64_t wave_pos_first = a.q_start + wave_row_first;
  const int64_t blk_last_row = min(blk_row0 + pf::kBlockRows, a.t) - 1;
  const int n_ktiles = static_cast<int>((a.q_start + blk_last_row) / pf::kKeyTile) + 1;
  const bool wave_active = wave_row_first < a.t;

  // Start loading key tile 0 before touching Q.
  stage_tile<DH>(lds_k[0], lds_v[0], kg, vg, row_stride_kv, 0, a.kv_len, wave, lane);

  // Q^T as the MFMA B operand: lane holds row `col`, dims ks*16 + half*8 .. +8.
  Frag8 qf[S::KSTEPS];
  {
    const bf16_t *qp = qg + (row_valid ? my_row : 0) * row_stride_q + (int64_t)h * DH + half * 8;
#pragma unroll
    for (int ks = 0; ks < S::KSTEPS; ++ks) qf[ks].u = row_valid ? ld16(qp + ks * 16) : make_uint4(0, 0, 0, 0);
  }

  floatx16 oacc[S::DSUB];
#pragma unroll
  for (int d = 0; d < S::DSUB; ++d) {
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[d][i] = 0.f;
  }
  float m_run = -INFINITY;  // reference max (log2 units) of this lane's query row
  float l_run = 0.f;        // this lane's share of the running sum

  for (int kt = 0; kt < n_ktiles; ++kt) {
    // Tile kt has landed for every wave, and every wave is done with tile kt-1,
    // whose buffer the next loads overwrite.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const int buf = kt & 1;
    if (kt + 1 < n_ktiles) {
      stage_tile<DH>(lds_k[buf ^ 1], lds_v[buf ^ 1], kg, vg, row_stride_kv, (int64_t)(kt + 1) * pf::kKeyTile,
                     a.kv_len, wave, lane);
    }
    const int64_t key0 = (int64_t)kt * pf::kKeyTile;
    if (!wave_active || key0 > wave_pos_last) continue;
    char *tk = lds_k[buf];
    char *tv = lds_v[buf];

    // ---- S^T = K Q^T for two 32-key sub-tiles ----
    floatx16 sacc[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[sub][i] = 0.f;
      const int krow = sub * 32 + col;
#pragma unroll
      for (int ks = 0; ks < S::KSTEPS; ++ks) {
        Frag8 af;
        af.u = *reinterpret_cast<const uint4 *>(tk + swz<DH>(krow, ks * 16 + half * 8));
        sacc[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af.v, qf[ks].v, sacc[sub], 0, 0, 0);
      }
    }
    // ---- causal mask (diagonal tiles only) and tile maximum ----
    // Accumulator element i of sub-tile `sub` is key
    //   key0 + sub*32 + (i/4)*8 + half*4 + (i%4)   for query row `col`.
    if (key0 + pf::kKeyTile - 1 > wave_pos_first) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int64_t key = key0 + sub * 32 + (i >> 2) * 8 + half * 4 + (i & 3);
          if (key > my_pos) sacc[sub][i] = -INFINITY;
        }
      }
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
      for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, sacc[sub][i]);
    }
    tmax = fmaxf(tmax, shfl_xor_f(tmax, 32)) * a.scale_log2;  // scale > 0 keeps the order
    // Lazy rescale (both lanes of a row take the same decision).
    const bool need = tmax > m_run + pf::kRescaleSlack;
    if (__any(need)) {
      if (need) {
        const float alpha = fast_exp2(m_run - tmax);  // m_run = -inf gives 0
        l_run *= alpha;
#pragma unroll
        for (int d = 0; d < S::DSUB; ++d) {
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[d][i] *= alpha;
        }
        m_run = tmax;
      }
    }
    // ---- P^T (bf16) as the B operand of O^T += V^T P^T ----
    Frag8 pfr[2][2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p0 = fast_exp2(fmaf(sacc[sub][kk * 8 + 2 * j], a.scale_log2, -m_run));
          const float p1 = fast_exp2(fmaf(sacc[sub][kk * 8 + 2 * j + 1], a.scale_log2, -m_run));
          l_run += p0 + p1;
          pfr[sub][kk].w[j] = cvt_pk_bf16(p0, p1);
        }
      }
    }
    // k-slot j of lane half `half` in step (sub, kk) is key
    //   sub*32 + kk*16 + (j/4)*8 + half*4 + (j%4).
    // A operand V^T via two transposed reads: in each 16-lane group, source
    // lane a + 4j points at key kb + j, dims dbase + 4a .. +3, and lane i of
    // the group receives keys kb..kb+3 of dim dbase + i.
    const int grp = lane >> 4;                 // 16-lane group
    const int src_a = lane & 3;
    const int src_j = (lane >> 2) & 3;
    const int dcol = (grp & 1) * 16 + src_a * 4;
#pragma unroll
    for (int d = 0; d < S::DSUB; ++d) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int kb = sub * 32 + kk * 16 + (grp >> 1) * 4 + src_j;
          Frag8 af;
          af.s4[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_shortx4_t *)(tv + swz<DH>(kb, d * 32 + dcol)));
          af.s4[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_shortx4_t *)(tv + swz<DH>(kb + 8, d * 32 + dcol)));
          oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af.v, pfr[sub][kk].v, oacc[d], 0, 0, 0);
        }
      }
    }
  }

  const float l_tot = l_run + shfl_xor_f(l_run, 32);
  if (!row_valid) return;
  const float inv = 1.0f / l_tot;
  // O^T accumulator element i of tile d is dim d*32 + (i/4)*8 + half*4 + (i%4)
  // of query row `col`.
  if (a.o_bf16) {
    bf16_t *op = static_cast<bf16_t *>(a.o) + my_row * row_stride_q + (int64_t)h * DH;
#pragma unroll
    for (int d = 0; d < S::DSUB; ++d) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int dim = d * 32 + i4 * 8 + half * 4;
        uint2 packed;
        packed.x = cvt_pk_bf16(oacc[d][i4 * 4 + 0] * inv, oacc[d][i4 * 4 + 1] * inv);
        packed.y = cvt_pk_bf16(oacc[d][i4 * 4 + 2] * inv, oacc[d][i4 * 4 + 3] * inv);
        *reinterpret_cast<uint2 *>(op + dim) = packed;
      }
    }
  } else {
    float *op = static_cast<float *>(a.o) + my_row * row_stride_q + (int64_t)h * DH;
#pragma unroll
    for (int d = 0; d < S::DSUB; ++d) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int dim = d * 32 + i4 * 8 + half * 4;
        float4 v = make_float4(oacc[d][i4 * 4 + 0] * inv, oacc[d][i4 * 4 + 1] * inv,
                               oacc[d][i4 * 4 + 2] * inv, oacc[d][i4 * 4 + 3] * inv);
        *reinterpret_cast<float4 *>(op + dim) = v;
      }
    }
  }
  if (a.lse != nullptr && half == 0) {
    a.lse[my_row * a.n_q_heads + h] = (m_run + log2f(l_tot)) * kLn2;
  }
}

// fp32 path: one lane per (query row, head); the 64 lanes of a wave are 64
// consecutive query rows of one head and read each K/V row together.
template <int DH>
__global__ __launch_bounds__(64) void prefill_f32_kernel(const PrefillArgs a) {
  const int lane = threadIdx.x;
  const int n_rtiles = static_cast<int>((a.t + 63) / 64);
  const int rtile = n_rtiles - 1 - static_cast<int>(blockIdx.x / a.n_q_heads);
  const int h = static_cast<int>(blockIdx.x % a.n_q_heads);
  const int g = h / (a.n_q_heads / a.n_kv_heads);
  const int64_t row = (int64_t)rtile * 64 + lane;
  const bool valid = row < a.t;
  const int64_t pos = a.q_start + (valid ? row : a.t - 1);
  const int64_t last_row = min((int64_t)rtile * 64 + 63, a.t - 1);
  const int64_t last_pos = a.q_start + last_row;

  const int64_t rs_q = (int64_t)a.n_q_heads * DH;
  const int64_t rs_kv = (int64_t)a.n_kv_heads * DH;
  const float *qp = static_cast<const float *>(a.q) + (valid ? row : 0) * rs_q + (int64_t)h * DH;
  const float *kg = static_cast<const float *>(a.k) + g * DH;
  const float *vg = static_cast<const float *>(a.v) + g * DH;

  float q[DH], acc[DH];
#pragma unroll
  for (int e = 0; e < DH; ++e) {
    q[e] = qp[e];
    acc[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int64_t j = 0; j <= last_pos; ++j) {
    const float *kr = kg + j * rs_kv;
    const float *vr = vg + j * rs_kv;
    float d = 0.f;
#pragma unroll
    for (int e = 0; e < DH; ++e) d = fmaf(q[e], kr[e], d);
    if (j <= pos) {
      const float x = d * a.scale_log2;
      const float mn = fmaxf(m, x);
      const float alpha = fast_exp2(m - mn);
      const float p = fast_exp2(x - mn);
      l = l * alpha + p;
#pragma unroll
      for (int e = 0; e < DH; ++e) acc[e] = fmaf(p, vr[e], acc[e] * alpha);
      m = mn;
    }
  }
  if (!valid) return;
  const float inv = 1.0f / l;
  if (a.o_bf16) {
    bf16_t *op = static_cast<bf16_t *>(a.o) + row * rs_q + (int64_t)h * DH;
#pragma unroll
    for (int e = 0; e < DH; ++e) op[e] = f32_to_bf16(acc[e] * inv);
  } else {
    float *op = static_cast<float *>(a.o) + row * rs_q + (int64_t)h * DH;
#pragma unroll
    for (int e = 0; e < DH; ++e) op[e] = acc[e] * inv;
  }
  if (a.lse != nullptr) a.lse[row * a.n_q_heads + h] = (m + log2f(l)) * kLn2;
}

hipError_t launch_prefill(const PrefillArgs &a, int dtype, int head_dim, hipStream_t s) {
  if (dtype == YOCO_DT_BF16) {
    const int64_t n_qtiles = (a.t + pf::kBlockRows - 1) / pf::kBlockRows;
    const int64_t n_units = n_qtiles * a.n_kv_heads;
    const int64_t group = a.n_q_heads / a.n_kv_heads;
    const unsigned int blocks =
        static_cast<unsigned int>(((n_units + pf::kXcds - 1) / pf::kXcds) * pf::kXcds * group);
    if (head_dim == 128) {
      hipLaunchKernelGGL(prefill_bf16_kernel<128>, dim3(blocks), dim3(pf::kThreads), 0, s, a);
    } else if (head_dim == 64) {
      hipLaunchKernelGGL(prefill_bf16_kernel<64>, dim3(blocks), dim3(pf::kThreads), 0, s, a);
    } else {
      return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  if (dtype == YOCO_DT_F32) {
    const unsigned int blocks = static_cast<unsigned int>((a.t + 63) / 64) * a.n_q_heads;
    if (head_dim == 128) {
      hipLaunchKernelGGL(prefill_f32_kernel<128>, dim3(blocks), dim3(64), 0, s, a);
    } else if (head_dim == 64) {
      hipLaunchKernelGGL(prefill_f32_kernel<64>, dim3(blocks), dim3(64), 0, s, a);
    } else {
      return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

}  // namespace yoco
