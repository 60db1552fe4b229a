// Causal cross-attention of a block of query rows over the shared cache
// (prefill / training forward).
//
// What it computes ([Notes] "YOCO：You Only Cache Once 中文精读笔记" s.2.1
// Eq. 3, causal mask m <= n, GQA; [Blog] "NeurIPS'24 | YOCO: 长上下文 LLM
// 为什么不必每层都存一份 KV Cache?" s.2): query row i at absolute position
// p = q_start + i, head h, reads cache rows 0..p of KV head g = h / G:
//   o = softmax(scale * q K^T) V,  lse = ln sum exp(scale * q K^T).
//
// bf16 path (dense contraction, so it runs on MFMA):
//   One workgroup = 4 waves = 128 query rows of one query head; each wave owns
//   32 rows.  Keys are processed in tiles of 64 rows staged in LDS: K row-major
//   (padded rows), V transposed (V^T[dim][key], padded) so that both MFMA
//   operands are read with contiguous LDS loads.
//   Scores are computed transposed, S^T = K Q^T, with
//   v_mfma_f32_32x32x16_bf16 (A = K from LDS, B = Q^T kept in registers), so
//   in the 32x32 accumulator layout every lane holds ONE query row (its
//   column) and 16 of the 32 keys; the other 16 keys of that row sit in lane
//   l ^ 32.  Row maxima therefore need one cross-lane exchange per tile and
//   the running sum stays lane-local.
//   The output is accumulated transposed too, O^T += V^T P^T, with P^T taken
//   straight from the score accumulators (rounded to bf16) as the B operand:
//   the k-index order of the MFMA is free as long as A and B agree, so the
//   keys a lane already holds define the order and the V^T operand is read
//   to match.  Each lane's O^T column is its own query row, so rescaling by
//   exp2(m_old - m_new) is lane-local.
//   Causality: a workgroup visits key tiles 0..(last position it needs)/64;
//   a wave skips tiles that lie wholly above its rows, and the diagonal tile
//   masks keys > p with -inf.  Workgroups are launched longest-first.
// fp32 path: plain fp32 VALU kernel (one lane per query row, exact online
// softmax) for fp32 caches.
#include "device_common.h"
#include "yoco_internal.h"

namespace yoco {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

namespace pf {
constexpr int kWaves = 4;
constexpr int kRowsPerWave = 32;
constexpr int kBlockRows = kWaves * kRowsPerWave;  // 128 query rows
constexpr int kKeyTile = 64;
constexpr int kThreads = kWaves * 64;
}  // namespace pf

union Frag8 {
  bf16x8_t v;
  uint4 u;
  uint32_t w[4];
  uint2 h[2];
};

template <int DH>
struct PrefillLds {
  static constexpr int KPAD = DH + 8;            // K row stride (bf16): 16 B pad
  static constexpr int VPAD = pf::kKeyTile + 4;  // V^T row stride (bf16): 8 B pad
  bf16_t k[pf::kKeyTile * KPAD];
  bf16_t vt[DH * VPAD];
};

template <int DH>
__global__ __launch_bounds__(pf::kThreads) void prefill_bf16_kernel(const PrefillArgs a) {
  using L = PrefillLds<DH>;
  __shared__ L lds;
  constexpr int KSTEPS = DH / 16;   // MFMA k-steps over head_dim for S^T
  constexpr int DSUB = DH / 32;     // 32-row MFMA tiles over head_dim for O^T

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;       // 0 or 1
  const int col = lane & 31;        // the query row this lane owns (within the wave)

  const int n_qtiles = static_cast<int>((a.t + pf::kBlockRows - 1) / pf::kBlockRows);
  const int qtile = n_qtiles - 1 - static_cast<int>(blockIdx.x / a.n_q_heads);  // longest first
  const int h = static_cast<int>(blockIdx.x % a.n_q_heads);
  const int g = h / (a.n_q_heads / a.n_kv_heads);

  const int64_t row_stride_q = (int64_t)a.n_q_heads * DH;
  const int64_t row_stride_kv = (int64_t)a.n_kv_heads * DH;
  const bf16_t *qg = static_cast<const bf16_t *>(a.q);
  const bf16_t *kg = static_cast<const bf16_t *>(a.k) + g * DH;
  const bf16_t *vg = static_cast<const bf16_t *>(a.v) + g * DH;

  const int64_t blk_row0 = (int64_t)qtile * pf::kBlockRows;
  const int64_t my_row = blk_row0 + wave * pf::kRowsPerWave + col;  // query row index
  const bool row_valid = my_row < a.t;
  const int64_t my_pos = a.q_start + (row_valid ? my_row : (a.t - 1));
  // Positions covered by this wave and by the whole workgroup.
  const int64_t wave_row_first = blk_row0 + wave * pf::kRowsPerWave;
  const int64_t wave_last_row = min(wave_row_first + pf::kRowsPerWave, a.t) - 1;
  const int64_t wave_pos_last = a.q_start + wave_last_row;
  const int64_t blk_last_row = min(blk_row0 + pf::kBlockRows, a.t) - 1;
  const int64_t blk_pos_last = a.q_start + blk_last_row;
  const int n_ktiles = static_cast<int>(blk_pos_last / pf::kKeyTile) + 1;
  const bool wave_active = wave_row_first < a.t;

  // Q^T as the MFMA B operand: lane holds row `col`, dims ks*16 + half*8 .. +8.
  Frag8 qf[KSTEPS];
  {
    const bf16_t *qp = qg + (row_valid ? my_row : 0) * row_stride_q + (int64_t)h * DH + half * 8;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      qf[ks].u = row_valid ? ld16(qp + ks * 16) : make_uint4(0, 0, 0, 0);
    }
  }

  floatx16 oacc[DSUB];
#pragma unroll
  for (int d = 0; d < DSUB; ++d) {
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[d][i] = 0.f;
  }
  float m_run = -INFINITY;  // running max (log2 units) of this lane's query row
  float l_run = 0.f;        // this lane's share of the running sum

  for (int kt = 0; kt < n_ktiles; ++kt) {
    const int64_t key0 = (int64_t)kt * pf::kKeyTile;
    // ---- stage K (row-major) and V (transposed) tiles in LDS ----
    constexpr int CHUNKS = pf::kKeyTile * DH / 8;  // 16-byte chunks per tile
#pragma unroll
    for (int cidx = tid; cidx < CHUNKS; cidx += pf::kThreads) {
      const int kr = cidx / (DH / 8);
      const int d0 = (cidx - kr * (DH / 8)) * 8;
      const int64_t key = key0 + kr;
      uint4 kvv = make_uint4(0, 0, 0, 0), vvv = make_uint4(0, 0, 0, 0);
      if (key < a.kv_len) {
        kvv = ld16(kg + key * row_stride_kv + d0);
        vvv = ld16(vg + key * row_stride_kv + d0);
      }
      *reinterpret_cast<uint4 *>(&lds.k[kr * L::KPAD + d0]) = kvv;
      const uint32_t vw[4] = {vvv.x, vvv.y, vvv.z, vvv.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        lds.vt[(d0 + 2 * j) * L::VPAD + kr] = static_cast<bf16_t>(vw[j] & 0xffffu);
        lds.vt[(d0 + 2 * j + 1) * L::VPAD + kr] = static_cast<bf16_t>(vw[j] >> 16);
      }
    }
    __syncthreads();

    if (wave_active && key0 <= wave_pos_last) {
      // ---- S^T = K Q^T for two 32-key sub-tiles ----
      floatx16 sacc[2];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[sub][i] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
          Frag8 af;
          af.u = *reinterpret_cast<const uint4 *>(&lds.k[(sub * 32 + col) * L::KPAD + ks * 16 + half * 8]);
          sacc[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af.v, qf[ks].v, sacc[sub], 0, 0, 0);
        }
      }
      // ---- scale, causal mask, running max ----
      // Accumulator element i of sub-tile `sub` is key
      //   key0 + sub*32 + (i/4)*8 + half*4 + (i%4)   for query row `col`.
      const bool diag = key0 + pf::kKeyTile - 1 > a.q_start + wave_row_first;
      float tmax = -INFINITY;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float x = sacc[sub][i] * a.scale_log2;
          if (diag) {
            const int64_t key = key0 + sub * 32 + (i >> 2) * 8 + half * 4 + (i & 3);
            if (key > my_pos) x = -INFINITY;
          }
          sacc[sub][i] = x;
          tmax = fmaxf(tmax, x);
        }
      }
      tmax = fmaxf(tmax, shfl_xor_f(tmax, 32));
      const float m_new = fmaxf(m_run, tmax);  // finite: key 0 is visible to every row
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < DSUB; ++d) {
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[d][i] *= alpha;
      }
      // ---- P^T (bf16) as the B operand of O^T += V^T P^T ----
      Frag8 pf8[2][2];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float p0 = fast_exp2(sacc[sub][kk * 8 + 2 * j] - m_new);
            const float p1 = fast_exp2(sacc[sub][kk * 8 + 2 * j + 1] - m_new);
            l_run += p0 + p1;
            pf8[sub][kk].w[j] = pack_bf16x2(p0, p1);
          }
        }
      }
      // k-slot j of lane half `half` in step (sub, kk) is key
      //   sub*32 + kk*16 + (j/4)*8 + half*4 + (j%4).
#pragma unroll
      for (int d = 0; d < DSUB; ++d) {
        const bf16_t *vrow = &lds.vt[(d * 32 + col) * L::VPAD];
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            const int kb = sub * 32 + kk * 16 + half * 4;
            Frag8 af;
            af.h[0] = *reinterpret_cast<const uint2 *>(vrow + kb);
            af.h[1] = *reinterpret_cast<const uint2 *>(vrow + kb + 8);
            oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af.v, pf8[sub][kk].v, oacc[d], 0, 0, 0);
          }
        }
      }
    }
    __syncthreads();
  }

  if (!row_valid) return;
  const float l_tot = l_run + shfl_xor_f(l_run, 32);
  // Note: the shuffle above runs before the early return for every lane in
  // the wave when the wave is partially valid; see the guard below.
  const float inv = 1.0f / l_tot;
  // O^T accumulator element i of tile d is dim d*32 + (i/4)*8 + half*4 + (i%4)
  // of query row `col`.
  if (a.o_bf16) {
    bf16_t *op = static_cast<bf16_t *>(a.o) + my_row * row_stride_q + (int64_t)h * DH;
#pragma unroll
    for (int d = 0; d < DSUB; ++d) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int dim = d * 32 + i4 * 8 + half * 4;
        uint2 packed;
        packed.x = pack_bf16x2(oacc[d][i4 * 4 + 0] * inv, oacc[d][i4 * 4 + 1] * inv);
        packed.y = pack_bf16x2(oacc[d][i4 * 4 + 2] * inv, oacc[d][i4 * 4 + 3] * inv);
        *reinterpret_cast<uint2 *>(op + dim) = packed;
      }
    }
  } else {
    float *op = static_cast<float *>(a.o) + my_row * row_stride_q + (int64_t)h * DH;
#pragma unroll
    for (int d = 0; d < DSUB; ++d) {
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
    const unsigned int blocks =
        static_cast<unsigned int>((a.t + pf::kBlockRows - 1) / pf::kBlockRows) * a.n_q_heads;
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
