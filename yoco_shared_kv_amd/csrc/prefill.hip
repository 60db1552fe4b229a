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
#include <type_traits>

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

__device__ __forceinline__ float dot2_bf16_f32(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
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

// Row-dependent XOR applied to the 16-byte chunk index of a tile row.
// Mode 0: row % chunks.  Mode 1 (head_dim 128): bits (r1 r0 r2) in the low
// three bits plus r3, so that 8 consecutive rows hit 8 distinct chunk slots
// mod 8 (16-byte K reads) and rows 4k..4k+3 with chunks c, c^1 hit 8
// distinct slots mod 8 (the 8-byte transposed V reads of one 16-lane group).
// Mode 2 (head_dim 128): (r1 r0) in bits 3..2 and (r3 r2) in bits 1..0.
template <int DH, int SWZ>
__device__ __forceinline__ int row_xor(int row) {
  using S = PrefillShape<DH>;
  if constexpr (SWZ == 1 && S::kChunks == 16) {
    return ((row & 3) << 1) | ((row >> 2) & 1) | (row & 8);
  } else if constexpr (SWZ == 2 && S::kChunks == 16) {
    return ((row & 3) << 2) | ((row >> 2) & 3);
  } else {
    return row & (S::kChunks - 1);
  }
}

// LDS byte offset of element `dim` (multiple of 4 for 8-byte reads, of 8 for
// 16-byte reads) of tile row `row`, with the XOR-swizzled chunk layout.
template <int DH, int SWZ>
__device__ __forceinline__ int swz(int row, int dim) {
  using S = PrefillShape<DH>;
  const int chunk = dim >> 3;
  const int slot = chunk ^ row_xor<DH, SWZ>(row);
  return row * S::kRowBytes + slot * 16 + (dim & 7) * 2;
}

// Per-lane element offsets (within a tile) of this wave's direct-to-LDS
// loads: load i of the wave fills 1 KiB block blk = wave * kLoadsPerWave + i,
// lane L writes LDS bytes blk*1024 + L*16 = (row, slot) and so reads global
// chunk slot ^ row_xor(row) of that row.
template <int DH, int SWZ>
struct StageOffsets {
  using S = PrefillShape<DH>;
  int row[S::kLoadsPerWave];
  int goff[S::kLoadsPerWave];  // row * row_stride + chunk * 8 (elements)
  __device__ __forceinline__ void init(int wave, int lane, int row_stride) {
#pragma unroll
    for (int i = 0; i < S::kLoadsPerWave; ++i) {
      const int blk = wave * S::kLoadsPerWave + i;
      row[i] = blk * S::kRowsPerLoad + lane / S::kChunks;
      const int chunk = (lane % S::kChunks) ^ row_xor<DH, SWZ>(row[i]);
      goff[i] = row[i] * row_stride + chunk * 8;
    }
  }
};

// Issue this wave's share of the direct-to-LDS loads of one K/V tile pair
// (tile rows key0 .. key0+63; rows at or past kv_len re-read row kv_len-1 and
// are masked by causality later).
template <int DH, int SWZ>
__device__ __forceinline__ void stage_tile(char *lds_k, char *lds_v, const bf16_t *kg, const bf16_t *vg,
                                           int row_stride, int64_t key0, int64_t kv_len, int wave,
                                           const StageOffsets<DH, SWZ> &so) {
  using S = PrefillShape<DH>;
  const int64_t tile_base = key0 * row_stride;
  const bf16_t *kt = kg + tile_base;
  const bf16_t *vt = vg + tile_base;
  const bool full = key0 + pf::kKeyTile <= kv_len;
#pragma unroll
  for (int i = 0; i < S::kLoadsPerWave; ++i) {
    const int blk = wave * S::kLoadsPerWave + i;
    int off = so.goff[i];
    if (!full && key0 + so.row[i] >= kv_len) {
      off += static_cast<int>(kv_len - 1 - key0 - so.row[i]) * row_stride;
    }
    __builtin_amdgcn_global_load_lds(static_cast<const void *>(kt + off),
                                     (lds_void_t *)(lds_k + blk * 1024), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(static_cast<const void *>(vt + off),
                                     (lds_void_t *)(lds_v + blk * 1024), 16, 0, 0);
  }
}

template <int DH, int SWZ>
__global__ __launch_bounds__(pf::kThreads, 2) void prefill_bf16_kernel(const PrefillArgs a) {
  using S = PrefillShape<DH>;
  // [buffer][K, V][tile]: every LDS read below is a per-lane offset plus a
  // compile-time immediate.
  __shared__ __attribute__((aligned(1024))) char lds[2][2][S::kTileBytes];

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
  const int row_stride_kv = a.n_kv_heads * DH;
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

  StageOffsets<DH, SWZ> so;
  so.init(wave, lane, row_stride_kv);
  // Start loading key tile 0 before touching Q.
  stage_tile<DH, SWZ>(lds[0][0], lds[0][1], kg, vg, row_stride_kv, 0, a.kv_len, wave, so);

  // Q^T as the MFMA B operand: lane holds row `col`, dims ks*16 + half*8 .. +8.
  Frag8 qf[S::KSTEPS];
  {
    const bf16_t *qp = qg + (row_valid ? my_row : 0) * row_stride_q + (int64_t)h * DH + half * 8;
#pragma unroll
    for (int ks = 0; ks < S::KSTEPS; ++ks) qf[ks].u = row_valid ? ld16(qp + ks * 16) : make_uint4(0, 0, 0, 0);
  }

  // LDS read offsets within a tile.  K (A operand of S^T): row sub*32 + col,
  // dims ks*16 + half*8; the row_xor of the swizzle depends only on row mod
  // 16, so sub adds the immediate sub*32*rowbytes.
  int koff[S::KSTEPS];
#pragma unroll
  for (int ks = 0; ks < S::KSTEPS; ++ks) koff[ks] = swz<DH, SWZ>(col, ks * 16 + half * 8);
  // V^T (A operand of O^T) via transposed reads: in each 16-lane group,
  // source lane a + 4j points at key kb + j, dims dbase + 4a .. +3, and lane
  // i of the group receives keys kb..kb+3 of dim dbase + i.  With
  // kb = sub*32 + kk*16 + (grp/2)*4 + j and the second read at kb + 8, only
  // (read r, dim tile d) changes the swizzled offset; sub and kk are
  // immediates.
  const int grp = lane >> 4;
  const int src_a = lane & 3;
  const int src_j = (lane >> 2) & 3;
  const int vrow = (grp >> 1) * 4 + src_j;
  const int dcol = (grp & 1) * 16 + src_a * 4;
  int voff[2][S::DSUB];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
#pragma unroll
    for (int d = 0; d < S::DSUB; ++d) voff[r][d] = swz<DH, SWZ>(vrow + 8 * r, d * 32 + dcol);
  }

  floatx16 oacc[S::DSUB];
#pragma unroll
  for (int d = 0; d < S::DSUB; ++d) {
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[d][i] = 0.f;
  }
  float m_run = -INFINITY;  // reference max (log2 units) of this lane's query row
  float l_run = 0.f;        // this lane's share of sum(p), from the bf16 p the MFMA uses
  const uint32_t kOnesBf16x2 = 0x3F803F80u;  // (1.0, 1.0) in bf16

  auto tile_step = [&](auto buf_c, int kt) {
    constexpr int BUF = decltype(buf_c)::value;
    // Tile kt has landed for every wave, and every wave is done with tile kt-1,
    // whose buffer the next loads overwrite.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (kt + 1 < n_ktiles) {
      stage_tile<DH, SWZ>(lds[BUF ^ 1][0], lds[BUF ^ 1][1], kg, vg, row_stride_kv,
                          (int64_t)(kt + 1) * pf::kKeyTile, a.kv_len, wave, so);
    }
    const int64_t key0 = (int64_t)kt * pf::kKeyTile;
    if (!wave_active || key0 > wave_pos_last) return;
    char *tk = lds[BUF][0];
    char *tv = lds[BUF][1];

    // ---- S^T = K Q^T for two 32-key sub-tiles ----
    floatx16 sacc[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[sub][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < S::KSTEPS; ++ks) {
        Frag8 af;
        af.u = *reinterpret_cast<const uint4 *>(tk + koff[ks] + sub * 32 * S::kRowBytes);
        sacc[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af.v, qf[ks].v, sacc[sub], 0, 0, 0);
      }
    }
    // ---- causal mask (diagonal tiles only) ----
    // Accumulator element i of sub-tile `sub` is key
    //   key0 + sub*32 + (i/4)*8 + half*4 + (i%4)   for query row `col`.
    if (key0 + pf::kKeyTile - 1 > wave_pos_first) {
      const int64_t rel64 = my_pos - key0;
      const int rel = rel64 < pf::kKeyTile ? static_cast<int>(rel64) : pf::kKeyTile;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if (sub * 32 + (i >> 2) * 8 + half * 4 + (i & 3) > rel) sacc[sub][i] = -INFINITY;
        }
      }
    }
    // ---- P^T (bf16) as the B operand of O^T += V^T P^T ----
    // Probabilities are formed against the current reference first (each
    // sub-tile as soon as its scores exist, so the exps of sub-tile 0 can
    // overlap the MFMAs of sub-tile 1); the tile maximum is checked
    // alongside, and in the rare case that it passes the reference by more
    // than the slack, O and l are rescaled and P is formed again.
    Frag8 pfr[2][2];
    auto make_p = [&](int sub) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p0 = fast_exp2(fmaf(sacc[sub][kk * 8 + 2 * j], a.scale_log2, -m_run));
          const float p1 = fast_exp2(fmaf(sacc[sub][kk * 8 + 2 * j + 1], a.scale_log2, -m_run));
          pfr[sub][kk].w[j] = cvt_pk_bf16(p0, p1);
        }
      }
    };
    make_p(0);
    make_p(1);
    float tmax = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
      for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, sacc[sub][i]);
    }
    tmax = fmaxf(tmax, shfl_xor_f(tmax, 32)) * a.scale_log2;  // scale > 0 keeps the order
    // Both lanes of a row take the same decision.
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
      make_p(0);
      make_p(1);
    }
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int j = 0; j < 4; ++j) l_run = dot2_bf16_f32(pfr[sub][kk].w[j], kOnesBf16x2, l_run);
      }
    }
    // k-slot j of lane half `half` in step (sub, kk) is key
    //   sub*32 + kk*16 + (j/4)*8 + half*4 + (j%4).
#pragma unroll
    for (int d = 0; d < S::DSUB; ++d) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int rows = (sub * 32 + kk * 16) * S::kRowBytes;
          Frag8 af;
          af.s4[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4_t *)(tv + voff[0][d] + rows));
          af.s4[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4_t *)(tv + voff[1][d] + rows));
          oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af.v, pfr[sub][kk].v, oacc[d], 0, 0, 0);
        }
      }
    }
  };

  for (int kt = 0; kt < n_ktiles; kt += 2) {
    tile_step(std::integral_constant<int, 0>(), kt);
    if (kt + 1 < n_ktiles) tile_step(std::integral_constant<int, 1>(), kt + 1);
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

constexpr int kPrefillSwizzle = 2;  // modes 1 and 2 both remove the 2-way V-read bank conflicts; 2 measured fastest

hipError_t launch_prefill(const PrefillArgs &a, int dtype, int head_dim, hipStream_t s) {
  if (dtype == YOCO_DT_BF16) {
    const int64_t n_qtiles = (a.t + pf::kBlockRows - 1) / pf::kBlockRows;
    const int64_t n_units = n_qtiles * a.n_kv_heads;
    const int64_t group = a.n_q_heads / a.n_kv_heads;
    const unsigned int blocks =
        static_cast<unsigned int>(((n_units + pf::kXcds - 1) / pf::kXcds) * pf::kXcds * group);
    if (head_dim == 128) {
      hipLaunchKernelGGL((prefill_bf16_kernel<128, kPrefillSwizzle>), dim3(blocks), dim3(pf::kThreads), 0, s, a);
    } else if (head_dim == 64) {
      hipLaunchKernelGGL((prefill_bf16_kernel<64, kPrefillSwizzle>), dim3(blocks), dim3(pf::kThreads), 0, s, a);
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
