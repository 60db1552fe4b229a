// Backward of causal cross-attention over the shared cache (training).
//
// What it computes: the gradient of [Notes] "YOCO：You Only Cache Once 中文精读
// 笔记" s.2.1 Eq. 3 (o = softmax(scale * q K^T) V over cache rows 0..p) with
// respect to the query, K^ and V^.  [Deep] "You Only Cache Once:
// Decoder-Decoder Architectures for Language Models" s.2.2: every cross layer
// reads the same K^/V^, so their gradients are the sums over the layers; each
// call ADDS its layer's dK, dV.  For query row i (position p), head h, KV head
// g = h / G, with P = softmax and dO the upstream gradient of o:
//   dP_j = <dO, v_j>,  D = sum_j P_j dP_j = <dO, o>,  dS_j = P_j (dP_j - D)
//   dq = scale * sum_j dS_j k_j;  dk_j += scale * dS_j q;  dv_j += P_j dO.
// P is recomputed from the forward's lse: P_j = exp(scale <q, k_j> - lse).
//
// Three kernels, no atomics (results are bitwise reproducible):
//   * bwd_rowstats_kernel: D = <dO, o> and lse * log2(e) per (row, head),
//     written transposed ([H_q][t]) into the caller's workspace.
//   * bwd_dq_kernel: the forward's layout (256 query rows of one query head
//     per workgroup, 32 per wave, K/V tiles of 64 rows double-buffered in
//     LDS by buffer loads).  Per 32-key half: S^T = K Q^T and dP^T = V dO^T
//     on MFMA (Q^T and dO^T in registers), dS^T formed in the accumulator
//     layout (one query row per lane), then dQ^T += K^T dS^T with K^T read
//     transposed from LDS.
//   * bwd_dkdv_kernel: one workgroup per (128 cache rows, KV head), 4 waves,
//     two workgroups per CU (so two waves per SIMD: one wave's exp and dS
//     work runs while the other's products occupy the matrix core), each
//     wave owning 32 cache rows whose K^T and V^T fragments stay in
//     registers.  Query rows of the G query heads stream through LDS
//     in tiles of 64 (Q, dO, lse, D).  Per 32-row half: S = Q K^T and
//     dP = dO V^T (one cache row per lane), P and dS formed there, then
//     dV += P^T dO and dK += dS^T Q with dO and Q read transposed from LDS.
//     The k order of the last two products follows the rows each lane holds
//     (any order works when both operands agree).
#include "attn_tiles.h"

namespace yoco {

namespace bw {
constexpr int kKvWaves = 4;                  // dK/dV workgroup: 4 waves, two workgroups per CU
constexpr int kKeysPerWave = 32;
constexpr int kBlockKeys = kKvWaves * kKeysPerWave;  // 128 cache rows per workgroup
constexpr int kKvThreads = kKvWaves * 64;
constexpr int kQTile = 64;                   // query rows per staged tile
constexpr int kSwizzle = 2;
}  // namespace bw

// ---------------------------------------------------------------------------
// D = <dO, o> and lse2 = lse * log2(e), transposed to [H_q][t].
// ---------------------------------------------------------------------------
template <int DH>
__global__ __launch_bounds__(256) void bwd_rowstats_kernel(const BwdArgs a) {
  constexpr int kLanes = DH / 8;  // lanes per (row, head), 8 elements each
  const int64_t items = a.t * a.n_q_heads;
  const int64_t item = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) / kLanes;
  const int sub = threadIdx.x % kLanes;
  float acc = 0.f;
  if (item < items) {
    const int64_t base = item * DH + sub * 8;
    Frag8 d;
    d.u = ld16(static_cast<const bf16_t *>(a.d_o) + base);
    float ov[8];
    if (a.o_bf16) {
      const uint4 r = ld16(static_cast<const bf16_t *>(a.o) + base);
      const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ov[2 * j] = bf16_lo(w[j]);
        ov[2 * j + 1] = bf16_hi(w[j]);
      }
    } else {
      const float *op = static_cast<const float *>(a.o) + base;
      const uint4 r0 = ld16(op), r1 = ld16(op + 4);
      ov[0] = __uint_as_float(r0.x), ov[1] = __uint_as_float(r0.y), ov[2] = __uint_as_float(r0.z);
      ov[3] = __uint_as_float(r0.w), ov[4] = __uint_as_float(r1.x), ov[5] = __uint_as_float(r1.y);
      ov[6] = __uint_as_float(r1.z), ov[7] = __uint_as_float(r1.w);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc = fmaf(bf16_lo(d.w[j]), ov[2 * j], acc);
      acc = fmaf(bf16_hi(d.w[j]), ov[2 * j + 1], acc);
    }
  }
  acc = group_sum<kLanes>(acc);  // every lane of the wave takes part
  if (item < items && sub == 0) {
    const int64_t i = item / a.n_q_heads;
    const int h = static_cast<int>(item % a.n_q_heads);
    a.ws_d[h * a.t + i] = acc;
    a.ws_lse2[h * a.t + i] = a.lse[item] * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// dQ: workgroup = 256 query rows of one query head.
// ---------------------------------------------------------------------------
template <int DH>
__global__ __launch_bounds__(pf::kThreads, 1) void bwd_dq_kernel(const BwdArgs a) {
  constexpr int SWZ = bw::kSwizzle;
  using S = PrefillShape<DH>;
  __shared__ __attribute__((aligned(1024))) char lds_k0[S::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char lds_k1[S::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char lds_v0[S::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char lds_v1[S::kTileBytes];
  auto kbuf = [&](int b) __attribute__((always_inline)) { return b ? lds_k1 : lds_k0; };
  auto vbuf = [&](int b) __attribute__((always_inline)) { return b ? lds_v1 : lds_v0; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int col = lane & 31;

  // Block -> (query tile, query head), longest first; the G heads of a unit
  // sit on one XCD (they read the same K/V tiles).
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
  const int row_stride_kv = a.kv_row_stride;
  const bf16_t *kg = static_cast<const bf16_t *>(a.k) + g * DH;
  const bf16_t *vg = static_cast<const bf16_t *>(a.v) + g * DH;

  const int t = static_cast<int>(a.t);
  const int q_start = static_cast<int>(a.q_start);
  const int kv_len = static_cast<int>(a.kv_len);
  const int blk_row0 = qtile * pf::kBlockRows;
  const int wave_row_first = blk_row0 + wave * pf::kRowsPerWave;
  const int my_row = wave_row_first + col;
  const bool row_valid = my_row < t;
  const int my_pos = q_start + (row_valid ? my_row : (t - 1));
  const bool wave_active = wave_row_first < t;
  const int wave_pos_last = q_start + min(wave_row_first + pf::kRowsPerWave, t) - 1;
  const int blk_last_row = min(blk_row0 + pf::kBlockRows, t) - 1;
  const int n_ktiles = (q_start + blk_last_row) / pf::kKeyTile + 1;
  const int n_half = wave_active ? wave_pos_last / 32 + 1 : 0;

  StageOffsets<DH, SWZ> so;
  so.init(wave, lane, row_stride_kv);
  stage_tile<DH, SWZ>(lds_k0, kg, row_stride_kv, 0, kv_len, wave, so);
  stage_tile<DH, SWZ>(lds_v0, vg, row_stride_kv, 0, kv_len, wave, so);

  // Q^T and dO^T as MFMA B operands: lane holds row `col`, dims ks*16 + half*8.
  Frag8 qf[S::KSTEPS], of[S::KSTEPS];
  float lse2 = 0.f, dterm = 0.f;
  {
    const int64_t off = (int64_t)(row_valid ? my_row : 0) * row_stride_q + (int64_t)h * DH + half * 8;
    const bf16_t *qp = static_cast<const bf16_t *>(a.q) + off;
    const bf16_t *op = static_cast<const bf16_t *>(a.d_o) + off;
#pragma unroll
    for (int ks = 0; ks < S::KSTEPS; ++ks) {
      qf[ks].u = row_valid ? ld16(qp + ks * 16) : make_uint4(0, 0, 0, 0);
      of[ks].u = row_valid ? ld16(op + ks * 16) : make_uint4(0, 0, 0, 0);
    }
    if (row_valid) {
      lse2 = a.ws_lse2[(int64_t)h * t + my_row];
      dterm = a.ws_d[(int64_t)h * t + my_row];
    }
  }

  int koff[S::KSTEPS];
#pragma unroll
  for (int ks = 0; ks < S::KSTEPS; ++ks) koff[ks] = swz<DH, SWZ>(col, ks * 16 + half * 8);
  const int grp = lane >> 4;
  const int src_a = lane & 3;
  const int src_j = (lane >> 2) & 3;
  const int trow = (grp >> 1) * 4 + src_j;
  const int tcol = (grp & 1) * 16 + src_a * 4;
  int toff[2][S::DSUB];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
#pragma unroll
    for (int d = 0; d < S::DSUB; ++d) toff[r][d] = swz<DH, SWZ>(trow + 8 * r, d * 32 + tcol);
  }
  auto read_rows = [&](const char *tile, int ks) __attribute__((always_inline)) {
    Frag8 f;
    f.u = *reinterpret_cast<const uint4 *>(tile + koff[ks]);
    return f;
  };
  // Transposed read: dim tile d, key step kk of a 32-row half.
  auto read_tr = [&](const char *tile, int d, int kk) __attribute__((always_inline)) {
    Frag8 f;
    f.s4[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4_t *)(tile + toff[0][d] + kk * 16 * S::kRowBytes));
    f.s4[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4_t *)(tile + toff[1][d] + kk * 16 * S::kRowBytes));
    return f;
  };

  floatx16 dqacc[S::DSUB];
#pragma unroll
  for (int d = 0; d < S::DSUB; ++d) {
#pragma unroll
    for (int i = 0; i < 16; ++i) dqacc[d][i] = 0.f;
  }
  constexpr int kHalfBytes = 32 * S::kRowBytes;

  // A whole tile without masks, scheduled by hand: the products of both
  // halves in the order S0, dP0, S1, dP1, dQ0, dQ1 (each half's dQ products
  // in the order of the per-half form, so the sums are the same), with the
  // LDS reads three products ahead and one piece of a half's dS work between
  // products: half 0's while S1 and dP1 run, half 1's while dQ0 runs.
  auto pair_step = [&](const char *tk, const char *tv) __attribute__((always_inline)) {
    constexpr int KS = S::KSTEPS;        // S (or dP) products per half
    constexpr int NS = 2 * KS;           // S and dP products per half
    constexpr int NQ = 2 * S::DSUB;      // dQ products per half
    constexpr int NM = 2 * NS + 2 * NQ;  // products of the tile
    constexpr int kAhead = 3;          // 4 spills at two waves per SIMD
    floatx16 sv[2], dpv[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sv[h][i] = 0.f;
        dpv[h][i] = 0.f;
      }
    }
    Frag8 dsf[2][2];
    auto read = [&](int i) __attribute__((always_inline)) {
      if (i < 2 * NS) {
        const int h = i / NS, r = i % NS;
        return read_rows((r < KS ? tk : tv) + h * kHalfBytes, r % KS);
      }
      const int h = (i - 2 * NS) / NQ, r = (i - 2 * NS) % NQ;
      return read_tr(tk + h * kHalfBytes, r >> 1, r & 1);
    };
    auto product = [&](int i, const Frag8 &op) __attribute__((always_inline)) {
      if (i < 2 * NS) {
        const int h = i / NS, r = i % NS;
        if (r < KS) {
          sv[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op.v, qf[r].v, sv[h], 0, 0, 0);
        } else {
          dpv[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op.v, of[r - KS].v, dpv[h], 0, 0, 0);
        }
      } else {
        const int h = (i - 2 * NS) / NQ, r = (i - 2 * NS) % NQ;
        dqacc[r >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op.v, dsf[h][r & 1].v, dqacc[r >> 1], 0, 0, 0);
      }
    };
    // Piece k (0..7) of half h: accumulator elements kk*8 + 2j, +1 with
    // kk = k / 4, j = k % 4 (k-slot j of key step kk).
    auto piece = [&](int h, int k) __attribute__((always_inline)) {
      const int kk = k >> 2, j = k & 3;
      float ds[2];
#pragma unroll
      for (int e2 = 0; e2 < 2; ++e2) {
        const int e = kk * 8 + 2 * j + e2;
        const float p = fast_exp2(fmaf(sv[h][e], a.scale_log2, -lse2));
        ds[e2] = p * (dpv[h][e] - dterm);
      }
      dsf[h][kk].w[j] = cvt_pk_bf16(ds[0], ds[1]);
    };
    Frag8 opnd[NM];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) opnd[i] = read(i);
#pragma clang loop unroll(full)
    for (int i = 0; i < NM; ++i) {
      if (i + kAhead < NM) opnd[i + kAhead] = read(i + kAhead);
      product(i, opnd[i]);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (i == NS + ((k + 1) * NS) / 8 - 1) piece(0, k);  // during S1, dP1
        if (i == 2 * NS + (k * NQ) / 8) piece(1, k);        // during dQ0
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Tile kt sits in buffers kt % 2; the loop runs two tiles per pass so the
  // buffer of each is a compile-time choice: the compiler can then tell
  // that the reads of tile kt do not alias the loads of tile kt+1 still
  // landing in the other buffers, and does not wait for them.
  auto tile = [&](auto b_c, int kt) __attribute__((always_inline)) {
    constexpr int b = decltype(b_c)::value;
    // Tile kt has landed for every wave, and every wave is done with tile
    // kt-1, whose buffers the next loads overwrite.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (kt + 1 < n_ktiles) {
      stage_tile<DH, SWZ>(kbuf(b ^ 1), kg, row_stride_kv, (kt + 1) * pf::kKeyTile, kv_len, wave, so);
      stage_tile<DH, SWZ>(vbuf(b ^ 1), vg, row_stride_kv, (kt + 1) * pf::kKeyTile, kv_len, wave, so);
    }
    // Both halves in range and every row of the wave a row of the block at
    // or past the tile's last key (wave-uniform): the pipelined pair.
    if (2 * kt + 1 < n_half && wave_row_first + 31 < t && q_start + wave_row_first >= kt * pf::kKeyTile + 63) {
      pair_step(kbuf(b), vbuf(b));
      return;
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int u = 2 * kt + hh;
      if (u < n_half) {
        const char *tk = kbuf(b) + hh * kHalfBytes;
        const char *tv = vbuf(b) + hh * kHalfBytes;
        floatx16 s, dp;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          s[i] = 0.f;
          dp[i] = 0.f;
        }
#pragma unroll
        for (int ks = 0; ks < S::KSTEPS; ++ks) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_rows(tk, ks).v, qf[ks].v, s, 0, 0, 0);
#pragma unroll
        for (int ks = 0; ks < S::KSTEPS; ++ks) dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_rows(tv, ks).v, of[ks].v, dp, 0, 0, 0);
        // Element i is key 32u + (i/4)*8 + half*4 + (i%4) of query row `col`.
        // kMask: the half reaches past the first row of the wave (near the
        // diagonal) or the wave has rows past the block; the other halves
        // skip the per-element test.
        Frag8 dsf[2];
        auto soft = [&](auto mask_c) __attribute__((always_inline)) {
          const int rel = min(my_pos - u * 32 - half * 4, 32);
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              float ds[2];
#pragma unroll
              for (int e2 = 0; e2 < 2; ++e2) {
                const int e = kk * 8 + 2 * j + e2;
                float p = fast_exp2(fmaf(s[e], a.scale_log2, -lse2));
                if constexpr (decltype(mask_c)::value) p = (e >> 2) * 8 + (e & 3) <= rel ? p : 0.f;
                ds[e2] = p * (dp[e] - dterm);
              }
              dsf[kk].w[j] = cvt_pk_bf16(ds[0], ds[1]);
            }
          }
        };
        // Every row of the wave is a row of the block at a position at or
        // past the half's last key (wave-uniform).
        if (wave_row_first + 31 < t && q_start + wave_row_first >= u * 32 + 31) {
          soft(std::false_type());
        } else {
          soft(std::true_type());
        }
#pragma unroll
        for (int i = 0; i < 2 * S::DSUB; ++i) {
          const int d = i >> 1, kk = i & 1;
          dqacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_tr(tk, d, kk).v, dsf[kk].v, dqacc[d], 0, 0, 0);
        }
      }
    }
  };
  for (int kt = 0; kt < n_ktiles; kt += 2) {
    tile(std::integral_constant<int, 0>(), kt);
    if (kt + 1 < n_ktiles) tile(std::integral_constant<int, 1>(), kt + 1);
  }
  if (!row_valid) return;
  // dQ^T element i of tile d is dim d*32 + (i/4)*8 + half*4 + (i%4) of row `col`.
  float *dqp = a.d_q + (int64_t)my_row * row_stride_q + (int64_t)h * DH;
#pragma unroll
  for (int d = 0; d < S::DSUB; ++d) {
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int dim = d * 32 + i4 * 8 + half * 4;
      *reinterpret_cast<float4 *>(dqp + dim) =
          make_float4(dqacc[d][i4 * 4 + 0] * a.scale, dqacc[d][i4 * 4 + 1] * a.scale,
                      dqacc[d][i4 * 4 + 2] * a.scale, dqacc[d][i4 * 4 + 3] * a.scale);
    }
  }
}

// ---------------------------------------------------------------------------
// dK, dV: workgroup = 128 cache rows of one KV head, all G query heads.
// ---------------------------------------------------------------------------
// Staging of a 64-row tile of one head by the 4 waves of the workgroup (the
// same swizzled layout as the forward's K/V tiles).
template <int DH>
struct KvStage {
  using S = PrefillShape<DH>;
  static constexpr int kLoadsPerWave = S::kLoadsPerTile / bw::kKvWaves;
  uint32_t boff[kLoadsPerWave];
  __device__ __forceinline__ void init(int wave, int lane, int row_stride) {
#pragma unroll
    for (int i = 0; i < kLoadsPerWave; ++i) {
      const int row = (wave * kLoadsPerWave + i) * S::kRowsPerLoad + lane / S::kChunks;
      const int chunk = (lane % S::kChunks) ^ row_xor<DH, bw::kSwizzle>(row);
      boff[i] = static_cast<uint32_t>(row * row_stride + chunk * 8) * 2u;
    }
  }
  // Rows row0.. of a [rows][row_stride] bf16 array with n_rows rows; rows
  // past the end land as zeros.
  __device__ __forceinline__ void tile(char *lds_dst, const bf16_t *src, int64_t row_stride, int row0, int n_rows,
                                       int wave) const {
    const int64_t valid = static_cast<int64_t>(n_rows - row0) * row_stride * 2;
    const int64_t tile_bytes = static_cast<int64_t>(bw::kQTile) * row_stride * 2;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_t *>(src + (int64_t)row0 * row_stride), 0,
        static_cast<int>(max(int64_t(0), min(valid, tile_bytes))), kBufferFlags);
#pragma unroll
    for (int i = 0; i < kLoadsPerWave; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t *)(lds_dst + (wave * kLoadsPerWave + i) * 1024), 16,
                                               boff[i], 0, 0, 0);
    }
  }
};

template <int DH>
__global__ __launch_bounds__(bw::kKvThreads, 2) void bwd_dkdv_kernel(const BwdArgs a) {
  constexpr int SWZ = bw::kSwizzle;
  using S = PrefillShape<DH>;
  __shared__ __attribute__((aligned(1024))) char lds_q0[S::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char lds_q1[S::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char lds_o0[S::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char lds_o1[S::kTileBytes];
  __shared__ __attribute__((aligned(256))) float lds_l0[bw::kQTile];
  __shared__ __attribute__((aligned(256))) float lds_l1[bw::kQTile];
  __shared__ __attribute__((aligned(256))) float lds_d0[bw::kQTile];
  __shared__ __attribute__((aligned(256))) float lds_d1[bw::kQTile];
  auto qbuf = [&](int b) __attribute__((always_inline)) { return b ? lds_q1 : lds_q0; };
  auto obuf = [&](int b) __attribute__((always_inline)) { return b ? lds_o1 : lds_o0; };
  auto lbuf = [&](int b) __attribute__((always_inline)) { return b ? lds_l1 : lds_l0; };
  auto dbuf = [&](int b) __attribute__((always_inline)) { return b ? lds_d1 : lds_d0; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int col = lane & 31;

  // Block -> (block of cache rows, KV head); the first rows (seen by the
  // most query rows) first.
  const int g = static_cast<int>(blockIdx.x % a.n_kv_heads);
  const int kblock = static_cast<int>(blockIdx.x / a.n_kv_heads);
  const int group = a.n_q_heads / a.n_kv_heads;
  const int t = static_cast<int>(a.t);
  const int q_start = static_cast<int>(a.q_start);
  const int kv_len = static_cast<int>(a.kv_len);
  const int key_blk0 = kblock * bw::kBlockKeys;
  if (key_blk0 >= kv_len) return;
  const int key0 = key_blk0 + wave * bw::kKeysPerWave;  // this wave's first cache row
  const int my_key = key0 + col;
  const bool wave_active = key0 < kv_len;

  const int64_t row_stride_q = (int64_t)a.n_q_heads * DH;
  const int64_t row_stride_kv = a.kv_row_stride;               // cache rows
  const int64_t row_stride_dkv = (int64_t)a.n_kv_heads * DH;   // d_k, d_v rows (dense)

  // Query rows that see this block: positions >= key_blk0.
  const int r_first = max(0, key_blk0 - q_start);
  const int qt0 = r_first / bw::kQTile;
  const int n_qt = (t + bw::kQTile - 1) / bw::kQTile - qt0;
  const int n_it = group * n_qt;

  KvStage<DH> st;
  st.init(wave, lane, static_cast<int>(row_stride_q));
  auto stage = [&](int it, int b) __attribute__((always_inline)) {
    const int h = g * group + it / n_qt;
    const int row0 = (qt0 + it % n_qt) * bw::kQTile;
    st.tile(qbuf(b), static_cast<const bf16_t *>(a.q) + (int64_t)h * DH, row_stride_q, row0, t, wave);
    st.tile(obuf(b), static_cast<const bf16_t *>(a.d_o) + (int64_t)h * DH, row_stride_q, row0, t, wave);
    if (wave == 0) {
      // 64 consecutive rows of lse2 and D of head h, one dword per lane.
      const int bytes = max(0, min(t - row0, bw::kQTile)) * 4;
      const __amdgpu_buffer_rsrc_t rl =
          __builtin_amdgcn_make_buffer_rsrc(a.ws_lse2 + (int64_t)h * t + row0, 0, bytes, kBufferFlags);
      const __amdgpu_buffer_rsrc_t rd =
          __builtin_amdgcn_make_buffer_rsrc(a.ws_d + (int64_t)h * t + row0, 0, bytes, kBufferFlags);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (lds_void_t *)lbuf(b), 4, lane * 4u, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (lds_void_t *)dbuf(b), 4, lane * 4u, 0, 0, 0);
    }
  };
  stage(0, 0);

  // K^T and V^T as MFMA B operands (stationary): lane holds cache row
  // `my_key`, dims ks*16 + half*8.
  Frag8 kf[S::KSTEPS], vf[S::KSTEPS];
  {
    const bool ok = my_key < kv_len;
    const int64_t off = (int64_t)(ok ? my_key : 0) * row_stride_kv + (int64_t)g * DH + half * 8;
    const bf16_t *kp = static_cast<const bf16_t *>(a.k) + off;
    const bf16_t *vp = static_cast<const bf16_t *>(a.v) + off;
#pragma unroll
    for (int ks = 0; ks < S::KSTEPS; ++ks) {
      kf[ks].u = ok ? ld16(kp + ks * 16) : make_uint4(0, 0, 0, 0);
      vf[ks].u = ok ? ld16(vp + ks * 16) : make_uint4(0, 0, 0, 0);
    }
  }

  // Row-read offsets are recomputed at each use (a few integer ops) rather
  // than held in registers.
  const int rx = row_xor<DH, SWZ>(col);
  const int rbase = col * S::kRowBytes;
  const int grp = lane >> 4;
  const int src_a = lane & 3;
  const int src_j = (lane >> 2) & 3;
  const int trow = (grp >> 1) * 4 + src_j;
  const int tcol = (grp & 1) * 16 + src_a * 4;
  int toff[2][S::DSUB];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
#pragma unroll
    for (int d = 0; d < S::DSUB; ++d) toff[r][d] = swz<DH, SWZ>(trow + 8 * r, d * 32 + tcol);
  }
  auto read_rows = [&](const char *tile, int ks) __attribute__((always_inline)) {
    Frag8 f;
    f.u = *reinterpret_cast<const uint4 *>(tile + rbase + (((2 * ks + half) ^ rx) << 4));
    return f;
  };
  auto read_tr = [&](const char *tile, int d, int kk) __attribute__((always_inline)) {
    Frag8 f;
    f.s4[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4_t *)(tile + toff[0][d] + kk * 16 * S::kRowBytes));
    f.s4[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4_t *)(tile + toff[1][d] + kk * 16 * S::kRowBytes));
    return f;
  };

  floatx16 dk[S::DSUB], dv[S::DSUB];
#pragma unroll
  for (int d = 0; d < S::DSUB; ++d) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dk[d][i] = 0.f;
      dv[d][i] = 0.f;
    }
  }
  constexpr int kHalfBytes = 32 * S::kRowBytes;

  for (int it = 0; it < n_it; ++it) {
    const int b = it & 1;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (it + 1 < n_it) stage(it + 1, b ^ 1);
    const int row0 = (qt0 + it % n_qt) * bw::kQTile;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int r0 = row0 + hh * 32;  // first query row of the half
      // Some row of the half sees some cache row of this wave.
      if (wave_active && r0 < t && q_start + r0 + 31 >= key0) {
        const char *tq = qbuf(b) + hh * kHalfBytes;
        const char *to = obuf(b) + hh * kHalfBytes;
        floatx16 s, dp;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          s[i] = 0.f;
          dp[i] = 0.f;
        }
#pragma unroll
        for (int ks = 0; ks < S::KSTEPS; ++ks) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_rows(tq, ks).v, kf[ks].v, s, 0, 0, 0);
#pragma unroll
        for (int ks = 0; ks < S::KSTEPS; ++ks) dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_rows(to, ks).v, vf[ks].v, dp, 0, 0, 0);
        // Element i is query row r0 + (i/4)*8 + half*4 + (i%4) of cache row
        // `my_key`; lse2 and D of those rows come as four float4 groups.
        const float *lq = lbuf(b) + hh * 32 + half * 4;
        const float *dq = dbuf(b) + hh * 32 + half * 4;
        Frag8 pf[2], sf[2];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 l4 = *reinterpret_cast<const float4 *>(lq + q4 * 8);
          const float4 d4 = *reinterpret_cast<const float4 *>(dq + q4 * 8);
          const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
          const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
          float p[4], ds[4];
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4) {
            const int e = q4 * 4 + e4;
            const int row = r0 + q4 * 8 + half * 4 + e4;
            const bool vis = row < t && my_key <= q_start + row;
            p[e4] = vis ? fast_exp2(fmaf(s[e], a.scale_log2, -lv[e4])) : 0.f;
            ds[e4] = p[e4] * (dp[e] - dv4[e4]);
          }
          // Accumulator element e = kk*8 + j is k-slot j of key step kk.
          const int kk = q4 >> 1, j0 = (q4 & 1) * 2;
          pf[kk].w[j0] = cvt_pk_bf16(p[0], p[1]);
          pf[kk].w[j0 + 1] = cvt_pk_bf16(p[2], p[3]);
          sf[kk].w[j0] = cvt_pk_bf16(ds[0], ds[1]);
          sf[kk].w[j0 + 1] = cvt_pk_bf16(ds[2], ds[3]);
        }
#pragma unroll
        for (int i = 0; i < 2 * S::DSUB; ++i) {
          const int d = i >> 1, kk = i & 1;
          dv[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pf[kk].v, read_tr(to, d, kk).v, dv[d], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 2 * S::DSUB; ++i) {
          const int d = i >> 1, kk = i & 1;
          dk[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sf[kk].v, read_tr(tq, d, kk).v, dk[d], 0, 0, 0);
        }
      }
    }
  }
  if (!wave_active) return;
  // Accumulator element i of dim tile d: cache row key0 + (i/4)*8 + half*4 +
  // (i%4), dim d*32 + col.  Added to what the caller's buffers hold.
#pragma unroll
  for (int d = 0; d < S::DSUB; ++d) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = key0 + (i >> 2) * 8 + half * 4 + (i & 3);
      if (key < kv_len) {
        const int64_t e = (int64_t)key * row_stride_dkv + (int64_t)g * DH + d * 32 + col;
        a.d_k[e] += dk[d][i] * a.scale;
        a.d_v[e] += dv[d][i];
      }
    }
  }
}

hipError_t launch_prefill_bwd(const BwdArgs &a, int head_dim, hipStream_t s) {
  if (head_dim != 128 && head_dim != 64) return hipErrorInvalidValue;
  const int64_t items = a.t * a.n_q_heads;
  const int lanes = head_dim / 8;
  const unsigned int rs_blocks = static_cast<unsigned int>((items * lanes + 255) / 256);
  const int64_t n_qtiles = (a.t + pf::kBlockRows - 1) / pf::kBlockRows;
  const int64_t n_units = n_qtiles * a.n_kv_heads;
  const int64_t group = a.n_q_heads / a.n_kv_heads;
  const unsigned int dq_blocks = static_cast<unsigned int>(((n_units + pf::kXcds - 1) / pf::kXcds) * pf::kXcds * group);
  const unsigned int kv_blocks =
      static_cast<unsigned int>(((a.kv_len + bw::kBlockKeys - 1) / bw::kBlockKeys) * a.n_kv_heads);
  if (head_dim == 128) {
    hipLaunchKernelGGL(bwd_rowstats_kernel<128>, dim3(rs_blocks), dim3(256), 0, s, a);
    hipLaunchKernelGGL(bwd_dq_kernel<128>, dim3(dq_blocks), dim3(pf::kThreads), 0, s, a);
    hipLaunchKernelGGL(bwd_dkdv_kernel<128>, dim3(kv_blocks), dim3(bw::kKvThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL(bwd_rowstats_kernel<64>, dim3(rs_blocks), dim3(256), 0, s, a);
    hipLaunchKernelGGL(bwd_dq_kernel<64>, dim3(dq_blocks), dim3(pf::kThreads), 0, s, a);
    hipLaunchKernelGGL(bwd_dkdv_kernel<64>, dim3(kv_blocks), dim3(bw::kKvThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace yoco
