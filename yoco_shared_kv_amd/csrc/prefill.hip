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
//   A workgroup is 8 waves = 256 query rows of one query head (one workgroup
//   per CU); each wave owns 32 rows.  Keys are staged in tiles of 64 rows and
//   computed in halves of 32.
//   * Staging: each K or V tile (64 rows x head_dim bf16) is copied straight
//     from global memory into LDS with 16-byte buffer loads to LDS (no
//     registers), two buffers each for K and V in separate arrays (so reads
//     of one buffer never wait for loads into the other).  The buffer
//     descriptor ends at the last cache row that holds data; the hardware
//     range check writes zeros for rows past it.  Rows are stored unpadded
//     with the 16-byte chunk index XOR-swizzled by the row, so the operand
//     reads below hit distinct LDS banks.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16 (A = K rows read from LDS, B = Q^T kept in
//     registers).  In the 32x32 accumulator layout each lane holds ONE query
//     row (its column) and 16 of the 32 keys of a half; the other 16 sit in
//     lane l ^ 32.  Row maxima need one cross-lane exchange per half and the
//     running sum stays lane-local.
//   * The output is accumulated transposed too, O^T += V^T P^T.  P^T comes
//     straight from the score accumulators (rounded to bf16) as the B
//     operand; the MFMA's k order is free as long as A and B agree, so the
//     keys each lane already holds define it.  The A operand V^T is read from
//     the row-major V tile with ds_read_b64_tr_b16, which hands each lane 4
//     consecutive keys of one head-dim column (two reads per MFMA).
//   * Software pipeline: the step for half u issues the PV MFMAs of half u-1
//     and the S MFMAs of half u+1 while the VALU forms P of half u, with the
//     VALU work split into small pieces placed between the MFMAs, so the
//     exps run under the matrix work of the same wave.
//   * Softmax without rescaling: each row's reference maximum comes from its
//     first 32 keys and never moves, so O is never rescaled inside the loop
//     (a rescale there would force the accumulators through a branch).
//     Probabilities above 1 are fine up to 2^64; a row whose later maximum
//     passes the reference by more than that makes the workgroup run a
//     second pass, in which that row uses its true maximum.
//   * Causality: a workgroup visits key tiles 0..(last position it needs)/64;
//     each wave stops after the last half its rows can see and masks keys > p
//     in halves on its diagonal.  Workgroups run longest first, and the G
//     query heads of a KV group for the same query tile are placed on the
//     same XCD so their K/V tiles are shared in that XCD's L2.
// fp32 path: plain fp32 VALU kernel (one lane per query row, exact online
// softmax) for fp32 caches.
#include "attn_tiles.h"

namespace yoco {

// RB: 32-row blocks of query rows per wave (1: 8 waves, two per SIMD; 2: 4
// waves of 64 rows, one per SIMD, every K and V operand read from LDS feeding
// two MFMAs).  Each row block keeps its own Q^T, S^T, P^T, O^T and softmax
// state and runs exactly the arithmetic of RB = 1, so results do not depend
// on RB.
template <int DH, int SWZ, int RB>
__global__ __launch_bounds__(pf::kThreads / RB, 1) void prefill_bf16_kernel(const PrefillArgs a) {
  using S = PrefillShape<DH>;
  constexpr int NW = pf::kWaves / RB;          // waves per workgroup
  constexpr int kWaveRows = pf::kRowsPerWave * RB;
  // K and V tiles, two buffers each, as four separate arrays: the compiler
  // can then tell that reads of one buffer do not alias the direct-to-LDS
  // loads into another, and need not wait for those loads to land.  Every
  // LDS read below is a per-lane offset plus a compile-time immediate.
  __shared__ __attribute__((aligned(1024))) char lds_k0[S::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char lds_k1[S::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char lds_v0[S::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char lds_v1[S::kTileBytes];
  auto kbuf = [&](int b) __attribute__((always_inline)) { return b ? lds_k1 : lds_k0; };
  auto vbuf = [&](int b) __attribute__((always_inline)) { return b ? lds_v1 : lds_v0; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int half = lane >> 5;       // 0 or 1
  const int col = lane & 31;        // the query row this lane owns in each row block

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
  const int row_stride_kv = a.kv_row_stride;
  const bf16_t *qg = static_cast<const bf16_t *>(a.q);
  const bf16_t *kg = static_cast<const bf16_t *>(a.k) + g * DH;
  const bf16_t *vg = static_cast<const bf16_t *>(a.v) + g * DH;

  // Positions fit in int32: the host caps the slab capacity below 2^31.
  const int t = static_cast<int>(a.t);
  const int q_start = static_cast<int>(a.q_start);
  const int kv_len = static_cast<int>(a.kv_len);
  const int blk_row0 = qtile * pf::kBlockRows;
  const int wave_row_first = blk_row0 + wave * kWaveRows;
  int my_row[RB], my_pos[RB];
  bool row_valid[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    my_row[rb] = wave_row_first + rb * 32 + col;
    row_valid[rb] = my_row[rb] < t;
    my_pos[rb] = q_start + (row_valid[rb] ? my_row[rb] : (t - 1));
  }
  const bool wave_active = wave_row_first < t;
  const int wave_last_row = min(wave_row_first + kWaveRows, t) - 1;
  const int wave_pos_last = q_start + wave_last_row;
  const int wave_pos_first = q_start + wave_row_first;
  const int blk_last_row = min(blk_row0 + pf::kBlockRows, t) - 1;
  const int n_ktiles = (q_start + blk_last_row) / pf::kKeyTile + 1;
  // 32-key halves this wave needs: 0 .. n_half-1 (keys up to its last row).
  const int n_half = wave_active ? wave_pos_last / 32 + 1 : 0;

  StageOffsets<DH, SWZ, NW> so;
  so.init(wave, lane, row_stride_kv);
  // Start loading key tile 0 before touching Q.
  stage_tile<DH, SWZ, NW>(lds_k0, kg, row_stride_kv, 0, kv_len, wave, so);

  // Q^T as the MFMA B operand: lane holds row `col` of each row block, dims
  // ks*16 + half*8 .. +8.
  Frag8 qf[RB][S::KSTEPS];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const bf16_t *qp = qg + (int64_t)(row_valid[rb] ? my_row[rb] : 0) * row_stride_q + (int64_t)h * DH + half * 8;
#pragma unroll
    for (int ks = 0; ks < S::KSTEPS; ++ks) qf[rb][ks].u = row_valid[rb] ? ld16(qp + ks * 16) : make_uint4(0, 0, 0, 0);
  }

  // LDS read offsets within a tile.  K (A operand of S^T): row col of the
  // 32-key half, dims ks*16 + half*8; the row_xor of the swizzle depends only
  // on row mod 16, so the half adds the immediate 32*rowbytes.
  int koff[S::KSTEPS];
#pragma unroll
  for (int ks = 0; ks < S::KSTEPS; ++ks) koff[ks] = swz<DH, SWZ>(col, ks * 16 + half * 8);
  // V^T (A operand of O^T) via transposed reads: in each 16-lane group,
  // source lane a + 4j points at key kb + j, dims dbase + 4a .. +3, and lane
  // i of the group receives keys kb..kb+3 of dim dbase + i.  With
  // kb = half32*32 + kk*16 + (grp/2)*4 + j and the second read at kb + 8,
  // only (read r, dim tile d) changes the swizzled offset; the 32-key half
  // and kk are immediates.
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

  floatx16 oacc[RB][S::DSUB];
  float l_run[RB];  // this lane's share of sum(p) per row block, from the bf16 p the MFMA uses
  // Reference maximum (log2 units) of each of this lane's query rows.  It is
  // fixed from the row's first 32 keys, so O never needs rescaling: later
  // probabilities may exceed 1.  A row whose probabilities sum to 2^60 or
  // more (or to inf/NaN) may have lost range, which makes the workgroup run
  // a pass that finds each row's largest maximum and then a final pass in
  // which that row's reference is its largest maximum (every probability of
  // the row is then <= 1); the other rows repeat their arithmetic.
  float m_ref[RB], m_seen[RB];
  bool row_ovf[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_ref[rb] = -INFINITY;
    m_seen[rb] = -INFINITY;  // largest half maximum of the row (generic steps)
    row_ovf[rb] = false;     // the row's sum reached the limit in the first pass
  }
  const uint32_t kOnesBf16x2 = 0x3F803F80u;  // (1.0, 1.0) in bf16
  __shared__ int redo_flag;
  if (tid == 0) redo_flag = 0;  // ordered before any update by the first barrier below

  // Software pipeline over 32-key halves u of the key range.  Step u issues
  //   PV(u-1): O^T += V^T P^T for half u-1      (MFMA)
  //   S(u+1):  S^T = K Q^T for half u+1          (MFMA)
  //   softmax of half u: P(u) from S(u)          (VALU)
  // for every row block, so the exps of one half run while the matrix cores
  // work on its neighbours.  Halves 2p-1 and 2p form period p, which reads K
  // tile p and V tile p-1 from LDS while K tile p+1 and V tile p are being
  // loaded.
  floatx16 sa[RB], sb[RB];       // S of the half being normalised / being computed
  Frag8 pa[RB][2], pb[RB][2];    // P of the half being multiplied / being formed

  // Operands of the step's MFMAs.  PV MFMA i (i < 2*DSUB) is dim tile i/2,
  // key step i%2 of the V half; S MFMA ks reads K rows of the K half.
  auto read_v = [&](const char *tv, int i) __attribute__((always_inline)) {
    const int d = i >> 1, kk = i & 1;
    Frag8 f;
    f.s4[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4_t *)(tv + voff[0][d] + kk * 16 * S::kRowBytes));
    f.s4[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4_t *)(tv + voff[1][d] + kk * 16 * S::kRowBytes));
    return f;
  };
  auto read_k = [&](const char *tk, int ks) __attribute__((always_inline)) {
    Frag8 f;
    f.u = *reinterpret_cast<const uint4 *>(tk + koff[ks]);
    return f;
  };
  // P for accumulator pair j of key step kk: k-slot j of lane half `half`
  // in step kk is key kk*16 + (j/4)*8 + half*4 + (j%4), which is S^T
  // accumulator element kk*8 + j.
  auto make_p_pair = [&](const floatx16 &sv, Frag8 (&p)[2], float mref, int kk, int j) __attribute__((always_inline)) {
    const float p0 = fast_exp2(fmaf(sv[kk * 8 + 2 * j], a.scale_log2, -mref));
    const float p1 = fast_exp2(fmaf(sv[kk * 8 + 2 * j + 1], a.scale_log2, -mref));
    p[kk].w[j] = cvt_pk_bf16(p0, p1);
  };

  // One step of the pipeline, scheduled by hand: chunk i issues MFMA i of
  // every row block (the PV MFMAs, then the S MFMAs), the LDS reads of the
  // operand of MFMA i+4 and one piece of each row block's softmax of half u,
  // with a scheduling fence between chunks, so the VALU work runs under the
  // matrix work and few operands are in flight.
  // The generic form (first, causal-diagonal and last halves) adds only
  // selects, never branches, so O and S stay in fixed registers:
  //  * the causal mask;
  //  * PV MFMAs without a previous half get a zero V operand (a select:
  //    LDS that was never written may hold NaN);
  //  * an S MFMA without a next half produces a value nobody reads;
  //  * P of a half outside the wave's range is zero, and l, the reference
  //    and the maxima are updated only for halves in range.
  // Fast steps of one period are linked: the first reads the V operands of
  // the second's first kAhead MFMAs in its last chunks (into `carry`), so
  // the second starts without waiting for LDS.  link_c: 0 none, 1 fill
  // carry from tv + one half, 2 start from carry.
  constexpr int kAhead = 4;  // LDS reads run this many operands ahead
  // The linked steps carry the next step's first kAhead operands, which must
  // all be V operands.
  static_assert(kAhead <= 2 * S::DSUB, "read-ahead deeper than one step's V operands");
  constexpr int kHalfBytes = 32 * S::kRowBytes;
  Frag8 carry[kAhead];
  auto step = [&](auto generic_c, auto link_c, int u, const char *tk, const char *tv, floatx16 (&s_cur)[RB],
                  floatx16 (&s_next)[RB], Frag8 (&p_prev)[RB][2], Frag8 (&p_cur)[RB][2]) __attribute__((always_inline)) {
    constexpr bool kGeneric = decltype(generic_c)::value;
    constexpr int kLink = decltype(link_c)::value;
    constexpr int NPV = 2 * S::DSUB;
    constexpr int NM = NPV + S::KSTEPS;
    // Softmax pieces of each row block: (generic only) the row maximum (4
    // pieces of 4 elements) and its cross-lane exchange, then the
    // probabilities (8 pieces of one packed pair) and the running sum of
    // P(u-1) (2 pieces).  The fast form needs no maximum: the reference is
    // fixed, and range is checked once, from the row sum, at the end of the
    // pass.
    constexpr int kMax0 = 0, kXchg = kGeneric ? 4 : -1;
    constexpr int kP0 = kGeneric ? 5 : 0, kL0 = kP0 + 8, kPieces = kL0 + 2;
    const bool do_pv = !kGeneric || (u >= 1 && u - 1 < n_half);
    const bool do_soft = !kGeneric || (u >= 0 && u < n_half);
    if constexpr (kGeneric) {
      // Causal mask: accumulator element i is key 32u + (i/4)*8 + half*4 +
      // (i%4) of query row `col` of the block (a no-op below its diagonal).
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int rel = min(my_pos[rb] - u * 32 - half * 4, 32);
#pragma unroll
        for (int i = 0; i < 16; ++i) s_cur[rb][i] = (i >> 2) * 8 + (i & 3) > rel ? -INFINITY : s_cur[rb][i];
      }
    }
    Frag8 opnd[NM];
    auto issue_read = [&](int i) __attribute__((always_inline)) {
      if (i < NPV) {
        opnd[i] = read_v(tv, i);
        if (kGeneric && !do_pv) opnd[i].u = make_uint4(0, 0, 0, 0);
      } else {
        opnd[i] = read_k(tk, i - NPV);
      }
    };
    float tmax[RB], tmax_other[RB], l_add[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      tmax[rb] = s_cur[rb][0];
      tmax_other[rb] = 0.f;
      l_add[rb] = 0.f;
    }
    auto piece = [&](int rb, int i) __attribute__((always_inline)) {
      if (kGeneric && i >= kMax0 && i < kMax0 + 4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) tmax[rb] = fmaxf(tmax[rb], s_cur[rb][(i - kMax0) * 4 + e]);
      } else if (kGeneric && i == kXchg) {
        tmax_other[rb] = shfl_xor_f(tmax[rb], 32);
        // The row's first half (key 0 is always visible) sets the reference.
        const float tt = fmaxf(tmax[rb], tmax_other[rb]) * a.scale_log2;
        m_ref[rb] = (do_soft && m_ref[rb] == -INFINITY) ? tt : m_ref[rb];
      } else if (i >= kP0 && i < kP0 + 8) {
        make_p_pair(s_cur[rb], p_cur[rb], m_ref[rb], (i - kP0) >> 2, (i - kP0) & 3);
      } else if (i >= kL0 && i < kL0 + 2) {
#pragma unroll
        for (int j = 0; j < 4; ++j) l_add[rb] = dot2_bf16_f32(p_prev[rb][i - kL0].w[j], kOnesBf16x2, l_add[rb]);
      }
    };
#pragma unroll
    for (int i = 0; i < kAhead; ++i) {
      if constexpr (kLink == 2) {
        opnd[i] = carry[i];
      } else {
        issue_read(i);
      }
    }
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      if (i + kAhead < NM) {
        issue_read(i + kAhead);
      } else if constexpr (kLink == 1) {
        carry[i + kAhead - NM] = read_v(tv + kHalfBytes, i + kAhead - NM);
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if (i < NPV) {
          oacc[rb][i >> 1] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(opnd[i].v, p_prev[rb][i & 1].v, oacc[rb][i >> 1], 0, 0, 0);
        } else {
          if (i == NPV) {
#pragma unroll
            for (int e = 0; e < 16; ++e) s_next[rb][e] = 0.f;
          }
          s_next[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opnd[i].v, qf[rb][i - NPV].v, s_next[rb], 0, 0, 0);
        }
        piece(rb, i);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = NM; i < kPieces; ++i) {  // head_dim 64: fewer MFMAs than pieces
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) piece(rb, i);
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if constexpr (kGeneric) {
        const float tt = fmaxf(tmax[rb], tmax_other[rb]) * a.scale_log2;
        l_run[rb] += do_pv ? l_add[rb] : 0.f;
        m_seen[rb] = do_soft ? fmaxf(m_seen[rb], tt) : m_seen[rb];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          if (!do_soft) p_cur[rb][kk].u = make_uint4(0, 0, 0, 0);
        }
      } else {
        l_run[rb] += l_add[rb];
      }
    }
  };

  // One period: barrier, start the next loads, then halves 2p-1 and 2p.
  // Step 2p-1 reads K half 2p (tile p, rows 0..31) and V half 2p-2 (tile
  // p-1, rows 0..31); step 2p the second halves.
  // `inner_c` (fast periods: p + 1 < n_ktiles) stages without a branch, so
  // the steps of consecutive periods share one basic block and the compiler
  // cannot move a step's softmax past the barrier, away from the MFMAs it
  // is scheduled against.
  auto period_start = [&](auto inner_c, int kb, int p) __attribute__((always_inline)) {
    // Every wave's loads of K tile p and V tile p-1 have landed, and every
    // wave is done with K tile p-1 and V tile p-2, whose buffers the next
    // loads overwrite.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (decltype(inner_c)::value || p + 1 < n_ktiles)
      stage_tile<DH, SWZ, NW>(kbuf(kb ^ 1), kg, row_stride_kv, (p + 1) * pf::kKeyTile, kv_len, wave, so);
    if (decltype(inner_c)::value || p < n_ktiles)
      stage_tile<DH, SWZ, NW>(vbuf(kb), vg, row_stride_kv, p * pf::kKeyTile, kv_len, wave, so);
  };
  auto period_fast = [&](auto buf_c, int p) __attribute__((always_inline)) {
    constexpr int KB = decltype(buf_c)::value;  // K tile p sits in buffer p % 2
    period_start(std::true_type(), KB, p);
    const char *tk = kbuf(KB);
    const char *tv = vbuf(KB ^ 1);
    step(std::false_type(), std::integral_constant<int, 1>(), 2 * p - 1, tk, tv, sa, sb, pa, pb);
    step(std::false_type(), std::integral_constant<int, 2>(), 2 * p, tk + kHalfBytes, tv + kHalfBytes, sb, sa, pb, pa);
  };
  auto period_generic = [&](int p) __attribute__((always_inline)) {
    const int kb = p & 1;
    period_start(std::false_type(), kb, p);
    const char *tk = kbuf(kb);
    const char *tv = vbuf(kb ^ 1);
    step(std::true_type(), std::integral_constant<int, 0>(), 2 * p - 1, tk, tv, sa, sb, pa, pb);
    step(std::true_type(), std::integral_constant<int, 0>(), 2 * p, tk + kHalfBytes, tv + kHalfBytes, sb, sa, pb, pa);
  };
  // Periods 1 .. p_fast_end-1 take the fast form: both steps have a previous
  // half, a next half and a half in range, neither half reaches past the
  // wave's first row (2p+1 < n_half and 64p+31 <= wave_pos_first), and the
  // workgroup stages K tile p+1 (p+1 < n_ktiles).  They run in pairs (K
  // buffers 1, 0), the rest in the generic form.
  int p_fast_end = 1;
  if (wave_active) {
    const int by_len = n_half / 2;                           // largest p with 2p+1 < n_half, plus one
    const int by_diag = wave_pos_first >= 31 ? (wave_pos_first - 31) / 64 + 1 : 0;
    p_fast_end = max(1, min(min(by_len, by_diag), n_ktiles - 1));
  }
  const int p_pair_end = 1 + ((p_fast_end - 1) & ~1);

  for (int pass = 0;; ++pass) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int d = 0; d < S::DSUB; ++d) {
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[rb][d][i] = 0.f;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sa[rb][i] = 0.f;
        sb[rb][i] = 0.f;
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        pa[rb][kk].u = make_uint4(0, 0, 0, 0);
        pb[rb][kk].u = make_uint4(0, 0, 0, 0);
      }
      l_run[rb] = 0.f;
    }
    if (pass > 0) stage_tile<DH, SWZ, NW>(lds_k0, kg, row_stride_kv, 0, kv_len, wave, so);
    period_generic(0);
    int p = 1;
    // The maximum-finding pass runs every period in the generic form.
    const int p_fast = pass == 1 ? 1 : p_pair_end;
    for (; p < p_fast; p += 2) {
      period_fast(std::integral_constant<int, 1>(), p);
      period_fast(std::integral_constant<int, 0>(), p + 1);
    }
    for (; p <= n_ktiles; ++p) period_generic(p);
    if (pass == 2) break;
    if (pass == 0) {
      // Range check: every probability of a row is below its sum.
      bool any_ovf = false;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float l_sum = l_run[rb] + shfl_xor_f(l_run[rb], 32);
        row_ovf[rb] = !(l_sum < pf::kSumLimit);
        any_ovf |= row_ovf[rb];
      }
      if (__any(any_ovf) && lane == 0) redo_flag = 1;
      __syncthreads();
      if (redo_flag == 0) break;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) m_seen[rb] = -INFINITY;
    } else {
      // Each row that overflowed takes its largest maximum as the reference
      // for the final pass; the other rows keep theirs and repeat the same
      // arithmetic, so a row's result never depends on the other rows of its
      // workgroup.
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) m_ref[rb] = row_ovf[rb] ? m_seen[rb] : m_ref[rb];
      __syncthreads();
    }
    // The barrier above also retires every read of the LDS tiles the next
    // pass overwrites.
  }

#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float l_tot = l_run[rb] + shfl_xor_f(l_run[rb], 32);
    if (!row_valid[rb]) continue;
    const float inv = 1.0f / l_tot;
    // O^T accumulator element i of tile d is dim d*32 + (i/4)*8 + half*4 + (i%4)
    // of query row `col` of the block.
    if (a.o_bf16) {
      bf16_t *op = static_cast<bf16_t *>(a.o) + (int64_t)my_row[rb] * row_stride_q + (int64_t)h * DH;
#pragma unroll
      for (int d = 0; d < S::DSUB; ++d) {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int dim = d * 32 + i4 * 8 + half * 4;
          uint2 packed;
          packed.x = cvt_pk_bf16(oacc[rb][d][i4 * 4 + 0] * inv, oacc[rb][d][i4 * 4 + 1] * inv);
          packed.y = cvt_pk_bf16(oacc[rb][d][i4 * 4 + 2] * inv, oacc[rb][d][i4 * 4 + 3] * inv);
          *reinterpret_cast<uint2 *>(op + dim) = packed;
        }
      }
    } else {
      float *op = static_cast<float *>(a.o) + (int64_t)my_row[rb] * row_stride_q + (int64_t)h * DH;
#pragma unroll
      for (int d = 0; d < S::DSUB; ++d) {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int dim = d * 32 + i4 * 8 + half * 4;
          float4 v = make_float4(oacc[rb][d][i4 * 4 + 0] * inv, oacc[rb][d][i4 * 4 + 1] * inv,
                                 oacc[rb][d][i4 * 4 + 2] * inv, oacc[rb][d][i4 * 4 + 3] * inv);
          *reinterpret_cast<float4 *>(op + dim) = v;
        }
      }
    }
    if (a.lse != nullptr && half == 0) {
      a.lse[(int64_t)my_row[rb] * a.n_q_heads + h] = (m_ref[rb] + log2f(l_tot)) * kLn2;
    }
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
  const int64_t rs_kv = a.kv_row_stride;
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

// 32-row blocks per wave.  2 (4 waves of 64 rows, one per SIMD) gives the same
// bits and halves the LDS reads per product, but ran slower.
constexpr int kPrefillRowBlocks = 1;
constexpr int kPrefillSwizzle = 2;  // modes 1 and 2 both remove the 2-way V-read bank conflicts; 2 measured fastest

hipError_t launch_prefill(const PrefillArgs &a, int dtype, int head_dim, hipStream_t s) {
  if (dtype == YOCO_DT_BF16) {
    const int64_t n_qtiles = (a.t + pf::kBlockRows - 1) / pf::kBlockRows;
    const int64_t n_units = n_qtiles * a.n_kv_heads;
    const int64_t group = a.n_q_heads / a.n_kv_heads;
    const unsigned int blocks =
        static_cast<unsigned int>(((n_units + pf::kXcds - 1) / pf::kXcds) * pf::kXcds * group);
    if (head_dim == 128) {
      hipLaunchKernelGGL((prefill_bf16_kernel<128, kPrefillSwizzle, kPrefillRowBlocks>), dim3(blocks),
                         dim3(pf::kThreads / kPrefillRowBlocks), 0, s, a);
    } else if (head_dim == 64) {
      hipLaunchKernelGGL((prefill_bf16_kernel<64, kPrefillSwizzle, kPrefillRowBlocks>), dim3(blocks),
                         dim3(pf::kThreads / kPrefillRowBlocks), 0, s, a);
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
