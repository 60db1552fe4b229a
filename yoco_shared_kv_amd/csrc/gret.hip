// Gated retention (gRet), the self-decoder's token mixer: recurrent steps
// for generation and a chunkwise form on the matrix cores for prefill.
//
// What it computes ([Notes] "YOCO：You Only Cache Once 中文精读笔记" s.2.2
// Eq. 4-5 and s.2.3; [Deep] "You Only Cache Once: Decoder-Decoder
// Architectures for Language Models" s.3.1): per head, with q_t, k_t, v_t of
// length D and the head-wise gate gamma_t = sigmoid(g_t)^(1/tau),
//   S_t = gamma_t S_{t-1} + k_t^T v_t,   o_t = q_t S_t           (Eq. 5)
// which equals the parallel form O = (Q K^T (.) D) V with
// D[t][m] = prod_{i=m+1..t} gamma_i (Eq. 4).  Decays are handled as
// cumulative sums of log gamma = logsigmoid(g) / tau, so every factor is
// exp of a difference <= 0 (no division by a vanishing product).
//
// Recurrent path (gret_recurrent_kernel): the state's columns evolve
// independently, so one workgroup per (sequence, head, 16 state columns)
// keeps its D x 16 slice of the fp32 state in registers and walks the tokens
// in order: state update, then o = q S for its columns with a reduction over
// rows (shuffles, then LDS).  Generation runs one token per sequence; fp32
// prefill runs all tokens of one sequence.
//
// Chunkwise path (bf16, D = 128), chunks of C = 128 positions
// ([Notes] s.2.3: parallel inside a chunk, a state passed between chunks):
//   with l_j the inclusive cumulative log gamma inside the chunk,
//   U_c     = sum_k exp(l_C - l_k) k_k^T v_k                  (chunk's own state)
//   R_{c+1} = exp(l_C) R_c + U_c,  R_0 = the start state       (state entering chunk c+1)
//   O_j     = sum_{k<=j} exp(l_j - l_k) (q_j . k_k) v_k + exp(l_j) q_j R_c
// The pass over chunks is split in two levels, so no per-chunk state ever
// goes to memory: chunks form groups of kGroup; inside group g the same
// recurrence started from zero gives the group's total T_g and its decay
// Lambda_g, and S_{g+1} = exp(Lambda_g) S_g + T_g (S_0 the start state)
// gives the state entering each group.
//   * gret_group_state_kernel: one workgroup per (group, head) forms the
//     group's total in one pass, T_g = K'^T V over the group's positions
//     with K' = exp(L_G - L_k) k_k rounded to bf16 (the same value as the
//     chunk recurrence from zero; weights applied to the transposed K
//     fragments), both operands from row-major LDS tiles, in fp32; it also
//     stores the chunk-local cumulative gates l for the output kernel.
//   * gret_group_scan_kernel: the short pass over groups, elementwise over
//     the state (S_g in fp32, the last state to state_out).
//   * gret_group_out_kernel: one workgroup per (group, head) walks the
//     group's chunks again, with A started at S_g, so before chunk c it
//     holds R_c.  Per chunk, 4 waves x 32 query rows: R_c is rounded to bf16
//     into LDS; the carried term O^T = R^T Q^T comes first, while the
//     chunk's K loads (then each lane scales its query row by exp(l_j)),
//     then per 32-key half S^T = K Q^T,
//     P = S exp(l_j - l_k) masked to k <= j and rounded to bf16 (formed
//     while V loads into the buffer R_c held), then O^T += V^T P^T -- the
//     layout of the causal prefill kernel (one query row per lane, Q^T in
//     registers) -- and last the state update of the chunk, as in the state
//     kernel.  Each chunk's k and v are read twice in all (once per
//     kernel); no state goes to memory per chunk.
// The stored states are transposed ([value dim][key dim]): the accumulator
// layout writes and reads four consecutive key dims per lane.
#include "attn_tiles.h"

namespace yoco {
namespace gr {
constexpr int kChunk = 128;        // positions per chunk
constexpr int kD = 128;            // head dim of the chunkwise path
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kSwz = 2;
constexpr int kRowBytes = kD * 2;                    // 256
constexpr int kTileBytes = kChunk * kRowBytes;       // 32 KiB: [128][128] bf16
constexpr int kLoadsPerWave = kTileBytes / 1024 / kWaves;  // 8 one-KiB loads
constexpr int kGroup = 8;          // chunks per group
constexpr int kScanAhead = 8;      // group states in flight per thread in the scan
// s_waitcnt immediate (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// in 6:4, lgkmcnt in 11:8) that waits for vector memory only, down to 4
// outstanding operations.
constexpr int kVmcnt4 = 4 | (7 << 4) | (15 << 8);
constexpr int kLgkm0 = 0xF | (7 << 4) | (3 << 14);  // LDS/scalar counter only, down to 0
}  // namespace gr

// log gamma = logsigmoid(g) / tau = (min(g, 0) - log1p(exp(-|g|))) / tau.
__device__ __forceinline__ float gret_log_gate(float g, float inv_tau) {
  return (fminf(g, 0.f) - log1pf(expf(-fabsf(g)))) * inv_tau;
}

// ---------------------------------------------------------------------------
// Recurrent steps.  Column e of the state evolves on its own (S_t[:, e] =
// gamma_t S_{t-1}[:, e] + k_t v_t[e]) and o_t[e] = q_t S_t[:, e] reads only
// that column, so a workgroup owns kGretCols columns of one (sequence, head)
// state for all D rows: thread t holds four consecutive columns
// 4 * (t % 4) .. +3 of rows t / 4 + 64 i.  The row sum of o goes through
// shuffles inside each wave (lane bits 2..5) and then LDS across the four
// waves, in a fixed order.
// ---------------------------------------------------------------------------
constexpr int kGretCols = 16;
template <typename T, int D>
__global__ __launch_bounds__(256) void gret_recurrent_kernel(const GretArgs a) {
  constexpr int kColThreads = kGretCols / 4;        // 4 threads per row
  constexpr int kGroups = 256 / kColThreads;        // 64 row groups
  constexpr int kRows = D / kGroups;                // rows per thread
  constexpr int kBlocks = D / kGretCols;            // column blocks per head
  static_assert(kRows >= 1 && D % kGroups == 0, "state rows");
  __shared__ float s_q[D], s_k[D], s_v[kGretCols];
  __shared__ float s_o[4][kGretCols];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c_local = (tid % kColThreads) * 4;
  const int grp = tid / kColThreads;
  const int cblk = blockIdx.x % kBlocks;
  const int bh = blockIdx.x / kBlocks;
  const int b = bh / a.heads;
  const int h = bh % a.heads;
  const int c0 = cblk * kGretCols + c_local;  // this thread's first state column
  const int64_t sbase = (static_cast<int64_t>(b) * a.heads + h) * D * D;
  float S[kRows][4];
#pragma unroll
  for (int i = 0; i < kRows; ++i) {
    const int row = grp + kGroups * i;
    if (a.state_in != nullptr) {
      const float4 t = *reinterpret_cast<const float4 *>(a.state_in + sbase + row * D + c0);
      S[i][0] = t.x, S[i][1] = t.y, S[i][2] = t.z, S[i][3] = t.w;
    } else {
      S[i][0] = S[i][1] = S[i][2] = S[i][3] = 0.f;
    }
  }
  // Token t's q, k, v and gate are loaded one token ahead (token 0 together
  // with the state), so a step waits for at most one memory round trip.
  float nq = 0.f, nk = 0.f, nv = 0.f, ng = 0.f;
  auto fetch = [&](int64_t t) __attribute__((always_inline)) {
    const int64_t tok = (static_cast<int64_t>(b) * a.n_tokens + t) * a.heads + h;
    if (tid < D) {
      nq = load_elem(static_cast<const T *>(a.q) + tok * D + tid);
      nk = load_elem(static_cast<const T *>(a.k) + tok * D + tid);
    }
    if (tid < kGretCols) nv = load_elem(static_cast<const T *>(a.v) + tok * D + cblk * kGretCols + tid);
    ng = a.gate[tok];
  };
  if (a.n_tokens > 0) fetch(0);
  for (int64_t t = 0; t < a.n_tokens; ++t) {
    const int64_t tok = (static_cast<int64_t>(b) * a.n_tokens + t) * a.heads + h;
    __syncthreads();  // the previous token's reads of s_q/s_k/s_v/s_o are done
    if (tid < D) {
      s_q[tid] = nq;
      s_k[tid] = nk;
    }
    if (tid < kGretCols) s_v[tid] = nv;
    const float gamma = expf(gret_log_gate(ng, a.inv_tau));
    if (t + 1 < a.n_tokens) fetch(t + 1);
    __syncthreads();
    float vv[4], o[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 4; ++e) vv[e] = s_v[c_local + e];
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
      const int row = grp + kGroups * i;
      const float kr = s_k[row], qr = s_q[row];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        S[i][e] = fmaf(gamma, S[i][e], kr * vv[e]);
        o[e] = fmaf(qr, S[i][e], o[e]);
      }
    }
    // Sum over the 16 row groups of the wave (lane bits 2..5), then waves.
#pragma unroll
    for (int sft = kColThreads; sft < 64; sft <<= 1) {
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] += __shfl_xor(o[e], sft, 64);
    }
    if (lane < kColThreads) {
#pragma unroll
      for (int e = 0; e < 4; ++e) s_o[wave][c_local + e] = o[e];
    }
    __syncthreads();
    if (tid < kGretCols) {
      const float acc = ((s_o[0][tid] + s_o[1][tid]) + s_o[2][tid]) + s_o[3][tid];
      a.o[tok * D + cblk * kGretCols + tid] = acc;
    }
  }
  if (a.state_out == nullptr) return;
#pragma unroll
  for (int i = 0; i < kRows; ++i) {
    const int row = grp + kGroups * i;
    *reinterpret_cast<float4 *>(a.state_out + sbase + row * D + c0) = make_float4(S[i][0], S[i][1], S[i][2], S[i][3]);
  }
}

namespace gr {
// Direct-to-LDS staging of a [128][128] bf16 tile whose row r starts at
// base + r * stride (elements): load i of wave w fills 1 KiB block
// b = w * kLoadsPerWave + i = rows 4b .. 4b+3; lane L writes (row 4b + L/16,
// slot L%16) holding global chunk slot ^ row_xor(row).  The descriptor ends
// with row rows-1, so rows past it land as zeros.
__device__ __forceinline__ void stage_rows(char *dst, const bf16_t *base, int stride, int rows, int wave, int lane) {
  const int bytes = rows > 0 ? ((rows - 1) * stride + kD) * 2 : 0;
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t *>(base), 0, bytes, kBufferFlags);
#pragma unroll
  for (int i = 0; i < kLoadsPerWave; ++i) {
    const int blk = wave * kLoadsPerWave + i;
    const int row = blk * 4 + (lane >> 4);
    const int chunk = (lane & 15) ^ row_xor<kD, kSwz>(row);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)(dst + blk * 1024), 16,
                                             static_cast<uint32_t>(row * stride * 2 + chunk * 16), 0, 0, 0);
  }
}

// Transposed reads of a row-major [k][128] tile: the A (or B) fragment for
// output index tile `dt` (32 wide) and k step ks (16 deep): lane i of each
// 16-lane group receives 4 consecutive k rows of index dt*32 + (group&1)*16
// + i per read, two reads per fragment.  The order of k within the step is
// free as long as both operands of a product agree:
//   kSplitHalves: lanes 0..31 take k rows 0..7 of the step, 32..63 rows
//                 8..15 (the order of a 16-byte read of a k-contiguous row);
//   kInterleave:  lanes 0..31 take rows 0..3 and 8..11, 32..63 rows 4..7
//                 and 12..15 (the order of the 32x32 accumulator rows, so a
//                 score accumulator serves directly as the other operand).
enum TrOrder { kSplitHalves = 0, kInterleave = 1 };
struct TrFrag {
  int off[2][4];
  // Byte offset of read r (0, 1) of index tile dt for this lane.
  static __device__ __forceinline__ int offset(int lane, TrOrder order, int r, int dt) {
    const int grp = lane >> 4;
    const int src_a = lane & 3;
    const int src_j = (lane >> 2) & 3;
    const int krow = order == kSplitHalves ? (grp >> 1) * 8 + src_j : (grp >> 1) * 4 + src_j;
    const int second = order == kSplitHalves ? 4 : 8;
    const int col = (grp & 1) * 16 + src_a * 4;
    return swz<kD, kSwz>(krow + second * r, dt * 32 + col);
  }
  __device__ __forceinline__ void init(int lane, TrOrder order) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
#pragma unroll
      for (int d = 0; d < 4; ++d) off[r][d] = offset(lane, order, r, d);
    }
  }
  static __device__ __forceinline__ bf16x8_t read_at(const char *tile, int off0, int off1, int ks) {
    Frag8 f;
    f.s4[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4_t *)(tile + off0 + ks * 16 * kRowBytes));
    f.s4[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4_t *)(tile + off1 + ks * 16 * kRowBytes));
    return f.v;
  }
  __device__ __forceinline__ bf16x8_t read(const char *tile, int dt, int ks) const {
    return read_at(tile, off[0][dt], off[1][dt], ks);
  }
};

// One chunk's step of a state held in the MFMA accumulators (wave w: key
// dims 32w .. 32w+31, acc[t] value dims 32t .. 32t+31):
//   A <- exp(l_C) A + K'^T V,  K' = exp(l_C - l_k) k_k rounded to bf16,
// with K and V as row-major [128][128] LDS tiles and the key weights
// exp(l_C - l_k) in w (zero past the chunk's rows).  ka0/ka1: this wave's
// K^T fragment offsets; fr: V's offsets in the same k order.
__device__ __forceinline__ void state_step(floatx16 (&acc)[4], const char *lds_k, const char *lds_v, const float *w,
                                           int ka0, int ka1, const TrFrag &fr, float dec, int half) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[t][e] *= dec;
  }
#pragma unroll
  for (int ks = 0; ks < kChunk / 16; ++ks) {
    // The K^T fragment holds key rows ks*16 + half*8 + i (i = 0..7) of
    // key dim 32*wave + col; each is weighted and rounded to bf16.
    Frag8 af;
    af.v = TrFrag::read_at(lds_k, ka0, ka1, ks);
    const float4 w0 = *reinterpret_cast<const float4 *>(w + ks * 16 + half * 8);
    const float4 w1 = *reinterpret_cast<const float4 *>(w + ks * 16 + half * 8 + 4);
    af.w[0] = cvt_pk_bf16(bf16_lo(af.w[0]) * w0.x, bf16_hi(af.w[0]) * w0.y);
    af.w[1] = cvt_pk_bf16(bf16_lo(af.w[1]) * w0.z, bf16_hi(af.w[1]) * w0.w);
    af.w[2] = cvt_pk_bf16(bf16_lo(af.w[2]) * w1.x, bf16_hi(af.w[2]) * w1.y);
    af.w[3] = cvt_pk_bf16(bf16_lo(af.w[3]) * w1.z, bf16_hi(af.w[3]) * w1.w);
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af.v, fr.read(lds_v, t, ks), acc[t], 0, 0, 0);
  }
}
}  // namespace gr

// ---------------------------------------------------------------------------
// Per (group of kGroup chunks, head): the group's total
//   T_g = sum_k exp(L_G - L_k) k_k^T v_k
// over its positions, L the inclusive cumulative log gamma from the group's
// start and L_G its value at the group's end (Lambda_g) -- the recurrence
// A <- exp(l_C) A + U_c over the group's chunks from A = 0, summed in one
// pass: no step depends on the previous one, so K and V stream through LDS
// in 32-row sub-tiles, a ring of three with two in flight.  Wave 0 first
// scans the group's
// gates: kGroup * 2 consecutive positions per lane, lane totals scanned over
// the wave for L and over each lane segment of one chunk for the chunk-local
// cumulative sums l that go to the workspace for the output kernel; the key
// weights exp(L_G - L_k) go to LDS.  The weighted K^T fragments are rounded
// to bf16.  T_g lives in the MFMA accumulators: wave w owns rows (key dims)
// 32w .. 32w+31, all 128 value dims; it is stored transposed ([value
// dim][key dim]).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(gr::kThreads, 3) void gret_group_state_kernel(const GretArgs a) {
  using namespace gr;
  constexpr int kSubRows = 32;                           // rows per streamed sub-tile
  constexpr int kSubBytes = kSubRows * kRowBytes;        // 8 KiB of K (and of V)
  constexpr int kStages = 3;                             // ring of sub-tiles: two in flight
  constexpr int kLoadsPerStage = 2 * kSubBytes / 1024 / kWaves;  // vector memory ops per wave per stage (K and V)
  constexpr int kGroupRows = kGroup * kChunk;            // positions per group
  constexpr int kPerLane = kGroupRows / 64;              // positions per lane of the scan
  constexpr int kChunkLanes = kChunk / kPerLane;         // lanes of the scan per chunk
  static_assert(kGroupRows % 64 == 0 && kChunk % kPerLane == 0, "whole chunks per lane segment");
  static_assert(kLoadsPerStage == 4, "the counted waits below assume 4 loads per wave per stage");
  // One array per ring slot, selected at compile time: the compiler can then
  // tell that reads of one slot do not alias the direct-to-LDS loads still
  // landing in the others, and waits only as the counted waits below say.
  // (Each slot holds the K sub-tile and, after it, the V sub-tile.)
  __shared__ __attribute__((aligned(1024))) char lds_kv0[2 * kSubBytes];
  __shared__ __attribute__((aligned(1024))) char lds_kv1[2 * kSubBytes];
  __shared__ __attribute__((aligned(1024))) char lds_kv2[2 * kSubBytes];
  __shared__ __attribute__((aligned(16))) float s_w[kGroupRows];
  auto kslot = [&](auto b_c) __attribute__((always_inline)) -> char * {
    constexpr int B = decltype(b_c)::value;
    if constexpr (B == 0) return lds_kv0;
    else if constexpr (B == 1) return lds_kv1;
    else return lds_kv2;
  };
  auto vslot = [&](auto b_c) __attribute__((always_inline)) -> char * { return kslot(b_c) + kSubBytes; };
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int col = lane & 31;
  const int g = blockIdx.x / a.heads;
  const int h = blockIdx.x % a.heads;
  const int64_t t0 = static_cast<int64_t>(g) * kGroupRows;
  const int rows = a.n_tokens - t0 < kGroupRows ? static_cast<int>(a.n_tokens - t0) : kGroupRows;
  const int n_sub = (rows + kSubRows - 1) / kSubRows;
  const int stride = a.heads * kD;
  const bf16_t *kg = static_cast<const bf16_t *>(a.k) + (t0 * a.heads + h) * kD;
  const bf16_t *vg = static_cast<const bf16_t *>(a.v) + (t0 * a.heads + h) * kD;
  // Sub-tile j: rows 32j .. 32j+31 of the group; wave w loads rows 8w ..
  // 8w+7 of K and of V (two 1-KiB loads of 4 rows each); rows past the
  // group's end land as zeros.  Sub-tiles past the group's last one are
  // staged too, through descriptors of zero size (no memory access; zeros
  // land in a slot nobody reads), so every step issues the same loads and
  // the compiler's own wait tracking never merges paths with different
  // loads in flight (where it does, it waits for all of them).
  auto stage = [&](auto b_c, int j) __attribute__((always_inline)) {
    char *dk = kslot(b_c);
    char *dv = vslot(b_c);
    const int r0 = j * kSubRows;
    const int valid = rows - r0 < kSubRows ? rows - r0 : kSubRows;
    // (valid <= 0 gives a negative span: stride >= kD.)
    const int bytes = max(0, ((valid - 1) * stride + kD) * 2);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_t *>(kg + static_cast<int64_t>(r0) * stride), 0, bytes, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_t *>(vg + static_cast<int64_t>(r0) * stride), 0, bytes, kBufferFlags);
#pragma unroll
    for (int i = 0; i < kSubBytes / 1024 / kWaves; ++i) {
      const int blk = wave * (kSubBytes / 1024 / kWaves) + i;
      const int row = blk * 4 + (lane >> 4);
      const uint32_t off = static_cast<uint32_t>(row * stride * 2 + (((lane & 15) ^ row_xor<kD, kSwz>(row)) * 16));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t *)(dk + blk * 1024), 16, off, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t *)(dv + blk * 1024), 16, off, 0, 0, 0);
    }
  };
  // Wave 0 loads the group's gates first (every load issued at once, at
  // clamped positions), then every wave starts the first three sub-tiles.
  float lg[kPerLane];
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
      const int p = min(lane * kPerLane + i, rows - 1);
      lg[i] = a.gate[(t0 + p) * a.heads + h];
    }
  }
  stage(std::integral_constant<int, 0>(), 0);
  stage(std::integral_constant<int, 1>(), 1);

  // Wave 0, while the first sub-tiles load: the group's cumulative gates.
  if (wave == 0) {
    float tot = 0.f;
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
      const int p = lane * kPerLane + i;
      lg[i] = p < rows ? gret_log_gate(lg[i], a.inv_tau) : 0.f;
      tot += lg[i];
    }
    // Inclusive scans of the lane totals: over the wave (L) and over each
    // segment of kChunkLanes lanes (the chunk).
    float incl = tot, seg = tot;
#pragma unroll
    for (int sft = 1; sft < 64; sft <<= 1) {
      const float o = __shfl_up(incl, sft, 64);
      if (lane >= sft) incl += o;
      if (sft < kChunkLanes) {
        const float os = __shfl_up(seg, sft, 64);
        if ((lane & (kChunkLanes - 1)) >= sft) seg += os;
      }
    }
    const float total = __shfl(incl, 63, 64);  // L_G (positions past the group add 0)
    float big = incl - tot, loc = seg - tot;   // exclusive prefixes
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
      const int p = lane * kPerLane + i;
      big += lg[i];
      loc += lg[i];
      s_w[p] = p < rows ? expf(total - big) : 0.f;
      if (p < rows) a.lcum[(t0 + p) * a.heads + h] = loc;
    }
    if (lane == 0) a.gdec[static_cast<int64_t>(g) * a.heads + h] = total;
  }

  TrFrag fr;  // both operands of K'^T V in the same k order
  fr.init(lane, kSplitHalves);
  // This wave's K^T fragment offsets (index tile = wave), kept out of the
  // per-tile table so no register array is indexed at run time.
  const int ka0 = TrFrag::offset(lane, kSplitHalves, 0, wave);
  const int ka1 = TrFrag::offset(lane, kSplitHalves, 1, wave);
  floatx16 acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[t][e] = 0.f;
  }
  // Sub-tile j sits in ring slot j % 3; the loop runs three sub-tiles per
  // pass so that every slot is a compile-time choice.
  auto step = [&](auto b_c, int j) __attribute__((always_inline)) {
    constexpr int B = decltype(b_c)::value;
    // Sub-tile j has landed for every wave: this wave waits until only the
    // loads of the next sub-tile it has issued are outstanding (the first
    // pass waits for everything, the gates included), then the barrier.
    // Every wave is then also done with sub-tile j-1, whose slot sub-tile
    // j+2 takes.
    if (j == 0) {
      __builtin_amdgcn_s_waitcnt(0);
    } else {
      __builtin_amdgcn_s_waitcnt(kVmcnt4);
    }
    // A plain barrier: __syncthreads() adds a workgroup release fence, which
    // would wait for every load still landing in LDS.  LDS is one memory for
    // the workgroup, so the counted wait above is what orders this wave's
    // landed sub-tile before the others' reads; the empty asm statements keep
    // the compiler from moving memory accesses across the barrier.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    stage(std::integral_constant<int, (B + kStages - 1) % kStages>(), j + kStages - 1);
    __builtin_amdgcn_sched_barrier(0);  // the loads go out before this sub-tile's reads
    if (j >= n_sub) return;  // a step past the end only keeps the staging uniform
    const char *tk = kslot(b_c);
    const char *tv = vslot(b_c);
    const float *w = s_w + j * kSubRows;
#pragma unroll
    for (int ks = 0; ks < kSubRows / 16; ++ks) {
      // The K^T fragment holds rows ks*16 + half*8 + i (i = 0..7) of the
      // sub-tile for key dim 32*wave + col; each is weighted and rounded to bf16.
      Frag8 af;
      af.v = TrFrag::read_at(tk, ka0, ka1, ks);
      const float4 w0 = *reinterpret_cast<const float4 *>(w + ks * 16 + half * 8);
      const float4 w1 = *reinterpret_cast<const float4 *>(w + ks * 16 + half * 8 + 4);
      af.w[0] = cvt_pk_bf16(bf16_lo(af.w[0]) * w0.x, bf16_hi(af.w[0]) * w0.y);
      af.w[1] = cvt_pk_bf16(bf16_lo(af.w[1]) * w0.z, bf16_hi(af.w[1]) * w0.w);
      af.w[2] = cvt_pk_bf16(bf16_lo(af.w[2]) * w1.x, bf16_hi(af.w[2]) * w1.y);
      af.w[3] = cvt_pk_bf16(bf16_lo(af.w[3]) * w1.z, bf16_hi(af.w[3]) * w1.w);
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af.v, fr.read(tv, t, ks), acc[t], 0, 0, 0);
    }
  };
  // Whole passes of three steps (steps past the last sub-tile stage and
  // wait like the others), so no step sits under a branch.
  for (int j = 0; j < n_sub; j += kStages) {
    step(std::integral_constant<int, 0>(), j);
    step(std::integral_constant<int, 1>(), j + 1);
    step(std::integral_constant<int, 2>(), j + 2);
  }
  // The loads of the sub-tiles past the end land before the LDS is released.
  __builtin_amdgcn_s_waitcnt(0);
  // T_g (fp32, transposed).
  float *tg = a.tg + (static_cast<int64_t>(g) * a.heads + h) * kD * kD;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      *reinterpret_cast<float4 *>(tg + (t * 32 + col) * kD + wave * 32 + q4 * 8 + half * 4) =
          make_float4(acc[t][q4 * 4 + 0], acc[t][q4 * 4 + 1], acc[t][q4 * 4 + 2], acc[t][q4 * 4 + 3]);
    }
  }
}

// ---------------------------------------------------------------------------
// The pass over groups: S_0 = start state, S_{g+1} = exp(Lambda_g) S_g + T_g.
// Thread owns 4 consecutive elements of one head's transposed state; S_g
// goes out in fp32 for the output kernel, the state after the last group
// (untransposed) to state_out.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gret_group_scan_kernel(const GretArgs a, int n_groups) {
  using namespace gr;
  constexpr int kPerHead = kD * kD / 4;  // float4s per state
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<int64_t>(a.heads) * kPerHead) return;
  const int h = static_cast<int>(idx / kPerHead);
  const int e4 = static_cast<int>(idx % kPerHead);
  const int vdim = e4 / (kD / 4);         // row of the transposed state
  const int kdim = (e4 % (kD / 4)) * 4;   // first of its four key dims
  float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
  if (a.state_in) {
    const float *si = a.state_in + static_cast<int64_t>(h) * kD * kD + vdim;
    r = make_float4(si[(kdim + 0) * kD], si[(kdim + 1) * kD], si[(kdim + 2) * kD], si[(kdim + 3) * kD]);
  }
  auto t_at = [&](int gg) __attribute__((always_inline)) {
    return reinterpret_cast<const float4 *>(a.tg + (static_cast<int64_t>(gg) * a.heads + h) * kD * kD)[e4];
  };
  // kScanAhead groups' totals in flight.  Every load is issued at a clamped
  // group index, never under a branch (a load under a branch makes the
  // compiler wait for it where the branch joins, which would leave one load
  // in flight).
  float4 ring[kScanAhead];
  float lring[kScanAhead];
#pragma unroll
  for (int j = 0; j < kScanAhead; ++j) {
    const int gj = min(j, n_groups - 1);
    ring[j] = t_at(gj);
    lring[j] = a.gdec[static_cast<int64_t>(gj) * a.heads + h];
  }
  for (int g0 = 0; g0 < n_groups; g0 += kScanAhead) {
#pragma unroll
    for (int j = 0; j < kScanAhead; ++j) {
      const int gg = g0 + j;
      if (gg < n_groups) {
        reinterpret_cast<float4 *>(a.sg + (static_cast<int64_t>(gg) * a.heads + h) * kD * kD)[e4] = r;
        const float dec = expf(lring[j]);
        const float4 t = ring[j];
        r.x = fmaf(dec, r.x, t.x);
        r.y = fmaf(dec, r.y, t.y);
        r.z = fmaf(dec, r.z, t.z);
        r.w = fmaf(dec, r.w, t.w);
      }
      const int gn = min(gg + kScanAhead, n_groups - 1);
      ring[j] = t_at(gn);
      lring[j] = a.gdec[static_cast<int64_t>(gn) * a.heads + h];
    }
  }
  if (a.state_out) {
    float *so = a.state_out + static_cast<int64_t>(h) * kD * kD + vdim;
    so[(kdim + 0) * kD] = r.x;
    so[(kdim + 1) * kD] = r.y;
    so[(kdim + 2) * kD] = r.z;
    so[(kdim + 3) * kD] = r.w;
  }
}

// ---------------------------------------------------------------------------
// Outputs of a group of chunks of one head, walking the group's chunks in
// order with the state in the MFMA accumulators (the state kernel's layout),
// started at S_g, so that before chunk c it holds R_c.  Wave w owns query
// rows 32w .. 32w+31 of each chunk.  64 KiB of LDS (two workgroups per CU):
// R_c is rounded to bf16 into the buffer that V takes afterwards, so V loads
// while the scores of the chunk are formed.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(gr::kThreads, 2) void gret_group_out_kernel(const GretArgs a) {
  using namespace gr;
  __shared__ __attribute__((aligned(1024))) char lds_k[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char lds_rv[kTileBytes];  // R_c, then V_c
  __shared__ __attribute__((aligned(16))) float s_l[kChunk];
  __shared__ __attribute__((aligned(16))) float s_w[kChunk];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int col = lane & 31;
  const int g = blockIdx.x / a.heads;
  const int h = blockIdx.x % a.heads;
  const int n_chunks = static_cast<int>((a.n_tokens + kChunk - 1) / kChunk);
  const int c_begin = g * kGroup;
  const int c_end = c_begin + kGroup < n_chunks ? c_begin + kGroup : n_chunks;
  const int stride = a.heads * kD;

  // S_g (fp32, transposed: element (value v, key k) at v * 128 + k) into
  // the accumulators: acc[t] element e is key dim 32*wave + (e/4)*8 +
  // half*4 + e%4, value dim t*32 + col.
  floatx16 acc[4];
  {
    const float *sg = a.sg + (static_cast<int64_t>(g) * a.heads + h) * kD * kD;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 v = *reinterpret_cast<const float4 *>(sg + (t * 32 + col) * kD + wave * 32 + q4 * 8 + half * 4);
        acc[t][q4 * 4 + 0] = v.x;
        acc[t][q4 * 4 + 1] = v.y;
        acc[t][q4 * 4 + 2] = v.z;
        acc[t][q4 * 4 + 3] = v.w;
      }
    }
  }

  const int my_row = wave * 32 + col;
  // Q^T of a chunk as the B operand: lane holds query row my_row, dims
  // ks*16 + half*8 .. +8.  The next chunk's rows load while the current
  // chunk's state step runs.
  Frag8 qf[kD / 16];
  auto load_q = [&](int c) __attribute__((always_inline)) {
    const int64_t t0 = static_cast<int64_t>(c) * kChunk;
    const bool ok = t0 + my_row < a.n_tokens;
    const bf16_t *qp = static_cast<const bf16_t *>(a.q) + ((t0 + (ok ? my_row : 0)) * a.heads + h) * kD + half * 8;
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) qf[ks].u = ok ? ld16(qp + ks * 16) : make_uint4(0, 0, 0, 0);
  };
  load_q(c_begin);
  // The chunk-local cumulative gate of this thread's position (threads <
  // 128), loaded a chunk ahead like the queries (its load is not waited for
  // at the chunk's start).
  auto load_l = [&](int c) __attribute__((always_inline)) {
    const int64_t t0 = static_cast<int64_t>(c) * kChunk;
    const int64_t p = t0 + (tid < kChunk ? tid : 0);
    return p < a.n_tokens ? a.lcum[p * a.heads + h] : 0.f;
  };
  float l_next = load_l(c_begin);

  for (int c = c_begin; c < c_end; ++c) {
    // LDS read offsets are derived inside each chunk from an opaque copy of
    // the lane index, so the compiler cannot keep them in registers across
    // the whole loop (the state, O and P take most of them).
    int lane_o = lane;
    asm volatile("" : "+v"(lane_o));
    int koff[kD / 16];  // 16-byte reads of a row-major [.][128] tile: row col, dims ks*16 + half*8
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) koff[ks] = swz<kD, kSwz>(lane_o & 31, ks * 16 + (lane_o >> 5) * 8);
    const int64_t t0 = static_cast<int64_t>(c) * kChunk;
    const int rows = a.n_tokens - t0 < kChunk ? static_cast<int>(a.n_tokens - t0) : kChunk;
    const bf16_t *kg = static_cast<const bf16_t *>(a.k) + (t0 * a.heads + h) * kD;
    const bf16_t *vg = static_cast<const bf16_t *>(a.v) + (t0 * a.heads + h) * kD;
    // Every wave is done with the previous chunk's K, V and key weights.
    __syncthreads();
    if (tid < kChunk) s_l[tid] = l_next;  // zero past the last position
    // R_c (bf16, transposed: row = value dim) into LDS: four consecutive key
    // dims per lane and (t, q4), 8-byte writes.
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        uint2 pk;
        pk.x = cvt_pk_bf16(acc[t][q4 * 4 + 0], acc[t][q4 * 4 + 1]);
        pk.y = cvt_pk_bf16(acc[t][q4 * 4 + 2], acc[t][q4 * 4 + 3]);
        *reinterpret_cast<uint2 *>(lds_rv + swz<kD, kSwz>(t * 32 + col, wave * 32 + q4 * 8 + half * 4)) = pk;
      }
    }
    // The K tile loads go out after this wave's LDS writes (an LDS write
    // issued after them would wait for them).
    asm volatile("" ::: "memory");
    stage_rows(lds_k, kg, stride, rows, wave, lane);
    const bool row_valid = my_row < rows;
    // R_c and s_l are in LDS for every wave.  A plain barrier after the LDS
    // writes only: the K tile keeps loading under the carried term, which
    // does not read it (__syncthreads() would wait for those loads too).
    __builtin_amdgcn_s_waitcnt(kLgkm0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // Key weights of the state step, exp(l_C - l_k) (read after a later barrier).
    const float lc = s_l[rows - 1];
    if (tid < kChunk) s_w[tid] = tid < rows ? expf(lc - s_l[tid]) : 0.f;

    floatx16 oacc[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[d][e] = 0.f;
    }
    // Carried state: O^T = R^T Q^T (R^T rows d*32 + col from 16-byte reads),
    // then row j times exp(l_j).
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        Frag8 rf;
        rf.u = *reinterpret_cast<const uint4 *>(lds_rv + d * 32 * kRowBytes + koff[ks]);
        oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rf.v, qf[ks].v, oacc[d], 0, 0, 0);
      }
    }
    const float l_row = s_l[row_valid ? my_row : 0];
    const float carry = expf(l_row);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[d][e] *= carry;
    }
    // Every wave is done with R_c (V takes its buffer), and the K tile has
    // landed for every wave.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    stage_rows(lds_rv, vg, stride, rows, wave, lane);

    // Per 32-key half u = 0 .. wave (keys <= the wave's rows): S^T = K Q^T,
    // P = S exp(l_j - l_k) masked to k <= j, in bf16, then O^T += V^T P^T
    // over the half's two 16-key steps.  The first half's scores are formed
    // while V loads.
    TrFrag fv;
    fv.init(lane_o, kInterleave);  // V^T against P^T (the score accumulator order)
#pragma unroll
    for (int u = 0; u < kWaves; ++u) {
      if (u > wave) break;
      floatx16 sc;
#pragma unroll
      for (int e = 0; e < 16; ++e) sc[e] = 0.f;
      const char *tk = lds_k + u * 32 * kRowBytes;
#pragma unroll
      for (int ks = 0; ks < kD / 16; ++ks) {
        Frag8 kf;
        kf.u = *reinterpret_cast<const uint4 *>(tk + koff[ks]);
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf.v, qf[ks].v, sc, 0, 0, 0);
      }
      // S^T element e is key 32u + (e/4)*8 + half*4 + e%4 of query row my_row.
      Frag8 pf[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float pv[2];
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            const int e = kk * 8 + 2 * j + x;
            const int key = u * 32 + (e >> 2) * 8 + half * 4 + (e & 3);
            pv[x] = (key <= my_row) ? sc[e] * expf(l_row - s_l[key]) : 0.f;
          }
          pf[kk].w[j] = cvt_pk_bf16(pv[0], pv[1]);
        }
      }
      if (u == 0) {
        // Every wave runs half 0: V has landed for every wave and the key
        // weights are in place.
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fv.read(lds_rv + u * 32 * kRowBytes, d, kk), pf[kk].v,
                                                            oacc[d], 0, 0, 0);
        }
      }
    }
    if (row_valid) {
      // oacc[d] element e is value dim d*32 + (e/4)*8 + half*4 + e%4 of row my_row.
      float *op = a.o + ((t0 + my_row) * a.heads + h) * kD;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          *reinterpret_cast<float4 *>(op + d * 32 + i4 * 8 + half * 4) =
              make_float4(oacc[d][i4 * 4 + 0], oacc[d][i4 * 4 + 1], oacc[d][i4 * 4 + 2], oacc[d][i4 * 4 + 3]);
        }
      }
    }
    // R_{c+1}; the state after the group's last chunk is the scan's.
    if (c + 1 < c_end) {
      l_next = load_l(c + 1);
      load_q(c + 1);
      TrFrag fr;
      fr.init(lane_o, kSplitHalves);  // V against K'^T
      const int ka0 = TrFrag::offset(lane_o, kSplitHalves, 0, wave);
      const int ka1 = TrFrag::offset(lane_o, kSplitHalves, 1, wave);
      state_step(acc, lds_k, lds_rv, s_w, ka0, ka1, fr, expf(lc), half);
    }
  }
}

bool gret_chunked_applies(int dtype, int head_dim) { return dtype == YOCO_DT_BF16 && head_dim == gr::kD; }

int64_t gret_n_chunks(int64_t n) { return (n + gr::kChunk - 1) / gr::kChunk; }

int64_t gret_n_groups(int64_t n) { return (gret_n_chunks(n) + gr::kGroup - 1) / gr::kGroup; }

hipError_t launch_gret_recurrent(const GretArgs &a, int dtype, int head_dim, int n_seq, hipStream_t s) {
  const int64_t blocks64 = static_cast<int64_t>(n_seq) * a.heads * (head_dim / kGretCols);
  if (blocks64 > 0x7fffffff) return hipErrorInvalidValue;
  const unsigned blocks = static_cast<unsigned>(blocks64);
  if (dtype == YOCO_DT_BF16) {
    if (head_dim == 128) hipLaunchKernelGGL((gret_recurrent_kernel<bf16_t, 128>), dim3(blocks), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((gret_recurrent_kernel<bf16_t, 64>), dim3(blocks), dim3(256), 0, s, a);
  } else {
    if (head_dim == 128) hipLaunchKernelGGL((gret_recurrent_kernel<float, 128>), dim3(blocks), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((gret_recurrent_kernel<float, 64>), dim3(blocks), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_gret_chunked(const GretArgs &a, hipStream_t s) {
  const int64_t n_groups = gret_n_groups(a.n_tokens);
  const int64_t blocks = n_groups * a.heads;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gret_group_state_kernel, dim3(static_cast<unsigned>(blocks)), dim3(gr::kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t scan_threads = static_cast<int64_t>(a.heads) * gr::kD * gr::kD / 4;
  hipLaunchKernelGGL(gret_group_scan_kernel, dim3(static_cast<unsigned>((scan_threads + 255) / 256)), dim3(256), 0, s,
                     a, static_cast<int>(n_groups));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(gret_group_out_kernel, dim3(static_cast<unsigned>(blocks)), dim3(gr::kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace yoco
