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
// The pass over chunks is split in two levels, so no per-chunk fp32 state
// ever goes to memory: chunks form groups of kGroup; inside group g the
// same recurrence started from zero gives A_c, the group's total T_g and
// its decay Lambda_g, and then S_{g+1} = exp(Lambda_g) S_g + T_g (S_0 the
// start state) gives R_c = A_c + exp(delta_c) S_g, delta_c the log decay
// from the group's start to chunk c.
//   * gret_group_state_kernel: one workgroup per (group, head) walks the
//     group's chunks with A in the MFMA accumulators: l for the chunk (a
//     wave scan), A_c out in bf16, then A <- exp(l_C) A + K'^T V with
//     K' = exp(l_C - l_k) k_k rounded to bf16 (weights applied to the
//     transposed K fragments), both operands from row-major LDS tiles.
//   * gret_group_scan_kernel: the short pass over groups, elementwise over
//     the state (S_g in fp32, the last state to state_out).
//   * gret_chunk_out_kernel: 4 waves x 32 query rows of a chunk.  R_c is
//     formed in fp32 from A_c and S_g and rounded to bf16 into LDS; the
//     carried term O^T = R^T Q^T comes first (then each lane scales its
//     query row by exp(l_j)), then per 32-key half S^T = K Q^T,
//     P = S exp(l_j - l_k) masked to k <= j and rounded to bf16 (formed
//     while V loads into the buffer R_c held), then O^T += V^T P^T -- the
//     layout of the causal prefill kernel (one query row per lane, Q^T in
//     registers).
// The stored states are transposed ([value dim][key dim]): the output
// kernel then reads R^T rows with plain 16-byte LDS reads, and the state
// kernel writes four consecutive key dims per lane.
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
constexpr int kGroup = 8;          // chunks per group of the state kernel
constexpr int kScanAhead = 8;      // group states in flight per thread in the scan
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
}  // namespace gr

// ---------------------------------------------------------------------------
// Per (group of kGroup chunks, head), walking the group's chunks in order:
// l (inclusive cumulative log gamma inside each chunk) and the log decay
// from the group's start to each chunk (delta_c) go to the workspace; the
// group-local state A_c (state before chunk c, counted from zero at the
// group's start) goes out in bf16 for every chunk but the group's first,
// A_{c+1} = exp(l_C) A_c + K'^T V with K' = exp(l_C - l_k) k_k rounded to
// bf16, and the group's total T_g = A after its last chunk in fp32, with
// its log decay Lambda_g.  A lives in the MFMA accumulators: wave w owns
// rows (key dims) 32w .. 32w+31, all 128 value dims.  States are stored
// transposed ([value dim][key dim]), the layout the output kernel reads.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(gr::kThreads, 2) void gret_group_state_kernel(const GretArgs a) {
  using namespace gr;
  __shared__ __attribute__((aligned(1024))) char lds_k[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char lds_v[kTileBytes];
  __shared__ __attribute__((aligned(16))) float s_w[kChunk];
  __shared__ float s_lc;
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
  float delta = 0.f;  // log decay from the group's start to chunk c
  for (int c = c_begin; c < c_end; ++c) {
    const int64_t t0 = static_cast<int64_t>(c) * kChunk;
    const int rows = a.n_tokens - t0 < kChunk ? static_cast<int>(a.n_tokens - t0) : kChunk;
    stage_rows(lds_k, static_cast<const bf16_t *>(a.k) + (t0 * a.heads + h) * kD, stride, rows, wave, lane);
    stage_rows(lds_v, static_cast<const bf16_t *>(a.v) + (t0 * a.heads + h) * kD, stride, rows, wave, lane);
    // Wave 0, while the tiles load: the chunk's cumulative log gates (lane
    // holds positions 2L, 2L+1) and the key weights exp(l_C - l_k).
    if (wave == 0) {
      float l0 = 0.f, l1 = 0.f;
      const int p0 = 2 * lane, p1 = 2 * lane + 1;
      if (p0 < rows) l0 = gret_log_gate(a.gate[(t0 + p0) * a.heads + h], a.inv_tau);
      if (p1 < rows) l1 = gret_log_gate(a.gate[(t0 + p1) * a.heads + h], a.inv_tau);
      l1 += l0;
      float incl = l1;  // inclusive scan of the pair sums over lanes
#pragma unroll
      for (int sft = 1; sft < 64; sft <<= 1) {
        const float o = __shfl_up(incl, sft, 64);
        if (lane >= sft) incl += o;
      }
      const float excl = incl - l1;
      const float c0v = excl + l0, c1v = excl + l1;
      const float last = __shfl(incl, 63, 64);  // l_C (rows past the chunk add 0)
      if (p0 < rows) a.lcum[(t0 + p0) * a.heads + h] = c0v;
      if (p1 < rows) a.lcum[(t0 + p1) * a.heads + h] = c1v;
      s_w[p0] = p0 < rows ? expf(last - c0v) : 0.f;
      s_w[p1] = p1 < rows ? expf(last - c1v) : 0.f;
      if (lane == 0) {
        s_lc = last;
        a.cdec[static_cast<int64_t>(c) * a.heads + h] = delta;
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const float lc = s_lc;
    // A_c out (bf16, transposed): acc[t] element e is A row (key dim)
    // 32*wave + (e/4)*8 + half*4 + e%4, column (value dim) t*32 + col, so a
    // lane's four consecutive e are four consecutive key dims: 8-byte stores.
    if (c > c_begin) {
      uint16_t *rl = a.rl + (static_cast<int64_t>(c) * a.heads + h) * kD * kD;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          uint2 pk;
          pk.x = cvt_pk_bf16(acc[t][q4 * 4 + 0], acc[t][q4 * 4 + 1]);
          pk.y = cvt_pk_bf16(acc[t][q4 * 4 + 2], acc[t][q4 * 4 + 3]);
          *reinterpret_cast<uint2 *>(rl + (t * 32 + col) * kD + wave * 32 + q4 * 8 + half * 4) = pk;
        }
      }
    }
    const float dec = expf(lc);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[t][e] *= dec;
    }
    delta += lc;
#pragma unroll
    for (int ks = 0; ks < kChunk / 16; ++ks) {
      // The K^T fragment holds key rows ks*16 + half*8 + i (i = 0..7) of
      // key dim 32*wave + col; each is weighted and rounded to bf16.
      Frag8 af;
      af.v = TrFrag::read_at(lds_k, ka0, ka1, ks);
      const float4 w0 = *reinterpret_cast<const float4 *>(s_w + ks * 16 + half * 8);
      const float4 w1 = *reinterpret_cast<const float4 *>(s_w + ks * 16 + half * 8 + 4);
      af.w[0] = cvt_pk_bf16(bf16_lo(af.w[0]) * w0.x, bf16_hi(af.w[0]) * w0.y);
      af.w[1] = cvt_pk_bf16(bf16_lo(af.w[1]) * w0.z, bf16_hi(af.w[1]) * w0.w);
      af.w[2] = cvt_pk_bf16(bf16_lo(af.w[2]) * w1.x, bf16_hi(af.w[2]) * w1.y);
      af.w[3] = cvt_pk_bf16(bf16_lo(af.w[3]) * w1.z, bf16_hi(af.w[3]) * w1.w);
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af.v, fr.read(lds_v, t, ks), acc[t], 0, 0, 0);
    }
    __syncthreads();  // the next chunk's tiles take the buffers
  }
  // T_g (fp32, transposed) and Lambda_g.
  float *tg = a.tg + (static_cast<int64_t>(g) * a.heads + h) * kD * kD;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      *reinterpret_cast<float4 *>(tg + (t * 32 + col) * kD + wave * 32 + q4 * 8 + half * 4) =
          make_float4(acc[t][q4 * 4 + 0], acc[t][q4 * 4 + 1], acc[t][q4 * 4 + 2], acc[t][q4 * 4 + 3]);
    }
  }
  if (tid == 0) a.gdec[static_cast<int64_t>(g) * a.heads + h] = delta;
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
  float4 ring[kScanAhead];
  float lring[kScanAhead];
#pragma unroll
  for (int j = 0; j < kScanAhead; ++j) {
    if (j < n_groups) {
      ring[j] = t_at(j);
      lring[j] = a.gdec[static_cast<int64_t>(j) * a.heads + h];
    }
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
        if (gg + kScanAhead < n_groups) {
          ring[j] = t_at(gg + kScanAhead);
          lring[j] = a.gdec[static_cast<int64_t>(gg + kScanAhead) * a.heads + h];
        }
      }
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
// Outputs of one chunk of one head: wave w owns query rows 32w .. 32w+31.
// 64 KiB of LDS (two workgroups per CU): the carried state R_c is formed in
// the buffer that V takes afterwards, so V loads while the scores of the
// chunk are formed.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(gr::kThreads, 2) void gret_chunk_out_kernel(const GretArgs a) {
  using namespace gr;
  __shared__ __attribute__((aligned(1024))) char lds_k[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char lds_rv[kTileBytes];  // R_c, then V
  __shared__ float s_l[kChunk];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int col = lane & 31;
  // Chunks in reverse order, so the ragged last chunk does not run last.
  const int n_chunks = static_cast<int>((a.n_tokens + kChunk - 1) / kChunk);
  const int chunk = n_chunks - 1 - static_cast<int>(blockIdx.x / a.heads);
  const int h = blockIdx.x % a.heads;
  const int64_t t0 = static_cast<int64_t>(chunk) * kChunk;
  const int rows = a.n_tokens - t0 < kChunk ? static_cast<int>(a.n_tokens - t0) : kChunk;
  const int stride = a.heads * kD;
  const bf16_t *kg = static_cast<const bf16_t *>(a.k) + (t0 * a.heads + h) * kD;
  const bf16_t *vg = static_cast<const bf16_t *>(a.v) + (t0 * a.heads + h) * kD;
  stage_rows(lds_k, kg, stride, rows, wave, lane);
  if (tid < kChunk) s_l[tid] = tid < rows ? a.lcum[(t0 + tid) * a.heads + h] : 0.f;
  // R_c = A_c + exp(delta_c) S_g (transposed: row = value dim), formed in
  // fp32 and rounded to bf16 into LDS; A_c is zero for a group's first chunk.
  {
    const int g = chunk / kGroup;
    const bool first = chunk == g * kGroup;
    const float dec = expf(a.cdec[static_cast<int64_t>(chunk) * a.heads + h]);
    const float *sg = a.sg + (static_cast<int64_t>(g) * a.heads + h) * kD * kD;
    const uint16_t *rl = a.rl + (static_cast<int64_t>(chunk) * a.heads + h) * kD * kD;
#pragma unroll
    for (int i = 0; i < kD * 16 / kThreads; ++i) {
      const int piece = i * kThreads + tid;
      const int row = piece >> 4;
      const int ch = piece & 15;
      const float4 s0 = *reinterpret_cast<const float4 *>(sg + row * kD + ch * 8);
      const float4 s1 = *reinterpret_cast<const float4 *>(sg + row * kD + ch * 8 + 4);
      Frag8 r;
      r.u = first ? make_uint4(0, 0, 0, 0) : ld16(reinterpret_cast<const bf16_t *>(rl) + row * kD + ch * 8);
      r.w[0] = cvt_pk_bf16(fmaf(dec, s0.x, bf16_lo(r.w[0])), fmaf(dec, s0.y, bf16_hi(r.w[0])));
      r.w[1] = cvt_pk_bf16(fmaf(dec, s0.z, bf16_lo(r.w[1])), fmaf(dec, s0.w, bf16_hi(r.w[1])));
      r.w[2] = cvt_pk_bf16(fmaf(dec, s1.x, bf16_lo(r.w[2])), fmaf(dec, s1.y, bf16_hi(r.w[2])));
      r.w[3] = cvt_pk_bf16(fmaf(dec, s1.z, bf16_lo(r.w[3])), fmaf(dec, s1.w, bf16_hi(r.w[3])));
      *reinterpret_cast<uint4 *>(lds_rv + swz<kD, kSwz>(row, ch * 8)) = r.u;
    }
  }

  // Q^T as the B operand: lane holds query row 32*wave + col, dims ks*16 + half*8 .. +8.
  const int my_row = wave * 32 + col;
  const bool row_valid = my_row < rows;
  Frag8 qf[kD / 16];
  {
    const bf16_t *qp = static_cast<const bf16_t *>(a.q) + ((t0 + (row_valid ? my_row : 0)) * a.heads + h) * kD + half * 8;
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) qf[ks].u = row_valid ? ld16(qp + ks * 16) : make_uint4(0, 0, 0, 0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  TrFrag fv;
  fv.init(lane, kInterleave);   // V^T against P^T (the score accumulator order)
  int koff[kD / 16];            // 16-byte reads of a row-major [.][128] tile: row col, dims ks*16 + half*8
#pragma unroll
  for (int ks = 0; ks < kD / 16; ++ks) koff[ks] = swz<kD, kSwz>(col, ks * 16 + half * 8);
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
  __syncthreads();  // every wave is done with R_c; V takes its buffer
  stage_rows(lds_rv, vg, stride, rows, wave, lane);

  // Scores of the chunk while V loads: 32-key halves u = 0 .. wave (keys <=
  // the wave's rows), P = S exp(l_j - l_k) masked to k <= j, in bf16.
  Frag8 p[kWaves][2];
#pragma unroll
  for (int u = 0; u < kWaves; ++u) {
    if (u > wave) break;
    floatx16 s;
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = 0.f;
    const char *tk = lds_k + u * 32 * kRowBytes;
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) {
      Frag8 kf;
      kf.u = *reinterpret_cast<const uint4 *>(tk + koff[ks]);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf.v, qf[ks].v, s, 0, 0, 0);
    }
    // S^T element e is key 32u + (e/4)*8 + half*4 + e%4 of query row my_row.
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float pv[2];
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          const int e = kk * 8 + 2 * j + x;
          const int key = u * 32 + (e >> 2) * 8 + half * 4 + (e & 3);
          pv[x] = (key <= my_row) ? s[e] * expf(l_row - s_l[key]) : 0.f;
        }
        p[u][kk].w[j] = cvt_pk_bf16(pv[0], pv[1]);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();  // V has landed for every wave
  // O^T += V^T P^T over each half's two 16-key steps.
#pragma unroll
  for (int u = 0; u < kWaves; ++u) {
    if (u > wave) break;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fv.read(lds_rv + u * 32 * kRowBytes, d, kk), p[u][kk].v, oacc[d], 0, 0, 0);
      }
    }
  }
  if (!row_valid) return;
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
  const int64_t n_chunks = gret_n_chunks(a.n_tokens);
  const int64_t n_groups = gret_n_groups(a.n_tokens);
  const int64_t blocks = n_chunks * a.heads;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gret_group_state_kernel, dim3(static_cast<unsigned>(n_groups * a.heads)), dim3(gr::kThreads), 0,
                     s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t scan_threads = static_cast<int64_t>(a.heads) * gr::kD * gr::kD / 4;
  hipLaunchKernelGGL(gret_group_scan_kernel, dim3(static_cast<unsigned>((scan_threads + 255) / 256)), dim3(256), 0, s,
                     a, static_cast<int>(n_groups));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(gret_chunk_out_kernel, dim3(static_cast<unsigned>(blocks)), dim3(gr::kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace yoco
