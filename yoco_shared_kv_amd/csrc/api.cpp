// Host side of the C ABI: argument validation, split planning and dispatch.
// Every check runs before anything is enqueued; on failure nothing is
// enqueued and no host length changes.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <initializer_list>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "yoco_internal.h"

namespace {

thread_local char g_err[512] = "";

yoco_status fail(yoco_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

yoco_status ok() {
  g_err[0] = '\0';
  return YOCO_OK;
}

bool dtype_ok(int32_t dt) { return dt == YOCO_DT_F32 || dt == YOCO_DT_BF16; }
size_t dtype_size(int32_t dt) { return dt == YOCO_DT_F32 ? 4 : 2; }
bool head_dim_ok(int32_t dh) { return dh == 64 || dh == 128; }
bool group_ok(int32_t g) { return g == 1 || g == 2 || g == 3 || g == 4 || g == 6 || g == 8; }

// The kernels are built for gfx950 only; refuse any other device loudly.
constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

yoco_status check_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(YOCO_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(YOCO_ERR_HIP, "device index %d out of range", dev);
  int st = g_dev_state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(YOCO_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_dev_state[dev].store(st, std::memory_order_release);
    if (st == 2) return fail(YOCO_ERR_HIP, "device %d is %s; this library is built for gfx950", dev, prop.gcnArchName);
  }
  if (st != 1) return fail(YOCO_ERR_HIP, "device %d is not gfx950", dev);
  return YOCO_OK;
}

yoco_status launched(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(YOCO_ERR_HIP, "%s launch: %s", what, hipGetErrorString(e));
  return ok();
}

// The kernels move tensors with 16-byte vector loads and stores, and
// per-row or per-head scalars with 4-byte ones.
struct Named {
  const void *p;
  const char *name;
};

yoco_status check_aligned(std::initializer_list<Named> ptrs, unsigned align) {
  for (const Named &x : ptrs) {
    if (x.p != nullptr && (reinterpret_cast<uintptr_t>(x.p) & (align - 1)) != 0)
      return fail(YOCO_ERR_ALIGNMENT, "%s (%p) is not %u-byte aligned", x.name, x.p, align);
  }
  return YOCO_OK;
}

constexpr int64_t kMaxRowStride = int64_t(1) << 20;

yoco_status check_row_stride(int64_t rs, int32_t n_kv_heads, int32_t head_dim, int32_t dtype) {
  if (rs == 0) return YOCO_OK;
  const int64_t dense = static_cast<int64_t>(n_kv_heads) * head_dim;
  if (rs < dense || rs > kMaxRowStride || (rs * static_cast<int64_t>(dtype_size(dtype))) % 16 != 0)
    return fail(YOCO_ERR_BAD_SHAPE, "row_stride %lld: must be 0 or in [%lld, %lld] with rows a multiple of 16 bytes",
                (long long)rs, (long long)dense, (long long)kMaxRowStride);
  return YOCO_OK;
}

// Elements from one cache row to the next.
int64_t row_stride_of(const yoco_kv_cache *c) {
  return c->row_stride != 0 ? c->row_stride : static_cast<int64_t>(c->n_kv_heads) * c->head_dim;
}

yoco_status check_cache(const yoco_kv_cache *c) {
  if (c == nullptr) return fail(YOCO_ERR_NULL_POINTER, "cache is NULL");
  if (c->k == nullptr || c->v == nullptr) return fail(YOCO_ERR_NULL_POINTER, "cache k or v is NULL");
  if (check_aligned({{c->k, "cache k"}, {c->v, "cache v"}}, 16) != YOCO_OK) return YOCO_ERR_ALIGNMENT;
  if (c->len_host == nullptr) return fail(YOCO_ERR_NULL_POINTER, "cache len_host is NULL");
  if (c->n_seq < 1 || c->n_seq > YOCO_MAX_SEQ)
    return fail(YOCO_ERR_BAD_SHAPE, "n_seq %d outside [1, %d]", c->n_seq, YOCO_MAX_SEQ);
  if (c->n_kv_heads < 1 || c->n_kv_heads > yoco::kMaxKvHeads)
    return fail(YOCO_ERR_BAD_SHAPE, "n_kv_heads %d outside [1, %d]", c->n_kv_heads, yoco::kMaxKvHeads);
  if (!head_dim_ok(c->head_dim)) return fail(YOCO_ERR_BAD_SHAPE, "head_dim %d is not 64 or 128", c->head_dim);
  if (c->seq_capacity < 1 || c->seq_capacity > (int64_t(1) << 31) - 1)
    return fail(YOCO_ERR_BAD_SHAPE, "seq_capacity %lld outside [1, 2^31)", (long long)c->seq_capacity);
  if (!dtype_ok(c->dtype)) return fail(YOCO_ERR_BAD_DTYPE, "cache dtype %d unknown", c->dtype);
  return check_row_stride(c->row_stride, c->n_kv_heads, c->head_dim, c->dtype);
}

yoco_status check_eps(float eps) {
  if (!std::isfinite(eps) || eps < 0.f) return fail(YOCO_ERR_BAD_VALUE, "eps %g must be finite and >= 0", eps);
  return YOCO_OK;
}

yoco_status check_heads(int32_t n_q_heads, int32_t n_kv_heads) {
  if (n_q_heads < 1 || n_q_heads % n_kv_heads != 0)
    return fail(YOCO_ERR_BAD_SHAPE, "n_q_heads %d is not a positive multiple of n_kv_heads %d", n_q_heads, n_kv_heads);
  if (!group_ok(n_q_heads / n_kv_heads))
    return fail(YOCO_ERR_BAD_SHAPE, "group size %d not in {1,2,3,4,6,8}", n_q_heads / n_kv_heads);
  return YOCO_OK;
}

yoco_status check_scale(float s) {
  if (!std::isfinite(s) || s <= 0.f) return fail(YOCO_ERR_BAD_VALUE, "softmax_scale %g must be finite and > 0", s);
  return YOCO_OK;
}

// ---- decode split planning -------------------------------------------------
// Library split size: enough splits that the decode grid fills the device in
// one resident round (CUs x resident workgroups per CU, capped), rounded to
// kDecodeAutoQuantum rows, at least kDecodeMinSplitRows.  The workspace bound
// below holds for any device because the target is capped.
struct DeviceInfo {
  std::atomic<int> cus{0};
  std::atomic<int> occ[2][2][9];  // [dtype][head_dim == 128][group]
};
DeviceInfo g_dev_info[kMaxDevices];

int decode_target_blocks(int dtype, int head_dim, int group) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  DeviceInfo &info = g_dev_info[dev];
  int cus = info.cus.load(std::memory_order_relaxed);
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    info.cus.store(cus, std::memory_order_relaxed);
  }
  std::atomic<int> &slot = info.occ[dtype == YOCO_DT_BF16 ? 1 : 0][head_dim == 128 ? 1 : 0][group];
  int occ = slot.load(std::memory_order_relaxed);
  if (occ == 0) {
    occ = yoco::decode_blocks_per_cu(dtype, head_dim, group);
    if (occ <= 0) occ = 1;
    slot.store(occ, std::memory_order_relaxed);
  }
  const int64_t target = static_cast<int64_t>(cus) * occ;
  return static_cast<int>(target < yoco::kDecodeMaxTargetBlocks ? target : yoco::kDecodeMaxTargetBlocks);
}

// Library split plan: the smallest split size R (a multiple of
// kDecodeAutoQuantum, at least kDecodeMinSplitRows) whose splits
// n_b = ceil(len_b / R) number at most target_blocks / n_kv_heads over the
// sequences (or one per sequence when there are more sequences than that),
// so the grid is one resident round; each sequence then cuts its rows into
// n_b equal splits (rounded up to the quantum), which keeps a ragged batch's
// workgroups close to the same length.  A single sequence of 131072 rows at
// 8 KV heads and 256 workgroups gets 32 splits of 4096 rows.
void auto_split_plan(const int64_t *lens, int n_seq, int n_kv_heads, int64_t target_blocks, int32_t *rows_out) {
  const int64_t budget = std::max<int64_t>(1, target_blocks / n_kv_heads);
  int64_t longest = 0;
  for (int b = 0; b < n_seq; ++b) longest = std::max(longest, lens[b]);
  auto splits_at = [&](int64_t r) {
    int64_t n = 0;
    for (int b = 0; b < n_seq; ++b) n += (lens[b] + r - 1) / r;
    return n;
  };
  const int64_t q = yoco::kDecodeAutoQuantum;
  int64_t lo = std::max<int64_t>(yoco::kDecodeMinSplitRows, q), hi = std::max(lo, ((longest + q - 1) / q) * q);
  if (splits_at(lo) <= budget) {
    hi = lo;
  } else {
    while (hi - lo > q) {  // splits_at(hi) <= max(budget, n_seq), splits_at(lo) > budget
      const int64_t mid = ((lo + hi) / 2 / q) * q;
      if (mid <= lo) break;
      if (splits_at(mid) <= budget) hi = mid; else lo = mid;
    }
  }
  for (int b = 0; b < n_seq; ++b) {
    const int64_t n = std::max<int64_t>(1, (lens[b] + hi - 1) / hi);
    int64_t r = (lens[b] + n - 1) / n;
    r = std::max<int64_t>(yoco::kDecodeMinSplitRows, ((r + q - 1) / q) * q);
    rows_out[b] = static_cast<int32_t>(std::min(r, hi));
  }
}

// Upper bound of total splits over every length <= capacity for a split size.
// Library choice: at most max(target/H, n_seq) <= target/H + n_seq splits,
// and every split is at least kDecodeMinSplitRows rows (unless it is its
// sequence's only one), which bounds them by n_seq*ceil(cap/kDecodeMinSplitRows).
int64_t max_total_splits(const yoco_kv_cache *c, int64_t rows_per_split) {
  if (rows_per_split == 0) {
    const int64_t fixed_bound =
        c->n_seq * ((c->seq_capacity + yoco::kDecodeMinSplitRows - 1) / yoco::kDecodeMinSplitRows);
    const int64_t growing_bound = (yoco::kDecodeMaxTargetBlocks + c->n_kv_heads - 1) / c->n_kv_heads + c->n_seq;
    return fixed_bound < growing_bound ? fixed_bound : growing_bound;
  }
  return c->n_seq * ((c->seq_capacity + rows_per_split - 1) / rows_per_split);
}

size_t decode_workspace_bytes(const yoco_kv_cache *c, int32_t n_q_heads, int64_t total_splits) {
  const int64_t group = n_q_heads / c->n_kv_heads;
  const int64_t prow = c->head_dim + 4;
  return YOCO_DECODE_COUNTER_BYTES +
         static_cast<size_t>(total_splits) * c->n_kv_heads * group * prow * sizeof(float);
}

yoco_status check_split_rows(int64_t rows_per_split) {
  if (rows_per_split < 0 || (rows_per_split % yoco::kDecodeSplitQuantum) != 0 ||
      rows_per_split > (int64_t(1) << 30))
    return fail(YOCO_ERR_BAD_VALUE, "rows_per_split %lld must be 0 or a positive multiple of %d",
                (long long)rows_per_split, yoco::kDecodeSplitQuantum);
  return YOCO_OK;
}

}  // namespace

extern "C" {

int yoco_abi_version(void) { return YOCO_ABI_VERSION; }

const char *yoco_last_error(void) { return g_err; }

yoco_status yoco_kv_cache_bytes(int32_t n_seq, int64_t seq_capacity, int32_t n_kv_heads, int32_t head_dim,
                                int32_t dtype, int64_t row_stride, size_t *bytes) {
  if (bytes == nullptr) return fail(YOCO_ERR_NULL_POINTER, "bytes is NULL");
  if (n_seq < 1 || seq_capacity < 1 || n_kv_heads < 1 || head_dim < 1)
    return fail(YOCO_ERR_BAD_SHAPE, "cache dimensions must be positive");
  if (!dtype_ok(dtype)) return fail(YOCO_ERR_BAD_DTYPE, "dtype %d unknown", dtype);
  yoco_status st = check_row_stride(row_stride, n_kv_heads, head_dim, dtype);
  if (st != YOCO_OK) return st;
  const int64_t rs = row_stride != 0 ? row_stride : static_cast<int64_t>(n_kv_heads) * head_dim;
  *bytes = static_cast<size_t>(n_seq) * static_cast<size_t>(seq_capacity) * static_cast<size_t>(rs) *
           dtype_size(dtype);
  return ok();
}

yoco_status yoco_kv_cache_row_stride(int32_t n_kv_heads, int32_t head_dim, int32_t dtype, int64_t *row_stride) {
  if (row_stride == nullptr) return fail(YOCO_ERR_NULL_POINTER, "row_stride is NULL");
  if (n_kv_heads < 1 || head_dim < 1) return fail(YOCO_ERR_BAD_SHAPE, "cache dimensions must be positive");
  if (!dtype_ok(dtype)) return fail(YOCO_ERR_BAD_DTYPE, "dtype %d unknown", dtype);
  const int64_t dense = static_cast<int64_t>(n_kv_heads) * head_dim;
  const int64_t esz = static_cast<int64_t>(dtype_size(dtype));
  const int64_t bytes = dense * esz;
  *row_stride = (bytes >= 1024 && bytes % 512 == 0) ? dense + 128 / esz : dense;
  return ok();
}

}  // extern "C"

namespace {

// Rotary position embedding requested by a *_rope entry point (theta 0: none).
struct RopeSpec {
  double theta = 0.0;
  const int64_t *pos_host = nullptr;  // q_project: per-row positions, or NULL
  int64_t pos0 = 0;                   // q_project: position of row 0 when pos_host is NULL
};

yoco_status check_rope(const RopeSpec &r) {
  if (r.theta == 0.0) return YOCO_OK;
  if (!std::isfinite(r.theta) || r.theta <= 1.0)
    return fail(YOCO_ERR_BAD_VALUE, "rope_theta %g must be finite and > 1", r.theta);
  return YOCO_OK;
}

// The few-row path (project_rows.hip) runs when the caller passes a
// workspace and the shapes allow it; without a workspace the strip kernel of
// project.hip takes the same rows.  A workspace that is given but too small
// for a call that would use it is an error.
struct RowsChoice {
  bool use = false;
  yoco::ProjRowsPlan plan{};
};

yoco_status choose_rows_path(int64_t n, int32_t d, int32_t ncols, int32_t n_out, int32_t w_dtype,
                             const void *workspace, size_t workspace_bytes, RowsChoice *c) {
  c->use = false;
  if (check_aligned({{workspace, "workspace"}}, 16) != YOCO_OK) return YOCO_ERR_ALIGNMENT;
  if (workspace == nullptr || n < 1 || n > yoco::kProjRowsMaxRows) return YOCO_OK;
  if (!yoco::project_rows_plan(d, ncols, n_out, w_dtype, &c->plan)) return YOCO_OK;
  const size_t need = yoco::project_rows_workspace_bytes(c->plan);
  if (workspace_bytes < need)
    return fail(YOCO_ERR_WORKSPACE, "workspace %zu bytes < %zu (yoco_project_workspace)", workspace_bytes, need);
  c->use = true;
  return YOCO_OK;
}

yoco_status launch_projection(const yoco::ProjArgs &a, const RowsChoice &rows, int x_dt, int w_dt, int o_dt,
                              void *workspace, void *stream, const char *what) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (rows.use) return launched(yoco::launch_project_rows(a, rows.plan, x_dt, w_dt, o_dt, workspace, s), what);
  return launched(yoco::launch_project(a, x_dt, w_dt, o_dt, s), what);
}

void set_rope(yoco::ProjArgs &a, const RopeSpec &r, int head_dim) {
  if (r.theta == 0.0) return;
  a.rope_out = 0;
  a.head_dim = head_dim;
  a.rope_log2_theta = std::log2(r.theta);
}

yoco_status kv_project_impl(const void *m, int32_t m_dtype, int64_t n, int32_t d_model, const float *gain,
                            float eps, const void *w_k, const void *w_v, int32_t w_dtype,
                            yoco_kv_cache *cache, int32_t seq, int64_t row_start, const RopeSpec &rope,
                            void *workspace, size_t workspace_bytes, void *stream) {
  yoco_status st = check_cache(cache);
  if (st != YOCO_OK) return st;
  if (m == nullptr || w_k == nullptr || w_v == nullptr) return fail(YOCO_ERR_NULL_POINTER, "m, w_k or w_v is NULL");
  if ((st = check_aligned({{m, "m"}, {w_k, "w_k"}, {w_v, "w_v"}, {gain, "gain"}}, 16)) != YOCO_OK) return st;
  if (d_model < 1) return fail(YOCO_ERR_BAD_SHAPE, "d_model %d < 1", d_model);
  if (seq < 0 || seq >= cache->n_seq) return fail(YOCO_ERR_BAD_SHAPE, "seq %d outside [0, %d)", seq, cache->n_seq);
  if (!dtype_ok(m_dtype) || !dtype_ok(w_dtype)) return fail(YOCO_ERR_BAD_DTYPE, "m or w dtype unknown");
  if ((st = check_eps(eps)) != YOCO_OK) return st;
  if ((st = check_rope(rope)) != YOCO_OK) return st;
  if (n < 0 || row_start < 0 || row_start > cache->seq_capacity - n)
    return fail(YOCO_ERR_OUT_OF_RANGE, "rows [%lld, %lld) outside capacity %lld", (long long)row_start,
                (long long)(row_start + n), (long long)cache->seq_capacity);
  RowsChoice rows;
  if ((st = choose_rows_path(n, d_model, cache->n_kv_heads * cache->head_dim, 2, w_dtype, workspace,
                             workspace_bytes, &rows)) != YOCO_OK)
    return st;
  if (n == 0) return ok();
  if ((st = check_device()) != YOCO_OK) return st;

  yoco::ProjArgs a{};
  a.x = m;
  a.gain = gain;
  a.w[0] = w_k;
  a.w[1] = w_v;
  a.out[0] = cache->k;
  a.out[1] = cache->v;
  a.n = n;
  a.dst_row_base = static_cast<int64_t>(seq) * cache->seq_capacity + row_start;
  a.d = d_model;
  a.ncols = cache->n_kv_heads * cache->head_dim;
  a.out_stride = row_stride_of(cache);
  a.n_out = 2;
  a.indexed = 0;
  a.eps = eps;
  set_rope(a, rope, cache->head_dim);  // K^ only; row r at position row_start + r
  a.pos_base = row_start;
  st = launch_projection(a, rows, m_dtype, w_dtype, cache->dtype, workspace, stream, "kv_project");
  if (st != YOCO_OK) return st;
  if (cache->len_host[seq] < row_start + n) cache->len_host[seq] = row_start + n;
  return ok();
}

yoco_status kv_append_impl(const void *m_new, int32_t m_dtype, int32_t d_model, const float *gain, float eps,
                           const void *w_k, const void *w_v, int32_t w_dtype, yoco_kv_cache *cache,
                           const RopeSpec &rope, void *workspace, size_t workspace_bytes, void *stream) {
  yoco_status st = check_cache(cache);
  if (st != YOCO_OK) return st;
  if (m_new == nullptr || w_k == nullptr || w_v == nullptr)
    return fail(YOCO_ERR_NULL_POINTER, "m_new, w_k or w_v is NULL");
  if ((st = check_aligned({{m_new, "m_new"}, {w_k, "w_k"}, {w_v, "w_v"}, {gain, "gain"}}, 16)) != YOCO_OK) return st;
  if (d_model < 1) return fail(YOCO_ERR_BAD_SHAPE, "d_model %d < 1", d_model);
  if (!dtype_ok(m_dtype) || !dtype_ok(w_dtype)) return fail(YOCO_ERR_BAD_DTYPE, "m or w dtype unknown");
  if ((st = check_eps(eps)) != YOCO_OK) return st;
  if ((st = check_rope(rope)) != YOCO_OK) return st;
  for (int b = 0; b < cache->n_seq; ++b) {
    const int64_t len = cache->len_host[b];
    if (len < 0 || len + 1 > cache->seq_capacity)
      return fail(YOCO_ERR_OUT_OF_RANGE, "sequence %d: length %lld leaves no room under capacity %lld", b,
                  (long long)len, (long long)cache->seq_capacity);
  }
  RowsChoice rows;
  if ((st = choose_rows_path(cache->n_seq, d_model, cache->n_kv_heads * cache->head_dim, 2, w_dtype, workspace,
                             workspace_bytes, &rows)) != YOCO_OK)
    return st;
  if ((st = check_device()) != YOCO_OK) return st;

  yoco::ProjArgs a{};
  a.x = m_new;
  a.gain = gain;
  a.w[0] = w_k;
  a.w[1] = w_v;
  a.out[0] = cache->k;
  a.out[1] = cache->v;
  a.n = cache->n_seq;
  a.dst_row_base = 0;
  a.d = d_model;
  a.ncols = cache->n_kv_heads * cache->head_dim;
  a.out_stride = row_stride_of(cache);
  a.n_out = 2;
  a.indexed = 1;
  a.eps = eps;
  for (int b = 0; b < cache->n_seq; ++b) a.dst_rows[b] = static_cast<int64_t>(b) * cache->seq_capacity + cache->len_host[b];
  set_rope(a, rope, cache->head_dim);  // the new row of sequence b sits at position len_b
  a.pos_indexed = 1;
  a.pos_stride = cache->seq_capacity;
  st = launch_projection(a, rows, m_dtype, w_dtype, cache->dtype, workspace, stream, "kv_append");
  if (st != YOCO_OK) return st;
  for (int b = 0; b < cache->n_seq; ++b) cache->len_host[b] += 1;
  return ok();
}

yoco_status q_project_impl(const void *x, int32_t x_dtype, int64_t n, int32_t d_model, const float *gain,
                           float eps, const void *w_q, int32_t w_dtype, int32_t n_q_heads, int32_t head_dim,
                           void *q_out, int32_t q_dtype, const RopeSpec &rope, void *workspace,
                           size_t workspace_bytes, void *stream) {
  if (x == nullptr || w_q == nullptr || q_out == nullptr) return fail(YOCO_ERR_NULL_POINTER, "x, w_q or q_out is NULL");
  if (check_aligned({{x, "x"}, {w_q, "w_q"}, {gain, "gain"}, {q_out, "q_out"}}, 16) != YOCO_OK)
    return YOCO_ERR_ALIGNMENT;
  if (d_model < 1 || n_q_heads < 1 || n < 0) return fail(YOCO_ERR_BAD_SHAPE, "d_model, n_q_heads and n must be positive");
  if (!head_dim_ok(head_dim)) return fail(YOCO_ERR_BAD_SHAPE, "head_dim %d is not 64 or 128", head_dim);
  if (!dtype_ok(x_dtype) || !dtype_ok(w_dtype) || !dtype_ok(q_dtype))
    return fail(YOCO_ERR_BAD_DTYPE, "x, w or q dtype unknown");
  yoco_status st = check_eps(eps);
  if (st != YOCO_OK) return st;
  if ((st = check_rope(rope)) != YOCO_OK) return st;
  if (rope.theta != 0.0) {
    if (rope.pos_host != nullptr) {
      if (n > YOCO_MAX_SEQ) return fail(YOCO_ERR_BAD_SHAPE, "a position table covers at most %d rows, got %lld",
                                        YOCO_MAX_SEQ, (long long)n);
      for (int64_t r = 0; r < n; ++r) {
        if (rope.pos_host[r] < 0) return fail(YOCO_ERR_OUT_OF_RANGE, "position %lld of row %lld is negative",
                                              (long long)rope.pos_host[r], (long long)r);
      }
    } else if (rope.pos0 < 0) {
      return fail(YOCO_ERR_OUT_OF_RANGE, "pos0 %lld is negative", (long long)rope.pos0);
    }
  }
  RowsChoice rows;
  if ((st = choose_rows_path(n, d_model, n_q_heads * head_dim, 1, w_dtype, workspace, workspace_bytes, &rows)) !=
      YOCO_OK)
    return st;
  if (n == 0) return ok();
  if ((st = check_device()) != YOCO_OK) return st;

  yoco::ProjArgs a{};
  a.x = x;
  a.gain = gain;
  a.w[0] = w_q;
  a.w[1] = nullptr;
  a.out[0] = q_out;
  a.out[1] = nullptr;
  a.n = n;
  a.dst_row_base = 0;
  a.d = d_model;
  a.ncols = n_q_heads * head_dim;
  a.out_stride = a.ncols;
  a.n_out = 1;
  a.indexed = 0;
  a.eps = eps;
  set_rope(a, rope, head_dim);
  if (rope.pos_host != nullptr) {
    // The destination rows are contiguous, so dst_rows holds the positions.
    a.pos_indexed = 1;
    a.pos_stride = 0;
    for (int64_t r = 0; r < n; ++r) a.dst_rows[r] = rope.pos_host[r];
  } else {
    a.pos_base = rope.pos0;
  }
  return launch_projection(a, rows, x_dtype, w_dtype, q_dtype, workspace, stream, "q_project");
}

}  // namespace

extern "C" {

yoco_status yoco_project_workspace(int64_t n, int32_t d_model, int32_t n_cols, int32_t n_out, int32_t w_dtype,
                                   size_t *bytes) {
  if (bytes == nullptr) return fail(YOCO_ERR_NULL_POINTER, "bytes is NULL");
  if (n < 0 || d_model < 1 || n_cols < 1 || (n_out != 1 && n_out != 2))
    return fail(YOCO_ERR_BAD_SHAPE, "n %lld, d_model %d, n_cols %d, n_out %d", (long long)n, d_model, n_cols, n_out);
  if (!dtype_ok(w_dtype)) return fail(YOCO_ERR_BAD_DTYPE, "w dtype %d unknown", w_dtype);
  yoco::ProjRowsPlan plan{};
  *bytes = (n >= 1 && n <= yoco::kProjRowsMaxRows && yoco::project_rows_plan(d_model, n_cols, n_out, w_dtype, &plan))
               ? yoco::project_rows_workspace_bytes(plan)
               : 0;
  return ok();
}

yoco_status yoco_fold_norm_gain(const void *w, int32_t w_dtype, const float *gain, int32_t d_model, int32_t n_cols,
                                void *w_out, void *stream) {
  if (w == nullptr || gain == nullptr || w_out == nullptr)
    return fail(YOCO_ERR_NULL_POINTER, "w, gain or w_out is NULL");
  if (d_model < 1 || n_cols < 1) return fail(YOCO_ERR_BAD_SHAPE, "d_model %d and n_cols %d must be >= 1", d_model, n_cols);
  if (!dtype_ok(w_dtype)) return fail(YOCO_ERR_BAD_DTYPE, "w dtype %d unknown", w_dtype);
  if (check_aligned({{w, "w"}, {gain, "gain"}, {w_out, "w_out"}}, 16) != YOCO_OK) return YOCO_ERR_ALIGNMENT;
  // In place only as the same bf16 array: any other overlap would let one
  // lane overwrite weights another lane has yet to read.
  const size_t n_elems = static_cast<size_t>(d_model) * static_cast<size_t>(n_cols);
  const uintptr_t in0 = reinterpret_cast<uintptr_t>(w), in1 = in0 + n_elems * dtype_size(w_dtype);
  const uintptr_t out0 = reinterpret_cast<uintptr_t>(w_out), out1 = out0 + n_elems * 2;
  const bool same = in0 == out0 && w_dtype == YOCO_DT_BF16;
  if (!same && in0 < out1 && out0 < in1)
    return fail(YOCO_ERR_BAD_VALUE, "w_out overlaps w (in place only as the same bf16 array)");
  yoco_status st = check_device();
  if (st != YOCO_OK) return st;
  return launched(yoco::launch_fold_gain(w, w_dtype, gain, d_model, n_cols, w_out, static_cast<hipStream_t>(stream)),
                  "fold_norm_gain");
}

yoco_status yoco_default_softmax_scale(int32_t head_dim, float *scale) {
  if (scale == nullptr) return fail(YOCO_ERR_NULL_POINTER, "scale is NULL");
  if (head_dim < 1) return fail(YOCO_ERR_BAD_SHAPE, "head_dim %d < 1", head_dim);
  *scale = static_cast<float>(1.0 / std::sqrt(static_cast<double>(head_dim)));
  return ok();
}

yoco_status yoco_kv_project(const void *m, int32_t m_dtype, int64_t n, int32_t d_model, const float *gain,
                            float eps, const void *w_k, const void *w_v, int32_t w_dtype,
                            yoco_kv_cache *cache, int32_t seq, int64_t row_start, void *workspace,
                            size_t workspace_bytes, void *stream) {
  return kv_project_impl(m, m_dtype, n, d_model, gain, eps, w_k, w_v, w_dtype, cache, seq, row_start, RopeSpec{},
                         workspace, workspace_bytes, stream);
}

yoco_status yoco_kv_project_rope(const void *m, int32_t m_dtype, int64_t n, int32_t d_model, const float *gain,
                                 float eps, const void *w_k, const void *w_v, int32_t w_dtype,
                                 yoco_kv_cache *cache, int32_t seq, int64_t row_start, double rope_theta,
                                 void *workspace, size_t workspace_bytes, void *stream) {
  RopeSpec r;
  r.theta = rope_theta;
  if (rope_theta == 0.0) return fail(YOCO_ERR_BAD_VALUE, "rope_theta must be finite and > 1");
  return kv_project_impl(m, m_dtype, n, d_model, gain, eps, w_k, w_v, w_dtype, cache, seq, row_start, r, workspace,
                         workspace_bytes, stream);
}

yoco_status yoco_kv_append(const void *m_new, int32_t m_dtype, int32_t d_model, const float *gain, float eps,
                           const void *w_k, const void *w_v, int32_t w_dtype, yoco_kv_cache *cache,
                           void *workspace, size_t workspace_bytes, void *stream) {
  return kv_append_impl(m_new, m_dtype, d_model, gain, eps, w_k, w_v, w_dtype, cache, RopeSpec{}, workspace,
                        workspace_bytes, stream);
}

yoco_status yoco_kv_append_rope(const void *m_new, int32_t m_dtype, int32_t d_model, const float *gain, float eps,
                                const void *w_k, const void *w_v, int32_t w_dtype, yoco_kv_cache *cache,
                                double rope_theta, void *workspace, size_t workspace_bytes, void *stream) {
  RopeSpec r;
  r.theta = rope_theta;
  if (rope_theta == 0.0) return fail(YOCO_ERR_BAD_VALUE, "rope_theta must be finite and > 1");
  return kv_append_impl(m_new, m_dtype, d_model, gain, eps, w_k, w_v, w_dtype, cache, r, workspace, workspace_bytes,
                        stream);
}

yoco_status yoco_q_project(const void *x, int32_t x_dtype, int64_t n, int32_t d_model, const float *gain,
                           float eps, const void *w_q, int32_t w_dtype, int32_t n_q_heads, int32_t head_dim,
                           void *q_out, int32_t q_dtype, void *workspace, size_t workspace_bytes, void *stream) {
  return q_project_impl(x, x_dtype, n, d_model, gain, eps, w_q, w_dtype, n_q_heads, head_dim, q_out, q_dtype,
                        RopeSpec{}, workspace, workspace_bytes, stream);
}

yoco_status yoco_q_project_rope(const void *x, int32_t x_dtype, int64_t n, int32_t d_model, const float *gain,
                                float eps, const void *w_q, int32_t w_dtype, int32_t n_q_heads, int32_t head_dim,
                                void *q_out, int32_t q_dtype, const int64_t *pos_host, int64_t pos0,
                                double rope_theta, void *workspace, size_t workspace_bytes, void *stream) {
  RopeSpec r;
  r.theta = rope_theta;
  r.pos_host = pos_host;
  r.pos0 = pos0;
  if (rope_theta == 0.0) return fail(YOCO_ERR_BAD_VALUE, "rope_theta must be finite and > 1");
  return q_project_impl(x, x_dtype, n, d_model, gain, eps, w_q, w_dtype, n_q_heads, head_dim, q_out, q_dtype, r,
                        workspace, workspace_bytes, stream);
}

yoco_status yoco_cross_attn_prefill(const void *q, int32_t q_dtype, int64_t q_start, int64_t t, int32_t n_q_heads,
                                    const yoco_kv_cache *cache, int32_t seq, float softmax_scale, void *o,
                                    int32_t o_dtype, float *lse, void *stream) {
  yoco_status st = check_cache(cache);
  if (st != YOCO_OK) return st;
  if (q == nullptr || o == nullptr) return fail(YOCO_ERR_NULL_POINTER, "q or o is NULL");
  if ((st = check_aligned({{q, "q"}, {o, "o"}}, 16)) != YOCO_OK) return st;
  if ((st = check_aligned({{lse, "lse"}}, 4)) != YOCO_OK) return st;
  if ((st = check_heads(n_q_heads, cache->n_kv_heads)) != YOCO_OK) return st;
  if (seq < 0 || seq >= cache->n_seq) return fail(YOCO_ERR_BAD_SHAPE, "seq %d outside [0, %d)", seq, cache->n_seq);
  if (q_dtype != cache->dtype) return fail(YOCO_ERR_BAD_DTYPE, "q dtype %d differs from cache dtype %d", q_dtype, cache->dtype);
  if (!dtype_ok(o_dtype)) return fail(YOCO_ERR_BAD_DTYPE, "o dtype %d unknown", o_dtype);
  if ((st = check_scale(softmax_scale)) != YOCO_OK) return st;
  const int64_t len = cache->len_host[seq];
  if (q_start < 0 || t < 0 || len > cache->seq_capacity || q_start > len - t)
    return fail(YOCO_ERR_OUT_OF_RANGE, "query rows at positions [%lld, %lld) exceed cache length %lld",
                (long long)q_start, (long long)(q_start + t), (long long)len);
  if (t == 0) return ok();
  if ((st = check_device()) != YOCO_OK) return st;

  const size_t esz = dtype_size(cache->dtype);
  const int64_t slab = static_cast<int64_t>(seq) * cache->seq_capacity * row_stride_of(cache);
  yoco::PrefillArgs a{};
  a.q = q;
  a.k = static_cast<const char *>(cache->k) + slab * esz;
  a.v = static_cast<const char *>(cache->v) + slab * esz;
  a.o = o;
  a.lse = lse;
  a.q_start = q_start;
  a.t = t;
  a.kv_len = len;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = cache->n_kv_heads;
  a.kv_row_stride = static_cast<int32_t>(row_stride_of(cache));
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.o_bf16 = (o_dtype == YOCO_DT_BF16) ? 1 : 0;
  return launched(yoco::launch_prefill(a, cache->dtype, cache->head_dim, static_cast<hipStream_t>(stream)),
                  "cross_attn_prefill");
}

yoco_status yoco_cross_attn_decode_workspace(const yoco_kv_cache *cache, int32_t n_q_heads, int64_t rows_per_split,
                                             size_t *bytes) {
  yoco_status st = check_cache(cache);
  if (st != YOCO_OK) return st;
  if (bytes == nullptr) return fail(YOCO_ERR_NULL_POINTER, "bytes is NULL");
  if ((st = check_heads(n_q_heads, cache->n_kv_heads)) != YOCO_OK) return st;
  if ((st = check_split_rows(rows_per_split)) != YOCO_OK) return st;
  *bytes = decode_workspace_bytes(cache, n_q_heads, max_total_splits(cache, rows_per_split));
  return ok();
}

}  // extern "C"

namespace {

// Shared by the decode with a caller's workspace and the variant that uses
// the library's static scratch (noalloc): the caller's workspace must hold
// the bound over every length up to capacity; the scratch only this call's
// split plan, within its fixed size.
yoco_status decode_impl(const void *q, int32_t q_dtype, int32_t n_q_heads, const yoco_kv_cache *cache,
                        float softmax_scale, float *o, float *lse, void *workspace, size_t workspace_bytes,
                        int64_t rows_per_split, void *stream, bool noalloc) {
  yoco_status st = check_cache(cache);
  if (st != YOCO_OK) return st;
  if (q == nullptr || o == nullptr || (!noalloc && workspace == nullptr))
    return fail(YOCO_ERR_NULL_POINTER, "q, o or workspace is NULL");
  if ((st = check_aligned({{q, "q"}, {o, "o"}, {workspace, "workspace"}}, 16)) != YOCO_OK) return st;
  if ((st = check_aligned({{lse, "lse"}}, 4)) != YOCO_OK) return st;
  if ((st = check_heads(n_q_heads, cache->n_kv_heads)) != YOCO_OK) return st;
  if (q_dtype != cache->dtype) return fail(YOCO_ERR_BAD_DTYPE, "q dtype %d differs from cache dtype %d", q_dtype, cache->dtype);
  if ((st = check_scale(softmax_scale)) != YOCO_OK) return st;
  if ((st = check_split_rows(rows_per_split)) != YOCO_OK) return st;
  for (int b = 0; b < cache->n_seq; ++b) {
    const int64_t len = cache->len_host[b];
    if (len < 1 || len > cache->seq_capacity)
      return fail(YOCO_ERR_OUT_OF_RANGE, "sequence %d: length %lld outside [1, %lld]", b, (long long)len,
                  (long long)cache->seq_capacity);
  }
  if (!noalloc) {
    const size_t bound = decode_workspace_bytes(cache, n_q_heads, max_total_splits(cache, rows_per_split));
    if (workspace_bytes < bound)
      return fail(YOCO_ERR_WORKSPACE, "workspace %zu bytes < %zu (yoco_cross_attn_decode_workspace)",
                  workspace_bytes, bound);
  }
  const int group = n_q_heads / cache->n_kv_heads;
  yoco::DecodeArgs a{};
  if (rows_per_split != 0) {
    for (int b = 0; b < cache->n_seq; ++b) a.split_rows[b] = static_cast<int32_t>(rows_per_split);
  } else {
    auto_split_plan(cache->len_host, cache->n_seq, cache->n_kv_heads,
                    decode_target_blocks(cache->dtype, cache->head_dim, group), a.split_rows);
  }
  int64_t total = 0;
  for (int b = 0; b < cache->n_seq; ++b) {
    a.split_begin[b] = static_cast<int32_t>(total);
    a.len[b] = static_cast<int32_t>(cache->len_host[b]);
    total += (cache->len_host[b] + a.split_rows[b] - 1) / a.split_rows[b];
  }
  a.split_begin[cache->n_seq] = static_cast<int32_t>(total);
  const size_t need = decode_workspace_bytes(cache, n_q_heads, total);
  if (noalloc && need > YOCO_DECODE_NOALLOC_SCRATCH_BYTES)
    return fail(YOCO_ERR_WORKSPACE,
                "this call's split plan needs %zu bytes of scratch, more than the %d the no-allocation decode has "
                "(use yoco_cross_attn_decode with a workspace, or larger rows_per_split)",
                need, YOCO_DECODE_NOALLOC_SCRATCH_BYTES);
  if (need > (noalloc ? size_t(YOCO_DECODE_NOALLOC_SCRATCH_BYTES) : workspace_bytes))
    return fail(YOCO_ERR_WORKSPACE, "split plan exceeds the workspace (internal bound violated)");
  if (total * cache->n_kv_heads > (int64_t(1) << 31) - 1)
    return fail(YOCO_ERR_BAD_VALUE, "too many splits (%lld)", (long long)total);
  if ((st = check_device()) != YOCO_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (noalloc) {
    const hipError_t e = yoco::decode_noalloc_scratch(&workspace, s);
    if (e != hipSuccess) return fail(YOCO_ERR_HIP, "no-allocation decode scratch: %s", hipGetErrorString(e));
  }

  a.k = cache->k;
  a.v = cache->v;
  a.q = q;
  a.o = o;
  a.lse = lse;
  a.counters = static_cast<unsigned int *>(workspace);
  a.part_acc = reinterpret_cast<float *>(static_cast<char *>(workspace) + YOCO_DECODE_COUNTER_BYTES);
  a.part_ml = nullptr;
  a.row_stride = row_stride_of(cache);
  a.seq_stride = cache->seq_capacity * a.row_stride;
  a.n_seq = cache->n_seq;
  a.n_kv_heads = cache->n_kv_heads;
  a.n_q_heads = n_q_heads;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.total_splits = static_cast<int32_t>(total);
  return launched(yoco::launch_decode(a, cache->dtype, cache->head_dim, group, s),
                  noalloc ? "cross_attn_decode_noalloc" : "cross_attn_decode");
}

}  // namespace

extern "C" {

yoco_status yoco_cross_attn_decode(const void *q, int32_t q_dtype, int32_t n_q_heads, const yoco_kv_cache *cache,
                                   float softmax_scale, float *o, float *lse, void *workspace,
                                   size_t workspace_bytes, int64_t rows_per_split, void *stream) {
  return decode_impl(q, q_dtype, n_q_heads, cache, softmax_scale, o, lse, workspace, workspace_bytes, rows_per_split,
                     stream, false);
}

yoco_status yoco_cross_attn_decode_noalloc(const void *q, int32_t q_dtype, int32_t n_q_heads,
                                           const yoco_kv_cache *cache, float softmax_scale, float *o, float *lse,
                                           int64_t rows_per_split, void *stream) {
  return decode_impl(q, q_dtype, n_q_heads, cache, softmax_scale, o, lse, nullptr, 0, rows_per_split, stream, true);
}


yoco_status yoco_cross_attn_prefill_bwd_workspace(int64_t t, int32_t n_q_heads, size_t *bytes) {
  if (bytes == nullptr) return fail(YOCO_ERR_NULL_POINTER, "bytes is NULL");
  if (t < 0 || n_q_heads <= 0) return fail(YOCO_ERR_BAD_SHAPE, "t %lld, n_q_heads %d", (long long)t, n_q_heads);
  *bytes = static_cast<size_t>(2 * t * n_q_heads) * sizeof(float);
  return ok();
}

yoco_status yoco_cross_attn_prefill_bwd(const void *q, const void *o, int32_t o_dtype, const void *d_o,
                                        const float *lse, int64_t q_start, int64_t t, int32_t n_q_heads,
                                        const yoco_kv_cache *cache, int32_t seq, float softmax_scale, float *d_q,
                                        float *d_k, float *d_v, void *workspace, size_t workspace_bytes,
                                        void *stream) {
  yoco_status st = check_cache(cache);
  if (st != YOCO_OK) return st;
  if (q == nullptr || o == nullptr || d_o == nullptr || lse == nullptr || d_q == nullptr || d_k == nullptr ||
      d_v == nullptr || workspace == nullptr)
    return fail(YOCO_ERR_NULL_POINTER, "q, o, d_o, lse, d_q, d_k, d_v or workspace is NULL");
  if ((st = check_aligned({{q, "q"}, {o, "o"}, {d_o, "d_o"}, {d_q, "d_q"}, {d_k, "d_k"}, {d_v, "d_v"},
                           {workspace, "workspace"}}, 16)) != YOCO_OK)
    return st;
  if ((st = check_aligned({{lse, "lse"}}, 4)) != YOCO_OK) return st;
  if ((st = check_heads(n_q_heads, cache->n_kv_heads)) != YOCO_OK) return st;
  if (seq < 0 || seq >= cache->n_seq) return fail(YOCO_ERR_BAD_SHAPE, "seq %d outside [0, %d)", seq, cache->n_seq);
  if (cache->dtype != YOCO_DT_BF16)
    return fail(YOCO_ERR_BAD_DTYPE, "the backward runs on bf16 caches (cache dtype %d)", cache->dtype);
  if (!dtype_ok(o_dtype)) return fail(YOCO_ERR_BAD_DTYPE, "o dtype %d unknown", o_dtype);
  if ((st = check_scale(softmax_scale)) != YOCO_OK) return st;
  const int64_t len = cache->len_host[seq];
  if (q_start < 0 || t < 0 || len > cache->seq_capacity || q_start > len - t)
    return fail(YOCO_ERR_OUT_OF_RANGE, "query rows at positions [%lld, %lld) exceed cache length %lld",
                (long long)q_start, (long long)(q_start + t), (long long)len);
  const size_t need = static_cast<size_t>(2 * t * n_q_heads) * sizeof(float);
  if (workspace_bytes < need)
    return fail(YOCO_ERR_WORKSPACE, "workspace %zu bytes < %zu (yoco_cross_attn_prefill_bwd_workspace)",
                workspace_bytes, need);
  if (t == 0) return ok();
  if ((st = check_device()) != YOCO_OK) return st;

  const int64_t slab = static_cast<int64_t>(seq) * cache->seq_capacity * row_stride_of(cache);
  yoco::BwdArgs a{};
  a.q = q;
  a.o = o;
  a.d_o = d_o;
  a.lse = lse;
  a.k = static_cast<const char *>(cache->k) + slab * 2;
  a.v = static_cast<const char *>(cache->v) + slab * 2;
  a.d_q = d_q;
  a.d_k = d_k;
  a.d_v = d_v;
  a.ws_d = static_cast<float *>(workspace);
  a.ws_lse2 = static_cast<float *>(workspace) + t * n_q_heads;
  a.q_start = q_start;
  a.t = t;
  a.kv_len = q_start + t;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = cache->n_kv_heads;
  a.kv_row_stride = static_cast<int32_t>(row_stride_of(cache));
  a.scale = softmax_scale;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.o_bf16 = (o_dtype == YOCO_DT_BF16) ? 1 : 0;
  return launched(yoco::launch_prefill_bwd(a, cache->head_dim, static_cast<hipStream_t>(stream)),
                  "cross_attn_prefill_bwd");
}

}  // extern "C"

namespace {

// Workspace regions of the projection backward, each 256-byte aligned.  The
// matrix-core regions are sized whenever the shapes allow that path, whatever
// the storage types, so one size serves every call with these shapes.
struct PbwdLayout {
  size_t inv_r = 0, ybf = 0, dzb[2] = {0, 0}, dw_part = 0, dgain_part = 0, total = 0;
  int32_t splits = 0, split_rows = 0;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

PbwdLayout pbwd_layout(int64_t n, int32_t d, int32_t ncols, int32_t n_out) {
  PbwdLayout L;
  size_t off = 0;
  L.inv_r = off;
  off = align256(off + static_cast<size_t>(n) * 4);
  const bool tiles = d % 256 == 0 && ncols % 256 == 0 && n > 0;
  if (tiles) {
    L.ybf = off;
    off = align256(off + static_cast<size_t>(n) * d * 2);
    for (int p = 0; p < n_out; ++p) {
      L.dzb[p] = off;
      off = align256(off + static_cast<size_t>(n) * ncols * 2);
    }
    yoco::project_bwd_split_plan(n, d, ncols, n_out, &L.splits, &L.split_rows);
    L.dw_part = off;
    off = align256(off + static_cast<size_t>(L.splits) * n_out * d * ncols * 4);
  }
  L.dgain_part = off;
  off = align256(off + static_cast<size_t>((n + yoco::kProjBwdFinRows - 1) / yoco::kProjBwdFinRows) * d * 4);
  L.total = off;
  return L;
}

yoco_status project_bwd_impl(const void *x, int32_t x_dtype, int64_t n, int32_t d_model, const float *gain,
                             float eps, const void *const w[2], int32_t w_dtype, int32_t ncols, int32_t n_out,
                             const void *const dz[2], int32_t dz_dtype, float *d_x, float *const d_w[2],
                             float *d_gain, void *workspace, size_t workspace_bytes, void *stream) {
  if (x == nullptr || d_x == nullptr || workspace == nullptr)
    return fail(YOCO_ERR_NULL_POINTER, "input, its gradient or workspace is NULL");
  for (int p = 0; p < n_out; ++p) {
    if (w[p] == nullptr || dz[p] == nullptr || d_w[p] == nullptr)
      return fail(YOCO_ERR_NULL_POINTER, "a weight, an output gradient or a weight gradient is NULL");
  }
  if (check_aligned({{x, "input"}, {gain, "gain"}, {d_x, "input gradient"}, {d_gain, "d_gain"},
                     {workspace, "workspace"}}, 16) != YOCO_OK)
    return YOCO_ERR_ALIGNMENT;
  for (int p = 0; p < n_out; ++p) {
    if (check_aligned({{w[p], "weight"}, {dz[p], "output gradient"}, {d_w[p], "weight gradient"}}, 16) != YOCO_OK)
      return YOCO_ERR_ALIGNMENT;
  }
  if (n < 0 || d_model < 1 || d_model > yoco::kProjBwdMaxD)
    return fail(YOCO_ERR_BAD_SHAPE, "n %lld must be >= 0 and d_model %d in [1, %d]", (long long)n, d_model,
                yoco::kProjBwdMaxD);
  if (!dtype_ok(x_dtype) || !dtype_ok(w_dtype) || !dtype_ok(dz_dtype))
    return fail(YOCO_ERR_BAD_DTYPE, "input, weight or gradient dtype unknown");
  yoco_status st = check_eps(eps);
  if (st != YOCO_OK) return st;
  const PbwdLayout L = pbwd_layout(n, d_model, ncols, n_out);
  if (workspace_bytes < L.total)
    return fail(YOCO_ERR_WORKSPACE, "workspace %zu bytes < %zu (yoco_project_bwd_workspace)", workspace_bytes,
                L.total);
  if (n == 0) return ok();
  if ((st = check_device()) != YOCO_OK) return st;

  char *ws = static_cast<char *>(workspace);
  yoco::ProjBwdArgs a{};
  a.x = x;
  a.gain = gain;
  a.dx = d_x;
  a.dgain = d_gain;
  for (int p = 0; p < n_out; ++p) {
    a.w[p] = w[p];
    a.dz[p] = dz[p];
    a.dw[p] = d_w[p];
  }
  a.n = n;
  a.d = d_model;
  a.ncols = ncols;
  a.n_out = n_out;
  a.x_bf16 = x_dtype == YOCO_DT_BF16;
  a.w_bf16 = w_dtype == YOCO_DT_BF16;
  a.dz_bf16 = dz_dtype == YOCO_DT_BF16;
  a.eps = eps;
  a.inv_r = reinterpret_cast<float *>(ws + L.inv_r);
  a.dgain_part = reinterpret_cast<float *>(ws + L.dgain_part);
  a.mfma = yoco::project_bwd_mfma_applies(n, d_model, ncols, x_dtype, w_dtype) ? 1 : 0;
  if (a.mfma) {
    a.ybf = reinterpret_cast<uint16_t *>(ws + L.ybf);
    for (int p = 0; p < n_out; ++p) {
      a.dzb[p] = a.dz_bf16 ? static_cast<uint16_t *>(const_cast<void *>(dz[p]))
                           : reinterpret_cast<uint16_t *>(ws + L.dzb[p]);
    }
    a.dw_part = reinterpret_cast<float *>(ws + L.dw_part);
    a.splits = L.splits;
    a.split_rows = L.split_rows;
  }
  return launched(yoco::launch_project_bwd(a, static_cast<hipStream_t>(stream)), "project_bwd");
}

}  // namespace

extern "C" {

yoco_status yoco_project_bwd_workspace(int64_t n, int32_t d_model, int32_t n_cols, int32_t n_out, size_t *bytes) {
  if (bytes == nullptr) return fail(YOCO_ERR_NULL_POINTER, "bytes is NULL");
  if (n < 0 || d_model < 1 || d_model > yoco::kProjBwdMaxD || n_cols < 1 || (n_out != 1 && n_out != 2))
    return fail(YOCO_ERR_BAD_SHAPE, "n %lld, d_model %d, n_cols %d, n_out %d", (long long)n, d_model, n_cols, n_out);
  *bytes = pbwd_layout(n, d_model, n_cols, n_out).total;
  return ok();
}

yoco_status yoco_kv_project_bwd(const void *m, int32_t m_dtype, int64_t n, int32_t d_model, const float *gain,
                                float eps, const void *w_k, const void *w_v, int32_t w_dtype, int32_t n_kv_heads,
                                int32_t head_dim, const void *dz_k, const void *dz_v, int32_t dz_dtype, float *d_m,
                                float *d_w_k, float *d_w_v, float *d_gain, void *workspace, size_t workspace_bytes,
                                void *stream) {
  if (n_kv_heads < 1 || n_kv_heads > yoco::kMaxKvHeads)
    return fail(YOCO_ERR_BAD_SHAPE, "n_kv_heads %d outside [1, %d]", n_kv_heads, yoco::kMaxKvHeads);
  if (!head_dim_ok(head_dim)) return fail(YOCO_ERR_BAD_SHAPE, "head_dim %d is not 64 or 128", head_dim);
  const void *w[2] = {w_k, w_v};
  const void *dz[2] = {dz_k, dz_v};
  float *dw[2] = {d_w_k, d_w_v};
  return project_bwd_impl(m, m_dtype, n, d_model, gain, eps, w, w_dtype, n_kv_heads * head_dim, 2, dz, dz_dtype,
                          d_m, dw, d_gain, workspace, workspace_bytes, stream);
}

yoco_status yoco_q_project_bwd(const void *x, int32_t x_dtype, int64_t n, int32_t d_model, const float *gain,
                               float eps, const void *w_q, int32_t w_dtype, int32_t n_q_heads, int32_t head_dim,
                               const void *dz_q, int32_t dz_dtype, float *d_x, float *d_w_q, float *d_gain,
                               void *workspace, size_t workspace_bytes, void *stream) {
  if (n_q_heads < 1 || n_q_heads > 4096) return fail(YOCO_ERR_BAD_SHAPE, "n_q_heads %d outside [1, 4096]", n_q_heads);
  if (!head_dim_ok(head_dim)) return fail(YOCO_ERR_BAD_SHAPE, "head_dim %d is not 64 or 128", head_dim);
  const void *w[2] = {w_q, nullptr};
  const void *dz[2] = {dz_q, nullptr};
  float *dw[2] = {d_w_q, nullptr};
  return project_bwd_impl(x, x_dtype, n, d_model, gain, eps, w, w_dtype, n_q_heads * head_dim, 1, dz, dz_dtype, d_x,
                          dw, d_gain, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// Workspace of the chunkwise gated-retention prefill, 256-byte aligned
// regions: cumulative log gates, per-group log decays, group totals and the
// states entering each group (fp32).
struct GretLayout {
  size_t lcum = 0, gdec = 0, tg = 0, sg = 0, total = 0;
};

GretLayout gret_layout(int64_t n, int32_t heads, int32_t head_dim, int32_t dtype) {
  GretLayout L;
  if (!yoco::gret_chunked_applies(dtype, head_dim) || n <= 0) return L;
  const size_t groups = static_cast<size_t>(yoco::gret_n_groups(n));
  const size_t state = static_cast<size_t>(head_dim) * head_dim;
  size_t off = 0;
  L.lcum = off;
  off = align256(off + static_cast<size_t>(n) * heads * 4);
  L.gdec = off;
  off = align256(off + groups * heads * 4);
  L.tg = off;
  off = align256(off + groups * heads * state * 4);
  L.sg = off;
  off = align256(off + groups * heads * state * 4);
  L.total = off;
  return L;
}

yoco_status check_gret(const void *q, const void *k, const void *v, const float *gate, const float *o, int32_t dtype,
                       int32_t heads, int32_t head_dim, float tau) {
  if (q == nullptr || k == nullptr || v == nullptr || gate == nullptr || o == nullptr)
    return fail(YOCO_ERR_NULL_POINTER, "q, k, v, gate_logits or o is NULL");
  if (check_aligned({{q, "q"}, {k, "k"}, {v, "v"}, {o, "o"}}, 16) != YOCO_OK) return YOCO_ERR_ALIGNMENT;
  if (check_aligned({{gate, "gate_logits"}}, 4) != YOCO_OK) return YOCO_ERR_ALIGNMENT;
  if (heads < 1 || heads > 4096) return fail(YOCO_ERR_BAD_SHAPE, "n_heads %d outside [1, 4096]", heads);
  if (!head_dim_ok(head_dim)) return fail(YOCO_ERR_BAD_SHAPE, "head_dim %d is not 64 or 128", head_dim);
  if (!dtype_ok(dtype)) return fail(YOCO_ERR_BAD_DTYPE, "dtype %d unknown", dtype);
  if (!std::isfinite(tau) || tau <= 0.f) return fail(YOCO_ERR_BAD_VALUE, "tau %g must be finite and > 0", tau);
  return YOCO_OK;
}

}  // namespace

extern "C" {

yoco_status yoco_gret_prefill_workspace(int64_t n, int32_t n_heads, int32_t head_dim, int32_t dtype, size_t *bytes) {
  if (bytes == nullptr) return fail(YOCO_ERR_NULL_POINTER, "bytes is NULL");
  if (n < 0 || n_heads < 1 || !head_dim_ok(head_dim))
    return fail(YOCO_ERR_BAD_SHAPE, "n %lld, n_heads %d, head_dim %d", (long long)n, n_heads, head_dim);
  if (!dtype_ok(dtype)) return fail(YOCO_ERR_BAD_DTYPE, "dtype %d unknown", dtype);
  *bytes = gret_layout(n, n_heads, head_dim, dtype).total;
  return ok();
}

yoco_status yoco_gret_prefill(const void *q, const void *k, const void *v, int32_t dtype, const float *gate_logits,
                              float tau, int64_t n, int32_t n_heads, int32_t head_dim, const float *state_in, float *o,
                              float *state_out, void *workspace, size_t workspace_bytes, void *stream) {
  yoco_status st = check_gret(q, k, v, gate_logits, o, dtype, n_heads, head_dim, tau);
  if (st != YOCO_OK) return st;
  if (n < 0) return fail(YOCO_ERR_BAD_SHAPE, "n %lld < 0", (long long)n);
  if ((st = check_aligned({{state_in, "state_in"}, {state_out, "state_out"}, {workspace, "workspace"}}, 16)) !=
      YOCO_OK)
    return st;
  const GretLayout L = gret_layout(n, n_heads, head_dim, dtype);
  if (L.total > 0 && (workspace == nullptr || workspace_bytes < L.total))
    return fail(YOCO_ERR_WORKSPACE, "workspace %zu bytes < %zu (yoco_gret_prefill_workspace)", workspace_bytes,
                L.total);
  if (n == 0) return ok();
  if ((st = check_device()) != YOCO_OK) return st;
  yoco::GretArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.gate = gate_logits;
  a.state_in = state_in;
  a.state_out = state_out;
  a.o = o;
  a.n_tokens = n;
  a.heads = n_heads;
  a.inv_tau = 1.0f / tau;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (L.total > 0) {
    char *ws = static_cast<char *>(workspace);
    a.lcum = reinterpret_cast<float *>(ws + L.lcum);
    a.gdec = reinterpret_cast<float *>(ws + L.gdec);
    a.tg = reinterpret_cast<float *>(ws + L.tg);
    a.sg = reinterpret_cast<float *>(ws + L.sg);
    return launched(yoco::launch_gret_chunked(a, s), "gret_prefill");
  }
  return launched(yoco::launch_gret_recurrent(a, dtype, head_dim, 1, s), "gret_prefill");
}

yoco_status yoco_gret_decode(const void *q, const void *k, const void *v, int32_t dtype, const float *gate_logits,
                             float tau, int32_t n_seq, int32_t n_heads, int32_t head_dim, float *state, float *o,
                             void *stream) {
  yoco_status st = check_gret(q, k, v, gate_logits, o, dtype, n_heads, head_dim, tau);
  if (st != YOCO_OK) return st;
  if (state == nullptr) return fail(YOCO_ERR_NULL_POINTER, "state is NULL");
  if ((st = check_aligned({{state, "state"}}, 16)) != YOCO_OK) return st;
  if (n_seq < 0 || static_cast<int64_t>(n_seq) * n_heads > 0x7fffffff)
    return fail(YOCO_ERR_BAD_SHAPE, "n_seq %d", n_seq);
  if (n_seq == 0) return ok();
  if ((st = check_device()) != YOCO_OK) return st;
  yoco::GretArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.gate = gate_logits;
  a.state_in = state;
  a.state_out = state;
  a.o = o;
  a.n_tokens = 1;
  a.heads = n_heads;
  a.inv_tau = 1.0f / tau;
  return launched(yoco::launch_gret_recurrent(a, dtype, head_dim, n_seq, static_cast<hipStream_t>(stream)),
                  "gret_decode");
}

}  // extern "C"
