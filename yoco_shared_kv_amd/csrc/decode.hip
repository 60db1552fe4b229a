// Launchers for the split-N decode kernel (the kernel itself is in
// decode_kernel.h).  Tuning per storage type: 8 waves per workgroup, each
// lane owning 8 elements of a head row (bf16: one 16-byte load per row),
// 8 passes per tile for bf16 and 4 for fp32, no register double buffering;
// measured on MI355X as the fastest of the swept shapes for the 128 Ki-row
// workload when the grid is one resident round.
#include <atomic>
#include <mutex>

#include "decode_kernel.h"

namespace yoco {

// Scratch of the decode variant that allocates nothing
// (yoco_cross_attn_decode_noalloc): arrival counters, then partial rows,
// laid out as the caller's workspace of yoco_cross_attn_decode.  Each device
// holds its own copy until the process ends.  Host code never uses the
// array's name as an address (on the host it is only a stand-in): the
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[YOCO_DECODE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kScratchDevices = 64;
std::atomic<void *> g_scratch_ptr[kScratchDevices];
std::mutex g_scratch_mutex;

__global__ void zero_words_kernel(unsigned int *p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}
}  // namespace

hipError_t decode_noalloc_scratch(void **ptr, hipStream_t s) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      // The counters must start at zero (every completed call leaves them
      // zero): clear them once, in stream order before the first decode,
      // with a kernel rather than a memset (a caller may be capturing the
      // stream into a graph).
      const int words = YOCO_DECODE_COUNTER_BYTES / 4;
      hipLaunchKernelGGL(zero_words_kernel, dim3((words + 255) / 256), dim3(256), 0, s,
                         static_cast<unsigned int *>(p), words);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

template <typename T>
using ProdTune = DecodeTune<8, 8, (sizeof(T) == 2 ? 8 : 4), false>;

template <typename T, int DH, int G>
static hipError_t launch_decode_t(const DecodeArgs &a, hipStream_t s) {
  using C = DecodeCfg<T, DH, G, ProdTune<T>>;
  const unsigned int blocks = static_cast<unsigned int>(a.total_splits) * a.n_kv_heads;
  hipLaunchKernelGGL((decode_kernel<T, DH, G, ProdTune<T>>), dim3(blocks), dim3(C::NT), 0, s, a);
  return hipGetLastError();
}

template <typename T, int DH, int G>
static int occupancy_t() {
  using C = DecodeCfg<T, DH, G, ProdTune<T>>;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_kernel<T, DH, G, ProdTune<T>>, C::NT, 0) !=
      hipSuccess)
    return 0;
  return n;
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

template <typename T, int DH>
static int occupancy_g(int group) {
  switch (group) {
    case 1: return occupancy_t<T, DH, 1>();
    case 2: return occupancy_t<T, DH, 2>();
    case 3: return occupancy_t<T, DH, 3>();
    case 4: return occupancy_t<T, DH, 4>();
    case 6: return occupancy_t<T, DH, 6>();
    case 8: return occupancy_t<T, DH, 8>();
    default: return 0;
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

int decode_blocks_per_cu(int dtype, int head_dim, int group) {
  if (dtype == YOCO_DT_BF16) {
    if (head_dim == 128) return occupancy_g<bf16_t, 128>(group);
    if (head_dim == 64) return occupancy_g<bf16_t, 64>(group);
  } else if (dtype == YOCO_DT_F32) {
    if (head_dim == 128) return occupancy_g<float, 128>(group);
    if (head_dim == 64) return occupancy_g<float, 64>(group);
  }
  return 0;
}

}  // namespace yoco
