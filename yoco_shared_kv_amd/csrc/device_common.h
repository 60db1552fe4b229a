// Device helpers for gfx950: bf16 packing, DPP reductions, 16-byte loads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace yoco {

typedef uint16_t bf16_t;  // raw bfloat16 bits

__device__ __forceinline__ float bf16_lo(uint32_t packed) {
  return __uint_as_float(packed << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t packed) {
  return __uint_as_float(packed & 0xffff0000u);
}
__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 with round-to-nearest-even (finite inputs; NaN stays NaN).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// --- DPP lane exchange (all 64 lanes active) --------------------------------
// dpp_ctrl encodings (GCN/CDNA DPP): quad_perm = p0|p1<<2|p2<<4|p3<<6,
// row_mirror = 0x140, row_half_mirror = 0x141.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int kDppQuadXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;  // lane i <-> 7-i within 8
constexpr int kDppRowMirror = 0x140;      // lane i <-> 15-i within 16

// Sum over aligned groups of N lanes (N = 4, 8 or 16); every lane of the
// group receives the group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 4 || N == 8 || N == 16, "group of 4, 8 or 16 lanes");
  x += dpp<kDppQuadXor1>(x);
  x += dpp<kDppQuadXor2>(x);
  if constexpr (N >= 8) x += dpp<kDppRowHalfMirror>(x);
  if constexpr (N >= 16) x += dpp<kDppRowMirror>(x);
  return x;
}

__device__ __forceinline__ float shfl_xor_f(float x, int mask) {
  return __shfl_xor(x, mask, 64);
}

// 16-byte global load / store.
__device__ __forceinline__ uint4 ld16(const void *p) {
  return *reinterpret_cast<const uint4 *>(p);
}
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_stream(const void *p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Eight consecutive elements (16 B of bf16 or 32 B of fp32) as fp32.
template <typename T>
struct Vec8;

template <>
struct Vec8<bf16_t> {
  uint4 raw;
  __device__ __forceinline__ void load(const bf16_t *p) { raw = ld16_stream(p); }
  __device__ __forceinline__ void zero() { raw = make_uint4(0, 0, 0, 0); }
  __device__ __forceinline__ float operator[](int i) const {
    uint32_t w = (i < 2) ? raw.x : (i < 4) ? raw.y : (i < 6) ? raw.z : raw.w;
    return (i & 1) ? bf16_hi(w) : bf16_lo(w);
  }
};

template <>
struct Vec8<float> {
  uint4 raw[2];
  __device__ __forceinline__ void load(const float *p) {
    raw[0] = ld16_stream(p);
    raw[1] = ld16_stream(p + 4);
  }
  __device__ __forceinline__ void zero() {
    raw[0] = make_uint4(0, 0, 0, 0);
    raw[1] = raw[0];
  }
  __device__ __forceinline__ float operator[](int i) const {
    const uint4 &r = raw[i >> 2];
    uint32_t w = ((i & 3) == 0) ? r.x : ((i & 3) == 1) ? r.y : ((i & 3) == 2) ? r.z : r.w;
    return __uint_as_float(w);
  }
};

template <typename T>
__device__ __forceinline__ float load_elem(const T *p);
template <>
__device__ __forceinline__ float load_elem<float>(const float *p) { return *p; }
template <>
__device__ __forceinline__ float load_elem<bf16_t>(const bf16_t *p) { return bf16_to_f32(*p); }

template <typename T>
__device__ __forceinline__ void store_elem(T *p, float v);
template <>
__device__ __forceinline__ void store_elem<float>(float *p, float v) { *p = v; }
template <>
__device__ __forceinline__ void store_elem<bf16_t>(bf16_t *p, float v) { *p = f32_to_bf16(v); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace yoco
