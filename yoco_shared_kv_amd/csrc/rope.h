// Rotary position embedding in the projection epilogues.
//
// What it computes ([Blog] "NeurIPS'24 | YOCO: 长上下文 LLM 为什么不必每层都存一份
// KV Cache?" s.7: the shared projection rotates K^ by position and each cross
// layer rotates its own Q; V is not rotated.  [Notes] "YOCO：You Only Cache
// Once 中文精读笔记" s.4.3, Table 7: the base theta of each training stage):
// pair i of a head, elements (2i, 2i+1), turns by pos * theta^(-2i/head_dim)
// radians, i.e. pos * rev_i turns with rev_i = theta^(-2i/head_dim) / (2 pi).
//
// Precision: the turn count pos * rev_i is formed in double precision and
// reduced to its fraction in [-1/2, 1/2] there (positions reach 2^20 and more,
// where a single-precision angle would be off by hundredths of a radian);
// the sine and cosine of the fraction come from v_sin_f32 / v_cos_f32, whose
// input is in turns; the rotation is applied to the fp32 projection result
// before it is rounded to the output type.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace yoco {

// Turns per position of pair i of a head.
__device__ __forceinline__ double rope_rev(int i, int head_dim, double log2_theta) {
  return exp2(-(2.0 * i / head_dim) * log2_theta) * 0.15915494309189535;  // 1 / (2 pi)
}

// (x0, x1) <- rotation of (x0, x1) by pos * rev turns.
__device__ __forceinline__ void rope_turn(float &x0, float &x1, int64_t pos, double rev) {
  const double turns = static_cast<double>(pos) * rev;
  const float frac = static_cast<float>(turns - rint(turns));
  const float s = __builtin_amdgcn_sinf(frac);
  const float c = __builtin_amdgcn_cosf(frac);
  const float a = x0;
  const float b = x1;
  x0 = a * c - b * s;
  x1 = a * s + b * c;
}

}  // namespace yoco
