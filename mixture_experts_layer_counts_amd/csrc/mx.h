// MXFP8 element and scale encoders shared by the quantiser, the MX gather and
// the MX epilogue of the up/gate GEMM (device code, gfx950).
#pragma once

#include "common.h"

namespace moe {

// X = floor(log2(amax)) - 8 clamped to [-127, 127]; amax == 0 (or below the
// normal range) gives -127.  Read off the fp32 exponent field.
__device__ __forceinline__ int mx_scale_exponent(float amax) {
  // a zero or subnormal amax (exponent field 0) lands below -127 and is clamped
  // there; a finite amax has field <= 254, so X <= 119
  const int e = static_cast<int>((__float_as_uint(amax) >> 23) & 0xff);
  return max(e - 127 - 8, -127);
}

// Nearest E4M3FN code of v, ties to even, saturating at +-448, sign kept.
// The subnormal and the normal code are both formed and one is selected, so
// that unrolled loops over many elements carry no branches.
__device__ __forceinline__ uint8_t e4m3_from_f32(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fminf(fabsf(v), 448.0f);
  // below 2^-6: multiples of 2^-9 (subnormals); 8 * 2^-9 is the smallest normal
  const uint32_t sub = static_cast<uint32_t>(rintf(a * 512.0f));
  uint32_t u = __float_as_uint(a);
  u += 0x7ffffu + ((u >> 20) & 1u);  // round to 3 mantissa bits, ties to even
  const uint32_t nrm = ((((u >> 23) & 0xffu) - 127u + 7u) << 3) | ((u >> 20) & 7u);
  return static_cast<uint8_t>((a < 0.015625f ? sub : nrm) | sign);
}

// One 32-element block, fp32 -> 32 E4M3 bytes (two 16-byte words, element i
// in byte i) and the E8M0 scale byte (returned).
__device__ __forceinline__ uint8_t quantize32_f32(const float (&v)[32], u32x4_t& lo, u32x4_t& hi) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int X = mx_scale_exponent(amax);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) word |= static_cast<uint32_t>(e4m3_from_f32(ldexpf(v[4 * i + j], -X))) << (8 * j);
    if (i < 4)
      lo[i] = word;
    else
      hi[i - 4] = word;
  }
  return static_cast<uint8_t>(X + 127);
}

}  // namespace moe
