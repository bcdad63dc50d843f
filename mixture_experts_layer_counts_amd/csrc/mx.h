// MXFP8 element and scale encoders shared by the quantiser, the MX gather and
// the MX epilogue of the up/gate GEMM (device code, gfx950).
#pragma once

#include "common.h"

namespace moe {

// X = floor(log2(amax)) - 8 clamped to [-127, 127]; amax == 0 (or below the
// normal range) gives -127.  Read off the fp32 exponent field.
__device__ __forceinline__ int mx_scale_exponent(float amax) {
  const int e = static_cast<int>((__float_as_uint(amax) >> 23) & 0xff);
  if (e == 0) return -127;  // zero or subnormal: floor(log2) - 8 < -127
  const int X = e - 127 - 8;  // e <= 254 (finite input) keeps X <= 119
  return X < -127 ? -127 : X;
}

// Nearest E4M3FN code of v, ties to even, saturating at +-448, sign kept.
__device__ __forceinline__ uint8_t e4m3_from_f32(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  float a = fminf(fabsf(v), 448.0f);
  uint32_t code;
  if (a < 0.015625f) {  // below 2^-6: multiples of 2^-9 (subnormals); 8 * 2^-9 is the smallest normal
    code = static_cast<uint32_t>(rintf(a * 512.0f));
  } else {
    uint32_t u = __float_as_uint(a);
    u += 0x7ffffu + ((u >> 20) & 1u);  // round to 3 mantissa bits, ties to even
    code = ((((u >> 23) & 0xffu) - 127u + 7u) << 3) | ((u >> 20) & 7u);
  }
  return static_cast<uint8_t>(code | sign);
}

}  // namespace moe
