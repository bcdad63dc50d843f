// Shared device helpers of the gfx950 MoE kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));  // 16-byte chunk held in registers

constexpr int kWave = 64;

// Device error bits (same values as MOE_DEVERR_* in include/moe.h).
constexpr int kErrExpertRange = 0x1;
constexpr int kErrRowOverflow = 0x2;
constexpr int kErrNonFinite = 0x4;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest even (NaN kept quiet).  Both results are
// formed and one selected, so that unrolled epilogues carry no branches.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t rne = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  const uint32_t qnan = (u >> 16) | 0x40u;
  return static_cast<uint16_t>((u & 0x7fffffffu) > 0x7f800000u ? qnan : rne);
}

// SiLU(g) * u, with the hardware reciprocal (about 1 ulp) in place of a
// correctly rounded division: the result is rounded to bf16 or E4M3 next.
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

__device__ __forceinline__ void raise_error(int* err, int bits) {
  if (err) atomicOr(err, bits);
}

__device__ __forceinline__ int lane_id() { return static_cast<int>(threadIdx.x) & (kWave - 1); }

}  // namespace moe
