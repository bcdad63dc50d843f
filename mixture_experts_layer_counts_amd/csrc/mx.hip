// MXFP8 quantisation on gfx950 (MoK paper "Mixture-of-Kittens: MoE Megakernel
// for NVL72s", §3.4 "MXFP8 Support": a dedicated kernel pre-quantises the
// expert weights; activation quantisation is fused into the dispatch and the
// gated activation).
//
// Format (OCP microscaling, E4M3 elements): blocks of 32 consecutive elements
// along the contraction axis share a power-of-two scale 2^X stored as the byte
// X + 127 (E8M0), X = floor(log2(amax)) - 8 (8 = exponent of the largest E4M3
// normal, 448 = 1.75 * 2^8), clamped to [-127, 127]; an all-zero block has
// X = -127.  Each element v / 2^X is rounded to the nearest E4M3FN value, ties
// to even, saturating at +-448; the sign is kept when the value rounds to 0.
// The rounding is done in integer arithmetic on the fp32 bits, so the result
// does not depend on any hardware conversion mode.

#include "common.h"
#include "kernels.h"
#include "mx.h"

namespace moe {

// One block of 32 bf16 values (64 bytes at `src`) -> 32 E4M3 bytes (in two
// 16-byte words) and the E8M0 scale byte (returned).
__device__ __forceinline__ uint8_t quantize_block32_words(const uint16_t* __restrict__ src, u32x4_t& lo,
                                                          u32x4_t& hi) {
  const u32x4_t* s = reinterpret_cast<const u32x4_t*>(src);
  float v[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4_t w = s[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * i + 2 * j] = __uint_as_float(w[j] << 16);
      v[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
  }
  return quantize32_f32(v, lo, hi);
}

__device__ __forceinline__ void quantize_block32(const uint16_t* __restrict__ src, uint8_t* __restrict__ q,
                                                 uint8_t* __restrict__ scale) {
  u32x4_t lo, hi;
  *scale = quantize_block32_words(src, lo, hi);
  u32x4_t* d = reinterpret_cast<u32x4_t*>(q);
  d[0] = lo;
  d[1] = hi;
}

__global__ __launch_bounds__(256) void quantize_mxfp8_kernel(const uint16_t* __restrict__ src, int64_t blocks,
                                                             uint8_t* __restrict__ q, uint8_t* __restrict__ scale) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= blocks) return;
  quantize_block32(src + i * 32, q + i * 32, scale + i);
}

hipError_t launch_quantize_mxfp8(const uint16_t* src, int64_t rows, int64_t K, uint8_t* q, uint8_t* scale,
                                 hipStream_t stream) {
  const int64_t blocks = rows * (K / 32);
  if (blocks <= 0) return hipSuccess;
  if ((blocks + 255) / 256 > 0x7fffffff) return hipErrorInvalidValue;
  quantize_mxfp8_kernel<<<static_cast<unsigned>((blocks + 255) / 256), 256, 0, stream>>>(src, blocks, q, scale);
  return hipGetLastError();
}

// Rows quantised with their scales written stage-major ([K/128][rows][4], the
// layout the MX GEMMs read activation scales in): one thread per 32-element
// block, the same encoder as above.
__global__ __launch_bounds__(256) void quantize_rows_mx_staged_kernel(const uint16_t* __restrict__ src, int64_t rows,
                                                                      int64_t K, uint8_t* __restrict__ q,
                                                                      uint8_t* __restrict__ scale) {
  const int64_t nb = K / 32;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= rows * nb) return;
  const int64_t row = i / nb, blk = i % nb;
  quantize_block32(src + i * 32, q + i * 32, scale + ((blk >> 2) * rows + row) * 4 + (blk & 3));
}

hipError_t launch_quantize_rows_mx_staged(const uint16_t* src, int64_t rows, int64_t K, uint8_t* q, uint8_t* scale,
                                          hipStream_t stream) {
  if (K % 128 != 0) return hipErrorInvalidValue;
  const int64_t blocks = rows * (K / 32);
  if (blocks <= 0) return hipSuccess;
  if ((blocks + 255) / 256 > 0x7fffffff) return hipErrorInvalidValue;
  quantize_rows_mx_staged_kernel<<<static_cast<unsigned>((blocks + 255) / 256), 256, 0, stream>>>(src, rows, K, q,
                                                                                                  scale);
  return hipGetLastError();
}

// Scale words into the layout the MX GEMM reads: row-major [groups][rows][K/32]
// -> stage-major [groups][K/128][rows][4] (one 4-byte word per row and 128-wide
// K stage; one thread moves one word).
__global__ __launch_bounds__(256) void pack_mx_scales_kernel(const uint32_t* __restrict__ src, int64_t words,
                                                             int64_t rows, int64_t stages,
                                                             uint32_t* __restrict__ dst) {
  const int64_t w = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (w >= words) return;
  const int64_t per_group = stages * rows;
  const int64_t g = w / per_group, rem = w - g * per_group;
  const int64_t st = rem / rows, r = rem - st * rows;
  dst[w] = src[(g * rows + r) * stages + st];
}

hipError_t launch_pack_mx_scales(const uint8_t* scale, int64_t groups, int64_t rows, int64_t K, uint8_t* packed,
                                 hipStream_t stream) {
  if (K % 128 != 0 || reinterpret_cast<uintptr_t>(scale) % 4 || reinterpret_cast<uintptr_t>(packed) % 4)
    return hipErrorInvalidValue;
  const int64_t stages = K / 128, words = groups * rows * stages;
  if (words <= 0) return hipSuccess;
  if ((words + 255) / 256 > 0x7fffffff) return hipErrorInvalidValue;
  pack_mx_scales_kernel<<<static_cast<unsigned>((words + 255) / 256), 256, 0, stream>>>(
      reinterpret_cast<const uint32_t*>(scale), words, rows, stages, reinterpret_cast<uint32_t*>(packed));
  return hipGetLastError();
}

// MX gather (§3.4: the activation quantisation rides on the dispatch).  As the
// bf16 gather, schedule position p reads source row sched_src[p] / k and fills
// ring slot p mod C, here as E4M3 bytes [C][D] and stage-major scale bytes
// [D/128][C][4] (the layout the MX GEMM reads); one thread quantises one
// 32-element block.
__global__ __launch_bounds__(256) void gather_mx_kernel(const uint16_t* __restrict__ x_src, int64_t src_rows, int D,
                                                        int k, const int32_t* __restrict__ sched_src,
                                                        const int32_t* __restrict__ offsets, int L, int64_t p_begin,
                                                        int64_t rows, int64_t ring_rows, uint8_t* __restrict__ ring_q,
                                                        uint8_t* __restrict__ ring_s, int* err) {
  const int nb = D / 32;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= rows * nb) return;
  const int64_t p = p_begin + i / nb;
  const int blk = static_cast<int>(i % nb);
  if (p >= offsets[L]) return;
  const int32_t route = sched_src[p];
  const int64_t src_row = route / k;
  if (route < 0 || src_row >= src_rows) {  // a table not built by the schedule kernels
    if (blk == 0) raise_error(err, kErrExpertRange);
    return;
  }
  const int64_t slot = p % ring_rows;
  quantize_block32(x_src + src_row * D + blk * 32, ring_q + slot * D + blk * 32,
                   ring_s + ((blk >> 2) * ring_rows + slot) * 4 + (blk & 3));
}

hipError_t launch_gather_mx(const uint16_t* x_src, int64_t src_rows, int D, int k, const int32_t* sched_src,
                            const int32_t* offsets, int L, int64_t p_begin, int64_t rows, int64_t ring_rows,
                            uint8_t* ring_q, uint8_t* ring_s, int* err, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  if (D % 128 != 0) return hipErrorInvalidValue;
  const int64_t n = rows * (D / 32);
  if ((n + 255) / 256 > 0x7fffffff) return hipErrorInvalidValue;
  gather_mx_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, stream>>>(
      x_src, src_rows, D, k, sched_src, offsets, L, p_begin, rows, ring_rows, ring_q, ring_s, err);
  return hipGetLastError();
}

// MX gather from the source side (R = 1, one minibatch holding every routed
// row): one thread quantises one 32-element block of a token once and writes
// it to the ring slots of the token's k routes.
__global__ __launch_bounds__(256) void gather_src_mx_kernel(const uint16_t* __restrict__ x, int T, int D, int k,
                                                            const int32_t* __restrict__ route_dst, int64_t P,
                                                            int64_t ring_rows, uint8_t* __restrict__ ring_q,
                                                            uint8_t* __restrict__ ring_s, int* err) {
  const int nb = D / 32;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= static_cast<int64_t>(T) * nb) return;
  const int64_t t = i / nb;
  const int blk = static_cast<int>(i % nb);
  u32x4_t lo, hi;
  const uint8_t sc = quantize_block32_words(x + t * D + blk * 32, lo, hi);
  for (int s = 0; s < k; ++s) {
    const int32_t p = route_dst[t * k + s];
    if (p < 0 || p >= P) {  // a table not built by the schedule kernels
      if (blk == 0) raise_error(err, kErrExpertRange);
      continue;
    }
    const int64_t slot = p % ring_rows;
    u32x4_t* d = reinterpret_cast<u32x4_t*>(ring_q + slot * D + blk * 32);
    d[0] = lo;
    d[1] = hi;
    ring_s[((blk >> 2) * ring_rows + slot) * 4 + (blk & 3)] = sc;
  }
}

hipError_t launch_gather_src_mx(const uint16_t* x, int T, int D, int k, const int32_t* route_dst, int64_t P,
                                int64_t ring_rows, uint8_t* ring_q, uint8_t* ring_s, int* err, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  if (D % 128 != 0) return hipErrorInvalidValue;
  const int64_t n = static_cast<int64_t>(T) * (D / 32);
  if ((n + 255) / 256 > 0x7fffffff) return hipErrorInvalidValue;
  gather_src_mx_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, stream>>>(x, T, D, k, route_dst, P,
                                                                                   ring_rows, ring_q, ring_s, err);
  return hipGetLastError();
}

}  // namespace moe
