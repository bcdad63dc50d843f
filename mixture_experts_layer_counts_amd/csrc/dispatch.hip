// Token movement on gfx950: gather into the ring buffer, and the combine.
//
// Gather (MoK paper "Mixture-of-Kittens: MoE Megakernel for NVL72s", §3.1
// "Scheduling": dispatch walks the schedule table row by row, and rows land
// directly in expert-contiguous buffer positions, with no other local copy;
// §3.3: the destination is a fixed-size ring buffer).  Position p of the
// schedule reads source row sched_src[p] / k and fills ring slot p mod C.
// One wave copies one 2*D-byte row with 16-byte loads and stores.
//
// Combine (§2.1 MoE equation, router-weighted sum; §3.4 "Determinism": no
// atomics, a fixed order): out32[t] = (sum over s in slot order of
// fma(g[t,s], y[t,s], .)) + shared[t], in fp32; out = bf16(out32).

#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace moe {

__global__ __launch_bounds__(256) void gather_kernel(const uint16_t* __restrict__ x_src, int64_t src_rows, int D,
                                                     int k, const int32_t* __restrict__ sched_src,
                                                     const int32_t* __restrict__ offsets, int L, int64_t p_begin,
                                                     int64_t rows, int64_t ring_rows, uint16_t* __restrict__ ring,
                                                     int* err) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / kWave;
  if (i >= rows) return;
  const int64_t p = p_begin + i;
  if (p >= offsets[L]) return;
  const int32_t route = sched_src[p];
  const int64_t src_row = route / k;
  if (route < 0 || src_row >= src_rows) {  // a table not built by the schedule kernels
    if (lane_id() == 0) raise_error(err, kErrExpertRange);
    return;
  }
  const uint4* __restrict__ s = reinterpret_cast<const uint4*>(x_src + src_row * D);
  uint4* __restrict__ d = reinterpret_cast<uint4*>(ring + (p % ring_rows) * D);
  const int n = D / 8;
  for (int c = lane_id(); c < n; c += kWave) d[c] = s[c];
}

hipError_t launch_gather(const uint16_t* x_src, int64_t src_rows, int D, int k, const int32_t* sched_src,
                         const int32_t* offsets, int L, int64_t p_begin, int64_t rows, int64_t ring_rows,
                         uint16_t* ring, int* err, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  gather_kernel<<<static_cast<unsigned>((rows + 3) / 4), 256, 0, stream>>>(x_src, src_rows, D, k, sched_src, offsets,
                                                                           L, p_begin, rows, ring_rows, ring, err);
  return hipGetLastError();
}

// The same placement walked from the source side, for one GPU (R = 1) when a
// single minibatch holds every routed row: one block per token reads the row
// once and writes it to the ring slots of the token's k routes (route_dst is
// the inverse of the schedule table), instead of reading it k times.
__global__ __launch_bounds__(256) void gather_src_kernel(const uint16_t* __restrict__ x, int T, int D, int k,
                                                         const int32_t* __restrict__ route_dst, int64_t P,
                                                         int64_t ring_rows, uint16_t* __restrict__ ring, int* err) {
  __shared__ int32_t slot_s[16];  // ring slot of each route (< ring_rows), or -1
  const int t = blockIdx.x, tid = threadIdx.x;
  if (tid < k) {
    const int32_t p = route_dst[static_cast<int64_t>(t) * k + tid];
    const bool ok = p >= 0 && p < P;
    if (!ok) raise_error(err, kErrExpertRange);  // a table not built by the schedule kernels
    slot_s[tid] = ok ? static_cast<int32_t>(p % ring_rows) : -1;
  }
  __syncthreads();
  int32_t slot[16];
#pragma unroll
  for (int s = 0; s < 16; ++s) slot[s] = s < k ? slot_s[s] : -1;
  const uint4* __restrict__ src = reinterpret_cast<const uint4*>(x + static_cast<int64_t>(t) * D);
  const int n = D / 8;
  for (int c = tid; c < n; c += 256) {
    const uint4 v = src[c];
#pragma unroll
    for (int s = 0; s < 16; ++s)
      if (slot[s] >= 0) reinterpret_cast<uint4*>(ring + static_cast<int64_t>(slot[s]) * D)[c] = v;
  }
}

hipError_t launch_gather_src(const uint16_t* x, int T, int D, int k, const int32_t* route_dst, int64_t P,
                             int64_t ring_rows, uint16_t* ring, int* err, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  if (k > 16) return hipErrorInvalidValue;
  gather_src_kernel<<<static_cast<unsigned>(T), 256, 0, stream>>>(x, T, D, k, route_dst, P, ring_rows, ring, err);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ Y, const float* __restrict__ sh,
                                                      const float* __restrict__ gate,
                                                      const int32_t* __restrict__ route_dst, int64_t route_base,
                                                      int D, int k, int by_route_dst, uint16_t* __restrict__ out,
                                                      float* __restrict__ out32) {
  __shared__ int64_t row_s[16];
  __shared__ float g_s[16];
  const int t = blockIdx.x, tid = threadIdx.x;
  if (tid < k) {
    const int64_t j = static_cast<int64_t>(t) * k + tid;
    g_s[tid] = gate[j];
    row_s[tid] = by_route_dst ? static_cast<int64_t>(route_dst[route_base + j]) : j;
  }
  __syncthreads();
  // Y rows are read once and the outputs are not read again here, so both
  // go through non-temporal loads and stores (measured 9% faster than the
  // default cache policy at the DeepSeek-V3 shape)
  for (int c = tid * 8; c < D; c += 256 * 8) {
    // every load of this chunk is issued before the fixed-order sum uses them
    u32x4_t y[16];
#pragma unroll
    for (int s = 0; s < 16; ++s)
      if (s < k && row_s[s] >= 0) y[s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(Y + row_s[s] * D + c));
    const float4* shp = reinterpret_cast<const float4*>(sh + static_cast<int64_t>(t) * D + c);
    const float4 s0 = shp[0], s1 = shp[1];
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      // a route to a remote expert (row < 0) is summed where its row returns
      if (s >= k || row_s[s] < 0) continue;
      const float g = g_s[s];
      const uint32_t w[4] = {y[s][0], y[s][1], y[s][2], y[s][3]};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = fmaf(g, __uint_as_float(w[i] << 16), acc[2 * i]);
        acc[2 * i + 1] = fmaf(g, __uint_as_float(w[i] & 0xffff0000u), acc[2 * i + 1]);
      }
    }
    acc[0] += s0.x;
    acc[1] += s0.y;
    acc[2] += s0.z;
    acc[3] += s0.w;
    acc[4] += s1.x;
    acc[5] += s1.y;
    acc[6] += s1.z;
    acc[7] += s1.w;
    const u32x4_t o = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
                       pack_bf16x2(acc[6], acc[7])};
    __builtin_nontemporal_store(o, reinterpret_cast<u32x4_t*>(out + static_cast<int64_t>(t) * D + c));
    if (out32) {
      f32x4_t* o32 = reinterpret_cast<f32x4_t*>(out32 + static_cast<int64_t>(t) * D + c);
      __builtin_nontemporal_store(f32x4_t{acc[0], acc[1], acc[2], acc[3]}, o32);
      __builtin_nontemporal_store(f32x4_t{acc[4], acc[5], acc[6], acc[7]}, o32 + 1);
    }
  }
}

hipError_t launch_combine(const uint16_t* Y, const float* shared_out, const float* gate, const int32_t* route_dst,
                          int64_t route_base, int T, int D, int k, bool by_route_dst, uint16_t* out, float* out32,
                          hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  combine_kernel<<<T, 256, 0, stream>>>(Y, shared_out, gate, route_dst, route_base, D, k, by_route_dst ? 1 : 0,
                                        out, out32);
  return hipGetLastError();
}

// K-tiling of bf16 matrices [groups][rows][K] -> [groups][K/64][rows][64]:
// one 16-byte chunk (eight elements) per thread and step; eight consecutive
// threads read 128 contiguous bytes of a row and write one whole 128-byte
// line of a plane.
__global__ __launch_bounds__(256) void tile_bf16_kernel(const uint16_t* __restrict__ src, int64_t rows, int64_t K,
                                                        int64_t chunks, uint16_t* __restrict__ dst,
                                                        int64_t plane_rows, int64_t row0, int64_t group_stride) {
  const int64_t per_row = K / 8, per_group = rows * per_row;
  for (int64_t q = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; q < chunks;
       q += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t g = q / per_group, rem = q - g * per_group;
    const int64_t r = rem / per_row, c = rem - r * per_row;
    const int64_t to = g * group_stride + ((c / 8) * plane_rows + row0 + r) * kTileK + (c % 8) * 8;
    *reinterpret_cast<uint4*>(dst + to) = *reinterpret_cast<const uint4*>(src + q * 8);
  }
}

hipError_t launch_tile_bf16(const uint16_t* src, int64_t groups, int64_t rows, int64_t K, uint16_t* dst,
                            hipStream_t stream, int64_t plane_rows, int64_t row0, int64_t group_stride) {
  if (groups <= 0 || rows <= 0 || K <= 0 || K % kTileK) return hipErrorInvalidValue;
  if (plane_rows == 0) plane_rows = rows;
  if (group_stride == 0) group_stride = plane_rows * K;
  if (row0 < 0 || row0 + rows > plane_rows || group_stride < plane_rows * K) return hipErrorInvalidValue;
  const int64_t chunks = groups * rows * (K / 8);
  const int64_t blocks = std::min<int64_t>((chunks + 255) / 256, 65536);
  tile_bf16_kernel<<<static_cast<unsigned>(blocks), 256, 0, stream>>>(src, rows, K, chunks, dst, plane_rows, row0,
                                                                      group_stride);
  return hipGetLastError();
}

__global__ void clear_int_kernel(int* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

hipError_t launch_clear_int(int* p, int n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  clear_int_kernel<<<(n + 255) / 256, 256, 0, stream>>>(p, n);
  return hipGetLastError();
}

}  // namespace moe
