// The memory-bound kernels of the MoE-layer backward pass on gfx950 (the
// GEMMs are gemm.hip's).
//
// MoK paper "Mixture-of-Kittens: MoE Megakernel for NVL72s": the backward
// walks the forward's dispatch table in reverse (§3.1: the same table serves
// both directions), replays the up/gate projections instead of keeping their
// outputs (§3.3 "Ring-Aware Forward Replay"), and takes the router-weight
// gradient from the gate gradients <dout, y> (§3.4 "Router Weight Gradient
// Computation").  With g_s the renormalised gate of slot s of a token:
//   dY[p]   = g dout[t]                  ring row p of route (t, s)
//   dg[t,s] = <dout[t], y[t,s]>          y the routed row the forward stored
//   dl[t,s] = g_s (dg_s - sum g dg)      the selected logits' gradient
//   h = SiLU(a_g) a_u,  da_g = dh a_u SiLU'(a_g),  da_u = dh SiLU(a_g)
//   dx[t]   = dx_shared[t] + dx_router[t] + sum_s dx_ring[route_dst[t k + s]]
// All sums run in a fixed order; no floating-point atomics.

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

// One wave per ring row: dY[p] = bf16(g * dout[t]) for the route sched_src[p].
__global__ __launch_bounds__(256) void dy_gather_kernel(const uint16_t* __restrict__ dout, const float* __restrict__ gate,
                                                        const int32_t* __restrict__ sched_src, int64_t P, int T, int D,
                                                        int k, uint16_t* __restrict__ dy, int* err) {
  const int64_t p = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / kWave;
  if (p >= P) return;
  const int32_t j = sched_src[p];
  if (j < 0 || j / k >= T) {
    if (lane_id() == 0) raise_error(err, kErrExpertRange);
    return;
  }
  const float g = gate[j];
  const uint16_t* __restrict__ src = dout + static_cast<int64_t>(j / k) * D;
  uint16_t* __restrict__ dst = dy + p * D;
  auto scale = [g](const u32x4_t& v) {
    u32x4_t o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float lo = g * bf16_to_f32(static_cast<uint16_t>(v[q] & 0xffffu));
      const float hi = g * bf16_to_f32(static_cast<uint16_t>(v[q] >> 16));
      o[q] = pack_bf16x2(lo, hi);
    }
    return o;
  };
  constexpr int kStep = kWave * 8;  // elements one pass of the wave covers
  int c = lane_id() * 8;
  // four 16-byte loads in flight per lane, then their stores; the row's last
  // chunks one at a time
  for (; c + 3 * kStep < D; c += 4 * kStep) {
    const u32x4_t v0 = *reinterpret_cast<const u32x4_t*>(src + c);
    const u32x4_t v1 = *reinterpret_cast<const u32x4_t*>(src + c + kStep);
    const u32x4_t v2 = *reinterpret_cast<const u32x4_t*>(src + c + 2 * kStep);
    const u32x4_t v3 = *reinterpret_cast<const u32x4_t*>(src + c + 3 * kStep);
    *reinterpret_cast<u32x4_t*>(dst + c) = scale(v0);
    *reinterpret_cast<u32x4_t*>(dst + c + kStep) = scale(v1);
    *reinterpret_cast<u32x4_t*>(dst + c + 2 * kStep) = scale(v2);
    *reinterpret_cast<u32x4_t*>(dst + c + 3 * kStep) = scale(v3);
  }
  for (; c < D; c += kStep) *reinterpret_cast<u32x4_t*>(dst + c) = scale(*reinterpret_cast<const u32x4_t*>(src + c));
}

// One wave per route j: dg[j] = <dout[j / k], y[j]>, each lane summing its
// own columns in order, then the lanes combined by a fixed butterfly.
__global__ __launch_bounds__(256) void route_grad_kernel(const uint16_t* __restrict__ dout,
                                                         const uint16_t* __restrict__ y, int64_t n_routes, int D, int k,
                                                         float* __restrict__ dg) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / kWave;
  if (j >= n_routes) return;
  const uint16_t* __restrict__ a = dout + (j / k) * D;
  const uint16_t* __restrict__ b = y + j * D;
  float acc = 0.f;
  for (int c = lane_id() * 8; c < D; c += kWave * 8) {
    const u32x4_t va = *reinterpret_cast<const u32x4_t*>(a + c);
    const u32x4_t vb = *reinterpret_cast<const u32x4_t*>(b + c);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc = fmaf(bf16_to_f32(static_cast<uint16_t>(va[q] & 0xffffu)), bf16_to_f32(static_cast<uint16_t>(vb[q] & 0xffffu)),
                 acc);
      acc = fmaf(bf16_to_f32(static_cast<uint16_t>(va[q] >> 16)), bf16_to_f32(static_cast<uint16_t>(vb[q] >> 16)), acc);
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane_id() == 0) dg[j] = acc;
}

// One block per token: the row of the logit gradient, zero off the
// selection, dl_s = g_s (dg_s - sum_s' g_s' dg_s') on it (bf16, row stride ld).
__global__ __launch_bounds__(256) void gate_grad_kernel(const float* __restrict__ gate, const float* __restrict__ dg,
                                                        const int32_t* __restrict__ idx, int T, int E, int ld, int k,
                                                        uint16_t* __restrict__ dl) {
  const int t = blockIdx.x;
  uint16_t* __restrict__ row = dl + static_cast<int64_t>(t) * ld;
  for (int e = threadIdx.x; e < ld; e += 256) row[e] = 0;
  __syncthreads();
  if (threadIdx.x == 0) {
    float s = 0.f;
    for (int q = 0; q < k; ++q) s = fmaf(gate[t * k + q], dg[t * k + q], s);
    for (int q = 0; q < k; ++q) {
      const int e = idx[t * k + q];
      if (e >= 0 && e < E) row[e] = f32_to_bf16(gate[t * k + q] * (dg[t * k + q] - s));
    }
  }
}

// Elementwise SwiGLU backward over rows x I: act = [a_g | a_u] (bf16, row
// stride 2I), dh (fp32, row stride I) -> h (bf16, stride I) and
// da = [da_g | da_u] (bf16, stride 2I).  Eight columns per thread.
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const uint16_t* __restrict__ act, const float* __restrict__ dh,
                                                         int64_t rows, int I, uint16_t* __restrict__ h,
                                                         uint16_t* __restrict__ da) {
  const int64_t q = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;  // 8-column group
  const int per_row = I / 8;
  if (q >= rows * per_row) return;
  const int64_t r = q / per_row;
  const int c = static_cast<int>(q % per_row) * 8;
  const u32x4_t vg = *reinterpret_cast<const u32x4_t*>(act + r * 2 * I + c);
  const u32x4_t vu = *reinterpret_cast<const u32x4_t*>(act + r * 2 * I + I + c);
  const f32x4_t d0 = *reinterpret_cast<const f32x4_t*>(dh + r * I + c);
  const f32x4_t d1 = *reinterpret_cast<const f32x4_t*>(dh + r * I + c + 4);
  u32x4_t oh, og, ou;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    float hv[2], gv[2], uv[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const float g = bf16_to_f32(static_cast<uint16_t>(half ? vg[w] >> 16 : vg[w] & 0xffffu));
      const float u = bf16_to_f32(static_cast<uint16_t>(half ? vu[w] >> 16 : vu[w] & 0xffffu));
      const float d = (w * 2 + half) < 4 ? d0[w * 2 + half] : d1[w * 2 + half - 4];
      const float s = __builtin_amdgcn_rcpf(1.0f + __expf(-g));
      const float silu = g * s;
      hv[half] = silu * u;
      gv[half] = d * u * (s * (1.0f + g * (1.0f - s)));
      uv[half] = d * silu;
    }
    oh[w] = pack_bf16x2(hv[0], hv[1]);
    og[w] = pack_bf16x2(gv[0], gv[1]);
    ou[w] = pack_bf16x2(uv[0], uv[1]);
  }
  *reinterpret_cast<u32x4_t*>(h + r * I + c) = oh;
  *reinterpret_cast<u32x4_t*>(da + r * 2 * I + c) = og;
  *reinterpret_cast<u32x4_t*>(da + r * 2 * I + I + c) = ou;
}

// Padded segment offsets: segment e (rows offsets[e] .. offsets[e+1]-1) takes
// columns padded[e] .. padded[e] + 64 ceil(n_e / 64) - 1 of the transposed
// layout; k_groups[e] = {padded[e], ceil(n_e / 64)}.  One block of 1024.
__global__ __launch_bounds__(1024) void pad_offsets_kernel(const int32_t* __restrict__ offsets, int L,
                                                           int32_t* __restrict__ padded, int2* __restrict__ k_groups) {
  __shared__ int part[1024];
  const int l = threadIdx.x;
  const int n = l < L ? (offsets[l + 1] - offsets[l] + 63) / 64 : 0;
  part[l] = n;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {  // inclusive scan (Hillis-Steele)
    const int v = l >= off ? part[l - off] : 0;
    __syncthreads();
    part[l] += v;
    __syncthreads();
  }
  const int start = (part[l] - n) * 64;
  if (l < L) {
    padded[l] = start;
    k_groups[l] = make_int2(start, n);
  }
  if (l == L - 1) padded[L] = start + n * 64;
}

// Transpose of row segments into padded columns: out [W][ld_out], column
// padded[e] + i holds row offsets[e] + i of src [rows][lda] (bf16), zero past
// the segment's rows.  A block moves a 64 x 64 tile through LDS with 16-byte
// global loads (8 columns of one source row) and 16-byte global stores (8
// rows of one source column); a 64-column chunk of the output lies in one
// segment, since padded starts are multiples of 64.  W, lda and ld_out are
// multiples of 8 and the bases 16-byte aligned (checked by the launcher).
__global__ __launch_bounds__(256) void seg_transpose_kernel(const uint16_t* __restrict__ src, int64_t lda, int W,
                                                            const int32_t* __restrict__ offsets,
                                                            const int32_t* __restrict__ padded, int L,
                                                            uint16_t* __restrict__ out, int64_t ld_out, bool tiled) {
  constexpr int kStride = 72;  // LDS row stride in elements (144 bytes: 16-byte aligned rows, spread banks)
  __shared__ __attribute__((aligned(16))) uint16_t tile[64 * kStride];
  const int64_t q0 = static_cast<int64_t>(blockIdx.x) * 64;  // output column chunk
  const int w0 = blockIdx.y * 64;                            // output row chunk (source column)
  if (q0 >= padded[L]) return;
  int lo = 0, hi = L - 1;  // the segment with padded[e] <= q0 < padded[e+1]
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (padded[mid] <= q0) lo = mid;
    else hi = mid - 1;
  }
  const int e = lo;
  const int64_t i0 = q0 - padded[e];
  const int64_t n_e = offsets[e + 1] - offsets[e];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int v = threadIdx.x + 256 * j;
    const int r = v >> 3, c = (v & 7) * 8;  // source row within the chunk, first of 8 source columns
    u32x4_t val = {0u, 0u, 0u, 0u};
    if (i0 + r < n_e && w0 + c < W)
      val = *reinterpret_cast<const u32x4_t*>(src + (offsets[e] + i0 + r) * lda + w0 + c);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      tile[(c + 2 * q) * kStride + r] = static_cast<uint16_t>(val[q] & 0xffffu);
      tile[(c + 2 * q + 1) * kStride + r] = static_cast<uint16_t>(val[q] >> 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int v = threadIdx.x + 256 * j;
    const int c = v >> 3, r = (v & 7) * 8;  // output row (source column), first of 8 output columns
    // the transposed operands (up to 1 GB each) are read back by the
    // weight-gradient GEMMs only after the other transposes: non-temporal
    // stores (measured 0.2% off the backward)
    // row-major [W][ld_out], or K-tiled: output column chunk q0 is one plane
    // of W rows, so the block's 64 x 64 tile is 8 KB of contiguous output
    const int64_t to = tiled ? ((q0 / kTileK) * W + w0 + c) * kTileK + r : static_cast<int64_t>(w0 + c) * ld_out + q0 + r;
    if (w0 + c < W)
      __builtin_nontemporal_store(*reinterpret_cast<const u32x4_t*>(tile + c * kStride + r),
                                  reinterpret_cast<u32x4_t*>(out + to));
  }
}

// Batched transpose: out[b][c][col0 + r] = in[b][r][c] for in [B][R][Cn]
// (bf16), out rows of stride ld_out, batch strides in_b / out_b; with
// plane_rows > 0 the output is K-tiled instead: element (row, col) of batch b
// at ((col / 64) * plane_rows + row) * 64 + col % 64.
__global__ __launch_bounds__(256) void transpose_kernel(const uint16_t* __restrict__ in, int R, int Cn, int64_t in_b,
                                                        uint16_t* __restrict__ out, int64_t ld_out, int64_t out_b,
                                                        int col0, int64_t plane_rows) {
  __shared__ uint16_t tile[64][66];
  const int b = blockIdx.z;
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const uint16_t* __restrict__ src = in + b * in_b;
  uint16_t* __restrict__ dst = out + b * out_b;
  for (int v = threadIdx.x; v < 64 * 64; v += 256) {
    const int r = v / 64, c = v % 64;
    tile[c][r] = (r0 + r < R && c0 + c < Cn) ? src[static_cast<int64_t>(r0 + r) * Cn + c0 + c] : 0;
  }
  __syncthreads();
  for (int v = threadIdx.x; v < 64 * 64; v += 256) {
    const int c = v / 64, r = v % 64;
    if (r0 + r >= R || c0 + c >= Cn) continue;
    const int64_t row = c0 + c, col = col0 + r0 + r;
    dst[plane_rows > 0 ? ((col / kTileK) * plane_rows + row) * kTileK + col % kTileK : row * ld_out + col] = tile[c][r];
  }
}

// dx[t] = dx_shared[t] + dx_router[t] + sum over slots s in order of
// dx_ring[route_dst[t k + s]] (fp32), four columns per thread.
__global__ __launch_bounds__(256) void dx_assemble_kernel(const float* __restrict__ dx_shared,
                                                          const float* __restrict__ dx_router,
                                                          const float* __restrict__ dx_ring,
                                                          const int32_t* __restrict__ route_dst, int T, int D, int k,
                                                          int64_t P, float* __restrict__ dx, int* err) {
  const int chunks = (D / 4 + 255) / 256;  // 1024-column chunks of a row
  const int t = static_cast<int>(blockIdx.x / chunks);
  const int c = (static_cast<int>(blockIdx.x % chunks) * 256 + threadIdx.x) * 4;
  if (c >= D) return;
  const int64_t o = static_cast<int64_t>(t) * D + c;
  f32x4_t acc = *reinterpret_cast<const f32x4_t*>(dx_shared + o);
  acc += *reinterpret_cast<const f32x4_t*>(dx_router + o);
  for (int s = 0; s < k; ++s) {
    const int32_t p = route_dst[static_cast<int64_t>(t) * k + s];
    if (p < 0 || p >= P) {
      if (c == 0) raise_error(err, kErrExpertRange);
      continue;
    }
    // each dx_ring row is read once, here: non-temporal loads, and a
    // non-temporal store of dx (measured 0.2% off the backward)
    acc += __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(dx_ring + static_cast<int64_t>(p) * D + c));
  }
  __builtin_nontemporal_store(acc, reinterpret_cast<f32x4_t*>(dx + o));
}

// One segment of `rows` rows (the shared expert's and the router's weight
// gradients): offsets {0, rows}, padded {0, 64 ceil(rows / 64)}, k_groups[0].
__global__ void single_segment_kernel(int rows, int32_t* __restrict__ offsets, int32_t* __restrict__ padded,
                                      int2* __restrict__ k_groups) {
  if (threadIdx.x == 0) {
    const int n = (rows + 63) / 64;
    offsets[0] = 0;
    offsets[1] = rows;
    padded[0] = 0;
    padded[1] = n * 64;
    k_groups[0] = make_int2(0, n);
  }
}

}  // namespace

hipError_t launch_single_segment(int rows, int32_t* offsets, int32_t* padded, int2* k_groups, hipStream_t s) {
  single_segment_kernel<<<1, 64, 0, s>>>(rows, offsets, padded, k_groups);
  return hipGetLastError();
}

hipError_t launch_dy_gather(const uint16_t* dout, const float* gate, const int32_t* sched_src, int64_t P, int T, int D,
                            int k, uint16_t* dy, int* err, hipStream_t s) {
  if (P <= 0) return hipSuccess;
  if (D % 8) return hipErrorInvalidValue;
  dy_gather_kernel<<<static_cast<unsigned>((P + 3) / 4), 256, 0, s>>>(dout, gate, sched_src, P, T, D, k, dy, err);
  return hipGetLastError();
}

hipError_t launch_route_grad(const uint16_t* dout, const uint16_t* y, int64_t n_routes, int D, int k, float* dg,
                             hipStream_t s) {
  if (n_routes <= 0) return hipSuccess;
  if (D % 8) return hipErrorInvalidValue;
  route_grad_kernel<<<static_cast<unsigned>((n_routes + 3) / 4), 256, 0, s>>>(dout, y, n_routes, D, k, dg);
  return hipGetLastError();
}

hipError_t launch_gate_grad(const float* gate, const float* dg, const int32_t* idx, int T, int E, int ld, int k,
                            uint16_t* dl, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  gate_grad_kernel<<<T, 256, 0, s>>>(gate, dg, idx, T, E, ld, k, dl);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const uint16_t* act, const float* dh, int64_t rows, int I, uint16_t* h, uint16_t* da,
                             hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (I % 8) return hipErrorInvalidValue;
  const int64_t n = rows * (I / 8);
  swiglu_bwd_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(act, dh, rows, I, h, da);
  return hipGetLastError();
}

hipError_t launch_pad_offsets(const int32_t* offsets, int L, int32_t* padded, int2* k_groups, hipStream_t s) {
  if (L <= 0 || L > 1024) return hipErrorInvalidValue;
  pad_offsets_kernel<<<1, 1024, 0, s>>>(offsets, L, padded, k_groups);
  return hipGetLastError();
}

hipError_t launch_seg_transpose(const uint16_t* src, int64_t lda, int W, const int32_t* offsets,
                                const int32_t* padded, int L, int64_t max_cols, uint16_t* out, int64_t ld_out,
                                hipStream_t s, bool tiled) {
  if (max_cols <= 0 || W <= 0) return hipSuccess;
  if (W % 8 || lda % 8 || ld_out % 64 || reinterpret_cast<uintptr_t>(src) % 16 ||
      reinterpret_cast<uintptr_t>(out) % 16)
    return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>((max_cols + 63) / 64), static_cast<unsigned>((W + 63) / 64));
  seg_transpose_kernel<<<grid, 256, 0, s>>>(src, lda, W, offsets, padded, L, out, ld_out, tiled);
  return hipGetLastError();
}

hipError_t launch_transpose(const uint16_t* in, int B, int R, int Cn, uint16_t* out, int64_t ld_out, int64_t out_b,
                            int col0, hipStream_t s, int64_t plane_rows) {
  if (B <= 0 || R <= 0 || Cn <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((R + 63) / 64), static_cast<unsigned>((Cn + 63) / 64), static_cast<unsigned>(B));
  transpose_kernel<<<grid, 256, 0, s>>>(in, R, Cn, static_cast<int64_t>(R) * Cn, out, ld_out, out_b, col0,
                                        plane_rows);
  return hipGetLastError();
}

hipError_t launch_dx_assemble(const float* dx_shared, const float* dx_router, const float* dx_ring,
                              const int32_t* route_dst, int T, int D, int k, int64_t P, float* dx, int* err,
                              hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (D % 4) return hipErrorInvalidValue;
  const int64_t blocks = static_cast<int64_t>(T) * ((D / 4 + 255) / 256);
  dx_assemble_kernel<<<static_cast<unsigned>(blocks), 256, 0, s>>>(dx_shared, dx_router, dx_ring, route_dst, T, D, k,
                                                                   P, dx, err);
  return hipGetLastError();
}

}  // namespace moe
