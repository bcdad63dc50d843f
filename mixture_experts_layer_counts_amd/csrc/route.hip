// Top-k expert selection and normalised gates on gfx950 (one wave64 per token).
//
// MoK paper "Mixture-of-Kittens: MoE Megakernel for NVL72s", §2.1: the router
// projection selects the k routed experts of each token and assigns each a
// router weight; the weights are normalised over the selected experts
// (g_i = s_i / sum_{j in E} s_j, MoK blog notation).  With s the softmax of
// the logits this is exp(l_i - l_max) / sum_{j in E} exp(l_j - l_max), which is
// what is evaluated here, in fp32, from the fp32 logits.
//
// Selection order: larger logit first, ties to the lower expert id.  Float
// comparison makes -0.0 and +0.0 equal.  A NaN logit sets the non-finite
// error bit and ranks below every number.

#include "common.h"
#include "kernels.h"

namespace moe {

// EPL = logits per lane (ceil(E / 64)), so the row lives in registers.
// The router GEMM may leave the logits as `parts` partial sums over K ranges
// (planes part_stride apart); they are added here in plane order, a fixed
// order, and the sums written back to `logits`.
template <int EPL>
__global__ __launch_bounds__(256) void topk_gate_kernel(const float* __restrict__ planes, int parts,
                                                        int64_t part_stride, float* __restrict__ logits, int T,
                                                        int E, int k, int32_t* __restrict__ idx,
                                                        float* __restrict__ gate, int* err) {
  const int token = blockIdx.x * 4 + static_cast<int>(threadIdx.x) / kWave;
  if (token >= T) return;
  const int lane = lane_id();
  const float* row = planes + static_cast<int64_t>(token) * E;

  float v[EPL];
  bool bad = false;
#pragma unroll
  for (int q = 0; q < EPL; ++q) {
    const int e = lane + kWave * q;
    float x = -INFINITY;
    if (e < E) {
      x = row[e];
      for (int pp = 1; pp < parts; ++pp) x += row[pp * part_stride + e];
      if (parts > 1) logits[static_cast<int64_t>(token) * E + e] = x;
      if (!__builtin_isfinite(x)) {
        bad = true;
        if (__builtin_isnan(x)) x = -INFINITY;
      }
    }
    v[q] = x;
  }
  if (__any(bad) && lane == 0) raise_error(err, kErrNonFinite);

  uint32_t taken = 0;
  float sel_v[16];
  int sel_i[16];
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    sel_v[s] = -INFINITY;
    sel_i[s] = 0;
  }
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    if (s >= k) continue;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < EPL; ++q) {
      const int e = lane + kWave * q;
      if (e < E && !((taken >> q) & 1u)) {
        if (v[q] > bv || (v[q] == bv && e < bi)) {
          bv = v[q];
          bi = e;
        }
      }
    }
    // wave-wide arg-max under the total order (value desc, id asc)
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & (kWave - 1)) == lane) taken |= 1u << (bi / kWave);
    sel_v[s] = bv;
    sel_i[s] = bi;
  }

  // gates: exp(l_s - l_0) / sum_s' exp(l_s' - l_0), summed in slot order
  float z[16];
  float sum = 0.f;
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    z[s] = 0.f;
    if (s < k) {
      z[s] = expf(sel_v[s] - sel_v[0]);
      sum += z[s];
    }
  }
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    if (s < k && lane == s) {
      idx[static_cast<int64_t>(token) * k + s] = sel_i[s];
      gate[static_cast<int64_t>(token) * k + s] = z[s] / sum;
    }
  }
}

hipError_t launch_topk_gate(const float* planes, int parts, int64_t part_stride, float* logits, int T, int E, int k,
                            int32_t* idx, float* gate, int* err, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  if (parts < 1) return hipErrorInvalidValue;
  const dim3 grid((T + 3) / 4), block(256);
  const int epl = (E + kWave - 1) / kWave;
  if (epl <= 1)
    topk_gate_kernel<1><<<grid, block, 0, stream>>>(planes, parts, part_stride, logits, T, E, k, idx, gate, err);
  else if (epl <= 2)
    topk_gate_kernel<2><<<grid, block, 0, stream>>>(planes, parts, part_stride, logits, T, E, k, idx, gate, err);
  else if (epl <= 4)
    topk_gate_kernel<4><<<grid, block, 0, stream>>>(planes, parts, part_stride, logits, T, E, k, idx, gate, err);
  else if (epl <= 6)
    topk_gate_kernel<6><<<grid, block, 0, stream>>>(planes, parts, part_stride, logits, T, E, k, idx, gate, err);
  else if (epl <= 8)
    topk_gate_kernel<8><<<grid, block, 0, stream>>>(planes, parts, part_stride, logits, T, E, k, idx, gate, err);
  else if (epl <= 16)
    topk_gate_kernel<16><<<grid, block, 0, stream>>>(planes, parts, part_stride, logits, T, E, k, idx, gate, err);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace moe
