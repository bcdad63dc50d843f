// Top-k expert selection and normalised gates on gfx950 (one wave64 per
// token; the selection itself is route_select.h's).

#include "common.h"
#include "kernels.h"
#include "route_select.h"

namespace moe {

// Four tokens per block of 256; the logits may arrive as `parts` partial sums
// over K ranges of the router GEMM (planes part_stride apart).
template <int EPL>
__global__ __launch_bounds__(256) void topk_gate_kernel(const float* __restrict__ planes, int parts,
                                                        int64_t part_stride, float* __restrict__ logits, int T,
                                                        int E, int k, int32_t* __restrict__ idx,
                                                        float* __restrict__ gate, int* err) {
  const int token = blockIdx.x * 4 + static_cast<int>(threadIdx.x) / kWave;
  if (token >= T) return;
  select_token<EPL>(planes, parts, part_stride, logits, token, E, k, idx, gate, err);
}

hipError_t launch_topk_gate(const float* planes, int parts, int64_t part_stride, float* logits, int T, int E, int k,
                            int32_t* idx, float* gate, int* err, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  if (parts < 1 || parts > kMaxRouterParts) return hipErrorInvalidValue;
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
