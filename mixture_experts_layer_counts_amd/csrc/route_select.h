// Per-token top-k selection and normalised gates on gfx950 (one wave64 per
// token), shared by the standalone top-k kernel and the fused router kernel.
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
#pragma once

#include "common.h"

namespace moe {

constexpr int kNoExpert = 0x7fffffff;  // id of an empty candidate

// (bv, bi) meets another lane's pair and keeps the larger under the order
// (value desc, id asc).
__device__ __forceinline__ void argmax_meet(float& bv, int& bi, float ov, int oi) {
  const bool take = ov > bv || (ov == bv && oi < bi);
  bv = take ? ov : bv;
  bi = take ? oi : bi;
}

// One step against the lane that the DPP control CTRL maps to this lane.
template <int CTRL>
__device__ __forceinline__ void argmax_dpp(float& bv, int& bi) {
  const float ov = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(bv), CTRL, 0xF, 0xF, false));
  const int oi = __builtin_amdgcn_mov_dpp(bi, CTRL, 0xF, 0xF, false);
  argmax_meet(bv, bi, ov, oi);
}

// Wave-wide arg-max; every lane ends with the result.  Within a 16-lane row
// the partners come by DPP: lane ^ 1 and lane ^ 2 (quad permutations), then
// the mirror within 8 lanes and within 16 lanes, each of which pairs lanes
// from the two halves that already agree; across rows by lane ^ 16 and
// lane ^ 32 through the LDS crossbar.
__device__ __forceinline__ void wave_argmax(float& bv, int& bi) {
  argmax_dpp<0xB1>(bv, bi);   // quad_perm [1, 0, 3, 2]
  argmax_dpp<0x4E>(bv, bi);   // quad_perm [2, 3, 0, 1]
  argmax_dpp<0x141>(bv, bi);  // row_half_mirror
  argmax_dpp<0x140>(bv, bi);  // row_mirror
  argmax_meet(bv, bi, __shfl_xor(bv, 16), __shfl_xor(bi, 16));
  argmax_meet(bv, bi, __shfl_xor(bv, 32), __shfl_xor(bi, 32));
}

// One wave, one token.  EPL = logits per lane (ceil(E / 64)), so the row
// lives in registers: lane l holds experts l, l + 64, ...  The token's logits
// are the sum of `parts` fp32 planes [T, E] (part_stride elements apart),
// added in plane order, a fixed order; when the planes are not `logits`
// itself the sums are written there.  Planes are loaded four at a time so
// that their loads are in flight together.  Then k rounds of a wave-wide
// arg-max: lane s keeps the id and the unnormalised gate of slot s, and the
// gate sum runs in slot order.
template <int EPL>
__device__ __forceinline__ void select_token(const float* __restrict__ planes, int parts, int64_t part_stride,
                                             float* __restrict__ logits, int token, int E, int k,
                                             int32_t* __restrict__ idx, float* __restrict__ gate, int* err) {
  const int lane = lane_id();
  const float* row = planes + static_cast<int64_t>(token) * E;
  float v[EPL];
  for (int base = 0; base < parts; base += 4) {
    float pv[4][EPL];
#pragma unroll
    for (int pp = 0; pp < 4; ++pp)
#pragma unroll
      for (int q = 0; q < EPL; ++q) {
        const int e = lane + kWave * q;
        pv[pp][q] = (base + pp < parts && e < E) ? row[(base + pp) * part_stride + e] : 0.f;
      }
#pragma unroll
    for (int q = 0; q < EPL; ++q) {
      float x = base == 0 ? pv[0][q] : v[q] + pv[0][q];
#pragma unroll
      for (int pp = 1; pp < 4; ++pp)
        if (base + pp < parts) x += pv[pp][q];
      v[q] = x;
    }
  }
  bool bad = false;
#pragma unroll
  for (int q = 0; q < EPL; ++q) {
    const int e = lane + kWave * q;
    float x = -INFINITY;
    if (e < E) {
      x = v[q];
      if (planes != logits) logits[static_cast<int64_t>(token) * E + e] = x;
      if (!__builtin_isfinite(x)) {
        bad = true;
        if (__builtin_isnan(x)) x = -INFINITY;
      }
    }
    v[q] = x;
  }
  if (__any(bad) && lane == 0) raise_error(err, kErrNonFinite);

  uint32_t taken = 0;
  float v0 = 0.f, sum = 0.f, my_z = 0.f;
  int my_i = 0;
  for (int s = 0; s < k; ++s) {
    float bv = -INFINITY;
    int bi = kNoExpert;
#pragma unroll
    for (int q = 0; q < EPL; ++q) {
      // ids rise with q, so an equal value never replaces an earlier candidate
      const int e = lane + kWave * q;
      const bool take = e < E && !((taken >> q) & 1u) && (v[q] > bv || bi == kNoExpert);
      bv = take ? v[q] : bv;
      bi = take ? e : bi;
    }
    wave_argmax(bv, bi);
    if ((bi & (kWave - 1)) == lane) taken |= 1u << (bi / kWave);
    if (s == 0) v0 = bv;
    // gates: exp(l_s - l_0) / sum_s' exp(l_s' - l_0)
    const float z = expf(bv - v0);
    sum += z;
    if (lane == s) {
      my_z = z;
      my_i = bi;
    }
  }
  if (lane < k) {
    idx[static_cast<int64_t>(token) * k + lane] = my_i;
    gate[static_cast<int64_t>(token) * k + lane] = my_z / sum;
  }
}

}  // namespace moe
