// Operand-stream probe on gfx950: the loads of a routed GEMM work item's K
// loop, with no arithmetic.  It measures what the expert GEMMs' load pipeline
// can reach on the chip, the floor their roofline fractions are read against;
// it is measurement, not a step of the layer.
//
// Work item i (one workgroup of 8 waves) walks row_bytes / 128 stages.  At
// each stage it moves 128 bytes of each of a_rows activation-like rows and of
// b_rows weight-like rows into two LDS rings with direct buffer->LDS loads
// (1 KB per wave instruction), with the routed GEMMs' ring protocol: a slot is
// refilled right after the barrier that ends the stage it held, the
// activation ring NSA slots deep and the weight ring NSB, one barrier per
// stage.  Items are cut into 8 contiguous runs, one per XCD, as the GEMMs cut
// theirs.  a_share consecutive items read the same activation rows (the N
// blocks of one row tile), so after the first fetch those come from the XCD's
// L2; every item reads weight rows of its own (a weight slab, streamed from
// HBM once).

#include "../../include/moe.h"
#include "common.h"
#include "gemm_common.h"

namespace moe {
namespace {

struct ProbeArgs {
  const char* act;
  const char* wts;
  int64_t row_bytes;
  int items, a_share, stages;
};

// AI, BI: 1 KB load instructions per wave per stage for the activation and
// weight rows (a_rows / 64, b_rows / 64 with 8 waves).
template <int AI, int BI, int NSA, int NSB>
__global__ __launch_bounds__(512) void stream_probe_kernel(const ProbeArgs p) {
  constexpr int ASLOT = AI * 8 * 1024, BSLOT = BI * 8 * 1024;  // bytes of one stage of each stream
  constexpr int LDS = NSA * ASLOT + NSB * BSLOT;
  static_assert(LDS > 0 && LDS <= 160 * 1024, "probe rings");
  __shared__ __attribute__((aligned(1024))) char smem[LDS];
  const int xcd = static_cast<int>(blockIdx.x) % kXcds, per = static_cast<int>(gridDim.x) / kXcds;
  const int item = xcd * per + static_cast<int>(blockIdx.x) / kXcds;
  if (item >= p.items) return;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  const int lane = static_cast<int>(threadIdx.x) % kWave;
  constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit elements
  const int64_t a_block = static_cast<int64_t>(AI) * 64 * p.row_bytes, b_block = static_cast<int64_t>(BI) * 64 * p.row_bytes;
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(p.act + (item / p.a_share) * a_block), 0, static_cast<int>(a_block), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(p.wts + static_cast<int64_t>(item) * b_block), 0, static_cast<int>(b_block), kRsrcWord3);
  // one instruction fills 8 rows of 128 bytes: lane l takes row l / 8, chunk l % 8
  uint32_t a_off[AI > 0 ? AI : 1], b_off[BI > 0 ? BI : 1];
#pragma unroll
  for (int j = 0; j < AI; ++j)
    a_off[j] = static_cast<uint32_t>(((wave * AI + j) * 8 + lane / 8) * p.row_bytes + (lane % 8) * 16);
#pragma unroll
  for (int j = 0; j < BI; ++j)
    b_off[j] = static_cast<uint32_t>(((wave * BI + j) * 8 + lane / 8) * p.row_bytes + (lane % 8) * 16);
  const int nk = p.stages;
  // past the last stage the loads repeat it, so that every step issues the
  // same number of loads (as in the GEMMs)
  auto issue_a = [&](int kt) __attribute__((always_inline)) {
    const int ko = (kt < nk ? kt : nk - 1) * 128;
#pragma unroll
    for (int j = 0; j < AI; ++j) dma16(ra, smem + (kt % NSA) * ASLOT + (wave * AI + j) * 1024, a_off[j], ko);
  };
  auto issue_b = [&](int kt) __attribute__((always_inline)) {
    const int ko = (kt < nk ? kt : nk - 1) * 128;
#pragma unroll
    for (int j = 0; j < BI; ++j)
      dma16(rb, smem + NSA * ASLOT + (kt % NSB) * BSLOT + (wave * BI + j) * 1024, b_off[j], ko);
  };
  // loads that may still be in flight once stage s has landed: those issued
  // after A(s), counted as in the GEMMs' K loop
  constexpr int VM_AFTER = NSB > NSA ? BI : 0;
  constexpr int VM_FIRST = VM_AFTER + (NSA - 1) * (AI + BI);
  constexpr int VM_STAGE = VM_AFTER + (NSA - 2) * (AI + BI);
  static_assert(NSA >= 2 && NSB >= NSA && VM_FIRST < 64, "ring depths");
#pragma unroll
  for (int v = -NSB; v < 0; ++v) {
    if (v + NSA >= 0) issue_a(v + NSA);
    issue_b(v + NSB);
  }
  asm volatile("s_waitcnt %0" ::"n"(waitcnt_imm(VM_FIRST, 15)) : "memory");
  __builtin_amdgcn_s_barrier();
  for (int kt = 0; kt < nk; ++kt) {
    asm volatile("s_waitcnt %0" ::"n"(waitcnt_imm(VM_STAGE, 15)) : "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    issue_a(kt + NSA);
    issue_b(kt + NSB);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no load may still target LDS when the workgroup ends
}

template <int AI, int BI, int NSA, int NSB>
hipError_t launch(const ProbeArgs& p, hipStream_t stream) {
  const int64_t grid = (static_cast<int64_t>(p.items) + kXcds - 1) / kXcds * kXcds;
  stream_probe_kernel<AI, BI, NSA, NSB><<<static_cast<unsigned>(grid), 512, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace
}  // namespace moe

extern "C" moe_status moe_stream_probe(const moe_stream_probe_args* a, void* stream) {
  using namespace moe;
  if (!a || a->items <= 0 || a->a_share <= 0 || a->row_bytes <= 0 || a->row_bytes % 128 != 0)
    return MOE_ERR_INVALID_ARG;
  if ((a->a_rows > 0 && !a->act) || (a->b_rows > 0 && !a->wts)) return MOE_ERR_INVALID_ARG;
  // each item's rows lie under one buffer resource (< 2^31 bytes)
  if (320 * a->row_bytes >= (int64_t(1) << 31) || a->items > (1 << 24)) return MOE_ERR_UNSUPPORTED;
  ProbeArgs p{static_cast<const char*>(a->act), static_cast<const char*>(a->wts), a->row_bytes, a->items,
              a->a_share, static_cast<int>(a->row_bytes / 128)};
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int A = a->a_rows, B = a->b_rows, NA = a->slots_a, NB = a->slots_b;
  hipError_t e;
  // the bf16 routed up/gate's stage (320 activation rows, 256 weight rows, 2 + 2 slots)
  if (A == 320 && B == 256 && NA == 2 && NB == 2) e = launch<5, 4, 2, 2>(p, s);
  else if (A == 320 && B == 0 && NA == 2 && NB == 2) e = launch<5, 0, 2, 2>(p, s);
  // the MXFP8 routed up/gate's stage (256 + 256 rows, 2 + 3 slots)
  else if (A == 256 && B == 256 && NA == 2 && NB == 3) e = launch<4, 4, 2, 3>(p, s);
  else if (A == 256 && B == 0 && NA == 2 && NB == 3) e = launch<4, 0, 2, 3>(p, s);
  // the same stage with both rings two slots deep (one stage in flight each)
  else if (A == 256 && B == 256 && NA == 2 && NB == 2) e = launch<4, 4, 2, 2>(p, s);
  // weight rows alone, at ring depths of 2 to 5 slots (1 to 4 stages in flight)
  else if (A == 0 && B == 256 && NA == NB && NB == 2) e = launch<0, 4, 2, 2>(p, s);
  else if (A == 0 && B == 256 && NA == 2 && NB == 3) e = launch<0, 4, 2, 3>(p, s);
  else if (A == 0 && B == 256 && NA == NB && NB == 3) e = launch<0, 4, 3, 3>(p, s);
  else if (A == 0 && B == 256 && NA == NB && NB == 4) e = launch<0, 4, 4, 4>(p, s);
  else if (A == 0 && B == 256 && NA == NB && NB == 5) e = launch<0, 4, 5, 5>(p, s);
  else return MOE_ERR_UNSUPPORTED;
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
