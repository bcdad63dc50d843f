// Grouped MXFP8 GEMMs of the routed expert FFNs on gfx950 scaled MFMA.
//
// MoK paper "Mixture-of-Kittens: MoE Megakernel for NVL72s", §3.4 "MXFP8
// Support": the routed experts run on MXFP8 operands; weights are quantised
// ahead of time and activations inside the dispatch (the gather) and inside
// the gated activation (the up/gate epilogue).  Operands are E4M3 bytes with
// one E8M0 scale per 32 consecutive elements along K, stored row-major as
// [rows][K] bytes and [rows][K/32] scale bytes.
//
// The matrix core does the block scaling itself: v_mfma_scale_f32_32x32x64_f8f6f4
// multiplies a 32x64 E4M3 block of A by a 64x32 block of B with one scale per
// row (column) and 32-wide K block, accumulating in fp32.  Lane l (h = l / 32)
// supplies row l % 32; its 32 bytes are K[16h, 16h+16) and K[32+16h, 32+16h+16)
// of the 64-wide step, and its scale byte is that row's scale of K block h.
//
// The pipeline is the bf16 kernel's: 256 x BN tiles, 4 waves, an LDS ring of
// two K stages fed by direct buffer->LDS loads, the same XOR swizzle of the
// 128-byte stage rows, the same expert-major XCD-aware work order over the
// balanced tile list.  A stage holds 128 K elements (one 128-byte line per
// row, two MFMA steps) plus a 4-byte scale word per row, itself loaded by
// 4-byte direct loads.  The K loop always runs from k = 0 in the same order,
// so a row's result does not depend on the tile or minibatch it falls in.
//
// Epilogues: SwiGLU with MX quantisation of h along I (a row's 32-column
// block lives in the 32 lanes of one half-wave, which reduce its largest
// magnitude by shuffles), and a plain bf16 store for the down projection,
// scattered to the row of the route it came from.

#include "common.h"
#include "gemm_common.h"
#include "kernels.h"
#include "mx.h"

namespace moe {

namespace {

constexpr int kMxBM = 256;     // tile rows (must match the tile lists, built with gemm_routed_bm())
constexpr int kMxStageK = 128;  // K elements (bytes) per stage row
constexpr int kMxStages = 2;
constexpr int kRB = kMxStageK;  // bytes of one stage row
constexpr int kSB = 4;          // scale bytes of one stage row (128 / 32)

struct MxSrc {
  __amdgpu_buffer_rsrc_t a, b0, b1, as, bs0, bs1;
};

// One direct 4-byte-per-lane load into LDS: lane l's word lands at lds + 4 l.
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t rsrc, char* lds, uint32_t voffset, int soffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds, 4, voffset, soffset, 0,
                                           0);
}

__device__ __forceinline__ f32x16_t mfma_mx(const i32x8_t& a, const i32x8_t& b, const f32x16_t& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

__device__ __forceinline__ i32x8_t cat8(u32x4_t lo, u32x4_t hi) {
  return reinterpret_cast<i32x8_t>(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// The K loop of one workgroup (see the bf16 kernel for the ring protocol).
// Per stage and wave: AI + BI 1 KB data loads and two 256-byte scale loads
// (A rows 64 w .. 64 w + 63, B rows likewise).
template <int BN, int NB, int FML, int FM, int FN, int AI, int BI>
__device__ __forceinline__ void k_loop_mx(char* smem, const MxSrc& src, const uint32_t (&a_off)[AI],
                                          const uint32_t (&b_off)[BI], uint32_t as_off, uint32_t bs_off, int nk,
                                          int a_rows, int tid, int wm, int wn, f32x16_t (&acc)[NB][FM][FN]) {
  constexpr int BM = kMxBM, BROWS = NB * BN;
  constexpr int WTM = BM / 2, WTN = BN / 2;
  constexpr int DATA = (BM + BROWS) * kRB;
  constexpr int STAGE = DATA + (BM + BROWS) * kSB;
  constexpr int ROWS_PER_LD = 1024 / kRB;
  static_assert(AI * ROWS_PER_LD * 4 == BM && BI * ROWS_PER_LD * 4 == BROWS, "data loads per wave per stage");
  static_assert(BM == 4 * 64 && BROWS == 4 * 64, "one scale load per wave per operand");
  constexpr int NLD = AI + BI + 2;
  constexpr int VM_AHEAD = (kMxStages - 2) * NLD;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;  // wave index is uniform
  const int frag_row = lane & 31, frag_h = lane >> 5;

  auto issue = [&](int kt) __attribute__((always_inline)) {
    const int buf = kt % kMxStages;
    const int kc = kt < nk ? kt : nk - 1;
    char* sa = smem + buf * STAGE;
    char* sb = sa + BM * kRB;
    char* ssa = sa + DATA;
    char* ssb = ssa + BM * kSB;
#pragma unroll
    for (int j = 0; j < AI; ++j)
      dma16(src.a, sa + (wave * AI + j) * 1024, (wave * AI + j) * ROWS_PER_LD < a_rows ? a_off[j] : a_off[0],
            kc * kRB);
#pragma unroll
    for (int j = 0; j < BI; ++j) {
      const int g = wave * BI + j;
      dma16((NB == 2 && g * ROWS_PER_LD >= BN) ? src.b1 : src.b0, sb + g * 1024, b_off[j], kc * kRB);
    }
    dma4(src.as, ssa + wave * 256, as_off, kc * kSB);
    dma4((NB == 2 && wave >= 2) ? src.bs1 : src.bs0, ssb + wave * 256, bs_off, kc * kSB);
  };

  struct Frags {
    i32x8_t a[FML > 0 ? FML : 1];
    i32x8_t b[NB][FN];
  };
  struct Scales {  // the stage's scale words of this lane's fragment rows (both steps)
    uint32_t a[FML > 0 ? FML : 1];
    uint32_t b[NB][FN];
  };
  auto read_frags = [&](int kt, int step, Frags& f) __attribute__((always_inline)) {
    const char* sa = smem + (kt % kMxStages) * STAGE;
    const char* sb = sa + BM * kRB;
    const int c0 = step * 4 + frag_h, c1 = c0 + 2;
#pragma unroll
    for (int fm = 0; fm < FML; ++fm) {
      const int row = wm * WTM + fm * 32 + frag_row;
      const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(sa + swz<kRB>(row, c0));
      const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(sa + swz<kRB>(row, c1));
      f.a[fm] = cat8(lo, hi);
    }
#pragma unroll
    for (int h = 0; h < NB; ++h)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int row = h * BN + wn * WTN + fn * 32 + frag_row;
        const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(sb + swz<kRB>(row, c0));
        const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(sb + swz<kRB>(row, c1));
        f.b[h][fn] = cat8(lo, hi);
      }
  };
  auto read_scales = [&](int kt, Scales& sc) __attribute__((always_inline)) {
    const char* ssa = smem + (kt % kMxStages) * STAGE + DATA;
    const char* ssb = ssa + BM * kSB;
#pragma unroll
    for (int fm = 0; fm < FML; ++fm)
      sc.a[fm] = *reinterpret_cast<const uint32_t*>(ssa + (wm * WTM + fm * 32 + frag_row) * kSB);
#pragma unroll
    for (int h = 0; h < NB; ++h)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        sc.b[h][fn] = *reinterpret_cast<const uint32_t*>(ssb + (h * BN + wn * WTN + fn * 32 + frag_row) * kSB);
  };
  // v_perm selector that replicates byte (2 step + h) of a scale word into all
  // four bytes: the K block of this lane's half of the step
  const uint32_t rep0 = (0 + frag_h) * 0x01010101u, rep1 = (2 + frag_h) * 0x01010101u;
  auto mfmas = [&](const Frags& f, const Scales& sc, int step) __attribute__((always_inline)) {
    const uint32_t rep = step ? rep1 : rep0;
#pragma unroll
    for (int fm = 0; fm < FML; ++fm) {
      const int sa = static_cast<int>(__builtin_amdgcn_perm(sc.a[fm], sc.a[fm], rep));
#pragma unroll
      for (int h = 0; h < NB; ++h)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          const int sb = static_cast<int>(__builtin_amdgcn_perm(sc.b[h][fn], sc.b[h][fn], rep));
          acc[h][fm][fn] = mfma_mx(f.a[fm], f.b[h][fn], acc[h][fm][fn], sa, sb);
        }
    }
  };
  constexpr int NMF = FML * NB * FN;
  constexpr int NRD = 2 * (FML + NB * FN);  // two 16-byte halves per fragment
  auto interleave = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NMF; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < NRD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };

#pragma unroll
  for (int s = 0; s < kMxStages - 1; ++s) issue(s);
  asm volatile("s_waitcnt %0" ::"n"(waitcnt_imm(VM_AHEAD, 15)) : "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  Frags f[2];
  Scales sc;
  if constexpr (FML > 0) {
    read_frags(0, 0, f[0]);
    read_scales(0, sc);
  }
  for (int kt = 0; kt < nk; ++kt) {
    issue(kt + kMxStages - 1);
    if constexpr (FML > 0) {
      read_frags(kt, 1, f[1]);
      mfmas(f[0], sc, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, NLD, 0);
      interleave();
    }
    asm volatile("s_waitcnt %0" ::"n"(waitcnt_imm(VM_AHEAD, 0)) : "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if constexpr (FML > 0) {
      // stage kt+1's first fragments (on the last step: a duplicate of the
      // last stage, loaded by the clamped issue above, and never used)
      const Scales cur = sc;
      read_frags(kt + 1, 0, f[0]);
      read_scales(kt + 1, sc);
      mfmas(f[1], cur, 1);
      interleave();
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <int BN, int EPI>
__global__ __launch_bounds__(256) void gemm_mx_kernel(const MxGemmArgs args) {
  constexpr int BM = kMxBM;
  constexpr int NB = (EPI == kEpiSwiGLU) ? 2 : 1;
  constexpr int BROWS = NB * BN;
  constexpr int WTM = BM / 2, WTN = BN / 2;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int ROWS_PER_LD = 1024 / kRB;
  constexpr int AI = BM / (4 * ROWS_PER_LD), BI = BROWS / (4 * ROWS_PER_LD);
  constexpr int STAGE = (BM + BROWS) * (kRB + kSB);

  __shared__ __attribute__((aligned(1024))) char smem[kMxStages * STAGE];

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave / 2, wn = wave % 2;

  const int n_blocks = (args.N + BN - 1) / BN;
  const int W = *args.tile_count * n_blocks;
  const int chunk = (W + kXcds - 1) / kXcds;
  const int local = static_cast<int>(blockIdx.x) / kXcds;
  if (local >= chunk) return;
  const int w = (static_cast<int>(blockIdx.x) % kXcds) * chunk + local;
  if (w >= W) return;
  const int4 g = args.tiles[w / n_blocks];
  const int nt = g.x >> 10, first = g.w;
  const int lw = w - first * n_blocks;
  const int nb = lw / nt;
  const int4 t = args.tiles[first + lw % nt];
  const int e = t.x & 1023;
  const int64_t p0 = t.y;
  const int nrows = t.z;
  const int n0 = nb * BN;
  const int K = args.K, KS = K / 32;

  constexpr int CH = kRB / 16;
  uint32_t a_off[AI];
#pragma unroll
  for (int j = 0; j < AI; ++j) {
    const int row = ROWS_PER_LD * (wave * AI + j) + lane / CH;
    const int c = (lane % CH) ^ ((row / (256 / kRB)) & (CH - 1));
    const int64_t p = p0 + (row < nrows ? row : nrows - 1);
    const int64_t arow = (p - args.a_sub) % args.a_mod;
    a_off[j] = static_cast<uint32_t>(arow * K + c * 16);
  }
  uint32_t b_off[BI];
#pragma unroll
  for (int j = 0; j < BI; ++j) {
    const int row = ROWS_PER_LD * (wave * BI + j) + lane / CH;
    const int c = (lane % CH) ^ ((row / (256 / kRB)) & (CH - 1));
    const int half = row / BN;
    int n = n0 + (row - half * BN);
    n = n < args.N ? n : args.N - 1;
    b_off[j] = static_cast<uint32_t>(static_cast<int64_t>(n) * K + c * 16);
  }
  // scale words: wave w loads the words of A rows 64 w + lane and of B stage
  // rows 64 w + lane (the gate half for waves 0-1 and the up half for 2-3
  // when NB == 2)
  uint32_t as_off, bs_off;
  {
    const int row = wave * 64 + lane;
    const int64_t p = p0 + (row < nrows ? row : nrows - 1);
    as_off = static_cast<uint32_t>(((p - args.a_sub) % args.a_mod) * KS);
    const int half = row / BN;
    int n = n0 + (row - half * BN);
    n = n < args.N ? n : args.N - 1;
    bs_off = static_cast<uint32_t>(static_cast<int64_t>(n) * KS);
  }
  constexpr int kRsrcWord3 = 0x00020000;
  MxSrc src;
  src.a = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(args.A), 0, static_cast<int>(args.a_rows * K),
                                            kRsrcWord3);
  src.as = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(args.As), 0, static_cast<int>(args.a_rows * KS),
                                             kRsrcWord3);
  const int b_bytes = args.N * K, bs_bytes = args.N * KS;
  src.b0 = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(args.B0 + static_cast<int64_t>(e) * b_bytes), 0,
                                             b_bytes, kRsrcWord3);
  src.bs0 = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(args.Bs0 + static_cast<int64_t>(e) * bs_bytes), 0,
                                              bs_bytes, kRsrcWord3);
  if constexpr (NB == 2) {
    src.b1 = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(args.B1 + static_cast<int64_t>(e) * b_bytes), 0,
                                               b_bytes, kRsrcWord3);
    src.bs1 = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(args.Bs1 + static_cast<int64_t>(e) * bs_bytes),
                                                0, bs_bytes, kRsrcWord3);
  } else {
    src.b1 = src.b0;
    src.bs1 = src.bs0;
  }
  f32x16_t acc[NB][FM][FN];
#pragma unroll
  for (int h = 0; h < NB; ++h)
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) acc[h][fm][fn] = f32x16_t{};

  int fm_live = (nrows - wm * WTM + 31) / 32;
  fm_live = fm_live < 0 ? 0 : (fm_live > FM ? FM : fm_live);
  const int nk = K / kMxStageK;
  switch (fm_live) {
#define MOE_CASE(n)                                                                                         \
  case n:                                                                                                   \
    if constexpr (n <= FM)                                                                                  \
      k_loop_mx<BN, NB, n, FM, FN, AI, BI>(smem, src, a_off, b_off, as_off, bs_off, nk, nrows, tid, wm, wn, acc); \
    break;
    MOE_CASE(0)
    MOE_CASE(1)
    MOE_CASE(2)
    MOE_CASE(3)
    MOE_CASE(4)
#undef MOE_CASE
    default:
      break;
  }

  // ---- epilogue: lane holds column (lane % 32) and rows 8*(r/4) + 4*(lane/32) + r%4 ----
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    if (fm >= fm_live) continue;  // wave-uniform
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int col = n0 + wn * WTN + fn * 32 + (lane & 31);
      const bool col_ok = n0 + wn * WTN + fn * 32 < args.N;  // N % 32 == 0: a 32-column block is all in or out
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row_t = wm * WTM + fm * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        const int64_t p = p0 + row_t;
        if constexpr (EPI == kEpiSwiGLU) {
          const float gv = acc[0][fm][fn][r], uv = acc[1][fm][fn][r];
          const float v = gv / (1.0f + __expf(-gv)) * uv;
          // largest magnitude of the row's 32-column block: the 32 lanes of this half-wave
          float amax = fabsf(v);
#pragma unroll
          for (int m = 16; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 32));
          const int X = mx_scale_exponent(amax);
          if (row_t < nrows && col_ok) {
            const int64_t crow = p - args.c_sub;
            static_cast<uint8_t*>(args.C)[crow * args.ldc + col] = e4m3_from_f32(ldexpf(v, -X));
            if ((lane & 31) == 0) args.Cs[crow * (args.ldc / 32) + col / 32] = static_cast<uint8_t>(X + 127);
          }
        } else {
          if (row_t < nrows && col_ok) {
            const int64_t crow = args.c_idx ? static_cast<int64_t>(args.c_idx[p]) : p - args.c_sub;
            static_cast<uint16_t*>(args.C)[crow * args.ldc + col] = f32_to_bf16(acc[0][fm][fn][r]);
          }
        }
      }
    }
  }
}

template <int BN, int EPI>
hipError_t run_mx(const MxGemmArgs& a, hipStream_t stream) {
  const int64_t n_blocks = (a.N + BN - 1) / BN;
  const int64_t work = static_cast<int64_t>(a.max_tiles) * n_blocks;
  const int64_t grid = (work + kXcds - 1) / kXcds * kXcds;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  gemm_mx_kernel<BN, EPI><<<static_cast<unsigned>(grid), 256, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_mx(const MxGemmArgs& a, int epilogue, hipStream_t stream) {
  if (gemm_routed_bm() != kMxBM) return hipErrorInvalidValue;
  if (a.K % kMxStageK != 0 || a.N <= 0 || a.N % 32 != 0 || a.a_rows <= 0 || !a.tiles || !a.tile_count)
    return hipErrorInvalidValue;
  // buffer resources address at most 2^31 bytes per operand here
  if (a.a_rows * a.K >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  if (static_cast<int64_t>(a.N) * a.K >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  switch (epilogue) {
    case kEpiSwiGLU:
      if (!a.Cs || a.ldc % 32 != 0) return hipErrorInvalidValue;
      return run_mx<128, kEpiSwiGLU>(a, stream);
    case kEpiBF16:
      return run_mx<256, kEpiBF16>(a, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace moe
