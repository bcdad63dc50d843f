// Grouped bf16 GEMMs of the expert FFNs on gfx950 MFMA.
//
// MoK paper "Mixture-of-Kittens: MoE Megakernel for NVL72s", §2.1: an
// expert's FFN is two input projections (up, gate) combined through a gated
// activation, then an output (down) projection; the MoK blog's notation makes
// the gate SiLU (SwiGLU).  The
// routed experts run as expert-grouped GEMMs over expert-contiguous row tiles
// of the ring buffer (§3.1, condition 3: rows of one expert sit contiguously,
// so no local reordering precedes the GEMMs).
//
// One workgroup (4 waves) computes a BM x BN output tile with
// v_mfma_f32_32x32x16_bf16: both operands are K-contiguous (rows of the
// activations and rows of the weights), so every lane feeds the matrix core
// with one 16-byte LDS read per operand.  Tiles of K = 64 are staged through
// LDS, double-buffered, with the next tile's global loads in flight while the
// current one is multiplied.  The K loop always runs in the same order from
// k = 0 and there is no split-K, so a row's result does not depend on which
// tile or minibatch it falls in.
//
// Epilogues: SwiGLU (gate and up tiles share the output coordinates; h =
// SiLU(g) * u rounded to bf16), plain bf16 store (routed down projection,
// optionally scattered to the row of the route it came from) and fp32 store
// (shared expert output, router logits).

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kBK = 64;
constexpr int kLdsLd = kBK + 8;  // padded LDS row (bf16 elements): conflict-free 16-byte reads

template <int BM, int BN, int WM, int WN, int EPI>
__global__ __launch_bounds__(256) void gemm_kernel(const GemmArgs args) {
  constexpr int NB = (EPI == kEpiSwiGLU) ? 2 : 1;  // B halves (gate, up)
  constexpr int BROWS = NB * BN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int A_LD = BM / 32, B_LD = BROWS / 32;  // 16-byte loads per thread per K tile
  static_assert(WM * WN == 4, "4 waves per workgroup");
  static_assert(FM >= 1 && FN >= 1 && BM % 32 == 0 && BROWS % 32 == 0, "tile shape");

  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (BM + BROWS) * kLdsLd];

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int wm = wave / WN, wn = wave % WN;

  const int n_blocks = (args.N + BN - 1) / BN;
  const int tcount = args.tiles ? *args.tile_count : (args.dense_rows + BM - 1) / BM;
  const int bid = blockIdx.x;
  if (bid >= tcount * n_blocks) return;
  const int tile = bid % tcount, nb = bid / tcount;
  int e, nrows;
  int64_t p0;
  if (args.tiles) {
    const int4 t = args.tiles[tile];
    e = t.x;
    p0 = t.y;
    nrows = t.z;
  } else {
    e = 0;
    p0 = static_cast<int64_t>(tile) * BM;
    nrows = args.dense_rows - static_cast<int>(p0) < BM ? args.dense_rows - static_cast<int>(p0) : BM;
  }
  const int n0 = nb * BN;
  const int K = args.K;

  // global source of each 16-byte chunk this thread stages (rows past the
  // tile or past N are clamped onto valid rows; their results are dropped)
  const int lrow = tid >> 3, lcol = (tid & 7) * 8;
  const uint16_t* a_src[A_LD];
#pragma unroll
  for (int it = 0; it < A_LD; ++it) {
    const int i = lrow + 32 * it;
    const int64_t p = p0 + (i < nrows ? i : nrows - 1);
    const int64_t arow = (p - args.a_sub) % args.a_mod;
    a_src[it] = args.A + arow * args.lda + lcol;
  }
  const uint16_t* b_src[B_LD];
#pragma unroll
  for (int it = 0; it < B_LD; ++it) {
    const int i = lrow + 32 * it;
    const int half = i / BN;
    int n = n0 + (i - half * BN);
    n = n < args.N ? n : args.N - 1;
    const uint16_t* base = (NB == 2 && half) ? args.B1 : args.B0;
    b_src[it] = base + static_cast<int64_t>(e) * args.b_expert_stride + static_cast<int64_t>(n) * K + lcol;
  }

  u32x4_t ra[A_LD], rb[B_LD];
#define MOE_GLOAD(kt)                                                                          \
  do {                                                                                         \
    _Pragma("unroll") for (int it = 0; it < A_LD; ++it) ra[it] =                               \
        *reinterpret_cast<const u32x4_t*>(a_src[it] + (kt) * kBK);                               \
    _Pragma("unroll") for (int it = 0; it < B_LD; ++it) rb[it] =                               \
        *reinterpret_cast<const u32x4_t*>(b_src[it] + (kt) * kBK);                               \
  } while (0)
#define MOE_SSTORE(buf)                                                                        \
  do {                                                                                         \
    uint16_t* as_ = smem + (buf) * (BM + BROWS) * kLdsLd;                                      \
    uint16_t* bs_ = as_ + BM * kLdsLd;                                                         \
    _Pragma("unroll") for (int it = 0; it < A_LD; ++it)                                        \
        *reinterpret_cast<u32x4_t*>(as_ + (lrow + 32 * it) * kLdsLd + lcol) = ra[it];            \
    _Pragma("unroll") for (int it = 0; it < B_LD; ++it)                                        \
        *reinterpret_cast<u32x4_t*>(bs_ + (lrow + 32 * it) * kLdsLd + lcol) = rb[it];            \
  } while (0)

  f32x16_t acc[NB][FM][FN];
#pragma unroll
  for (int h = 0; h < NB; ++h)
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) acc[h][fm][fn] = f32x16_t{};

  const int nk = K / kBK;
  MOE_GLOAD(0);
  MOE_SSTORE(0);
  __syncthreads();
  const int frag_row = lane & 31, frag_k = (lane >> 5) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) MOE_GLOAD(kt + 1);
    const uint16_t* as = smem + cur * (BM + BROWS) * kLdsLd;
    const uint16_t* bs = as + BM * kLdsLd;
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 16) {
      bf16x8_t af[FM], bfr[NB][FN];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
        af[fm] = *reinterpret_cast<const bf16x8_t*>(as + (wm * WTM + fm * 32 + frag_row) * kLdsLd + kk + frag_k);
#pragma unroll
      for (int h = 0; h < NB; ++h)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
          bfr[h][fn] = *reinterpret_cast<const bf16x8_t*>(
              bs + (h * BN + wn * WTN + fn * 32 + frag_row) * kLdsLd + kk + frag_k);
#pragma unroll
      for (int h = 0; h < NB; ++h)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
          for (int fn = 0; fn < FN; ++fn)
            acc[h][fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[fm], bfr[h][fn], acc[h][fm][fn], 0, 0, 0);
    }
    if (kt + 1 < nk) MOE_SSTORE(cur ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds column (lane % 32) and rows 8*(r/4) + 4*(lane/32) + r%4
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row_t = wm * WTM + fm * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
      if (row_t >= nrows) continue;
      const int64_t p = p0 + row_t;
      const int64_t crow = args.c_idx ? static_cast<int64_t>(args.c_idx[p]) : p - args.c_sub;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int col = n0 + wn * WTN + fn * 32 + (lane & 31);
        if (col >= args.N) continue;
        float v = acc[0][fm][fn][r];
        if constexpr (EPI == kEpiSwiGLU) {
          const float u = acc[NB - 1][fm][fn][r];
          v = v / (1.0f + __expf(-v)) * u;
        }
        if constexpr (EPI == kEpiF32) {
          static_cast<float*>(args.C)[crow * args.ldc + col] = v;
        } else {
          static_cast<uint16_t*>(args.C)[crow * args.ldc + col] = f32_to_bf16(v);
        }
      }
    }
  }
#undef MOE_GLOAD
#undef MOE_SSTORE
}

template <int BM, int BN, int WM, int WN, int EPI>
hipError_t run(const GemmArgs& a, hipStream_t stream) {
  const int tiles = a.tiles ? a.max_tiles : (a.dense_rows + BM - 1) / BM;
  const int n_blocks = (a.N + BN - 1) / BN;
  const int64_t grid = static_cast<int64_t>(tiles) * n_blocks;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  gemm_kernel<BM, BN, WM, WN, EPI><<<static_cast<unsigned>(grid), 256, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

constexpr int kRoutedBM = 128;

int gemm_routed_bm() { return kRoutedBM; }

int gemm_tiles_bound(int64_t rows, int groups, int bm) {
  // every group (expert segment) adds at most one partial tile
  const int64_t bound = (rows + bm - 1) / bm + (groups < rows ? groups : rows);
  return static_cast<int>(bound);
}

hipError_t launch_gemm(const GemmArgs& a, int epilogue, hipStream_t stream) {
  if (a.K % kBK != 0 || a.N <= 0) return hipErrorInvalidValue;
  switch (epilogue) {
    case kEpiSwiGLU:
      return run<kRoutedBM, 64, 2, 2, kEpiSwiGLU>(a, stream);
    case kEpiBF16:
      return run<kRoutedBM, 128, 2, 2, kEpiBF16>(a, stream);
    case kEpiF32:
      return run<kRoutedBM, 128, 2, 2, kEpiF32>(a, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace moe
