// Grouped MXFP8 GEMMs of the expert FFNs on gfx950 scaled MFMA.
//
// MoK paper "Mixture-of-Kittens: MoE Megakernel for NVL72s", §3.4 "MXFP8
// Support": the routed experts run on MXFP8 operands; weights are quantised
// ahead of time and activations inside the dispatch (the gather) and inside
// the gated activation (the up/gate epilogue).  Operands are E4M3 bytes with
// one E8M0 scale per 32 consecutive elements along K: data row-major [rows][K],
// scales stage-major [K/128][rows][4] (the 4 scale bytes of a row's 128-wide K
// stage form one word, and the words of consecutive rows are adjacent).
//
// The matrix core does the block scaling itself: v_mfma_scale_f32_32x32x64_f8f6f4
// multiplies a 32x64 E4M3 block of A by a 64x32 block of B with one scale per
// row (column) and 32-wide K block, accumulating in fp32.  Lane l (h = l / 32)
// supplies row l % 32; its 32 bytes are K[16h, 16h+16) and K[32+16h, 32+16h+16)
// of the 64-wide step, and its scale byte is that row's scale of K block h.
//
// The pipeline is the bf16 kernel's: 256 x BN tiles, 8 waves, K stages of
// 128 bytes per row (two MFMA steps) in two LDS rings fed by direct
// buffer->LDS loads (activation rows one stage ahead, weight rows two), the
// same XOR swizzle, the same expert-major XCD-aware work order over the
// balanced tile list, 32-row blocks dealt to the wave row groups in turn.
// Each lane loads the scale words of its own fragment rows (4 bytes = the 4
// K blocks of a stage) straight into registers, one stage ahead; with the
// stage-major scale layout the 32 rows of a fragment share one 128-byte line
// (row-major scales would touch 32 lines per load and cost about a quarter of
// the up/gate kernel's time).  The K loop always runs from k = 0 in the same
// order, so a row's result does not depend on the tile or minibatch it falls
// in.
//
// Epilogues, staged through LDS so that rows leave in 16-byte stores: SwiGLU
// with MX quantisation of h along I (staged as fp32; one thread then
// quantises one 32-column block of a row), bf16 for the down projection,
// scattered to the row of the route it came from, and fp32 in 128-row bands
// (the shared expert's down projection when it runs in MXFP8: a dense GEMM
// through a tile list holding its T rows as one segment).

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "common.h"
#include "gemm_common.h"
#include "kernels.h"
#include "mx.h"

namespace moe {

namespace {

constexpr int kMxBM = 256;      // tile rows (the tile lists are built with gemm_mx_routed_bm())
constexpr int kMxStageK = 128;  // K elements (bytes) per stage row
constexpr int kRB = kMxStageK;  // bytes of one stage row
constexpr int kNSA = 2, kNSB = 3;  // ring slots: activation rows, weight rows
// 8 waves (4 x 2), two per SIMD: one wave's MFMAs issue while the other waits
constexpr int kWM = 4, kWN = 2;
constexpr int kNW = kWM * kWN;

struct MxSrc {
  __amdgpu_buffer_rsrc_t a, b0, b1, as, bs0, bs1;
};

__device__ __forceinline__ f32x16_t mfma_mx(const i32x8_t& a, const i32x8_t& b, const f32x16_t& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

__device__ __forceinline__ i32x8_t cat8(u32x4_t lo, u32x4_t hi) {
  return reinterpret_cast<i32x8_t>(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Row of the tile held by 32-row MFMA block fm of a wave in row group wm.
__device__ __forceinline__ int mx_tile_row(int wm, int fm) { return (fm * kWM + wm) * 32; }

// Per-lane scale sources: the byte offset of the scale row of each fragment
// row this lane supplies (A: block fm; B: half h, block fn).
template <int FM, int NB, int FN>
struct MxScaleOff {
  uint32_t a[FM];
  uint32_t b[NB][FN];
};

template <int FML, int NB, int FN>
struct MxScales {  // one stage's scale words (4 K blocks) of this lane's fragment rows
  uint32_t a[FML > 0 ? FML : 1];
  uint32_t b[NB][FN];
};

// The K loop of one workgroup (the bf16 kernel's ring protocol).  Per stage
// and wave: AI + BI 1 KB direct loads and FML + NB*FN 4-byte scale loads.
template <int BN, int NB, int FML, int FM, int FN, int AI, int BI>
__device__ __forceinline__ void k_loop_mx(char* smem, const MxSrc& src, const uint32_t (&a_off)[AI],
                                          const uint32_t (&b_off)[BI], int b_stage, const MxScaleOff<FM, NB, FN>& so,
                                          int nk,
                                          int a_rows, int as_stage, int bs_stage, int tid, int wm, int wn,
                                          f32x16_t (&acc)[NB][FM][FN]) {
  constexpr int BM = kMxBM, BROWS = NB * BN;
  constexpr int WTN = BN / kWN;
  constexpr int ASLOT = BM * kRB, BSLOT = BROWS * kRB;
  constexpr int ROWS_PER_LD = 1024 / kRB;
  static_assert(AI * ROWS_PER_LD * kNW == BM && BI * ROWS_PER_LD * kNW == BROWS, "data loads per wave per stage");
  static_assert(BI < 16, "vmcnt range");
  char* const sa0 = smem;
  char* const sb0 = smem + kNSA * ASLOT;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;  // wave index is uniform
  const int frag_row = lane & 31, frag_h = lane >> 5;

  // a stage past the last (in the prologue of a K range shorter than the
  // rings) loads the last stage again, into a free slot, so that the
  // prologue issues the same number of loads
  auto issue_a = [&](int kt, MxScales<FML, NB, FN>& sc) __attribute__((always_inline)) {
    const int kc = kt < nk ? kt : nk - 1;
    char* sa = sa0 + (kt % kNSA) * ASLOT;
#pragma unroll
    for (int j = 0; j < AI; ++j)
      dma16(src.a, sa + (wave * AI + j) * 1024, (wave * AI + j) * ROWS_PER_LD < a_rows ? a_off[j] : a_off[0],
            kc * kRB);
    // the scale words of stage kt (A and B) ride with the A loads
#pragma unroll
    for (int fm = 0; fm < FML; ++fm) sc.a[fm] = __builtin_amdgcn_raw_buffer_load_b32(src.as, so.a[fm], kc * as_stage, 0);
#pragma unroll
    for (int h = 0; h < NB; ++h)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        sc.b[h][fn] = __builtin_amdgcn_raw_buffer_load_b32(h ? src.bs1 : src.bs0, so.b[h][fn], kc * bs_stage, 0);
  };
  auto issue_b = [&](int kt) __attribute__((always_inline)) {
    const int kc = kt < nk ? kt : nk - 1;
    char* sb = sb0 + (kt % kNSB) * BSLOT;
#pragma unroll
    for (int j = 0; j < BI; ++j) {
      const int g = wave * BI + j;
      dma16((NB == 2 && g * ROWS_PER_LD >= BN) ? src.b1 : src.b0, sb + g * 1024, b_off[j], kc * b_stage);
    }
  };

  struct Frags {
    i32x8_t a[FML > 0 ? FML : 1];
    i32x8_t b[NB][FN];
  };
  // LDS byte offsets of this lane's fragment halves within a slot, per MFMA
  // step and half j.  The swizzle term depends on (row / 2) % 8 alone, which
  // all fragment rows of a lane share (they differ by multiples of 32), so a
  // fragment's halves sit at these offsets plus a constant: the reads need
  // no address registers of their own.
  static_assert((BN / 2) % 8 == 0, "fragment rows share the swizzle term");
  uint32_t abase[2][2], bbase[2][2];
#pragma unroll
  for (int step = 0; step < 2; ++step)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = step * 4 + frag_h + 2 * j;
      abase[step][j] = swz<kRB>(mx_tile_row(wm, 0) + frag_row, c);
      bbase[step][j] = swz<kRB>(wn * WTN + frag_row, c);
    }
  auto read_frags = [&](int kt, int step, Frags& f) __attribute__((always_inline)) {
    const char* sa = sa0 + (kt % kNSA) * ASLOT;
    const char* sb = sb0 + (kt % kNSB) * BSLOT;
    const char* a0 = sa + abase[step][0];
    const char* a1 = sa + abase[step][1];
    const char* b0 = sb + bbase[step][0];
    const char* b1 = sb + bbase[step][1];
    constexpr int kFragA = kWM * 32 * kRB;  // bytes between a lane's A fragment rows
#pragma unroll
    for (int fm = 0; fm < FML; ++fm)
      f.a[fm] = cat8(*reinterpret_cast<const u32x4_t*>(a0 + fm * kFragA),
                     *reinterpret_cast<const u32x4_t*>(a1 + fm * kFragA));
#pragma unroll
    for (int h = 0; h < NB; ++h)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int off = (h * BN + fn * 32) * kRB;
        f.b[h][fn] = cat8(*reinterpret_cast<const u32x4_t*>(b0 + off), *reinterpret_cast<const u32x4_t*>(b1 + off));
      }
  };
  // v_perm selector that replicates byte (2 step + h) of a scale word into all
  // four bytes: the K block of this lane's half of the step
  const uint32_t rep0 = (0 + frag_h) * 0x01010101u, rep1 = (2 + frag_h) * 0x01010101u;
  auto mfmas = [&](const Frags& f, const MxScales<FML, NB, FN>& sc, int step) __attribute__((always_inline)) {
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
  constexpr int NSC = FML + NB * FN;        // scale loads per stage
  // fragment reads spread under the MFMAs; in step 0 also the A and scale
  // loads, one per MFMA
  auto interleave = [&](int step, bool loads) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NMF; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (2 * NMF <= NRD || (i & 1) == 0)
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      else
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (loads && step == 0 && i < AI + NSC) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
  };

  MxScales<FML, NB, FN> sc_cur, sc_next;
  issue_a(0, sc_cur);
  issue_b(0);
  issue_b(1);
  asm volatile("s_waitcnt %0" ::"n"(waitcnt_imm(BI, 15)) : "memory");  // A(0), scales(0), B(0) landed
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  Frags f[2];
  if constexpr (FML > 0) read_frags(0, 0, f[0]);
  // One step per stage.  In the down projection (one B operand) the last two
  // steps do not refetch the last stage (those loads only kept the per-step
  // load count uniform for the counted wait): step nk-2 issues A(nk-1) but
  // no B, step nk-1 nothing, and both wait by draining the counter.  An item
  // (K = 2048, 16 stages) thereby loses 3 of its 35 stage loads: 7% off the
  // step's time.  The up/gate (56 stages) keeps the uniform steps: the extra
  // code of the tail cost it 3-5%, more than its 3 refetches of 59.
  auto step = [&](int kt, auto load_a, auto load_b) __attribute__((always_inline)) {
    constexpr bool kA = decltype(load_a)::value, kB = decltype(load_b)::value;
    if constexpr (kA) issue_a(kt + 1, sc_next);
    if constexpr (FML > 0) {
      read_frags(kt, 1, f[1]);
      mfmas(f[0], sc_cur, 0);
      interleave(0, kA);
    }
    if constexpr (kB) issue_b(kt + 2);
    // A(kt+1), its scales and B(kt+1) have landed (B(kt+2) may still be in
    // flight) and this wave's reads of stage kt are done
    if constexpr (kB)
      asm volatile("s_waitcnt %0" ::"n"(waitcnt_imm(BI, 0)) : "memory");
    else
      asm volatile("s_waitcnt %0" ::"n"(waitcnt_imm(0, 0)) : "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if constexpr (FML > 0) {
      // stage kt+1's first fragments (past the last stage: a slot whose
      // data is never used)
      read_frags(kt + 1, 0, f[0]);
      mfmas(f[1], sc_cur, 1);
      interleave(1, false);
    }
    if constexpr (kA) sc_cur = sc_next;
  };
  if constexpr (NB == 1) {
    int kt = 0;
    for (; kt < nk - 2; ++kt) step(kt, std::true_type{}, std::true_type{});
    if (kt == nk - 2) step(kt++, std::true_type{}, std::false_type{});
    step(kt, std::false_type{}, std::false_type{});  // kt == nk - 1
  } else {
    // the same steps, written out: the compiler places its own waits on the
    // scale words differently when this loop goes through the step above,
    // and that measured 4-5% slower
    for (int kt = 0; kt < nk; ++kt) {
      issue_a(kt + 1, sc_next);
      if constexpr (FML > 0) {
        read_frags(kt, 1, f[1]);
        mfmas(f[0], sc_cur, 0);
        interleave(0, true);
      }
      issue_b(kt + 2);
      asm volatile("s_waitcnt %0" ::"n"(waitcnt_imm(BI, 0)) : "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if constexpr (FML > 0) {
        read_frags(kt + 1, 0, f[0]);
        mfmas(f[1], sc_cur, 1);
        interleave(1, false);
      }
      sc_cur = sc_next;
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no DMA may still target LDS when the workgroup ends
}

// One work item (row tile, N block): its K loop and its epilogue.  The
// workgroup's LDS is free on entry and on return.
template <int BN, int EPI>
__device__ __forceinline__ void gemm_mx_item(const MxGemmArgs& args, int w, int n_blocks, char* smem, int wave0) {
  constexpr int BM = kMxBM;
  constexpr int NB = (EPI == kEpiSwiGLU) ? 2 : 1;
  constexpr int BROWS = NB * BN;
  constexpr int WTN = BN / kWN;
  constexpr int FM = BM / kWM / 32, FN = WTN / 32;
  constexpr int ROWS_PER_LD = 1024 / kRB;
  constexpr int AI = BM / (kNW * ROWS_PER_LD), BI = BROWS / (kNW * ROWS_PER_LD);
  constexpr int LDS_BYTES = kNSA * BM * kRB + kNSB * BROWS * kRB;

  constexpr bool kItemLoop = EPI == kEpiBF16;  // resident workgroups walk several items
  const int tid = kItemLoop ? item_thread_index(wave0) : static_cast<int>(threadIdx.x);
  const int lane = tid & (kWave - 1), wave = kItemLoop ? wave0 : __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave / kWN, wn = wave % kWN;

  const int4 g = kItemLoop ? load_uniform(args.tiles + w / n_blocks) : args.tiles[w / n_blocks];
  const int nt = g.x >> 10, first = g.w;
  int nb, lt;
  grouped_item(w - first * n_blocks, nt, n_blocks, nb, lt);
  const int4 t = kItemLoop ? load_uniform(args.tiles + first + lt) : args.tiles[first + lt];
  const int e = t.x & 1023;
  const int64_t p0 = t.y;
  const int nrows = t.z;
  const int n0 = nb * BN;
  const int K = args.K, KS = K / 32;

  // ---- byte offsets of the 16-byte chunks this lane fetches ----
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
  // weights K-tiled: a stage's weight rows sit in one plane of N rows, kRB
  // bytes apart, and the next stage's plane follows
  const bool b_tiled = args.b_plane > 0;
  const int b_stage = b_tiled ? static_cast<int>(args.b_plane * kRB) : kRB;
  uint32_t b_off[BI];
#pragma unroll
  for (int j = 0; j < BI; ++j) {
    const int row = ROWS_PER_LD * (wave * BI + j) + lane / CH;
    const int c = (lane % CH) ^ ((row / (256 / kRB)) & (CH - 1));
    const int half = row / BN;
    int n = n0 + (row - half * BN);
    n = n < args.N ? n : args.N - 1;
    b_off[j] = b_tiled ? static_cast<uint32_t>(n * kRB + c * 16) : static_cast<uint32_t>(static_cast<int64_t>(n) * K + c * 16);
  }
  // ---- scale words of this lane's fragment rows in stage 0 (rows past the
  // tile or N are clamped; their products only reach dropped outputs); stage
  // kc's word sits kc * rows * 4 bytes further ----
  MxScaleOff<FM, NB, FN> so;
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    const int row = mx_tile_row(wm, fm) + (lane & 31);
    const int64_t p = p0 + (row < nrows ? row : nrows - 1);
    so.a[fm] = static_cast<uint32_t>(((p - args.a_sub) % args.a_mod) * 4);
  }
#pragma unroll
  for (int h = 0; h < NB; ++h)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      int n = n0 + wn * WTN + fn * 32 + (lane & 31);
      n = n < args.N ? n : args.N - 1;
      so.b[h][fn] = static_cast<uint32_t>(n * 4);
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

  // 32-row MFMA blocks of this wave that hold tile rows (wave-uniform)
  int fm_live = ((nrows + 31) / 32 - wm + kWM - 1) / kWM;
  fm_live = fm_live < 0 ? 0 : (fm_live > FM ? FM : fm_live);
  const int nk = K / kMxStageK;
  const int as_stage = static_cast<int>(args.a_rows * 4), bs_stage = args.N * 4;
  switch (fm_live) {
#define MOE_CASE(n)                                                                                         \
  case n:                                                                                                   \
    if constexpr (n <= FM)                                                                                  \
      k_loop_mx<BN, NB, n, FM, FN, AI, BI>(smem, src, a_off, b_off, b_stage, so, nk, nrows, as_stage, bs_stage, tid, \
                                            wm, wn, acc);                                                \
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

  // ---- epilogue, staged through LDS so that rows leave in 16-byte pieces ----
  // The MFMA layout gives lane l column l % 32 of rows 8*(r/4) + 4*(l/32) +
  // r%4 of each 32 x 32 block.
  __syncthreads();  // every wave is done with the K loop's LDS
  if constexpr (EPI == kEpiSwiGLU) {
    // SwiGLU, then MX quantisation of h along I, in two passes.  Pass 1: the
    // lanes write SiLU(g) * u of their entries to LDS as fp32.  Pass 2: each
    // thread takes one 32-column block of a row, finds its largest
    // magnitude and writes the 32 E4M3 bytes and the scale byte.  Nothing
    // crosses lanes and nothing branches per element.
    constexpr int VS = BN * 4 + 16;  // fp32 row stride: an odd number of 16-byte units
    static_assert(BM * VS <= LDS_BYTES, "staged tile fits");
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      if (fm >= fm_live) continue;  // wave-uniform
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int col_l = wn * WTN + fn * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row_t = mx_tile_row(wm, fm) + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
          *reinterpret_cast<float*>(smem + row_t * VS + col_l * 4) = silu_mul(acc[0][fm][fn][r], acc[1][fm][fn][r]);
        }
      }
    }
    __syncthreads();
    constexpr int BPR = BN / 32;  // 32-column blocks per row
    // consecutive threads take consecutive rows of one block column: with the
    // odd row stride their 16-byte reads fall on distinct banks
    for (int it = tid; it < nrows * BPR; it += 64 * kNW) {
      const int blk = it / nrows, row = it - blk * nrows;
      const int col = n0 + blk * 32;
      if (col >= args.N) continue;  // N % 32 == 0: a block is all in or out
      float v[32];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const f32x4_t q = *reinterpret_cast<const f32x4_t*>(smem + row * VS + blk * 128 + i * 16);
        v[4 * i] = q[0];
        v[4 * i + 1] = q[1];
        v[4 * i + 2] = q[2];
        v[4 * i + 3] = q[3];
      }
      u32x4_t lo, hi;
      const uint8_t sc = quantize32_f32(v, lo, hi);
      const int64_t p = p0 + row;
      const int64_t crow = args.c_idx ? static_cast<int64_t>(args.c_idx[p]) : p - args.c_sub;
      u32x4_t* d = reinterpret_cast<u32x4_t*>(static_cast<char*>(args.C) + crow * args.ldc + col);
      d[0] = lo;
      d[1] = hi;
      args.Cs[((col / kMxStageK) * args.cs_rows + (p - args.c_sub)) * 4 + (col / 32) % 4] = sc;
    }
  } else if constexpr (EPI == kEpiF32) {
    // fp32 rows (the shared expert's output): one 128-row band per 32-row
    // block index fm (block fm of the four row groups covers tile rows fm*128
    // .. fm*128+127), staged through LDS and copied out in 16-byte stores
    constexpr int CS = BN * 4 + 16;  // fp32 row stride of a staged band
    constexpr int BAND = kWM * 32;
    static_assert(BAND * CS <= LDS_BYTES, "staged band fits");
    constexpr int CPR = BN * 4 / 16;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      if (fm * BAND >= nrows) break;  // workgroup-uniform
      if (fm > 0) __syncthreads();    // the previous band's copy-out is done with the LDS
      if (fm < fm_live) {             // wave-uniform
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          const int col_l = wn * WTN + fn * 32 + (lane & 31);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row_b = wm * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
            *reinterpret_cast<float*>(smem + row_b * CS + col_l * 4) = acc[0][fm][fn][r];
          }
        }
      }
      __syncthreads();
      const int band_rows = min(BAND, nrows - fm * BAND);
      for (int idx = tid; idx < band_rows * CPR; idx += 64 * kNW) {
        const int row = idx / CPR, ch = idx - row * CPR;
        const int col = n0 + ch * 4;
        if (col >= args.N) continue;  // N % 32 == 0: a chunk is all in or out
        const int64_t p = p0 + fm * BAND + row;
        *reinterpret_cast<f32x4_t*>(static_cast<char*>(args.C) + ((p - args.c_sub) * args.ldc + col) * 4) =
            *reinterpret_cast<const f32x4_t*>(smem + row * CS + ch * 16);
      }
    }
  } else {
    constexpr int CS = BN * 2 + 16;  // bf16 row stride of the staged tile
    static_assert(BM * CS <= LDS_BYTES, "staged tile fits");
    constexpr int CPR = BN * 2 / 16;
    // Copy-out mapping: in pass `it`, wave w stores tile rows it * RSTEP +
    // w * RPI + lane / CPR.  A row table's entries are read once, before
    // any store (lane q * RPI + j of wave w holds tile row q * RSTEP + w *
    // RPI + j) and passed on by a cross-lane read: a table load inside the
    // store loop would wait for all earlier stores (one counter tracks both).
    constexpr int RPI = 64 / CPR, RSTEP = RPI * kNW;
    static_assert(64 % CPR == 0 && BM <= 64 * kNW, "copy-out mapping");
    int row_entry = 0;
    if (args.c_idx) {
      const int r = (lane / RPI) * RSTEP + wave * RPI + lane % RPI;
      if (r < nrows) row_entry = args.c_idx[p0 + r];
    }
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      if (fm >= fm_live) continue;  // wave-uniform
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int col_l = wn * WTN + fn * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row_t = mx_tile_row(wm, fm) + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
          *reinterpret_cast<uint16_t*>(smem + row_t * CS + col_l * 2) = f32_to_bf16(acc[0][fm][fn][r]);
        }
      }
    }
    __syncthreads();
    for (int it = 0; it * RSTEP < nrows; ++it) {
      const int row = it * RSTEP + wave * RPI + lane / CPR, ch = lane % CPR;
      const int entry = args.c_idx ? __shfl(row_entry, it * RPI + lane / CPR) : 0;
      const int col = n0 + ch * 8;
      if (row >= nrows || col >= args.N) continue;  // N % 32 == 0: a chunk is all in or out
      const int64_t p = p0 + row;
      const int64_t crow = args.c_idx ? static_cast<int64_t>(entry) : p - args.c_sub;
      // the rows are next read by the combine, long after they leave the
      // caches: non-temporal stores
      __builtin_nontemporal_store(*reinterpret_cast<const u32x4_t*>(smem + row * CS + ch * 16),
                                  reinterpret_cast<u32x4_t*>(static_cast<char*>(args.C) + (crow * args.ldc + col) * 2));
    }
  }
}

// Work items are cut into 8 contiguous runs, one per XCD: runs of equal item
// count, or the list's cost-balanced runs (tile_runs) when it comes with
// them.  Workgroup b takes item b / 8 of the run of XCD b mod 8,
// and the grid holds, per XCD, as many workgroups as the longest run may have
// items.  The down projection instead launches only as many workgroups as fit
// on the chip at once, and they walk their XCD's run side by side (workgroup
// b takes items b / 8, b / 8 + G, ... with G workgroups per XCD), so that one
// item's output stores drain under the next item's first loads.  (A loop over
// items in the up/gate kernel measured 5% slower: it raises its register
// pressure.)
template <int BN, int EPI>
__global__ __launch_bounds__(64 * kNW) void gemm_mx_kernel(const MxGemmArgs args) {
  constexpr int NB = (EPI == kEpiSwiGLU) ? 2 : 1;
  __shared__ __attribute__((aligned(1024))) char smem[kNSA * kMxBM * kRB + kNSB * NB * BN * kRB];
  const int n_blocks = (args.N + BN - 1) / BN;
  const int xcd = static_cast<int>(blockIdx.x) % kXcds;
  int run0, len;
  if (args.tile_runs) {  // positions in 1/kTileRunFrac of a tile
    run0 = static_cast<int>(static_cast<int64_t>(__builtin_amdgcn_readfirstlane(args.tile_runs[xcd])) * n_blocks /
                            kTileRunFrac);
    len = static_cast<int>(static_cast<int64_t>(__builtin_amdgcn_readfirstlane(args.tile_runs[xcd + 1])) * n_blocks /
                           kTileRunFrac) -
          run0;
  } else {
    const int W = *args.tile_count * n_blocks;
    const int chunk = (W + kXcds - 1) / kXcds;
    run0 = xcd * chunk;
    len = W - run0 < chunk ? W - run0 : chunk;
  }
  const int first = static_cast<int>(blockIdx.x) / kXcds;
  const int per_xcd = static_cast<int>(gridDim.x) / kXcds;  // the grid is a multiple of kXcds
  const int wave0 = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  if constexpr (EPI != kEpiBF16) {
    if (first < len) gemm_mx_item<BN, EPI>(args, run0 + first, n_blocks, smem, wave0);
  } else {
    for (int local = first; local < len; local += per_xcd) {
      // the previous item's copy-out has read the LDS before this item's loads refill it
      if (local > first) __syncthreads();
      gemm_mx_item<BN, EPI>(args, __builtin_amdgcn_readfirstlane(run0 + local), n_blocks, smem, wave0);
    }
  }
}

template <int BN, int EPI>
hipError_t run_mx(const MxGemmArgs& a, hipStream_t stream) {
  const int64_t n_blocks = (a.N + BN - 1) / BN;
  const int64_t work = static_cast<int64_t>(a.max_tiles) * n_blocks;
  if (work <= 0) return hipSuccess;
  if (work > 0x7ffffff0) return hipErrorInvalidValue;
  auto kernel = gemm_mx_kernel<BN, EPI>;
  // resident workgroups walk several items only for the down projection,
  // whose items end in large output stores; the up/gate items measured faster
  // one per workgroup, with room for balanced runs of up to tile_run_cap
  // tiles on every XCD
  int64_t cap = a.tile_runs ? int64_t(kXcds) * tile_run_cap(a.max_tiles) * n_blocks : work;
  if (EPI == kEpiBF16) {
    static std::atomic<int64_t> resident_cache{0};
    int64_t resident = resident_cache.load(std::memory_order_relaxed);
    if (resident <= 0) {
      resident = resident_workgroups(reinterpret_cast<const void*>(kernel), 64 * kNW);
      if (resident <= 0) return hipErrorInvalidValue;
      resident_cache.store(resident, std::memory_order_relaxed);
    }
    cap = std::min(work, resident);
  }
  const int64_t grid = (cap + kXcds - 1) / kXcds * kXcds;
  kernel<<<static_cast<unsigned>(grid), 64 * kNW, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

int gemm_mx_routed_bm() { return kMxBM; }

hipError_t launch_gemm_mx(const MxGemmArgs& a, int epilogue, hipStream_t stream) {
  if (a.K % kMxStageK != 0 || a.N <= 0 || a.N % 32 != 0 || a.a_rows <= 0 || !a.tiles || !a.tile_count)
    return hipErrorInvalidValue;
  // buffer resources address at most 2^31 bytes per operand here
  if (a.a_rows * a.K >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  if (static_cast<int64_t>(a.N) * a.K >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  if (a.b_plane != 0 && a.b_plane != a.N) return hipErrorInvalidValue;  // K-tiled weights: planes of all N rows
  // 16-byte output stores: the base and the row strides keep 16-byte alignment
  if (reinterpret_cast<uintptr_t>(a.C) % 16 != 0) return hipErrorInvalidValue;
  switch (epilogue) {
    case kEpiSwiGLU:
      // h scales are stage-major [ldc/128][cs_rows][4]
      if (!a.Cs || a.ldc % kMxStageK != 0 || a.cs_rows <= 0 || a.cs_rows * a.ldc >= (int64_t(1) << 31))
        return hipErrorInvalidValue;
      return run_mx<128, kEpiSwiGLU>(a, stream);
    case kEpiBF16:
      if (a.ldc % 8 != 0) return hipErrorInvalidValue;
      return run_mx<256, kEpiBF16>(a, stream);
    case kEpiF32:  // rows in tile order only (no row table)
      if (a.ldc % 4 != 0 || a.c_idx) return hipErrorInvalidValue;
      return run_mx<256, kEpiF32>(a, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace moe
