// Grouped bf16 GEMMs of the expert FFNs on gfx950 MFMA.
//
// MoK paper "Mixture-of-Kittens: MoE Megakernel for NVL72s", §2.1: an
// expert's FFN is two input projections (up, gate) combined through a gated
// activation, then an output (down) projection; the MoK blog's notation makes
// the gate SiLU (SwiGLU).  The routed experts run as expert-grouped GEMMs over
// expert-contiguous row tiles of the ring buffer (§3.1, condition 3: rows of
// one expert sit contiguously, so no local reordering precedes the GEMMs).
//
// Tiling.  A workgroup of 8 waves (two per SIMD, so that one wave's MFMAs
// issue while the other waits on a load or the barrier) computes a BM x BN
// output tile with v_mfma_f32_32x32x16_bf16; the waves form a WM x WN grid
// (4 x 2 for 256-row dense tiles, 2 x 4 for 320-row routed tiles), and the
// 32-row MFMA blocks of the tile are dealt to the row groups in turn.  Both
// operands are K-contiguous (activation rows and weight rows), so each lane
// feeds the matrix core with one 16-byte LDS read per operand.  K tiles of 64
// are staged through LDS rings by direct loads, each slot refilled as soon as
// its last reads are done: activation rows one stage ahead, weight rows two
// (they stream from HBM), or one where LDS cannot hold a third weight slot.
// The K loop always runs from k = 0 in the same order and there is no
// split-K, so a row's result does not depend on the tile or minibatch it
// falls in.
//
// Work order (routed).  The 256 MI355X CUs sit in 8 XCDs, each with its own
// L2, and workgroups are dealt to XCDs round-robin.  Work items are ordered
// expert-major, then by group of row tiles, then by N block, then by row tile
// in the group (grouped_item), and cut into 8 contiguous runs, one per XCD
// (balanced by an estimate of each tile's cost when the tile list comes with
// runs, else of equal item count), whose workgroups walk it side by side: so
// the row tiles of one (expert, N block) (which share the same weight rows)
// and the N-block tiles of one group (which share the same activation rows)
// run close together on one XCD and meet in its L2, while every weight byte
// is fetched from HBM about once
// for each group of row tiles.  With BM = 256 an expert's rows at the
// DeepSeek-V3 shape (about 256 per expert) mostly fit in one tile; 32-row
// blocks past the end of a tile are not multiplied.
//
// Epilogues: SwiGLU (gate and up tiles share output coordinates; h =
// SiLU(g) * u rounded to bf16), plain bf16 store (routed down projection,
// optionally scattered to the row of the route it came from, reusing the
// schedule table as in §3.1) and fp32 store (shared expert output, router
// logits).

#include <algorithm>
#include <atomic>
#include <cmath>
#include <type_traits>

#include "common.h"
#include "gemm_common.h"
#include "kernels.h"

namespace moe {

namespace {

#ifndef MOE_GEMM_BK
#define MOE_GEMM_BK 64
#endif
// Dense tiles: workgroups of 8 waves (4 row groups x 2 column groups, two
// waves per SIMD): while one wave of a SIMD waits on a load or a barrier the
// other issues its MFMAs.  Each wave owns a 64 x 128 block of a 256 x 256
// tile (128 accumulator registers).
constexpr int kWM = 4, kWN = 2;
constexpr int kStageK = MOE_GEMM_BK;    // K elements per pipeline stage (dense tiles)
constexpr int kLdsBytes = 160 * 1024;  // LDS of one CU (gfx950)

// LDS ring slots.  A slot is refilled at the barrier that ends the reads of
// the stage it held, so a ring of n slots issues its rows n - 1 stages ahead.
// The leads are set in K elements: weight rows stream from HBM and get twice
// the activation rows' lead; the weight ring gives up slots (down to the
// activation ring's count) where LDS would not hold it.
#ifndef MOE_GEMM_LEAD_A
#define MOE_GEMM_LEAD_A 64
#endif
#ifndef MOE_GEMM_LEAD_B
#define MOE_GEMM_LEAD_B 128
#endif
constexpr int ring_a_slots(int bk) { return 1 + MOE_GEMM_LEAD_A / bk; }
constexpr int ring_b_slots(int bk, int a_stage_bytes, int b_stage_bytes) {
  int n = 1 + MOE_GEMM_LEAD_B / bk;
  while (n > ring_a_slots(bk) && ring_a_slots(bk) * a_stage_bytes + n * b_stage_bytes > kLdsBytes) --n;
  return n;
}
// LDS bytes of both rings for a BM-row tile with brows weight rows per stage.
constexpr int ring_bytes(int bm, int brows, int bk) {
  return ring_a_slots(bk) * bm * bk * 2 + ring_b_slots(bk, bm * bk * 2, brows * bk * 2) * brows * bk * 2;
}


// Row of the tile held by 32-row MFMA block fm of a wave in row group wm:
// blocks are dealt to the WM row groups in turn, so that a partly filled
// tile keeps every wave busy.
template <int WM>
__device__ __forceinline__ int tile_row(int wm, int fm) {
  return (fm * WM + wm) * 32;
}

// The K loop of one workgroup.  BK-wide K tiles are staged through two LDS
// rings fed by direct buffer->LDS loads (lane l's 16 bytes land at base + 16 l,
// so one wave instruction fills 1 KB; each lane fetches the global chunk the
// swizzle maps to its slot): activation rows in 2 slots and weight rows in
// NSB slots, since weights stream from HBM and need the longer lead.  The
// 16-wide K sub-steps run back to back with the next sub-step's fragments read
// under the current MFMAs.  Before the last sub-step's MFMAs of stage kt the
// wave waits for A(kt+1) and B(kt+1) and passes the one barrier of the step;
// right after it, the slots stage kt used are refilled with A(kt+2) and
// B(kt+NSB), issued under those MFMAs while stage kt+1's first fragments are
// read.  FML = 32-row MFMA blocks of this wave that hold tile rows.
template <int BM, int BN, int WM, int WN, int NB, int FML, int FM, int FN, int BK, int AI, int BI>
__device__ __forceinline__ void k_loop(char* smem, const TileSrc& src, const uint32_t (&a_off)[AI],
                                       const uint32_t (&b_off)[BI], int nk, int a_rows, int a_stage, int b_stage,
                                       int tid, int wm, int wn, f32x16_t (&acc)[NB][FM][FN]) {
  constexpr int RB = BK * 2;  // bytes of one row of a stage
  constexpr int BROWS = NB * BN;
  constexpr int NSA = ring_a_slots(BK), NSB = ring_b_slots(BK, BM * RB, BROWS * RB);  // ring slots
  static_assert(NSA >= 2 && NSB >= NSA, "ring depths");
  constexpr int WTN = BN / WN;
  constexpr int KS = BK / 16;  // 16-wide K sub-steps per stage
  static_assert(KS >= 2, "fragment reads alternate between two register sets");
  constexpr int ROWS_PER_LD = 1024 / RB;
  static_assert(AI * ROWS_PER_LD * WM * WN == BM && BI * ROWS_PER_LD * WM * WN == BROWS,
                "DMA instructions per wave per stage");
  constexpr int ASLOT = BM * RB, BSLOT = BROWS * RB;
  char* const sa0 = smem;
  char* const sb0 = smem + NSA * ASLOT;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;  // wave index is uniform
  const int frag_row = lane & 31, frag_c = lane >> 5;

  // a stage past the last (in the prologue of a K range shorter than the
  // rings) loads the last stage again, into a free slot, so that the
  // prologue issues the same number of loads
  // a_stage, b_stage: bytes from one K stage of a row to the next (RB
  // row-major, a whole plane K-tiled)
  auto issue_a = [&](int kt) __attribute__((always_inline)) {
    const int ko = (kt < nk ? kt : nk - 1) * a_stage;
    char* sa = sa0 + (kt % NSA) * ASLOT;
    // A row groups past the tile are not fetched (their rows only feed dropped
    // outputs); a reload of the group's first row keeps the per-wave load
    // count, which the vmcnt waits rely on, the same for every wave
#pragma unroll
    for (int j = 0; j < AI; ++j)
      dma16(src.a, sa + (wave * AI + j) * 1024, (wave * AI + j) * ROWS_PER_LD < a_rows ? a_off[j] : a_off[0], ko);
  };
  // b_stage: bytes from one K stage of a weight row to the next (RB
  // row-major, a whole plane of N rows K-tiled)
  auto issue_b = [&](int kt) __attribute__((always_inline)) {
    const int ko = (kt < nk ? kt : nk - 1) * b_stage;
    char* sb = sb0 + (kt % NSB) * BSLOT;
#pragma unroll
    for (int j = 0; j < BI; ++j) {
      const int g = wave * BI + j;  // ROWS_PER_LD-row group of the B stage
      dma16((NB == 2 && g * ROWS_PER_LD >= BN) ? src.b1 : src.b0, sb + g * 1024, b_off[j], ko);
    }
  };
  using frag_a_t = bf16x8_t[FML > 0 ? FML : 1];
  using frag_b_t = bf16x8_t[NB][FN];
  auto read_frags = [&](int kt, int step, frag_a_t& af, frag_b_t& bfr) __attribute__((always_inline)) {
    const char* sa = sa0 + (kt % NSA) * ASLOT;
    const char* sb = sb0 + (kt % NSB) * BSLOT;
    const int c = step * 2 + frag_c;
#pragma unroll
    for (int fm = 0; fm < FML; ++fm)
      af[fm] = *reinterpret_cast<const bf16x8_t*>(sa + swz<RB>(tile_row<WM>(wm, fm) + frag_row, c));
#pragma unroll
    for (int h = 0; h < NB; ++h)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        bfr[h][fn] = *reinterpret_cast<const bf16x8_t*>(sb + swz<RB>(h * BN + wn * WTN + fn * 32 + frag_row, c));
  };
  auto mfmas = [&](const frag_a_t& af, const frag_b_t& bfr) __attribute__((always_inline)) {
#pragma unroll
    for (int fm = 0; fm < FML; ++fm)
#pragma unroll
      for (int h = 0; h < NB; ++h)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
          acc[h][fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[fm], bfr[h][fn], acc[h][fm][fn], 0, 0, 0);
  };
  constexpr int NMF = FML * NB * FN;  // MFMAs per 16-wide sub-step
  constexpr int NRD = FML + NB * FN;  // fragment reads per 16-wide sub-step
  // one fragment read under each MFMA; in the sub-step after the barrier
  // also the stage's loads (A, then B), one under each MFMA
  auto interleave = [&](int ks, bool loads) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NMF; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < NRD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (loads && ks == KS && i < AI + BI) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
  };

  // Ring protocol: a slot is refilled as soon as the barrier after its last
  // reads has passed.  At the barrier that ends stage kt's reads, A(kt+NSA)
  // goes to A slot kt % NSA and B(kt+NSB) to B slot kt % NSB.  The prologue
  // issues in the same order, as if the barriers of stages -NSB .. -1 had run.
  // Loads that may still be in flight once A(s) and B(s) have landed are the
  // ones issued after A(s): B(s-NSA+NSB) at the same barrier (unless NSB ==
  // NSA, when that is B(s) itself) and the NSA - 1 (prologue) or NSA - 2
  // (loop) later barriers' loads.
  constexpr int VM_AFTER = NSB > NSA ? BI : 0;
  constexpr int VM_FIRST = VM_AFTER + (NSA - 1) * (AI + BI);
  constexpr int VM_STAGE = VM_AFTER + (NSA - 2) * (AI + BI);
  static_assert(VM_FIRST < 64, "vmcnt range");
#pragma unroll
  for (int v = -NSB; v < 0; ++v) {
    if (v + NSA >= 0) issue_a(v + NSA);
    issue_b(v + NSB);
  }
  // A(0) and B(0) have landed
  asm volatile("s_waitcnt %0" ::"n"(waitcnt_imm(VM_FIRST, 15)) : "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  frag_a_t af[2];
  frag_b_t bf[2];
  if constexpr (FML > 0) read_frags(0, 0, af[0], bf[0]);
  auto step = [&](int kt, auto loads) __attribute__((always_inline)) {
    constexpr bool kLoads = decltype(loads)::value;
    if constexpr (FML > 0) {
#pragma unroll
      for (int ks = 0; ks + 1 < KS; ++ks) {
        read_frags(kt, ks + 1, af[(ks + 1) & 1], bf[(ks + 1) & 1]);
        mfmas(af[ks & 1], bf[ks & 1]);
        interleave(ks, kLoads);
      }
    }
    // A(kt+1) and B(kt+1) have landed and this wave's reads of stage kt are
    // done, before any wave refills a slot (in the tail, where fewer loads
    // are in flight than VM_STAGE counts on, by draining the counter)
    if constexpr (kLoads)
      asm volatile("s_waitcnt %0" ::"n"(waitcnt_imm(VM_STAGE, 0)) : "memory");
    else
      asm volatile("s_waitcnt %0" ::"n"(waitcnt_imm(0, 0)) : "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if constexpr (kLoads) {
      issue_a(kt + NSA);
      issue_b(kt + NSB);
    } else if constexpr (NSB > NSA) {
      if (kt + NSA < nk) issue_a(kt + NSA);  // a stage still to come (uniform branch)
    }
    if constexpr (FML > 0) {
      // past the last stage this reads a slot whose data is not used
      read_frags(kt + 1, 0, af[KS & 1], bf[KS & 1]);
      mfmas(af[(KS - 1) & 1], bf[(KS - 1) & 1]);
      interleave(KS, kLoads);
    }
  };
  // The last NSB steps issue no refetch of the last stage (the loads past it
  // only kept the count of loads per step uniform for the counted waits):
  // they load only the activation stages still to come, and wait by
  // draining the counter.  With both rings two slots deep every wait drains
  // it anyway.  The routed down item (K = 2048, 32 stages) thereby loses 2
  // of its 34 stage loads; a weight-gradient item (K = an expert's rows,
  // about 4 stages) 5 of its 13.
  int kt = 0;
  for (; kt < nk - NSB; ++kt) step(kt, std::true_type{});
  for (; kt < nk; ++kt) step(kt, std::false_type{});
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no DMA may still target LDS when the workgroup ends
}

// One work item (row tile, N block, K range) of the GEMM: its K loop and its
// epilogue.  The workgroup's LDS is free on entry and on return.
template <int BM, int BN, int WM, int WN, int EPI, bool ROUTED, int BK>
__device__ __forceinline__ void gemm_item(const GemmArgs& args, int w, int n_blocks, int S, char* smem, int wave0) {
  constexpr int NB = (EPI == kEpiSwiGLU) ? 2 : 1;  // B halves (gate, up)
  constexpr int BROWS = NB * BN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int RB = BK * 2;                                // bytes of one row of a stage
  constexpr int ROWS_PER_LD = 1024 / RB;                    // rows one 1 KB direct load fills
  constexpr int NW = WM * WN;                                                     // waves per workgroup
  constexpr int AI = BM / (NW * ROWS_PER_LD), BI = BROWS / (NW * ROWS_PER_LD);  // per wave per stage
  static_assert(FM >= 1 && FN >= 1 && AI * NW * ROWS_PER_LD == BM && BI * NW * ROWS_PER_LD == BROWS, "tile shape");

  constexpr bool kItemLoop = EPI == kEpiBF16 && ROUTED;  // resident workgroups walk several items
  const int tid = kItemLoop ? item_thread_index(wave0) : static_cast<int>(threadIdx.x);
  const int lane = tid & (kWave - 1), wave = kItemLoop ? wave0 : __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave / WN, wn = wave % WN;

  int e = 0, nrows, tile, nb, ks = 0, group = 0;
  int64_t p0;
  if constexpr (ROUTED) {
    // a tile of the expert group that owns item w
    const int4 g = kItemLoop ? load_uniform(args.tiles + w / n_blocks) : args.tiles[w / n_blocks];
    const int nt = g.x >> 10, first = g.w;
    int lt;
    grouped_item(w - first * n_blocks, nt, n_blocks, nb, lt);
    tile = first + lt;
    const int4 t = kItemLoop ? load_uniform(args.tiles + tile) : args.tiles[tile];
    e = t.x & 1023;
    p0 = t.y;
    nrows = t.z;
  } else {
    // dense: row tile outer, so the workgroups of one XCD share activation
    // rows in L2 and stream the (small) weight matrix; the K ranges of one
    // output tile are neighbours
    if (args.k_groups) {  // grouped K: the group's items are contiguous
      const int per = ((args.dense_rows + BM - 1) / BM) * n_blocks;
      group = w / per;
      w -= group * per;
    }
    ks = w % S;
    nb = (w / S) % n_blocks;
    tile = w / S / n_blocks;
    p0 = static_cast<int64_t>(tile) * BM;
    nrows = args.dense_rows - static_cast<int>(p0) < BM ? args.dense_rows - static_cast<int>(p0) : BM;
  }
  const int n0 = nb * BN;
  const int K = args.K;
  int k0 = ks * (K / S);  // first K element of this workgroup's range
  int nk = K / S / BK;    // its K stages
  if (!ROUTED && args.k_groups) {
    const int2 kg = args.k_groups[group];
    k0 = kg.x;
    nk = kg.y;
  }
  const int64_t ldb = args.ldb ? args.ldb : K;
  char* const cbase = static_cast<char*>(args.C) +
                      (ks * args.c_split_stride + group * args.c_group_stride) * (EPI == kEpiF32 ? 4 : 2);

  // ---- byte offsets of the 16-byte chunks this lane fetches ----
  // Direct load j of wave w fills rows ROWS_PER_LD (w * AI + j) + lane / CH of
  // a stage; the lane's slot is chunk lane % CH, so it fetches the global chunk
  // the swizzle maps there.  Rows past the tile are clamped onto its last row
  // and rows past N onto row N-1: their products only reach output rows and
  // columns that are dropped.
  constexpr int CH = RB / 16;
  // K-tiled operands (BK is the tiling's plane width): a stage's rows sit in
  // one plane, RB bytes apart, and the next stage's plane follows
  static_assert(BK == kTileK, "K stages are the tiling's planes");
  const bool a_tiled = args.a_plane > 0;
  const int a_stage = a_tiled ? static_cast<int>(args.a_plane * RB) : RB;
  uint32_t a_off[AI];
#pragma unroll
  for (int j = 0; j < AI; ++j) {
    const int row = ROWS_PER_LD * (wave * AI + j) + lane / CH;
    const int c = (lane % CH) ^ ((row / (256 / RB)) & (CH - 1));
    const int64_t p = p0 + (row < nrows ? row : nrows - 1);
    const int64_t arow = (p - args.a_sub) % args.a_mod;
    a_off[j] = a_tiled ? static_cast<uint32_t>(((k0 / BK) * args.a_plane + arow) * RB + c * 16)
                       : static_cast<uint32_t>((arow * args.lda + k0 + c * 8) * 2);
  }
  const bool b_tiled = args.b_plane > 0;
  const int b_stage = b_tiled ? static_cast<int>(args.b_plane * RB) : RB;
  uint32_t b_off[BI];
#pragma unroll
  for (int j = 0; j < BI; ++j) {
    const int row = ROWS_PER_LD * (wave * BI + j) + lane / CH;
    const int c = (lane % CH) ^ ((row / (256 / RB)) & (CH - 1));
    const int half = row / BN;
    int n = n0 + (row - half * BN);
    n = n < args.N ? n : args.N - 1;
    b_off[j] = b_tiled ? static_cast<uint32_t>(((k0 / BK) * args.b_plane + n) * RB + c * 16)
                       : static_cast<uint32_t>((static_cast<int64_t>(n) * ldb + k0 + c * 8) * 2);
  }
  constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit elements
  TileSrc src;
  src.a = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(args.A), 0, static_cast<int>(args.a_bytes),
                                            kRsrcWord3);
  const int b_bytes = static_cast<int>(args.N * ldb * 2);
  src.b0 = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(args.B0 + static_cast<int64_t>(e) * args.b_expert_stride), 0, b_bytes, kRsrcWord3);
  src.b1 = NB == 2 ? __builtin_amdgcn_make_buffer_rsrc(
                         const_cast<uint16_t*>(args.B1 + static_cast<int64_t>(e) * args.b_expert_stride), 0, b_bytes,
                         kRsrcWord3)
                   : src.b0;
  f32x16_t acc[NB][FM][FN];
#pragma unroll
  for (int h = 0; h < NB; ++h)
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) acc[h][fm][fn] = f32x16_t{};

  // 32-row MFMA blocks of this wave that hold tile rows (wave-uniform); the
  // K loop is instantiated per count so that its body is one straight block
  int fm_live = ((nrows + 31) / 32 - wm + WM - 1) / WM;
  fm_live = fm_live < 0 ? 0 : (fm_live > FM ? FM : fm_live);
  // an empty K range (a grouped-K group with no rows) skips the K loop: its
  // accumulators stay zero and the epilogue stores zeros
  switch (nk > 0 ? fm_live : -1) {
#define MOE_CASE(n)                                                                       \
  case n:                                                                                 \
    if constexpr (n <= FM)                                                                \
      k_loop<BM, BN, WM, WN, NB, n, FM, FN, BK, AI, BI>(smem, src, a_off, b_off, nk, nrows, a_stage, b_stage, tid, wm, \
                                                        wn, acc);                                               \
    break;
    MOE_CASE(0)
    MOE_CASE(1)
    MOE_CASE(2)
    MOE_CASE(3)
    MOE_CASE(4)
    MOE_CASE(5)
    MOE_CASE(6)
    MOE_CASE(7)
    MOE_CASE(8)
#undef MOE_CASE
    default:
      break;
  }

  // ---- epilogue, staged through LDS so that rows leave in 16-byte pieces ----
  // The MFMA layout gives lane l column l % 32 of rows 8*(r/4) + 4*(l/32) +
  // r%4; written straight out that is a 2- or 4-byte store per lane.  The
  // tile (or, for fp32 outputs, a band of it) is first written to LDS row by
  // row, then copied out by all threads in 16-byte chunks of whole rows.
  constexpr int ESZ = (EPI == kEpiF32) ? 4 : 2;  // bytes per output element
  constexpr int CS = BN * ESZ + 16;              // LDS row stride of the staged tile (padded against bank conflicts)
  constexpr int LDS_BYTES = ring_bytes(BM, BROWS, BK);
  constexpr int FMP_FIT = LDS_BYTES / CS / (WM * 32);  // 32-row blocks per row group that fit at once
  constexpr int FMP = FMP_FIT < FM ? FMP_FIT : FM;  // (the last band may hold fewer)
  constexpr int NBANDS = (FM + FMP - 1) / FMP;
  static_assert(FMP >= 1, "epilogue bands");
  constexpr int BAND = FMP * WM * 32;         // tile rows per band
  constexpr int CPR = BN * ESZ / 16;          // 16-byte chunks per staged row
  constexpr int EPC = 16 / ESZ;               // elements per chunk
  const bool vec_ok = ((args.ldc * ESZ) % 16 == 0) && (reinterpret_cast<uintptr_t>(cbase) % 16 == 0);
  // Copy-out mapping: in pass `it` of a band, wave w stores tile rows
  // it * RSTEP + w * RPI + lane / CPR, 16 bytes per lane.  Where output rows
  // come from a row table (the scatter of the routed down projection), each
  // row's entry is read once, before the first store: lane q * RPI + j of
  // wave w holds the entry of tile row q * RSTEP + w * RPI + j and passes it
  // on by a cross-lane read.  A table load inside the store loop would make
  // every pass wait for all earlier stores, since one counter tracks both.
  constexpr int RPI = 64 / CPR, RSTEP = RPI * NW;
  static_assert(64 % CPR == 0 && BM <= 64 * NW && BAND % RSTEP == 0, "copy-out mapping");
  int row_entry = 0;
  if (args.c_idx) {
    const int r = (lane / RPI) * RSTEP + wave * RPI + lane % RPI;
    if (r < nrows) row_entry = args.c_idx[p0 + r];
  }
  __syncthreads();  // every wave is done with the K loop's LDS
#pragma unroll
  for (int band = 0; band < NBANDS; ++band) {
#pragma unroll
    for (int fm = band * FMP; fm < (band + 1) * FMP && fm < FM; ++fm) {
      if (fm >= fm_live) continue;  // wave-uniform
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row_b = tile_row<WM>(wm, fm) - band * BAND + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          const int col_l = wn * WTN + fn * 32 + (lane & 31);
          float v = acc[0][fm][fn][r];
          if constexpr (EPI == kEpiSwiGLU) {
            const float u = acc[NB - 1][fm][fn][r];
            v = silu_mul(v, u);
          }
          if constexpr (EPI == kEpiF32) {
            *reinterpret_cast<float*>(smem + row_b * CS + col_l * 4) = v;
          } else {
            *reinterpret_cast<uint16_t*>(smem + row_b * CS + col_l * 2) = f32_to_bf16(v);
          }
        }
      }
    }
    __syncthreads();
    const int band_rows = min(BAND, nrows - band * BAND);
    for (int it = 0; it * RSTEP < band_rows; ++it) {
      const int row_b = it * RSTEP + wave * RPI + lane / CPR, ch = lane % CPR;
      const int entry = args.c_idx ? __shfl(row_entry, (band * BAND / RSTEP + it) * RPI + lane / CPR) : 0;
      const int col = n0 + ch * EPC;
      if (row_b >= band_rows || col >= args.N) continue;
      const int64_t p = p0 + band * BAND + row_b;
      const int64_t crow = args.c_idx ? static_cast<int64_t>(entry) : p - args.c_sub;
      const char* src_l = smem + row_b * CS + ch * 16;
      char* dst = cbase + (crow * args.ldc + col) * ESZ;
      if (vec_ok && col + EPC <= args.N) {
        // bf16 outputs and routed fp32 outputs take non-temporal stores:
        // most are read long after they leave the caches (the routed down
        // projection's rows by the combine, the weight gradients by the
        // optimiser), and the backward's routed fp32 rows (dh, dx_ring, 0.5
        // and 1.9 GB at the DeepSeek-V3 shape) do not fit the MALL anyway.
        // Measured: the routed down projection 3% faster, the weight
        // gradients 1.5%, the data-gradient GEMMs 2.7%, and no slower for
        // the shared expert's activations in the backward.  The dense fp32
        // outputs (the shared expert's, the router's logits) are read next
        // and keep plain stores.
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(src_l);
        if constexpr (EPI == kEpiBF16 || (EPI == kEpiF32 && ROUTED))
          __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(dst));
        else
          *reinterpret_cast<u32x4_t*>(dst) = v;
      } else {
        const int n_el = min(EPC, args.N - col);
        for (int e = 0; e < n_el; ++e) {
          if constexpr (ESZ == 4)
            reinterpret_cast<float*>(dst)[e] = reinterpret_cast<const float*>(src_l)[e];
          else
            reinterpret_cast<uint16_t*>(dst)[e] = reinterpret_cast<const uint16_t*>(src_l)[e];
        }
      }
    }
    if (band + 1 < NBANDS) __syncthreads();  // the next band reuses the LDS
  }
}

// Work items are split into 8 contiguous runs, one per XCD (workgroups are
// dealt to XCDs round-robin, so workgroup b sits on XCD b mod 8): runs of
// equal item count, or, for a routed list that comes with them, the list's
// cost-balanced runs (tile_runs).  Workgroup b takes item b / 8 of its XCD's
// run; the grid holds, per XCD, as many workgroups as the longest run may
// have items (tile_run_cap tiles' worth for balanced runs).
// The routed down projection instead launches only as many workgroups as fit
// on the chip at once, and workgroup b walks items b / 8, b / 8 + G, b / 8 +
// 2G, ... of its run (G = workgroups per XCD), so the XCD's workgroups still
// move through the run side by side: a workgroup that stays resident overlaps
// one item's output stores with the next item's first loads, where a fresh
// workgroup would first wait for the stores to drain and then for its loads.
// (A loop over items in the other kernels measured slower: it raises their
// register pressure.)
template <int BM, int BN, int WM, int WN, int EPI, bool ROUTED, int BK>
__global__ __launch_bounds__(64 * WM * WN) void gemm_kernel(const GemmArgs args) {
  constexpr int NB = (EPI == kEpiSwiGLU) ? 2 : 1;
  constexpr int LDS_BYTES = ring_bytes(BM, NB * BN, BK);
  static_assert(LDS_BYTES <= kLdsBytes, "LDS rings");
  __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];
  const int n_blocks = (args.N + BN - 1) / BN;
  const int xcd = static_cast<int>(blockIdx.x) % kXcds;
  int run0, len;
  if (ROUTED && args.tile_runs) {  // positions in 1/kTileRunFrac of a tile
    run0 = static_cast<int>(static_cast<int64_t>(__builtin_amdgcn_readfirstlane(args.tile_runs[xcd])) * n_blocks /
                            kTileRunFrac);
    len = static_cast<int>(static_cast<int64_t>(__builtin_amdgcn_readfirstlane(args.tile_runs[xcd + 1])) * n_blocks /
                           kTileRunFrac) -
          run0;
  } else {
    const int tcount = ROUTED ? *args.tile_count : (args.dense_rows + BM - 1) / BM;
    const int S = ROUTED ? 1 : args.k_splits;
    const int W = tcount * n_blocks * S * (!ROUTED && args.k_groups ? args.n_groups : 1);
    const int chunk = (W + kXcds - 1) / kXcds;
    run0 = xcd * chunk;
    len = W - run0 < chunk ? W - run0 : chunk;
  }
  const int S = ROUTED ? 1 : args.k_splits;  // K ranges (dense only), each with its own output plane
  const int first = static_cast<int>(blockIdx.x) / kXcds;
  const int per_xcd = static_cast<int>(gridDim.x) / kXcds;  // the grid is a multiple of kXcds
  const int wave0 = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  if constexpr (!(EPI == kEpiBF16 && ROUTED)) {
    if (first < len) gemm_item<BM, BN, WM, WN, EPI, ROUTED, BK>(args, run0 + first, n_blocks, S, smem, wave0);
  } else {
    for (int local = first; local < len; local += per_xcd) {
      // the previous item's copy-out has read the LDS before this item's loads refill it
      if (local > first) __syncthreads();
      gemm_item<BM, BN, WM, WN, EPI, ROUTED, BK>(args, __builtin_amdgcn_readfirstlane(run0 + local), n_blocks, S,
                                                 smem, wave0);
    }
  }
}

template <int BM, int BN, int WM, int WN, int EPI, bool ROUTED, int BK = kStageK>
hipError_t run(const GemmArgs& a, hipStream_t stream) {
  const int64_t tiles = ROUTED ? a.max_tiles : (a.dense_rows + BM - 1) / BM;
  const int64_t n_blocks = (a.N + BN - 1) / BN;
  const int64_t work = tiles * n_blocks * (ROUTED ? 1 : a.k_splits) * (!ROUTED && a.k_groups ? a.n_groups : 1);
  if (work <= 0) return hipSuccess;
  if (work > 0x7ffffff0) return hipErrorInvalidValue;
  auto kernel = gemm_kernel<BM, BN, WM, WN, EPI, ROUTED, BK>;
  // Resident workgroups walk several items only for the routed down
  // projection, whose items end in large output stores (a 320 x 256 bf16
  // tile after 32 K stages); elsewhere one item per workgroup measured as
  // fast or faster, and a list with balanced XCD runs gets room for runs of
  // up to tile_run_cap tiles on every XCD.
  int64_t cap = (ROUTED && a.tile_runs) ? int64_t(kXcds) * tile_run_cap(a.max_tiles) * n_blocks : work;
  if (EPI == kEpiBF16 && ROUTED) {
    static std::atomic<int64_t> resident_cache{0};
    int64_t resident = resident_cache.load(std::memory_order_relaxed);
    if (resident <= 0) {
      resident = resident_workgroups(reinterpret_cast<const void*>(kernel), 64 * WM * WN);
      if (resident <= 0) return hipErrorInvalidValue;
      resident_cache.store(resident, std::memory_order_relaxed);
    }
    cap = std::min(work, resident);
  }
  const int64_t grid = (cap + kXcds - 1) / kXcds * kXcds;
  kernel<<<static_cast<unsigned>(grid), 64 * WM * WN, 0, stream>>>(a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// The routed minibatch loop as one persistent kernel.
//
// MoK paper §3.2 ("Maximally Deferred Synchronization", "Kernel Fusion") and
// §3.4 ("Computation-Communication SM Tuning"): one resident kernel walks the
// minibatches; a set of workgroups moves rows (the gathers into the ring) while
// the rest run the expert GEMMs, and each step waits only for the steps whose
// data it reads, through device-side counters, instead of for everything
// launched before it.  On one GPU the gathers are local copies rather than
// pulls over a fabric, but the overlap is the same: while the GEMMs of
// minibatch m run, the rows of later minibatches are gathered, and the up/gate
// GEMM of minibatch m+1 runs beside the down GEMM of m.
//
// Steps and what each waits for (counters count finished work items):
//   G(m)  gather of minibatch m into ring slots p mod C: done by the memory
//         workgroups for m >= C/b (the first C/b are gathered before the
//         kernel, by the whole chip); waits until U(m - C/b) has read the
//         slots it overwrites;
//   U(m)  up/gate + SwiGLU of minibatch m into h buffer m mod H: waits for
//         G(m) and for D(m - H), the last reader of that h buffer;
//   D(m)  down projection of minibatch m: each item waits for the up/gate
//         items of its own row tile (all N blocks of that tile's h rows).
// H (2 to 4) follows the ring: C/b minibatches fit in it, so up/gate can run
// up to C/b - 1 minibatches ahead of down.  The GEMM workgroups take the U and
// D work items in the order U(0) .. U(H - 2), then for each m: U(m + H - 1),
// D(m), so that several up/gate steps fill the chip while the down steps
// trail them (a small minibatch's up/gate alone gives fewer work items than
// there are CUs, each as long as the whole K loop).  U(m + H - 1) waits for
// D(m - 1), the step just before it: every step waits only for steps earlier
// in that order (and G(m) only for U(m - C/b), earlier still).
// The items of a step are cut into 8 runs, one per XCD, as in the
// stream-ordered launches, and an XCD's GEMM workgroups take the items of its
// runs, in step order, from one queue (an atomic counter): a workgroup that
// finishes early takes the next item (with a single minibatch they are dealt
// round-robin instead, in the same order).  All workgroups are resident at once
// (the grid is the chip's occupancy), so the kernel cannot deadlock: the
// earliest unfinished item waits for nothing unfinished, and it is either
// running or the next item of its XCD's queue, which every item taken before
// it has finished and so left a workgroup free to take it.  A wait that spins
// past about a second (a workgroup that cannot be resident, for instance)
// sets MOE_DEVERR_PIPELINE and stops waiting, so the kernel always ends.
//
// Visibility: a finished step's writers drain their stores (s_waitcnt), pass a
// barrier, and one thread adds to the counter with an agent-scope release,
// which writes the XCD's L2 back; waiters poll with agent-scope acquires,
// which invalidate their caches before the data is read.  The work items are
// the stream-ordered path's own (gemm_item), so results are bitwise the same.
// ---------------------------------------------------------------------------
constexpr int kErrPipeline = 0x8;  // MOE_DEVERR_PIPELINE
constexpr int kSpinCap = 1 << 23;  // polls of about 0.1 us each

// Wait until *ctr >= target.  One lane polls with relaxed loads (which read
// past the caches and invalidate nothing), then one agent-scope acquire
// invalidates this CU's stale lines once, and a barrier releases the
// workgroup.  An acquire per poll would invalidate the caches the working
// GEMMs of the same XCD depend on at every poll (measured: 2-20x slower).
// Every wave of the workgroup must call this at the same point.
__device__ __forceinline__ void wait_count(int* ctr, int target, int* err) {
  if (target > 0 && threadIdx.x == 0) {
    for (int spins = 0;; ++spins) {
      if (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target) break;
      if ((spins & 63) == 63 &&
          (spins > kSpinCap || (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & kErrPipeline))) {
        raise_error(err, kErrPipeline);
        break;
      }
      __builtin_amdgcn_s_sleep(4);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
}

// This workgroup's writes are visible device-wide, then *ctr += n.
__device__ __forceinline__ void signal_count(int* ctr, int n) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's stores have completed
  __syncthreads();                                   // and every wave's
  if (threadIdx.x == 0) __hip_atomic_fetch_add(ctr, n, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

template <int BMU, int BNU, int WMU, int WNU, int BMD, int BND, int WMD, int WND>
__global__ __launch_bounds__(512) void pipeline_kernel(const PipeArgs pa) {
  static_assert(WMU * WNU == 8 && WMD * WND == 8, "8 waves");
  constexpr int LDS_U = ring_bytes(BMU, 2 * BNU, kStageK), LDS_D = ring_bytes(BMD, BND, kStageK);
  constexpr int LDS_BYTES = LDS_U > LDS_D ? LDS_U : LDS_D;
  static_assert(LDS_BYTES <= kLdsBytes, "LDS rings");
  __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];
  const int xcd = static_cast<int>(blockIdx.x) % kXcds, rx = static_cast<int>(blockIdx.x) / kXcds;
  const int mem_per_xcd = pa.n_mem / kXcds;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  const int lane = lane_id();
  const int64_t P = pa.offsets[pa.L] < pa.max_rows ? static_cast<int64_t>(pa.offsets[pa.L]) : pa.max_rows;
  const int nbu = (pa.up.N + BNU - 1) / BNU, nbd = (pa.down.N + BND - 1) / BND;
  const int64_t ring_mb = pa.C / pa.b;  // minibatches the ring holds
  auto n_items = [&](int m, int nb) { return __builtin_amdgcn_readfirstlane(pa.up.tile_count[m]) * nb; };

  if (rx < mem_per_xcd) {
    // ---- memory workgroup j: G(m) for m >= C/b ----
    const int j = rx * kXcds + xcd;
    for (int m = static_cast<int>(ring_mb); m < pa.n_mb; ++m) {
      wait_count(pa.upg + (m - ring_mb), n_items(static_cast<int>(m - ring_mb), nbu), pa.err);
      const int64_t lo = static_cast<int64_t>(m) * pa.b, hi = lo + pa.b < P ? lo + pa.b : P;
      const int n16 = pa.D / 8;  // 16-byte chunks per row
      for (int64_t p = lo + static_cast<int64_t>(j) * 8 + wave; p < hi; p += static_cast<int64_t>(pa.n_mem) * 8) {
        const int32_t route = pa.sched_src[p];
        const int64_t src_row = route / pa.k;
        if (route < 0 || src_row >= pa.src_rows) {  // a table not built by the schedule kernels
          if (lane == 0) raise_error(pa.err, kErrExpertRange);
          continue;
        }
        const uint4* __restrict__ s = reinterpret_cast<const uint4*>(pa.x_src + src_row * pa.D);
        uint4* __restrict__ d = reinterpret_cast<uint4*>(pa.ring + (p % pa.C) * pa.D);
        // eight 16-byte loads in flight per lane, then their stores; the
        // row's last chunks one at a time
        int c = lane;
        for (; c + 7 * kWave < n16; c += 8 * kWave) {
          const uint4 v0 = s[c], v1 = s[c + kWave], v2 = s[c + 2 * kWave], v3 = s[c + 3 * kWave];
          const uint4 v4 = s[c + 4 * kWave], v5 = s[c + 5 * kWave], v6 = s[c + 6 * kWave], v7 = s[c + 7 * kWave];
          d[c] = v0;
          d[c + kWave] = v1;
          d[c + 2 * kWave] = v2;
          d[c + 3 * kWave] = v3;
          d[c + 4 * kWave] = v4;
          d[c + 5 * kWave] = v5;
          d[c + 6 * kWave] = v6;
          d[c + 7 * kWave] = v7;
        }
        for (; c < n16; c += kWave) d[c] = s[c];
      }
      signal_count(pa.gathered + m, 1);
    }
    return;
  }

  // ---- GEMM workgroup: items of its XCD's runs, taken from the XCD's queue ----
  // The items of a step are cut into 8 runs, one per XCD, as in the
  // stream-ordered launches.  An XCD's runs of all steps, in step order, are
  // numbered consecutively; a GEMM workgroup takes the next number from its
  // XCD's queue head (one atomic), runs that item and takes another, so a
  // workgroup whose items were short takes more of them (an up/gate item runs
  // the whole K = D loop, a down item K = I).  Every workgroup of the XCD walks
  // the same steps to map its number to (step, item).  Which workgroup runs an
  // item does not change the item's arithmetic.
  // With one minibatch there is nothing to even out between steps, and the
  // numbers are dealt statically instead (the XCD's GEMM workgroup r takes
  // r, r + nr, ...), which saves each item the queue's atomic round trip.
  int* const head = pa.queue + xcd;
  int* const slot = pa.queue + kXcds + blockIdx.x;
  const int r = rx - mem_per_xcd, nr = static_cast<int>(gridDim.x) / kXcds - mem_per_xcd;
  const bool from_queue = pa.n_mb > 1;
  int dealt = r - nr;
  auto take = [&]() __attribute__((always_inline)) {
    if (!from_queue) return dealt += nr;
    __syncthreads();  // every wave has read the previous number
    if (threadIdx.x == 0)
      __hip_atomic_store(slot, __hip_atomic_fetch_add(head, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __syncthreads();
    return __builtin_amdgcn_readfirstlane(__hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
  };
  // this XCD's run of minibatch m's step with nb N blocks: [run0, run0 + len)
  auto xcd_run = [&](int m, int nb, int& run0) __attribute__((always_inline)) {
    if (pa.up.tile_runs) {
      const int32_t* tr = pa.up.tile_runs + static_cast<int64_t>(m) * kTileRunBounds;
      run0 = static_cast<int>(static_cast<int64_t>(__builtin_amdgcn_readfirstlane(tr[xcd])) * nb / kTileRunFrac);
      return static_cast<int>(static_cast<int64_t>(__builtin_amdgcn_readfirstlane(tr[xcd + 1])) * nb / kTileRunFrac) -
             run0;
    }
    const int n = n_items(m, nb), chunk = (n + kXcds - 1) / kXcds;
    run0 = xcd * chunk;
    const int run1 = min(n, (xcd + 1) * chunk);
    return run1 > run0 ? run1 - run0 : 0;
  };
  // row tile of item w of a step with nb N blocks (the decoding gemm_item uses)
  auto item_tile = [&](const int4* tiles, int w, int nb) __attribute__((always_inline)) {
    const int4 g = load_uniform(tiles + w / nb);
    int nblk, lt;
    grouped_item(w - g.w * nb, g.x >> 10, nb, nblk, lt);
    return g.w + lt;
  };
  auto up_item = [&](int m, int w) __attribute__((always_inline)) {
    // G(m) (memory workgroups, or before the kernel) and D(m - n_h), the
    // last reader of h buffer m mod n_h
    if (m >= ring_mb) wait_count(pa.gathered + m, pa.n_mem, pa.err);
    if (m >= pa.n_h) wait_count(pa.down_done + (m - pa.n_h), n_items(m - pa.n_h, nbd), pa.err);
    GemmArgs a = pa.up;
    a.tiles = pa.up.tiles + static_cast<int64_t>(m) * pa.up.max_tiles;
    a.tile_count = pa.up.tile_count + m;
    a.C = pa.h + static_cast<int64_t>(m % pa.n_h) * pa.b * pa.up.N;
    a.c_sub = static_cast<int64_t>(m) * pa.b;
    gemm_item<BMU, BNU, WMU, WNU, kEpiSwiGLU, true, kStageK>(a, w, nbu, 1, smem, wave);
    // the tile's h columns of this item are written: count it for the
    // tile's down items (a release: they read those h rows) and for the step
    // (relaxed: its waiters, the gathers, only need this item's loads of the
    // ring rows to have landed, which the wait on the load counter gives)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
      int* const tile_ctr = pa.upg_tile + static_cast<int64_t>(m) * pa.up.max_tiles;
      __hip_atomic_fetch_add(tile_ctr + item_tile(a.tiles, w, nbu), 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_add(pa.upg + m, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };
  auto down_item = [&](int m, int w) __attribute__((always_inline)) {
    GemmArgs a = pa.down;
    a.tiles = pa.up.tiles + static_cast<int64_t>(m) * pa.up.max_tiles;
    a.tile_count = pa.up.tile_count + m;
    a.A = pa.h + static_cast<int64_t>(m % pa.n_h) * pa.b * pa.up.N;
    a.a_sub = static_cast<int64_t>(m) * pa.b;
    // every up/gate item of this item's row tile: its h rows (the barrier
    // inside also lets this item refill the LDS)
    const int* const tile_ctr = pa.upg_tile + static_cast<int64_t>(m) * pa.up.max_tiles;
    wait_count(const_cast<int*>(tile_ctr) + item_tile(a.tiles, w, nbd), nbu, pa.err);
    gemm_item<BMD, BND, WMD, WND, kEpiBF16, true, kStageK>(a, w, nbd, 1, smem, wave);
    // relaxed, and with no wait on this item's output stores: the waiter
    // (up/gate of m + n_h) only needs this item's loads of the h rows it will
    // overwrite to have landed, and every wave's K loop ends with its loads
    // drained, before the barrier that opens the epilogue
    if (threadIdx.x == 0) __hip_atomic_fetch_add(pa.down_done + m, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  // up/gate runs `ahead` minibatches in front of down: U(0) .. U(ahead - 1),
  // then U(m + ahead), D(m) for each m
  const int ahead = pa.n_h - 1;
  int number = take(), base = 0;  // this workgroup's queue number; the XCD's items in the steps walked so far
  // (one loop per item kind, so that each loop holds one GEMM's code)
  auto step_up = [&](int m) __attribute__((always_inline)) {
    int run0;
    const int len = xcd_run(m, nbu, run0);
    for (; number < base + len; number = take()) up_item(m, run0 + number - base);
    base += len;
  };
  auto step_down = [&](int m) __attribute__((always_inline)) {
    int run0;
    const int len = xcd_run(m, nbd, run0);
    for (; number < base + len; number = take()) down_item(m, run0 + number - base);
    base += len;
  };
  for (int m = 0; m < ahead && m < pa.n_mb; ++m) step_up(m);
  for (int m = 0; m < pa.n_mb; ++m) {
    if (m + ahead < pa.n_mb) step_up(m + ahead);
    step_down(m);
  }
}

template <int BMU, int BNU, int WMU, int WNU, int BMD, int BND, int WMD, int WND>
hipError_t run_pipeline(const PipeArgs& pa, hipStream_t stream) {
  auto kernel = pipeline_kernel<BMU, BNU, WMU, WNU, BMD, BND, WMD, WND>;
  static std::atomic<int64_t> resident_cache{0};
  int64_t resident = resident_cache.load(std::memory_order_relaxed);
  if (resident <= 0) {
    resident = resident_workgroups(reinterpret_cast<const void*>(kernel), 512);
    if (resident <= 0) return hipErrorInvalidValue;
    resident_cache.store(resident, std::memory_order_relaxed);
  }
  const int64_t grid = resident / kXcds * kXcds;
  // GEMM workgroups on every XCD, and memory workgroups when some minibatch is gathered in the kernel
  if (pa.n_mem % kXcds || grid - pa.n_mem < kXcds) return hipErrorInvalidValue;
  if (pa.n_h < 2 || pa.n_h > kMaxPipeH || grid > kPipeMaxGrid || !pa.queue) return hipErrorInvalidValue;
  if (pa.n_mb > pa.C / pa.b && pa.n_mem <= 0) return hipErrorInvalidValue;
  kernel<<<static_cast<unsigned>(grid), 512, 0, stream>>>(pa);
  return hipGetLastError();
}

}  // namespace

// Routed tiles: 320 rows on a 2 x 4 wave grid (five 32-row blocks per row
// group), so that an expert segment of up to 320 rows (DeepSeek-V3 routing
// gives 200-320 per expert) is one tile and its weights pass through LDS once.
// They pay off when segments commonly exceed 256 rows (192 or more per expert
// on average) and a minibatch gives at least half as many up/gate work items
// as there are CUs.  Otherwise 256-row tiles are faster: their weight ring is
// a stage deeper, each loads fewer activation rows, and a small minibatch
// splits into more of them.
constexpr int kRoutedBM = 320, kRoutedWM = 2, kRoutedWN = 4;
constexpr int kSmallBM = 256;
constexpr int kShortBM = 128;

// Tiling for a minibatch of mb_rows rows.  Large minibatches of large expert
// segments take 320-row tiles (above).  Otherwise 256-row tiles with up/gate
// items 128 columns wide (gate and up each) and down items 256 wide, as long
// as a minibatch gives at least half the CUs an up/gate item.  Small
// minibatches hold only a few expert segments: their work is then cut finer,
// into 128-row tiles with up/gate items 64 columns wide and down items as wide
// as still gives half the CUs an item.  A CU streams its tiles' operands at a
// rate that hardly depends on the tile shape, so a minibatch that leaves most
// CUs idle streams its weights slowly; finer items cost more re-reads of the
// activation rows but keep the CUs busy.  Measured against every combination
// of these tile shapes on MI355X, this rule picked the fastest or one within
// 5% at every granularity of the DeepSeek-V3 layer (512-65,536 rows), its
// EP-64 rank share (512-32,768) and the mid layer (512-32,768); 512-row
// minibatches took 18.8 instead of 26.3 ms (DeepSeek-V3), 6.7 instead of 12.3
// ms (EP-64 share) and 3.2 instead of 5.0 ms (mid).  No choice changes the K
// order of any output, so the results stay bitwise the same.
//
// The persistent routed kernel runs the up/gate of minibatch m+1 beside the
// down of m, so the chip is shared by two steps and a step needs fewer items
// of its own: there the larger tiles are kept down to a sixth of the CUs'
// worth of items per step (measured on the same workloads: DeepSeek-V3 at
// 512 rows 14.8 ms with 256-row tiles against 18.9 ms with 128-row tiles, at
// 1,024 rows 12.8 ms with 320-row tiles against 16.6 ms; the mid layer at
// 2,048 rows 1.09 against 1.69 ms; the EP-64 share at 512 rows keeps 128-row
// tiles, 5.7 against 6.5 ms).
RoutedTiling gemm_routed_tiling(int64_t mb_rows, int64_t max_rows, int64_t experts, int64_t I, int64_t D,
                                bool pipeline) {
  experts = experts > 0 ? experts : 1;
  const int64_t cus = device_compute_units();
  const double cu = cus > 0 ? static_cast<double>(cus) : 256.0;
  const bool big_segments = max_rows >= 192 * experts;
  const int64_t items = mb_rows / kRoutedBM * ((I + 127) / 128);  // up/gate tiles are 128 columns wide
  if (big_segments && items >= (pipeline ? cu / 6.0 : 128.0)) return RoutedTiling{kRoutedBM, 128, 256};
  const double half = pipeline ? cu / 6.0 : 0.5 * cu;
  // expert segments of one minibatch: how many experts it overlaps (b / rows
  // per expert + 1 when it is cut from a longer schedule) and their rows
  const double avg = std::max(1.0, static_cast<double>(max_rows) / static_cast<double>(experts));
  const bool whole = mb_rows >= max_rows;
  const double segs = whole ? static_cast<double>(experts)
                            : std::min(static_cast<double>(experts), static_cast<double>(mb_rows) / avg + 1.0);
  const double seg_rows = whole ? avg : static_cast<double>(mb_rows) / segs;
  auto tiles = [&](int bm) { return segs * std::ceil(seg_rows / bm); };
  if (tiles(kSmallBM) * std::ceil(static_cast<double>(I) / 128.0) >= half) return RoutedTiling{kSmallBM, 128, 256};
  int bn_down = 256;
  while (bn_down > 64 && tiles(kShortBM) * std::ceil(static_cast<double>(D) / bn_down) < half) bn_down /= 2;
  return RoutedTiling{kShortBM, 64, bn_down};
}

// Tile height of a dense fp32-output GEMM (the shared expert's down
// projection): 320-row tiles cost about 1.25x a 256-row tile, so they win when
// they save a whole round of workgroups over the chip's compute units (8192
// rows: 3 rounds of 320-row items against 4 of 256-row items, measured 6%
// faster; 4096 rows: 2 rounds either way, and 256-row tiles measured 12%
// faster).
int dense_f32_bm(int64_t rows, int N) {
  const int64_t cus = device_compute_units();
  if (cus <= 0) return kSmallBM;
  const int64_t nb = (N + 255) / 256;
  const int64_t r256 = ((rows + 255) / 256 * nb + cus - 1) / cus;
  const int64_t r320 = ((rows + 319) / 320 * nb + cus - 1) / cus;
  return r320 * 320 < r256 * 256 ? kRoutedBM : kSmallBM;
}

int gemm_tiles_bound(int64_t rows, int groups, int bm) {
  // every group (expert segment) adds at most one partial tile
  const int64_t bound = (rows + bm - 1) / bm + (groups < rows ? groups : rows);
  return static_cast<int>(bound);
}

hipError_t launch_gemm(const GemmArgs& a, int epilogue, hipStream_t stream) {
  const bool routed = a.tiles != nullptr;
  if (a.N <= 0 || a.k_splits < 1 || (routed && a.k_splits != 1)) return hipErrorInvalidValue;
  if (a.k_groups && (routed || a.k_splits != 1 || a.n_groups < 1)) return hipErrorInvalidValue;
  if (!a.k_groups && a.K % (kStageK * a.k_splits) != 0) return hipErrorInvalidValue;
  const int64_t ldb = a.ldb ? a.ldb : a.K;
  if (ldb % 8 != 0) return hipErrorInvalidValue;  // 16-byte aligned B rows
  // K-tiled weights: planes of all N rows, K in whole planes (routed), or
  // grouped K over a K extent ldb; K-tiled A: grouped K only
  if (a.b_plane != 0 && (a.b_plane != a.N || (routed ? (ldb != a.K || a.K % kTileK) : (!a.k_groups || ldb % kTileK))))
    return hipErrorInvalidValue;
  if (a.a_plane < 0 || (a.a_plane > 0 && (!a.k_groups || a.lda % kTileK || a.a_plane < a.dense_rows)))
    return hipErrorInvalidValue;
  // buffer resources address at most 2^31 bytes per operand here
  if (a.a_bytes <= 0 || a.a_bytes >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  if (static_cast<int64_t>(a.N) * ldb * 2 >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  if (routed && a.tile_rows != kRoutedBM && a.tile_rows != kSmallBM && a.tile_rows != kShortBM)
    return hipErrorInvalidValue;
  const bool big = routed && a.tile_rows == kRoutedBM;
  const int bn = a.tile_cols;
  switch (epilogue) {
    case kEpiSwiGLU:
      if (!routed) return run<256, 128, kWM, kWN, kEpiSwiGLU, false>(a, stream);
      if (big) return bn == 128 ? run<kRoutedBM, 128, kRoutedWM, kRoutedWN, kEpiSwiGLU, true>(a, stream)
                                : hipErrorInvalidValue;
      if (a.tile_rows == kSmallBM) return bn == 128 ? run<kSmallBM, 128, kWM, kWN, kEpiSwiGLU, true>(a, stream)
                                                    : hipErrorInvalidValue;
      return bn == 64 ? run<kShortBM, 64, kWM, kWN, kEpiSwiGLU, true>(a, stream) : hipErrorInvalidValue;
    case kEpiBF16:
      if (!routed) return run<256, 256, kWM, kWN, kEpiBF16, false>(a, stream);
      if (big) return bn == 256 ? run<kRoutedBM, 256, kRoutedWM, kRoutedWN, kEpiBF16, true>(a, stream)
                                : hipErrorInvalidValue;
      if (a.tile_rows == kSmallBM) return bn == 256 ? run<kSmallBM, 256, kWM, kWN, kEpiBF16, true>(a, stream)
                                                    : hipErrorInvalidValue;
      if (bn == 256) return run<kShortBM, 256, kWM, kWN, kEpiBF16, true>(a, stream);
      if (bn == 128) return run<kShortBM, 128, kWM, kWN, kEpiBF16, true>(a, stream);
      if (bn == 64) return run<kShortBM, 64, kWM, kWN, kEpiBF16, true>(a, stream);
      return hipErrorInvalidValue;
    case kEpiF32:
      if (big) return run<kRoutedBM, 256, kRoutedWM, kRoutedWN, kEpiF32, true>(a, stream);
      if (routed) return run<kSmallBM, 256, kWM, kWN, kEpiF32, true>(a, stream);
      if (a.N <= 256 || a.k_splits > 1) return run<128, 128, kWM, kWN, kEpiF32, false>(a, stream);
      return dense_f32_bm(a.dense_rows, a.N) == kRoutedBM
                 ? run<kRoutedBM, 256, kRoutedWM, kRoutedWN, kEpiF32, false>(a, stream)
                 : run<256, 256, kWM, kWN, kEpiF32, false>(a, stream);
    default:
      return hipErrorInvalidValue;
  }
}

// Workgroups the persistent routed kernel runs with for `tiling` (all
// resident at once): 0 when the runtime cannot say.
int pipeline_workgroups(const RoutedTiling& t) {
  const void* k = nullptr;
  if (t.bm == kRoutedBM) k = reinterpret_cast<const void*>(pipeline_kernel<320, 128, 2, 4, 320, 256, 2, 4>);
  else if (t.bm == kSmallBM) k = reinterpret_cast<const void*>(pipeline_kernel<256, 128, 4, 2, 256, 256, 4, 2>);
  else if (t.bn_down == 256) k = reinterpret_cast<const void*>(pipeline_kernel<128, 64, 4, 2, 128, 256, 4, 2>);
  else if (t.bn_down == 128) k = reinterpret_cast<const void*>(pipeline_kernel<128, 64, 4, 2, 128, 128, 4, 2>);
  else k = reinterpret_cast<const void*>(pipeline_kernel<128, 64, 4, 2, 128, 64, 4, 2>);
  return static_cast<int>(resident_workgroups(k, 512) / kXcds * kXcds);
}

hipError_t launch_pipeline(const PipeArgs& pa, const RoutedTiling& t, hipStream_t stream) {
  if (pa.up.tile_rows != t.bm || pa.down.tile_rows != t.bm || pa.up.tile_cols != t.bn_up ||
      pa.down.tile_cols != t.bn_down || pa.b <= 0 || pa.C % pa.b || pa.D % 8)
    return hipErrorInvalidValue;
  if (t.bm == kRoutedBM && t.bn_up == 128 && t.bn_down == 256)
    return run_pipeline<320, 128, 2, 4, 320, 256, 2, 4>(pa, stream);
  if (t.bm == kSmallBM && t.bn_up == 128 && t.bn_down == 256)
    return run_pipeline<256, 128, 4, 2, 256, 256, 4, 2>(pa, stream);
  if (t.bm == kShortBM && t.bn_up == 64) {
    if (t.bn_down == 256) return run_pipeline<128, 64, 4, 2, 128, 256, 4, 2>(pa, stream);
    if (t.bn_down == 128) return run_pipeline<128, 64, 4, 2, 128, 128, 4, 2>(pa, stream);
    if (t.bn_down == 64) return run_pipeline<128, 64, 4, 2, 128, 64, 4, 2>(pa, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
