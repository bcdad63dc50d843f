// Host-side launchers of the gfx950 MoE kernels (internal to libmoe.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Workspace pieces used by the schedule kernels.
struct SchedScratch {
  int32_t* ord_local;  // [R*N*k] chunk-local ordinal of each route
  int32_t* chunk_cnt;  // [R][n_chunks][L] histogram, then exclusive chunk base
  int32_t* M;          // [R][L] routes per (source rank, local expert)
};

int sched_chunks(int NK);

// Top-k and gates from `parts` (1 .. kMaxRouterParts) fp32 planes [T, E]
// (stride part_stride elements), summed in plane order; with parts > 1 the
// sums are written to `logits`.
constexpr int kMaxRouterParts = 4;
hipError_t launch_topk_gate(const float* planes, int parts, int64_t part_stride, float* logits, int T, int E, int k,
                            int32_t* idx, float* gate, int* err, hipStream_t stream);

hipError_t launch_schedule(const int32_t* routes, int R, int NK, int c, int L, int E_total, int64_t max_rows,
                           int32_t* counts, int32_t* offsets, int32_t* sched_src, int32_t* route_dst,
                           const SchedScratch& s, int* err, hipStream_t stream);

// XCD runs of a tile list: the GEMM kernels cut a list's work items (in
// their work order, n_blocks per row tile) into one contiguous run per XCD.
// The boundaries are positions counted in 1/kTileRunFrac of a tile: with N
// blocks of nb items per tile, run x holds items [floor(runs[x] nb /
// kTileRunFrac), floor(runs[x + 1] nb / kTileRunFrac)); runs[0] = 0 and
// runs[8] = kTileRunFrac times the tile count.
constexpr int kTileRunBounds = 9;
constexpr int kTileRunFrac = 64;
// Most tiles one run may span, for lists of at most max_tiles tiles: twice
// the equal share of the largest list.  The up/gate GEMMs launch this many
// tiles' items per XCD, one workgroup each.
__host__ __device__ inline int tile_run_cap(int max_tiles) { return (max_tiles + 3) / 4; }
// `runs` (kTileRunBounds words per minibatch, each run spanning at most
// tile_run_cap(max_tiles) tiles) may be NULL: the kernels then cut the items
// into runs of equal count.
hipError_t launch_build_tiles(const int32_t* offsets, int L, int64_t b, int64_t max_rows, int BM, int n_minibatches,
                              int max_tiles, int4* tiles, int32_t* tile_count, int32_t* runs, hipStream_t stream);

// Tile list of a dense GEMM run through the routed kernels: rows 0 .. rows-1 as
// one segment of expert 0, cut into ceil(rows / BM) tiles of equal height
// (rounded up to 32), in the same format as the routed lists.
int dense_tiles_bound(int64_t rows, int BM);
hipError_t launch_dense_tiles(int64_t rows, int BM, int4* tiles, int32_t* tile_count, hipStream_t stream);

// ---------------------------------------------------------------------------
// Grouped GEMM  C[rows, N] = A[rows, K] * B[e][N, K]^T  (bf16 in, fp32 accumulate)
// ---------------------------------------------------------------------------
enum GemmEpilogue : int {
  kEpiSwiGLU = 0,  // B0 = gate, B1 = up: C = bf16(SiLU(A B0^T) * (A B1^T))
  kEpiBF16 = 1,    // C = bf16(A B0^T)
  kEpiF32 = 2,     // C = A B0^T in fp32
};

// K-tiled layout of a bf16 matrix [R][K]: element (r, k) at
// ((k / kTileK) * R + r) * kTileK + k % kTileK (moe_tile_bf16).
constexpr int kTileK = 64;
// dst group g (group_stride elements apart; 0: rows * K) takes src group g
// as rows row0 .. row0 + rows - 1 of its planes of plane_rows rows (0: rows).
hipError_t launch_tile_bf16(const uint16_t* src, int64_t groups, int64_t rows, int64_t K, uint16_t* dst,
                            hipStream_t stream, int64_t plane_rows = 0, int64_t row0 = 0, int64_t group_stride = 0);

struct GemmArgs {
  const uint16_t* A;  // bf16; tile position p reads row (p - a_sub) mod a_mod
  int64_t a_bytes;    // extent of A in bytes (< 2^31)
  int64_t lda;
  int64_t a_sub;
  int64_t a_mod;
  // 0: A row-major (lda); > 0 (grouped K only): A K-tiled with planes of
  // a_plane rows, A pointing at the first of its rows in a plane
  int64_t a_plane;
  const uint16_t* B0;  // bf16 [experts][N][K]
  const uint16_t* B1;  // second operand of the SwiGLU epilogue (same layout)
  int64_t b_expert_stride;
  // 0: each expert's B row-major [N][K] (row stride ldb); N (routed, or
  // grouped K with ldb the K extent): K-tiled [K/kTileK][N][kTileK], so
  // that one K stage's rows are one plane
  int64_t b_plane;
  int N;
  int K;
  void* C;  // output row = c_idx ? c_idx[p] : p - c_sub
  int64_t ldc;
  const int32_t* c_idx;
  int64_t c_sub;
  const int4* tiles;         // routed: {expert, p0, rows, 0}; NULL: dense rows 0..dense_rows-1
  const int32_t* tile_count;  // routed: number of valid tiles
  const int32_t* tile_runs;   // routed, or NULL: the list's XCD runs (kTileRunBounds tile indices)
  int tile_rows;              // routed: the height the tile lists were built with (gemm_routed_tiling)
  int tile_cols;              // routed: output columns per work item (gemm_routed_tiling's bn_up or bn_down)
  int dense_rows;
  int max_tiles;
  int k_splits;            // dense only: K is cut into this many equal ranges, one output plane each
  int64_t c_split_stride;  // elements between the output planes of the K ranges
  int64_t ldb;             // B row stride in elements (0: K)
  // Dense only, grouped K: group g multiplies K elements [k_groups[g].x,
  // + 64 * k_groups[g].y) of the A and B rows (a zero count gives zeros) into
  // its own output block at C + g * c_group_stride; k_splits must be 1.
  const int2* k_groups;
  int n_groups;
  int64_t c_group_stride;
};

// Grouped MXFP8 GEMM over a tile list (routed experts, or a dense GEMM through
// a one-expert list): E4M3 operands with one E8M0 scale per 32 elements along
// K, fp32 accumulate.  Data row-major, scales stage-major (the
// byte of row r, K block j at ((j / 4) * rows + r) * 4 + j % 4): A [a_rows][K]
// + [K/128][a_rows][4]; B per expert [N][K] + [K/128][N][4].
struct MxGemmArgs {
  const uint8_t* A;  // tile position p reads row (p - a_sub) mod a_mod
  const uint8_t* As;
  int64_t a_rows;  // rows of A (a_rows * K < 2^31)
  int64_t a_sub;
  int64_t a_mod;
  const uint8_t* B0;  // gate (SwiGLU) or the only operand
  const uint8_t* B1;  // up (SwiGLU)
  const uint8_t* Bs0;
  const uint8_t* Bs1;
  int64_t b_plane;  // 0: each expert's B row-major [N][K]; N: K-tiled [K/128][N][128] (one plane per K stage)
  int N;
  int K;
  void* C;      // SwiGLU: E4M3 [.][ldc], scales to Cs [ldc/128][cs_rows][4]; BF16: bf16 [.][ldc]; F32: fp32 [.][ldc]
  uint8_t* Cs;  // output row = c_idx ? c_idx[p] : p - c_sub
  int64_t cs_rows;
  int64_t ldc;
  const int32_t* c_idx;
  int64_t c_sub;
  const int4* tiles;
  const int32_t* tile_count;
  const int32_t* tile_runs;  // or NULL: the list's XCD runs (kTileRunBounds tile indices)
  int max_tiles;
};
hipError_t launch_gemm_mx(const MxGemmArgs& args, int epilogue, hipStream_t stream);
// Tile rows of the routed MXFP8 GEMM kernels (their tile lists are built with it).
int gemm_mx_routed_bm();

// Tiling of the routed bf16 GEMMs for minibatches of mb_rows rows, max_rows
// routed rows in all over `experts` local experts, intermediate width I and
// hidden width D: the tile height bm (the tile lists are built with it) and
// the output columns per work item of the up/gate (gate and up columns each)
// and of the down projection; `pipeline` for the persistent routed kernel.
struct RoutedTiling {
  int bm, bn_up, bn_down;
};
RoutedTiling gemm_routed_tiling(int64_t mb_rows, int64_t max_rows, int64_t experts, int64_t I, int64_t D,
                                bool pipeline);
hipError_t launch_gemm(const GemmArgs& args, int epilogue, hipStream_t stream);
int gemm_tiles_bound(int64_t rows, int groups, int bm);

// The routed minibatch loop as one persistent kernel (gather, up/gate +
// SwiGLU, down for every minibatch, with device-side counters between them).
// `up` and `down` are minibatch 0's GEMM arguments (tiles, tile_count and
// tile_runs of minibatch 0; the kernel steps them by minibatch); h holds n_h
// buffers of b * I bf16.  gathered / upg / down_done count finished work per
// minibatch, upg_tile per row tile; all must be zero at launch.  Minibatches
// below C / b are gathered before the launch; n_mem workgroups (a multiple of
// 8) gather the others.
struct PipeArgs {
  GemmArgs up, down;
  const uint16_t* x_src;
  int64_t src_rows;
  const int32_t* sched_src;
  const int32_t* offsets;
  int L, k, D, n_mb, n_mem;
  int64_t b, C, max_rows;
  uint16_t* ring;
  uint16_t* h;    // n_h buffers of [b, I]: minibatch m writes buffer m mod n_h
  int n_h;        // 2 .. kMaxPipeH; up/gate runs up to n_h - 1 minibatches ahead of down
  int *gathered, *upg, *down_done;
  int* upg_tile;  // [n_mb][up.max_tiles]: finished up/gate items of each row tile
  int* queue;     // [kPipeQueueInts]: 8 per-XCD item queue heads, then one word per workgroup; zero on entry
  int* err;
};
constexpr int kPipeMaxGrid = 1024;
constexpr int kPipeQueueInts = 8 + kPipeMaxGrid;
constexpr int kMaxPipeH = 4;
// h buffers of the persistent kernel for ring rows C and minibatch rows b:
// C / b clamped to 2 .. kMaxPipeH (the ring bounds how far the gathers, and so
// the up/gate steps, can run ahead).
inline int pipeline_h_buffers(int64_t b, int64_t C) {
  const int64_t q = b > 0 ? C / b : 2;
  return static_cast<int>(q < 2 ? 2 : (q > kMaxPipeH ? kMaxPipeH : q));
}
// Workgroups the persistent kernel runs with for a tiling (all resident).
int pipeline_workgroups(const RoutedTiling& tiling);
hipError_t launch_pipeline(const PipeArgs& args, const RoutedTiling& tiling, hipStream_t stream);

// ---------------------------------------------------------------------------
// Backward pass (backward.hip)
// ---------------------------------------------------------------------------
// dY[p] = bf16(gate[j] * dout[j / k]) for j = sched_src[p], p < P
hipError_t launch_dy_gather(const uint16_t* dout, const float* gate, const int32_t* sched_src, int64_t P, int T, int D,
                            int k, uint16_t* dy, int* err, hipStream_t s);
// dg[j] = <dout[j / k], y[j]> (fp32, fixed order) for the n_routes routes
hipError_t launch_route_grad(const uint16_t* dout, const uint16_t* y, int64_t n_routes, int D, int k, float* dg,
                             hipStream_t s);
// dl [T][ld] bf16: g_s (dg_s - sum g dg) at the selected experts, zero elsewhere
hipError_t launch_gate_grad(const float* gate, const float* dg, const int32_t* idx, int T, int E, int ld, int k,
                            uint16_t* dl, hipStream_t s);
// act [rows][2I] = [a_g | a_u], dh [rows][I] fp32 -> h [rows][I], da [rows][2I] = [da_g | da_u] (bf16)
hipError_t launch_swiglu_bwd(const uint16_t* act, const float* dh, int64_t rows, int I, uint16_t* h, uint16_t* da,
                             hipStream_t s);
// segments of offsets[] padded to 64 rows: padded [L+1], k_groups [L] = {padded[e], stages}
hipError_t launch_pad_offsets(const int32_t* offsets, int L, int32_t* padded, int2* k_groups, hipStream_t s);
// out [W][ld_out]: column padded[e] + i = row offsets[e] + i of src [.][lda] (zero past the segment)
hipError_t launch_seg_transpose(const uint16_t* src, int64_t lda, int W, const int32_t* offsets,
                                const int32_t* padded, int L, int64_t max_cols, uint16_t* out, int64_t ld_out,
                                hipStream_t s, bool tiled = false);
// offsets {0, rows}, padded {0, ceil64(rows)}, k_groups[0] = {0, ceil(rows / 64)} for one dense segment
hipError_t launch_single_segment(int rows, int32_t* offsets, int32_t* padded, int2* k_groups, hipStream_t s);
// out[b][c][col0 + r] = in[b][r][c], in [B][R][Cn] contiguous, out rows ld_out, batches out_b apart; with
// plane_rows > 0 each batch of the output is K-tiled with planes of plane_rows rows
hipError_t launch_transpose(const uint16_t* in, int B, int R, int Cn, uint16_t* out, int64_t ld_out, int64_t out_b,
                            int col0, hipStream_t s, int64_t plane_rows = 0);
// dx[t] = dx_shared[t] + dx_router[t] + sum_s dx_ring[route_dst[t k + s]] (fp32, in that order)
hipError_t launch_dx_assemble(const float* dx_shared, const float* dx_router, const float* dx_ring,
                              const int32_t* route_dst, int T, int D, int k, int64_t P, float* dx, int* err,
                              hipStream_t s);

// ---------------------------------------------------------------------------
// Data movement
// ---------------------------------------------------------------------------
hipError_t launch_gather(const uint16_t* x_src, int64_t src_rows, int D, int k, const int32_t* sched_src,
                         const int32_t* offsets, int L, int64_t p_begin, int64_t rows, int64_t ring_rows,
                         uint16_t* ring, int* err, hipStream_t stream);

hipError_t launch_combine(const uint16_t* Y, const float* shared_out, const float* gate, const int32_t* route_dst,
                          int64_t route_base, int T, int D, int k, bool by_route_dst, uint16_t* out, float* out32,
                          hipStream_t stream);

// MX gather: ring_q[p mod C] / ring_s[p mod C] = MX(x_src[sched_src[p] / k]),
// scales stage-major [D/128][C][4].
hipError_t launch_gather_mx(const uint16_t* x_src, int64_t src_rows, int D, int k, const int32_t* sched_src,
                            const int32_t* offsets, int L, int64_t p_begin, int64_t rows, int64_t ring_rows,
                            uint8_t* ring_q, uint8_t* ring_s, int* err, hipStream_t stream);

// Source-side gathers for R = 1 when one minibatch holds every routed row:
// each token row is read once and written to its k ring slots.
hipError_t launch_gather_src(const uint16_t* x, int T, int D, int k, const int32_t* route_dst, int64_t P,
                             int64_t ring_rows, uint16_t* ring, int* err, hipStream_t stream);
hipError_t launch_gather_src_mx(const uint16_t* x, int T, int D, int k, const int32_t* route_dst, int64_t P,
                                int64_t ring_rows, uint8_t* ring_q, uint8_t* ring_s, int* err, hipStream_t stream);

hipError_t launch_clear_int(int* p, int n, hipStream_t stream);

// MXFP8: rows x K bf16 -> E4M3 codes + one E8M0 scale per 32 elements along K.
hipError_t launch_quantize_mxfp8(const uint16_t* src, int64_t rows, int64_t K, uint8_t* q, uint8_t* scale,
                                 hipStream_t stream);
// rows x K bf16 -> E4M3 codes [rows][K] + E8M0 scales stage-major [K/128][rows][4]
// (the layout the MX GEMMs read activation scales in); K a multiple of 128.
hipError_t launch_quantize_rows_mx_staged(const uint16_t* src, int64_t rows, int64_t K, uint8_t* q, uint8_t* scale,
                                          hipStream_t stream);
// Row-major scales [groups][rows][K/32] -> stage-major [groups][K/128][rows][4].
hipError_t launch_pack_mx_scales(const uint8_t* scale, int64_t groups, int64_t rows, int64_t K, uint8_t* packed,
                                 hipStream_t stream);

}  // namespace moe
