// C ABI of libmoe.so: shape validation, workspace carving and the stream-ordered
// launch sequence of the MoE-layer forward.  See include/moe.h for the contract.

#include <algorithm>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/moe.h"
#include "common.h"
#include "kernels.h"

// Scratch of moe_schedule_static, the entry point that allocates nothing:
// per-route ordinals, per-chunk histograms and M of the schedule kernels.
// Each GPU holds its own copy until the process ends.  Host code must not
// pass `scratch` itself to a kernel (on the host it is only a stand-in for
// the symbol): it uses the device address looked up by static_scratch().
constexpr size_t kStaticScratchBytes = MOE_SCHEDULE_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Layout {
  size_t err, ord_local, chunk_cnt, M, tiles, tile_count, tile_runs, ring, ring_s, h, h_s, Y, h_shared, shared_out, router_parts,
      xs_q, xs_s, hs_s, shared_tiles, shared_tile_count, total;
  int router_splits;
  int64_t n_minibatches;
  int max_tiles;
  int routed_bm;      // tile height of the routed GEMMs' tile lists
  int bn_up, bn_down;  // output columns per work item of the routed bf16 GEMMs
  size_t pipe_counters;  // pipeline == 1: (3 + max_tiles) * n_minibatches ints, then the work queues
  int64_t y_rows;
};

// The GEMMs read every operand through a buffer resource, which addresses
// fewer than 2^31 bytes.  Each operand a launch would read that way must fit,
// so that an oversized shape is refused here, before any launch:
//   x (router, shared expert)  T*D*2     ring      C*D*e      routed h  b*I*e
//   shared h                   T*I_s*e_s one routed weight matrix I*D*e
//   shared weight matrix       I_s*D*e_s
// with e (e_s) = 2 bytes per element in bf16 and 1 in MXFP8.  T, D, I and
// I_s are already bounded when this runs; the router weights, E_total*D*2,
// stay below 2^28 under the bounds E_total <= 1024 and D <= 65536.
bool operands_addressable(const moe_shape* s) {
  constexpr int64_t kLimit = int64_t(1) << 31;
  if (s->ring_rows >= kLimit || s->minibatch_rows >= kLimit) return false;
  const int64_t e = s->precision == MOE_MXFP8 ? 1 : 2;
  const int64_t es = s->shared_precision == MOE_MXFP8 ? 1 : 2;
  // every factor is now below 2^31 and every multiplier below 2^17: no int64 overflow
  const int64_t bytes[] = {s->T * s->D * 2,         s->ring_rows * s->D * e, s->minibatch_rows * s->I * e,
                           s->T * s->I_shared * es, s->I * s->D * e,         s->I_shared * s->D * es};
  for (const int64_t v : bytes)
    if (v >= kLimit) return false;
  return true;
}

bool valid_shape(const moe_shape* s, moe_status* why) {
  *why = MOE_ERR_INVALID_ARG;
  if (!s) return false;
  if (s->shared_precision != MOE_BF16 && s->shared_precision != MOE_MXFP8) return false;
  if (s->T < 0 || s->D <= 0 || s->I <= 0 || s->I_shared <= 0 || s->E_total <= 0 || s->k <= 0) return false;
  if (s->k > s->E_total) return false;
  if (s->num_src_ranks < 1 || s->rank < 0 || s->rank >= s->num_src_ranks) return false;
  if (s->experts_per_rank < 1 || s->num_src_ranks * s->experts_per_rank != s->E_total) return false;
  if (s->tokens_per_src_rank != s->T) return false;
  if (s->minibatch_rows < 1 || s->ring_rows < s->minibatch_rows || s->ring_rows % s->minibatch_rows != 0)
    return false;
  if (s->max_rows < 0) return false;
  if (s->num_src_ranks == 1 && s->max_rows != s->T * s->k) return false;
  if (s->max_rows > s->num_src_ranks * s->T * s->k) return false;
  if (s->precision != MOE_BF16 && s->precision != MOE_MXFP8) return false;
  if (s->pipeline != 0 && s->pipeline != 1) return false;
  if (s->pipeline && (s->mem_workgroups < 0 || s->mem_workgroups % 8)) return false;
  if (s->weights_tiled != 0 && s->weights_tiled != 1) return false;
  *why = MOE_ERR_UNSUPPORTED;
  if (s->pipeline && s->precision != MOE_BF16) return false;
  if (s->D % 64 || s->I % 64 || s->I_shared % 64) return false;
  if (s->k > 16 || s->E_total > 1024 || s->experts_per_rank > 1024) return false;
  if (s->num_src_ranks * s->T * s->k >= (int64_t(1) << 31)) return false;
  if (s->max_rows >= (int64_t(1) << 31) || s->T >= (int64_t(1) << 31)) return false;
  if (s->D > 65536 || s->I > 65536 || s->I_shared > 65536) return false;
  // MXFP8 GEMM stages are 128 elements of K wide (D for up/gate, I for down)
  if (s->precision == MOE_MXFP8 && (s->D % 128 || s->I % 128)) return false;
  if (s->shared_precision == MOE_MXFP8 && (s->D % 128 || s->I_shared % 128)) return false;
  if (!operands_addressable(s)) return false;
  *why = MOE_OK;
  return true;
}

// K ranges of the router GEMM: with few output tiles (T/128 x E/128 well
// under the 256 CUs) the K axis is cut into equal ranges whose partial
// logits the top-k kernel adds in a fixed order.  The ranges double while
// the work items stay at most 512 (two per CU): at 8192 tokens that is 4
// ranges for 256 experts and 2 for 384, the fastest router + top-k of 1, 2
// and 4 ranges measured for each.
int router_splits(const moe_shape* s) {
  const int64_t tiles = ((s->T + 127) / 128) * ((s->E_total + 127) / 128);
  const int64_t stages = s->D / 64;
  int S = 1;
  while (2 * S <= moe::kMaxRouterParts && tiles * S * 2 <= 512 && stages % (2 * S) == 0) S *= 2;
  return S;
}

Layout layout_of(const moe_shape* s) {
  Layout L{};
  L.router_splits = router_splits(s);
  const int64_t R = s->num_src_ranks, NK = s->T * s->k, Lx = s->experts_per_rank;
  const int64_t mb_rows = std::min<int64_t>(s->minibatch_rows, std::max<int64_t>(s->max_rows, 1));
  const moe::RoutedTiling tiling = s->precision == MOE_MXFP8
                                       ? moe::RoutedTiling{moe::gemm_mx_routed_bm(), 0, 0}
                                       : moe::gemm_routed_tiling(mb_rows, s->max_rows, Lx, s->I, s->D,
                                                                 s->pipeline != 0);
  const int bm = tiling.bm;
  L.routed_bm = bm;
  L.bn_up = tiling.bn_up;
  L.bn_down = tiling.bn_down;
  L.n_minibatches = s->max_rows > 0 ? (s->max_rows + s->minibatch_rows - 1) / s->minibatch_rows : 0;
  L.max_tiles = moe::gemm_tiles_bound(mb_rows, static_cast<int>(Lx), bm);
  L.y_rows = (R == 1) ? NK : s->max_rows;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  L.err = take(sizeof(int32_t));
  L.ord_local = take(sizeof(int32_t) * R * NK);
  L.chunk_cnt = take(sizeof(int32_t) * R * moe::sched_chunks(static_cast<int>(NK)) * Lx);
  L.M = take(sizeof(int32_t) * R * Lx);
  L.tiles = take(sizeof(int4) * L.n_minibatches * L.max_tiles);
  L.tile_count = take(sizeof(int32_t) * std::max<int64_t>(L.n_minibatches, 1));
  L.tile_runs = take(sizeof(int32_t) * moe::kTileRunBounds * std::max<int64_t>(L.n_minibatches, 1));
  if (s->precision == MOE_MXFP8) {  // E4M3 bytes + one E8M0 byte per 32 along K
    L.ring = take(s->ring_rows * s->D);
    L.ring_s = take(s->ring_rows * (s->D / 32));
    L.h = take(s->minibatch_rows * s->I);
    L.h_s = take(s->minibatch_rows * (s->I / 32));
  } else {
    L.ring = take(sizeof(uint16_t) * s->ring_rows * s->D);
    // the persistent kernel runs up/gate up to H - 1 minibatches ahead of
    // down: H h buffers, H = C / b clamped to 2 .. 4
    L.h = take(sizeof(uint16_t) * s->minibatch_rows * s->I *
               (s->pipeline ? moe::pipeline_h_buffers(s->minibatch_rows, s->ring_rows) : 1));
  }
  L.pipe_counters = take(s->pipeline ? sizeof(int32_t) * ((3 + L.max_tiles) * std::max<int64_t>(L.n_minibatches, 1) +
                                                          moe::kPipeQueueInts)
                                     : 0);
  L.Y = take(sizeof(uint16_t) * L.y_rows * s->D);
  L.shared_out = take(sizeof(float) * s->T * s->D);
  if (s->shared_precision == MOE_MXFP8) {  // x and h of the shared expert in E4M3 + stage-major E8M0
    L.xs_q = take(s->T * s->D);
    L.xs_s = take(s->T * (s->D / 32));
    L.h_shared = take(s->T * s->I_shared);
    L.hs_s = take(s->T * (s->I_shared / 32));
    L.shared_tiles = take(sizeof(int4) * moe::dense_tiles_bound(s->T, moe::gemm_mx_routed_bm()));
    L.shared_tile_count = take(sizeof(int32_t));
  } else {
    L.h_shared = take(sizeof(uint16_t) * s->T * s->I_shared);
  }
  L.router_parts = take(L.router_splits > 1 ? sizeof(float) * L.router_splits * s->T * s->E_total : 0);
  L.total = off;
  return L;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

#define MOE_TRY_HIP(expr)                       \
  do {                                          \
    const hipError_t e_ = (expr);               \
    if (e_ != hipSuccess) return MOE_ERR_HIP;   \
  } while (0)

// Benchmark probe: event pairs around the launches of one kernel.
struct Probe {
  int kernel = -1;
  int max_launches = 0;
  int used = 0;
  std::vector<hipEvent_t> start, stop;
};
Probe g_probe;

struct ProbeScope {  // records around one launch of `kernel` when the probe asks for it
  int slot = -1;
  hipStream_t stream;
  ProbeScope(int kernel, hipStream_t s) : stream(s) {
    if (g_probe.kernel == kernel && g_probe.used < g_probe.max_launches) {
      slot = g_probe.used++;
      (void)hipEventRecord(g_probe.start[slot], stream);
    }
  }
  ~ProbeScope() {
    if (slot >= 0) (void)hipEventRecord(g_probe.stop[slot], stream);
  }
};

moe_status check_ws(const moe_shape* s, const void* ws, size_t ws_bytes, Layout* L) {
  moe_status why;
  if (!valid_shape(s, &why)) return why;
  *L = layout_of(s);
  if (!ws) return MOE_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(ws) % kAlign) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < L->total) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

// Device address of `scratch` on the current device, looked up once per
// device with that device current (each GPU has its own copy of the array).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

moe_status static_scratch(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MOE_OK;
}

// The schedule kernels' scratch carved from one base (256-byte aligned pieces).
struct SchedPieces {
  size_t ord_local, chunk_cnt, M, total;
};

SchedPieces sched_pieces(const moe_shape* s) {
  const int64_t R = s->num_src_ranks, NK = s->T * s->k, Lx = s->experts_per_rank;
  SchedPieces p{};
  p.ord_local = 0;
  p.chunk_cnt = align_up(sizeof(int32_t) * R * NK);
  p.M = p.chunk_cnt + align_up(sizeof(int32_t) * R * moe::sched_chunks(static_cast<int>(NK)) * Lx);
  p.total = p.M + align_up(sizeof(int32_t) * R * Lx);
  return p;
}

// The shared expert in MXFP8, an option beside the MoK paper's bf16 shared
// expert (§3.4, "MXFP8 Support"): x is MX-quantised along D, the up/gate GEMM
// quantises h along I_shared in its epilogue, and the down GEMM writes fp32
// rows for the combine.  Both GEMMs are the routed MX kernels over a tile list
// holding the T rows as one segment of "expert" 0.
hipError_t shared_expert_mx(const moe_shape* shape, const moe_weights* w, const void* x_local, const Layout& L,
                            void* ws, hipStream_t s) {
  const int64_t T = shape->T, D = shape->D, Is = shape->I_shared;
  uint8_t* xq = at<uint8_t>(ws, L.xs_q);
  uint8_t* xs = at<uint8_t>(ws, L.xs_s);
  uint8_t* hq = at<uint8_t>(ws, L.h_shared);
  uint8_t* hs = at<uint8_t>(ws, L.hs_s);
  int4* tiles = at<int4>(ws, L.shared_tiles);
  int32_t* count = at<int32_t>(ws, L.shared_tile_count);
  const int bm = moe::gemm_mx_routed_bm();
  {
    ProbeScope probe(MOE_K_SHARED_UP, s);
    hipError_t e = moe::launch_quantize_rows_mx_staged(static_cast<const uint16_t*>(x_local), T, D, xq, xs, s);
    if (e == hipSuccess) e = moe::launch_dense_tiles(T, bm, tiles, count, s);
    if (e != hipSuccess) return e;
    moe::MxGemmArgs u{};
    u.A = xq;
    u.As = xs;
    u.a_rows = T;
    u.a_sub = 0;
    u.a_mod = INT64_MAX;
    u.B0 = static_cast<const uint8_t*>(w->ws_gate);
    u.B1 = static_cast<const uint8_t*>(w->ws_up);
    u.Bs0 = w->ss_gate;
    u.Bs1 = w->ss_up;
    u.N = static_cast<int>(Is);
    u.K = static_cast<int>(D);
    u.C = hq;
    u.Cs = hs;
    u.cs_rows = T;
    u.ldc = Is;
    u.c_idx = nullptr;
    u.c_sub = 0;
    u.tiles = tiles;
    u.tile_count = count;
    u.max_tiles = moe::dense_tiles_bound(T, bm);
    e = moe::launch_gemm_mx(u, moe::kEpiSwiGLU, s);
    if (e != hipSuccess) return e;
  }
  moe::MxGemmArgs d{};
  d.A = hq;
  d.As = hs;
  d.a_rows = T;
  d.a_sub = 0;
  d.a_mod = INT64_MAX;
  d.B0 = static_cast<const uint8_t*>(w->ws_down);
  d.B1 = nullptr;
  d.Bs0 = w->ss_down;
  d.Bs1 = nullptr;
  d.N = static_cast<int>(D);
  d.K = static_cast<int>(Is);
  d.C = at<float>(ws, L.shared_out);
  d.Cs = nullptr;
  d.cs_rows = 0;
  d.ldc = D;
  d.c_idx = nullptr;
  d.c_sub = 0;
  d.tiles = tiles;
  d.tile_count = count;
  d.max_tiles = moe::dense_tiles_bound(T, bm);
  ProbeScope probe(MOE_K_SHARED_DOWN, s);
  return moe::launch_gemm_mx(d, moe::kEpiF32, s);
}

// One minibatch of the routed experts in MXFP8 (MoK paper §3.4 "MXFP8
// Support"): the gather quantises x along D into the ring, the up/gate GEMM
// quantises h along I in its epilogue, the down GEMM writes bf16 rows.
hipError_t routed_minibatch_mx(const moe_shape* shape, const moe_weights* w, const void* x_src,
                               const int32_t* sched_src, const int32_t* expert_offsets, const int32_t* route_dst,
                               const Layout& L, void* ws, int64_t m, int64_t p_begin, int64_t rows, hipStream_t s) {
  const int D = static_cast<int>(shape->D), I = static_cast<int>(shape->I), k = static_cast<int>(shape->k);
  const int Lx = static_cast<int>(shape->experts_per_rank);
  const int64_t b = shape->minibatch_rows, C = shape->ring_rows, R = shape->num_src_ranks;
  uint8_t* ring_q = at<uint8_t>(ws, L.ring);
  uint8_t* ring_s = at<uint8_t>(ws, L.ring_s);
  uint8_t* h_q = at<uint8_t>(ws, L.h);
  uint8_t* h_s = at<uint8_t>(ws, L.h_s);
  const int4* tiles = at<int4>(ws, L.tiles) + m * L.max_tiles;
  const int32_t* tile_count = at<int32_t>(ws, L.tile_count) + m;
  const int32_t* tile_runs = at<int32_t>(ws, L.tile_runs) + m * moe::kTileRunBounds;
  {
    ProbeScope probe(MOE_K_GATHER, s);
    const hipError_t e =
        (R == 1 && L.n_minibatches == 1)
            ? moe::launch_gather_src_mx(static_cast<const uint16_t*>(x_src), static_cast<int>(shape->T), D, k,
                                        route_dst, shape->max_rows, C, ring_q, ring_s, at<int>(ws, L.err), s)
            : moe::launch_gather_mx(static_cast<const uint16_t*>(x_src), R * shape->T, D, k, sched_src,
                                    expert_offsets, Lx, p_begin, rows, C, ring_q, ring_s, at<int>(ws, L.err), s);
    if (e != hipSuccess) return e;
  }
  moe::MxGemmArgs u{};
  u.A = ring_q;
  u.As = ring_s;
  u.a_rows = C;
  u.a_sub = 0;
  u.a_mod = C;
  u.B0 = static_cast<const uint8_t*>(w->w_gate);
  u.B1 = static_cast<const uint8_t*>(w->w_up);
  u.Bs0 = w->s_gate;
  u.Bs1 = w->s_up;
  u.b_plane = shape->weights_tiled ? I : 0;
  u.N = I;
  u.K = D;
  u.C = h_q;
  u.Cs = h_s;
  u.cs_rows = b;
  u.ldc = I;
  u.c_sub = p_begin;
  u.tiles = tiles;
  u.tile_count = tile_count;
  u.tile_runs = tile_runs;
  u.max_tiles = L.max_tiles;
  {
    ProbeScope probe(MOE_K_UP_GATE, s);
    const hipError_t e = moe::launch_gemm_mx(u, moe::kEpiSwiGLU, s);
    if (e != hipSuccess) return e;
  }
  moe::MxGemmArgs d{};
  d.A = h_q;
  d.As = h_s;
  d.a_rows = b;
  d.a_sub = p_begin;
  d.a_mod = INT64_MAX;
  d.B0 = static_cast<const uint8_t*>(w->w_down);
  d.B1 = nullptr;
  d.Bs0 = w->s_down;
  d.Bs1 = nullptr;
  d.b_plane = shape->weights_tiled ? D : 0;
  d.N = D;
  d.K = I;
  d.C = at<uint16_t>(ws, L.Y);
  d.ldc = D;
  d.c_idx = (R == 1) ? sched_src : nullptr;
  d.c_sub = 0;
  d.tiles = tiles;
  d.tile_count = tile_count;
  d.tile_runs = tile_runs;
  d.max_tiles = L.max_tiles;
  ProbeScope probe(MOE_K_DOWN, s);
  return moe::launch_gemm_mx(d, moe::kEpiBF16, s);
}

}  // namespace

extern "C" {

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_str(moe_status st) {
  switch (st) {
    case MOE_OK:
      return "ok";
    case MOE_ERR_INVALID_ARG:
      return "invalid argument";
    case MOE_ERR_UNSUPPORTED:
      return "unsupported shape or precision";
    case MOE_ERR_WORKSPACE:
      return "workspace too small";
    case MOE_ERR_HIP:
      return "HIP runtime error";
  }
  return "unknown status";
}

moe_status moe_workspace_bytes(const moe_shape* shape, size_t* bytes) {
  moe_status why;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  if (!valid_shape(shape, &why)) return why;
  *bytes = layout_of(shape).total;
  return MOE_OK;
}

moe_status moe_workspace_init(const moe_shape* shape, void* ws, size_t ws_bytes, void* stream) {
  Layout L;
  const moe_status st = check_ws(shape, ws, ws_bytes, &L);
  if (st != MOE_OK) return st;
  return hip_status(moe::launch_clear_int(at<int>(ws, L.err), 1, static_cast<hipStream_t>(stream)));
}

moe_status moe_route(const moe_shape* shape, const void* x, const void* w_router, float* logits, int32_t* topk_idx,
                     float* topk_gate, void* ws, size_t ws_bytes, void* stream) {
  Layout L;
  const moe_status st = check_ws(shape, ws, ws_bytes, &L);
  if (st != MOE_OK) return st;
  if (!logits || !topk_idx || !topk_gate || (x && !w_router)) return MOE_ERR_INVALID_ARG;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int T = static_cast<int>(shape->T), E = static_cast<int>(shape->E_total), k = static_cast<int>(shape->k);
  if (T == 0) return MOE_OK;
  if (x) {
    moe::GemmArgs g{};
    g.k_splits = 1;
    g.A = static_cast<const uint16_t*>(x);
    g.a_bytes = shape->T * shape->D * 2;
    g.lda = shape->D;
    g.a_sub = 0;
    g.a_mod = INT64_MAX;
    g.B0 = static_cast<const uint16_t*>(w_router);
    g.B1 = nullptr;
    g.b_expert_stride = 0;
    g.N = E;
    g.K = static_cast<int>(shape->D);
    g.C = L.router_splits > 1 ? static_cast<void*>(at<float>(ws, L.router_parts)) : static_cast<void*>(logits);
    g.ldc = E;
    g.k_splits = L.router_splits;
    g.c_split_stride = static_cast<int64_t>(T) * E;
    g.c_idx = nullptr;
    g.c_sub = 0;
    g.tiles = nullptr;
    g.tile_count = nullptr;
    g.dense_rows = T;
    ProbeScope probe(MOE_K_ROUTER_GEMM, s);
    MOE_TRY_HIP(moe::launch_gemm(g, moe::kEpiF32, s));
  }
  ProbeScope probe(MOE_K_TOPK, s);
  const bool parts = x && L.router_splits > 1;
  return hip_status(moe::launch_topk_gate(parts ? at<float>(ws, L.router_parts) : logits,
                                          parts ? L.router_splits : 1, static_cast<int64_t>(T) * E, logits, T, E, k,
                                          topk_idx, topk_gate, at<int>(ws, L.err), s));
}

moe_status moe_schedule(const moe_shape* shape, const int32_t* routes, int32_t* expert_counts,
                        int32_t* expert_offsets, int32_t* sched_src, int32_t* route_dst, void* ws, size_t ws_bytes,
                        void* stream) {
  Layout L;
  const moe_status st = check_ws(shape, ws, ws_bytes, &L);
  if (st != MOE_OK) return st;
  const int64_t NK = shape->T * shape->k;
  if (!expert_counts || !expert_offsets || !route_dst || (NK > 0 && !routes) || (shape->max_rows > 0 && !sched_src))
    return MOE_ERR_INVALID_ARG;
  moe::SchedScratch sc{at<int32_t>(ws, L.ord_local), at<int32_t>(ws, L.chunk_cnt), at<int32_t>(ws, L.M)};
  ProbeScope probe(MOE_K_SCHEDULE, static_cast<hipStream_t>(stream));
  return hip_status(moe::launch_schedule(
      routes, static_cast<int>(shape->num_src_ranks), static_cast<int>(NK), static_cast<int>(shape->rank),
      static_cast<int>(shape->experts_per_rank), static_cast<int>(shape->E_total), shape->max_rows, expert_counts,
      expert_offsets, sched_src, route_dst, sc, at<int>(ws, L.err), static_cast<hipStream_t>(stream)));
}

moe_status moe_schedule_static(const moe_shape* shape, const int32_t* routes, int32_t* expert_counts,
                               int32_t* expert_offsets, int32_t* sched_src, int32_t* route_dst, int32_t* dev_error,
                               void* stream) {
  moe_status why;
  if (!valid_shape(shape, &why)) return why;
  const int64_t NK = shape->T * shape->k;
  if (!expert_counts || !expert_offsets || !route_dst || !dev_error || (NK > 0 && !routes) ||
      (shape->max_rows > 0 && !sched_src))
    return MOE_ERR_INVALID_ARG;
  const SchedPieces pc = sched_pieces(shape);
  if (pc.total > kStaticScratchBytes) return MOE_ERR_UNSUPPORTED;
  void* base = nullptr;
  const moe_status st = static_scratch(&base);
  if (st != MOE_OK) return st;
  // every scratch entry a later kernel reads is written first by the same
  // call, so nothing needs clearing between calls
  moe::SchedScratch sc{at<int32_t>(base, pc.ord_local), at<int32_t>(base, pc.chunk_cnt), at<int32_t>(base, pc.M)};
  ProbeScope probe(MOE_K_SCHEDULE, static_cast<hipStream_t>(stream));
  return hip_status(moe::launch_schedule(
      routes, static_cast<int>(shape->num_src_ranks), static_cast<int>(NK), static_cast<int>(shape->rank),
      static_cast<int>(shape->experts_per_rank), static_cast<int>(shape->E_total), shape->max_rows, expert_counts,
      expert_offsets, sched_src, route_dst, sc, dev_error, static_cast<hipStream_t>(stream)));
}

moe_status moe_forward(const moe_shape* shape, const moe_weights* w, const void* x_src, const void* x_local,
                       const float* topk_gate, const int32_t* expert_offsets, const int32_t* sched_src,
                       const int32_t* route_dst, void* out, float* out32, void* ws, size_t ws_bytes,
                       void* stream) {
  Layout L;
  const moe_status st = check_ws(shape, ws, ws_bytes, &L);
  if (st != MOE_OK) return st;
  const bool mx = shape->precision == MOE_MXFP8;
  if (!w || !w->w_gate || !w->w_up || !w->w_down || !w->ws_gate || !w->ws_up || !w->ws_down) return MOE_ERR_INVALID_ARG;
  if (mx && (!w->s_gate || !w->s_up || !w->s_down)) return MOE_ERR_INVALID_ARG;
  const bool shared_mx = shape->shared_precision == MOE_MXFP8;
  if (shared_mx && (!w->ss_gate || !w->ss_up || !w->ss_down)) return MOE_ERR_INVALID_ARG;
  if (!expert_offsets || !route_dst || !topk_gate || !out) return MOE_ERR_INVALID_ARG;
  if (shape->T > 0 && !x_local) return MOE_ERR_INVALID_ARG;
  if (shape->max_rows > 0 && (!x_src || !sched_src)) return MOE_ERR_INVALID_ARG;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int T = static_cast<int>(shape->T), D = static_cast<int>(shape->D), I = static_cast<int>(shape->I);
  const int Is = static_cast<int>(shape->I_shared), k = static_cast<int>(shape->k);
  const int Lx = static_cast<int>(shape->experts_per_rank);
  const int64_t b = shape->minibatch_rows, C = shape->ring_rows, R = shape->num_src_ranks;
  if (T == 0 && shape->max_rows == 0) return MOE_OK;
  if (shape->pipeline) {
    // the persistent kernel's grid is every workgroup the chip holds at once
    // (a host query): at least 8 of them must be left for the GEMMs, and some
    // must gather when the ring holds fewer than all minibatches
    const int grid = moe::pipeline_workgroups(moe::RoutedTiling{L.routed_bm, L.bn_up, L.bn_down});
    if (grid <= 0) return MOE_ERR_HIP;
    if (shape->mem_workgroups > grid - 8) return MOE_ERR_INVALID_ARG;
    if (L.n_minibatches > C / b && shape->mem_workgroups == 0) return MOE_ERR_INVALID_ARG;
  }

  uint16_t* ring = at<uint16_t>(ws, L.ring);
  uint16_t* h = at<uint16_t>(ws, L.h);
  uint16_t* Y = at<uint16_t>(ws, L.Y);
  uint16_t* h_sh = at<uint16_t>(ws, L.h_shared);
  float* sh_out = at<float>(ws, L.shared_out);
  int4* tiles = at<int4>(ws, L.tiles);
  int32_t* tile_count = at<int32_t>(ws, L.tile_count);
  int32_t* tile_runs = at<int32_t>(ws, L.tile_runs);
  const int bm = L.routed_bm;

  // 1. tile lists of every minibatch (and their XCD runs), from the
  // device-side expert offsets
  {
    ProbeScope probe(MOE_K_TILES, s);
    MOE_TRY_HIP(moe::launch_build_tiles(expert_offsets, Lx, b, shape->max_rows, bm,
                                        static_cast<int>(L.n_minibatches), L.max_tiles,
                                        tiles, tile_count, tile_runs, s));
  }

  // 2. shared expert on this rank's tokens (MoK paper §3.4, "Shared Expert":
  //    it needs no dispatch, so it goes first)
  if (T > 0 && shared_mx) {
    MOE_TRY_HIP(shared_expert_mx(shape, w, x_local, L, ws, s));
  } else if (T > 0) {
    moe::GemmArgs g{};
    g.k_splits = 1;
    g.A = static_cast<const uint16_t*>(x_local);
    g.a_bytes = static_cast<int64_t>(T) * D * 2;
    g.lda = D;
    g.a_sub = 0;
    g.a_mod = INT64_MAX;
    g.B0 = static_cast<const uint16_t*>(w->ws_gate);
    g.B1 = static_cast<const uint16_t*>(w->ws_up);
    g.b_expert_stride = 0;
    g.N = Is;
    g.K = D;
    g.C = h_sh;
    g.ldc = Is;
    g.dense_rows = T;
    {
      ProbeScope probe(MOE_K_SHARED_UP, s);
      MOE_TRY_HIP(moe::launch_gemm(g, moe::kEpiSwiGLU, s));
    }
    moe::GemmArgs d{};
    d.k_splits = 1;
    d.A = h_sh;
    d.a_bytes = static_cast<int64_t>(T) * Is * 2;
    d.lda = Is;
    d.a_sub = 0;
    d.a_mod = INT64_MAX;
    d.B0 = static_cast<const uint16_t*>(w->ws_down);
    d.b_expert_stride = 0;
    d.N = D;
    d.K = Is;
    d.C = sh_out;
    d.ldc = D;
    d.dense_rows = T;
    ProbeScope probe(MOE_K_SHARED_DOWN, s);
    MOE_TRY_HIP(moe::launch_gemm(d, moe::kEpiF32, s));
  }

  // 3. routed experts, one minibatch of b schedule rows at a time
  // (bf16 GEMM arguments of minibatch m: up/gate reads ring slots p mod C and
  // writes h rows p - m*b; down reads them and writes each row to its route,
  // or to outbox row p when R > 1)
  auto up_args = [&](int64_t m, uint16_t* hbuf) {
    moe::GemmArgs u{};
    u.k_splits = 1;
    u.A = ring;
    u.a_bytes = C * D * 2;
    u.lda = D;
    u.a_sub = 0;
    u.a_mod = C;
    u.B0 = static_cast<const uint16_t*>(w->w_gate);
    u.B1 = static_cast<const uint16_t*>(w->w_up);
    u.b_expert_stride = static_cast<int64_t>(I) * D;
    u.b_plane = shape->weights_tiled ? I : 0;
    u.N = I;
    u.K = D;
    u.C = hbuf;
    u.ldc = I;
    u.c_idx = nullptr;
    u.c_sub = m * b;
    u.tiles = tiles + m * L.max_tiles;
    u.tile_count = tile_count + m;
    u.tile_runs = tile_runs + m * moe::kTileRunBounds;
    u.max_tiles = L.max_tiles;
    u.tile_rows = L.routed_bm;
    u.tile_cols = L.bn_up;
    return u;
  };
  auto down_args = [&](int64_t m, const uint16_t* hbuf) {
    moe::GemmArgs d{};
    d.k_splits = 1;
    d.A = hbuf;
    d.a_bytes = b * I * 2;
    d.lda = I;
    d.a_sub = m * b;
    d.a_mod = INT64_MAX;
    d.B0 = static_cast<const uint16_t*>(w->w_down);
    d.b_expert_stride = static_cast<int64_t>(D) * I;
    d.b_plane = shape->weights_tiled ? D : 0;
    d.N = D;
    d.K = I;
    d.C = Y;
    d.ldc = D;
    d.c_idx = (R == 1) ? sched_src : nullptr;  // push each row back to its route (§3.1 table reuse)
    d.c_sub = 0;
    d.tiles = tiles + m * L.max_tiles;
    d.tile_count = tile_count + m;
    d.tile_runs = tile_runs + m * moe::kTileRunBounds;
    d.max_tiles = L.max_tiles;
    d.tile_rows = L.routed_bm;
    d.tile_cols = L.bn_down;
    return d;
  };
  auto gather = [&](int64_t m) {
    const int64_t p_begin = m * b, rows = std::min<int64_t>(b, shape->max_rows - p_begin);
    ProbeScope probe(MOE_K_GATHER, s);
    if (R == 1 && L.n_minibatches == 1)  // one minibatch holds every row: read each token once
      return moe::launch_gather_src(static_cast<const uint16_t*>(x_src), T, D, k, route_dst, shape->max_rows, C, ring,
                                    at<int>(ws, L.err), s);
    return moe::launch_gather(static_cast<const uint16_t*>(x_src), R * shape->T, D, k, sched_src, expert_offsets, Lx,
                              p_begin, rows, C, ring, at<int>(ws, L.err), s);
  };
  if (shape->pipeline && L.n_minibatches > 0) {
    // the minibatches the ring holds at once are gathered by the whole chip;
    // the persistent kernel gathers the rest while it runs the GEMMs
    const int64_t pre = std::min<int64_t>(C / b, L.n_minibatches);
    int32_t* counters = at<int32_t>(ws, L.pipe_counters);
    const int64_t n_counters = (3 + L.max_tiles) * L.n_minibatches;
    MOE_TRY_HIP(moe::launch_clear_int(counters, static_cast<int>(n_counters + moe::kPipeQueueInts), s));
    for (int64_t m = 0; m < pre; ++m) MOE_TRY_HIP(gather(m));
    moe::PipeArgs pa{};
    pa.up = up_args(0, h);
    pa.down = down_args(0, h);
    pa.x_src = static_cast<const uint16_t*>(x_src);
    pa.src_rows = R * shape->T;
    pa.sched_src = sched_src;
    pa.offsets = expert_offsets;
    pa.L = Lx;
    pa.k = k;
    pa.D = D;
    pa.n_mb = static_cast<int>(L.n_minibatches);
    // memory workgroups only when some minibatch is gathered inside the
    // kernel; otherwise every workgroup runs GEMM items
    pa.n_mem = L.n_minibatches > C / b ? shape->mem_workgroups : 0;
    pa.b = b;
    pa.C = C;
    pa.max_rows = shape->max_rows;
    pa.ring = ring;
    pa.h = h;
    pa.n_h = moe::pipeline_h_buffers(b, C);
    pa.gathered = counters;
    pa.upg = counters + L.n_minibatches;
    pa.down_done = counters + 2 * L.n_minibatches;
    pa.upg_tile = counters + 3 * L.n_minibatches;
    pa.queue = counters + n_counters;
    pa.err = at<int>(ws, L.err);
    {
      ProbeScope probe(MOE_K_PIPELINE, s);
      MOE_TRY_HIP(moe::launch_pipeline(pa, moe::RoutedTiling{L.routed_bm, L.bn_up, L.bn_down}, s));
    }
  } else {
    for (int64_t m = 0; m < L.n_minibatches; ++m) {
      const int64_t p_begin = m * b;
      const int64_t rows = std::min<int64_t>(b, shape->max_rows - p_begin);
      if (mx) {
        MOE_TRY_HIP(
            routed_minibatch_mx(shape, w, x_src, sched_src, expert_offsets, route_dst, L, ws, m, p_begin, rows, s));
        continue;
      }
      MOE_TRY_HIP(gather(m));
      {
        ProbeScope probe(MOE_K_UP_GATE, s);
        MOE_TRY_HIP(moe::launch_gemm(up_args(m, h), moe::kEpiSwiGLU, s));
      }
      ProbeScope probe(MOE_K_DOWN, s);
      MOE_TRY_HIP(moe::launch_gemm(down_args(m, h), moe::kEpiBF16, s));
    }
  }

  // 4. fixed-order gate-weighted combine
  ProbeScope probe(MOE_K_COMBINE, s);
  return hip_status(moe::launch_combine(Y, sh_out, topk_gate, route_dst, shape->rank * T * static_cast<int64_t>(k), T,
                                        D, k, R > 1, static_cast<uint16_t*>(out), out32, s));
}

moe_status moe_routed_rows(const moe_shape* shape, const void* ws, size_t ws_bytes, const void** rows,
                           int64_t* n_rows) {
  Layout L;
  const moe_status st = check_ws(shape, ws, ws_bytes, &L);
  if (st != MOE_OK) return st;
  if (!rows || !n_rows) return MOE_ERR_INVALID_ARG;
  *rows = static_cast<const char*>(ws) + L.Y;
  *n_rows = L.y_rows;
  return MOE_OK;
}

moe_status moe_tile_bf16(const void* src, int64_t groups, int64_t rows, int64_t K, void* dst, void* stream) {
  if (groups < 0 || rows < 0 || K <= 0 || K % moe::kTileK != 0) return MOE_ERR_INVALID_ARG;
  if (groups == 0 || rows == 0) return MOE_OK;
  if (!src || !dst || src == dst) return MOE_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(src) % 16 || reinterpret_cast<uintptr_t>(dst) % 16) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_tile_bf16(static_cast<const uint16_t*>(src), groups, rows, K,
                                          static_cast<uint16_t*>(dst), static_cast<hipStream_t>(stream)));
}

moe_status moe_quantize_mxfp8(const void* src, int64_t rows, int64_t K, uint8_t* q, uint8_t* scale, void* stream) {
  if (rows < 0 || K <= 0 || K % 32 != 0) return MOE_ERR_INVALID_ARG;
  if (rows == 0) return MOE_OK;
  if (!src || !q || !scale) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_quantize_mxfp8(static_cast<const uint16_t*>(src), rows, K, q, scale,
                                               static_cast<hipStream_t>(stream)));
}

moe_status moe_mxfp8_pack_scales(const uint8_t* scale, int64_t groups, int64_t rows, int64_t K, uint8_t* packed,
                                 void* stream) {
  if (groups < 0 || rows < 0 || K <= 0 || K % 128 != 0) return MOE_ERR_INVALID_ARG;
  if (groups == 0 || rows == 0) return MOE_OK;
  if (!scale || !packed || scale == packed) return MOE_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(scale) % 4 || reinterpret_cast<uintptr_t>(packed) % 4) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_pack_mx_scales(scale, groups, rows, K, packed, static_cast<hipStream_t>(stream)));
}

moe_status moe_probe_begin(int32_t kernel_id, int32_t max_launches) {
  if (kernel_id < 0 || kernel_id >= MOE_K_COUNT || max_launches < 1 || max_launches > (1 << 20))
    return MOE_ERR_INVALID_ARG;
  double ms;
  int32_t n;
  if (g_probe.kernel >= 0) moe_probe_end(&ms, &n);
  g_probe.start.assign(max_launches, nullptr);
  g_probe.stop.assign(max_launches, nullptr);
  for (int i = 0; i < max_launches; ++i) {
    if (hipEventCreate(&g_probe.start[i]) != hipSuccess || hipEventCreate(&g_probe.stop[i]) != hipSuccess) {
      g_probe.max_launches = i;
      g_probe.kernel = kernel_id;
      moe_probe_end(&ms, &n);
      return MOE_ERR_HIP;
    }
  }
  g_probe.kernel = kernel_id;
  g_probe.max_launches = max_launches;
  g_probe.used = 0;
  return MOE_OK;
}

moe_status moe_probe_end(double* total_ms, int32_t* launches) {
  if (!total_ms || !launches) return MOE_ERR_INVALID_ARG;
  *total_ms = 0.0;
  *launches = 0;
  moe_status st = MOE_OK;
  if (g_probe.kernel >= 0 && g_probe.used > 0) {
    if (hipDeviceSynchronize() != hipSuccess) st = MOE_ERR_HIP;
    for (int i = 0; i < g_probe.used && st == MOE_OK; ++i) {
      float ms = 0.f;
      if (hipEventElapsedTime(&ms, g_probe.start[i], g_probe.stop[i]) != hipSuccess) st = MOE_ERR_HIP;
      *total_ms += ms;
    }
    *launches = g_probe.used;
  }
  for (size_t i = 0; i < g_probe.start.size(); ++i) {
    if (g_probe.start[i]) (void)hipEventDestroy(g_probe.start[i]);
    if (g_probe.stop[i]) (void)hipEventDestroy(g_probe.stop[i]);
  }
  g_probe = Probe{};
  return st;
}

moe_status moe_get_device_error(const moe_shape* shape, const void* ws, size_t ws_bytes, void* stream,
                                int32_t* host_code) {
  Layout L;
  const moe_status st = check_ws(shape, ws, ws_bytes, &L);
  if (st != MOE_OK) return st;
  if (!host_code) return MOE_ERR_INVALID_ARG;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  MOE_TRY_HIP(hipMemcpyAsync(host_code, static_cast<const char*>(ws) + L.err, sizeof(int32_t), hipMemcpyDeviceToHost, s));
  return hip_status(hipStreamSynchronize(s));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Backward pass
// ---------------------------------------------------------------------------
namespace {

int64_t pad64(int64_t v) { return (v + 63) / 64 * 64; }

struct BwdLayout {
  size_t tiles, tile_count, tile_runs, padded, k_groups, seg_off, seg_pad, seg_kg, ring, dy, act, dh, h, da, dx_ring, dyT, hT, daT,
      xT, dg, dl, dlT, act_s, dh_s, h_s, da_s, dx_s, doutT, h_sT, da_sT, x_T, dx_r, total;
  int64_t P, Ppad, Tpad, Ep;
  moe::RoutedTiling tiling;
  int max_tiles;
};

// Backward shapes: one GPU, bf16 routed and shared experts; every GEMM
// operand (read through a buffer resource) below 2^31 bytes.
bool valid_bwd_shape(const moe_shape* s, moe_status* why) {
  if (!valid_shape(s, why)) return false;
  *why = MOE_ERR_UNSUPPORTED;
  if (s->num_src_ranks != 1 || s->precision != MOE_BF16 || s->shared_precision != MOE_BF16 || s->weights_tiled)
    return false;
  constexpr int64_t kLimit = int64_t(1) << 31;
  const int64_t P = s->T * s->k, Ppad = pad64(P) + 64 * s->experts_per_rank, Tpad = pad64(s->T);
  const int64_t Ep = pad64(s->E_total);
  const int64_t bytes[] = {P * s->D * 2,       P * 2 * s->I * 2,         s->D * Ppad * 2,        2 * s->I * Ppad * 2,
                           s->T * 2 * s->I_shared * 2, s->D * Tpad * 2, 2 * s->I_shared * Tpad * 2, s->T * Ep * 2,
                           Ep * Tpad * 2,      s->D * Ep * 2,            2 * s->I * s->D * 2};
  for (const int64_t v : bytes)
    if (v >= kLimit) return false;
  *why = MOE_OK;
  return true;
}

BwdLayout bwd_layout_of(const moe_shape* s) {
  BwdLayout L{};
  const int64_t T = s->T, D = s->D, I = s->I, Is = s->I_shared, Lx = s->experts_per_rank;
  L.P = T * s->k;
  L.Ppad = pad64(L.P) + 64 * Lx;  // every segment padded to 64 rows
  L.Tpad = pad64(T);
  L.Ep = pad64(s->E_total);
  L.tiling = moe::gemm_routed_tiling(L.P, L.P, Lx, I, D, false);
  L.max_tiles = moe::gemm_tiles_bound(L.P, static_cast<int>(Lx), L.tiling.bm);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  L.tiles = take(sizeof(int4) * L.max_tiles);
  L.tile_count = take(sizeof(int32_t));
  L.tile_runs = take(sizeof(int32_t) * moe::kTileRunBounds);
  L.padded = take(sizeof(int32_t) * (Lx + 1));
  L.k_groups = take(sizeof(int2) * Lx);
  L.seg_off = take(sizeof(int32_t) * 2);
  L.seg_pad = take(sizeof(int32_t) * 2);
  L.seg_kg = take(sizeof(int2));
  L.ring = take(2 * L.P * D);
  L.dy = take(2 * L.P * D);
  L.act = take(2 * L.P * 2 * I);
  L.dh = take(4 * L.P * I);
  L.h = take(2 * L.P * I);
  L.da = take(2 * L.P * 2 * I);
  L.dx_ring = take(4 * L.P * D);
  L.dyT = take(2 * D * L.Ppad);
  L.hT = take(2 * I * L.Ppad);
  L.daT = take(2 * 2 * I * L.Ppad);
  L.xT = take(2 * D * L.Ppad);
  L.dg = take(4 * L.P);
  L.dl = take(2 * T * L.Ep);
  L.dlT = take(2 * L.Ep * L.Tpad);
  L.act_s = take(2 * T * 2 * Is);
  L.dh_s = take(4 * T * Is);
  L.h_s = take(2 * T * Is);
  L.da_s = take(2 * T * 2 * Is);
  L.dx_s = take(4 * T * D);
  L.doutT = take(2 * D * L.Tpad);
  L.h_sT = take(2 * Is * L.Tpad);
  L.da_sT = take(2 * 2 * Is * L.Tpad);
  L.x_T = take(2 * D * L.Tpad);
  L.dx_r = take(4 * T * D);
  L.total = off;
  return L;
}

// C = A B^T over dense rows (M x N, K-contiguous operands), optionally with
// grouped K ranges (groups stacked in the output `group_stride` elements
// apart).
moe::GemmArgs dense_args(const void* A, int64_t lda, int64_t M, const void* B, int64_t ldb, int N, int K, void* C,
                         int64_t ldc) {
  moe::GemmArgs g{};
  g.k_splits = 1;
  g.A = static_cast<const uint16_t*>(A);
  g.a_bytes = M * lda * 2;
  g.lda = lda;
  g.a_sub = 0;
  g.a_mod = INT64_MAX;
  g.B0 = static_cast<const uint16_t*>(B);
  g.ldb = ldb;
  g.N = N;
  g.K = K;
  g.C = C;
  g.ldc = ldc;
  g.dense_rows = static_cast<int>(M);
  return g;
}

}  // namespace

extern "C" {

moe_status moe_backward_workspace_bytes(const moe_shape* shape, size_t* bytes) {
  moe_status why;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  if (!valid_bwd_shape(shape, &why)) return why;
  *bytes = bwd_layout_of(shape).total;
  return MOE_OK;
}

moe_status moe_backward_prepare(const moe_shape* shape, const moe_weights* w, const void* w_router,
                                const moe_bwd_weights* bw, void* stream) {
  moe_status why;
  if (!valid_bwd_shape(shape, &why)) return why;
  if (!w || !bw || !w_router || !w->w_gate || !w->w_up || !w->w_down || !w->ws_gate || !w->ws_up || !w->ws_down)
    return MOE_ERR_INVALID_ARG;
  if (!bw->w_gu || !bw->w_gu_t || !bw->w_down_t || !bw->ws_gu || !bw->ws_gu_t || !bw->ws_down_t || !bw->w_router_t)
    return MOE_ERR_INVALID_ARG;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int L = static_cast<int>(shape->experts_per_rank), D = static_cast<int>(shape->D);
  const int I = static_cast<int>(shape->I), Is = static_cast<int>(shape->I_shared), E = static_cast<int>(shape->E_total);
  const int64_t Ep = pad64(E);
  // the routed copies are K-tiled (the backward's routed GEMMs read one
  // plane per K stage, as the forward's do with K-tiled weights):
  // w_gu: gate rows then up rows of each expert, [L, D/64, 2I, 64]
  const uint16_t* wg = static_cast<const uint16_t*>(w->w_gate);
  const uint16_t* wu = static_cast<const uint16_t*>(w->w_up);
  const uint16_t* wd = static_cast<const uint16_t*>(w->w_down);
  auto* gu = static_cast<uint16_t*>(bw->w_gu);
  const int64_t gu_stride = static_cast<int64_t>(2) * I * D;
  MOE_TRY_HIP(moe::launch_tile_bf16(wg, L, I, D, gu, s, 2 * I, 0, gu_stride));
  MOE_TRY_HIP(moe::launch_tile_bf16(wu, L, I, D, gu, s, 2 * I, I, gu_stride));
  // w_gu_t: [W_gate^T | W_up^T], [L, 2I/64, D, 64]; w_down_t: [L, D/64, I, 64]
  auto* gut = static_cast<uint16_t*>(bw->w_gu_t);
  MOE_TRY_HIP(moe::launch_transpose(wg, L, I, D, gut, 2 * I, static_cast<int64_t>(D) * 2 * I, 0, s, D));
  MOE_TRY_HIP(moe::launch_transpose(wu, L, I, D, gut, 2 * I, static_cast<int64_t>(D) * 2 * I, I, s, D));
  MOE_TRY_HIP(moe::launch_transpose(wd, L, D, I, static_cast<uint16_t*>(bw->w_down_t), D,
                                    static_cast<int64_t>(I) * D, 0, s, I));
  const size_t sslab = static_cast<size_t>(Is) * D * 2;
  MOE_TRY_HIP(hipMemcpyAsync(bw->ws_gu, w->ws_gate, sslab, hipMemcpyDeviceToDevice, s));
  MOE_TRY_HIP(hipMemcpyAsync(static_cast<char*>(bw->ws_gu) + sslab, w->ws_up, sslab, hipMemcpyDeviceToDevice, s));
  auto* sgut = static_cast<uint16_t*>(bw->ws_gu_t);
  MOE_TRY_HIP(moe::launch_transpose(static_cast<const uint16_t*>(w->ws_gate), 1, Is, D, sgut, 2 * Is, 0, 0, s));
  MOE_TRY_HIP(moe::launch_transpose(static_cast<const uint16_t*>(w->ws_up), 1, Is, D, sgut, 2 * Is, 0, Is, s));
  MOE_TRY_HIP(moe::launch_transpose(static_cast<const uint16_t*>(w->ws_down), 1, D, Is,
                                    static_cast<uint16_t*>(bw->ws_down_t), D, 0, 0, s));
  // W_r^T with its columns past E_total zero
  MOE_TRY_HIP(moe::launch_clear_int(static_cast<int*>(bw->w_router_t), static_cast<int>(D * Ep / 2), s));
  MOE_TRY_HIP(moe::launch_transpose(static_cast<const uint16_t*>(w_router), 1, E, D,
                                    static_cast<uint16_t*>(bw->w_router_t), Ep, 0, 0, s));
  return MOE_OK;
}

moe_status moe_backward(const moe_shape* shape, const moe_bwd_weights* bw, const void* x, const int32_t* topk_idx,
                        const float* topk_gate, const int32_t* expert_offsets, const int32_t* sched_src,
                        const int32_t* route_dst, const void* y_routes, const void* dout, const moe_grads* g,
                        int32_t* dev_error, void* ws, size_t ws_bytes, void* stream) {
  moe_status why;
  if (!valid_bwd_shape(shape, &why)) return why;
  const BwdLayout L = bwd_layout_of(shape);
  if (!ws || reinterpret_cast<uintptr_t>(ws) % kAlign) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (!bw || !g || !dev_error || !x || !topk_idx || !topk_gate || !expert_offsets || !sched_src || !route_dst ||
      !y_routes || !dout)
    return MOE_ERR_INVALID_ARG;
  // rows are read in 16-byte pieces
  for (const void* p : {x, y_routes, dout})
    if (reinterpret_cast<uintptr_t>(p) % 16) return MOE_ERR_INVALID_ARG;
  if (!bw->w_gu || !bw->w_gu_t || !bw->w_down_t || !bw->ws_gu || !bw->ws_gu_t || !bw->ws_down_t || !bw->w_router_t)
    return MOE_ERR_INVALID_ARG;
  if (!g->dx || !g->dw_gate || !g->dw_up || !g->dw_down || !g->dws_gate || !g->dws_up || !g->dws_down ||
      !g->dw_router)
    return MOE_ERR_INVALID_ARG;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int T = static_cast<int>(shape->T), D = static_cast<int>(shape->D), I = static_cast<int>(shape->I);
  const int Is = static_cast<int>(shape->I_shared), k = static_cast<int>(shape->k);
  const int E = static_cast<int>(shape->E_total), Lx = static_cast<int>(shape->experts_per_rank);
  const int64_t P = L.P, Ppad = L.Ppad, Tpad = L.Tpad, Ep = L.Ep;
  if (T == 0) return MOE_OK;
  int4* tiles = at<int4>(ws, L.tiles);
  int32_t* tile_count = at<int32_t>(ws, L.tile_count);
  int32_t* tile_runs = at<int32_t>(ws, L.tile_runs);
  uint16_t* ring = at<uint16_t>(ws, L.ring);
  uint16_t* dy = at<uint16_t>(ws, L.dy);
  uint16_t* act = at<uint16_t>(ws, L.act);
  float* dh = at<float>(ws, L.dh);
  uint16_t* h = at<uint16_t>(ws, L.h);
  uint16_t* da = at<uint16_t>(ws, L.da);
  float* dx_ring = at<float>(ws, L.dx_ring);
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const uint16_t* dob = static_cast<const uint16_t*>(dout);

  // ---- routed experts: the forward's rows again, in schedule order ----
  MOE_TRY_HIP(moe::launch_build_tiles(expert_offsets, Lx, P, P, L.tiling.bm, 1, L.max_tiles, tiles, tile_count,
                                      tile_runs, s));
  MOE_TRY_HIP(moe::launch_gather_src(xb, T, D, k, route_dst, P, P, ring, dev_error, s));
  MOE_TRY_HIP(moe::launch_dy_gather(dob, topk_gate, sched_src, P, T, D, k, dy, dev_error, s));
  auto routed = [&](const void* A, int64_t lda, const void* B, int64_t b_stride, int N, int K, void* C, int64_t ldc) {
    moe::GemmArgs a{};
    a.k_splits = 1;
    a.A = static_cast<const uint16_t*>(A);
    a.a_bytes = P * lda * 2;
    a.lda = lda;
    a.a_sub = 0;
    a.a_mod = INT64_MAX;
    a.B0 = static_cast<const uint16_t*>(B);
    a.b_expert_stride = b_stride;
    a.b_plane = N;  // the prepared routed weights are K-tiled
    a.N = N;
    a.K = K;
    a.C = C;
    a.ldc = ldc;
    a.tiles = tiles;
    a.tile_count = tile_count;
    a.tile_runs = tile_runs;
    a.max_tiles = L.max_tiles;
    a.tile_rows = L.tiling.bm;
    a.tile_cols = 256;
    return a;
  };
  {
    ProbeScope probe(MOE_K_BWD_REPLAY, s);  // act = [a_g | a_u] of every routed row
    MOE_TRY_HIP(moe::launch_gemm(routed(ring, D, bw->w_gu, int64_t(2) * I * D, 2 * I, D, act, 2 * I),
                                 moe::kEpiBF16, s));
  }
  {
    ProbeScope probe(MOE_K_BWD_DGRAD, s);  // dh = dY W_down, then dx_ring = da [W_gate; W_up]
    MOE_TRY_HIP(moe::launch_gemm(routed(dy, D, bw->w_down_t, int64_t(I) * D, I, D, dh, I), moe::kEpiF32, s));
    MOE_TRY_HIP(moe::launch_swiglu_bwd(act, dh, P, I, h, da, s));
    MOE_TRY_HIP(moe::launch_gemm(routed(da, 2 * I, bw->w_gu_t, int64_t(D) * 2 * I, D, 2 * I, dx_ring, D),
                                 moe::kEpiF32, s));
  }
  {
    // weight gradients: per expert, K = its rows (padded to 64 with zeros)
    ProbeScope probe(MOE_K_BWD_WGRAD, s);
    int32_t* padded = at<int32_t>(ws, L.padded);
    int2* kg = at<int2>(ws, L.k_groups);
    uint16_t* dyT = at<uint16_t>(ws, L.dyT);
    uint16_t* hT = at<uint16_t>(ws, L.hT);
    uint16_t* daT = at<uint16_t>(ws, L.daT);
    uint16_t* xT = at<uint16_t>(ws, L.xT);
    MOE_TRY_HIP(moe::launch_pad_offsets(expert_offsets, Lx, padded, kg, s));
    // the transposed operands are K-tiled (planes of 64 rows of the segment
    // axis), so each K stage of the grouped GEMMs reads contiguous planes
    MOE_TRY_HIP(moe::launch_seg_transpose(dy, D, D, expert_offsets, padded, Lx, Ppad, dyT, Ppad, s, true));
    MOE_TRY_HIP(moe::launch_seg_transpose(h, I, I, expert_offsets, padded, Lx, Ppad, hT, Ppad, s, true));
    MOE_TRY_HIP(moe::launch_seg_transpose(da, 2 * I, 2 * I, expert_offsets, padded, Lx, Ppad, daT, Ppad, s, true));
    MOE_TRY_HIP(moe::launch_seg_transpose(ring, D, D, expert_offsets, padded, Lx, Ppad, xT, Ppad, s, true));
    // A: M rows starting at row a0 of planes of a_rows rows; B: planes of N rows
    auto grouped = [&](const uint16_t* A, int64_t M, int64_t a_rows, int64_t a0, const uint16_t* B, int N, void* C,
                       int64_t ldc, int64_t gs) {
      moe::GemmArgs a = dense_args(A + a0 * moe::kTileK, Ppad, M, B, Ppad, N, 0, C, ldc);
      a.a_plane = a_rows;
      a.a_bytes = (a_rows * Ppad - a0 * moe::kTileK) * 2;
      a.b_plane = N;
      a.k_groups = kg;
      a.n_groups = Lx;
      a.c_group_stride = gs;
      return a;
    };
    MOE_TRY_HIP(moe::launch_gemm(grouped(dyT, D, D, 0, hT, I, g->dw_down, I, int64_t(D) * I), moe::kEpiBF16, s));
    MOE_TRY_HIP(moe::launch_gemm(grouped(daT, I, 2 * I, 0, xT, D, g->dw_gate, D, int64_t(I) * D), moe::kEpiBF16, s));
    MOE_TRY_HIP(moe::launch_gemm(grouped(daT, I, 2 * I, I, xT, D, g->dw_up, D, int64_t(I) * D), moe::kEpiBF16, s));
  }

  // ---- the shared expert, on every token with dy = dout ----
  uint16_t* act_s = at<uint16_t>(ws, L.act_s);
  float* dh_s = at<float>(ws, L.dh_s);
  uint16_t* h_s = at<uint16_t>(ws, L.h_s);
  uint16_t* da_s = at<uint16_t>(ws, L.da_s);
  float* dx_s = at<float>(ws, L.dx_s);
  MOE_TRY_HIP(moe::launch_gemm(dense_args(xb, D, T, bw->ws_gu, 0, 2 * Is, D, act_s, 2 * Is), moe::kEpiBF16, s));
  MOE_TRY_HIP(moe::launch_gemm(dense_args(dob, D, T, bw->ws_down_t, 0, Is, D, dh_s, Is), moe::kEpiF32, s));
  MOE_TRY_HIP(moe::launch_swiglu_bwd(act_s, dh_s, T, Is, h_s, da_s, s));
  MOE_TRY_HIP(moe::launch_gemm(dense_args(da_s, 2 * Is, T, bw->ws_gu_t, 0, D, 2 * Is, dx_s, D), moe::kEpiF32, s));
  int32_t* seg_off = at<int32_t>(ws, L.seg_off);
  int32_t* seg_pad = at<int32_t>(ws, L.seg_pad);
  int2* seg_kg = at<int2>(ws, L.seg_kg);
  uint16_t* doutT = at<uint16_t>(ws, L.doutT);
  uint16_t* h_sT = at<uint16_t>(ws, L.h_sT);
  uint16_t* da_sT = at<uint16_t>(ws, L.da_sT);
  uint16_t* x_T = at<uint16_t>(ws, L.x_T);
  MOE_TRY_HIP(moe::launch_single_segment(T, seg_off, seg_pad, seg_kg, s));
  MOE_TRY_HIP(moe::launch_seg_transpose(dob, D, D, seg_off, seg_pad, 1, Tpad, doutT, Tpad, s, true));
  MOE_TRY_HIP(moe::launch_seg_transpose(h_s, Is, Is, seg_off, seg_pad, 1, Tpad, h_sT, Tpad, s, true));
  MOE_TRY_HIP(moe::launch_seg_transpose(da_s, 2 * Is, 2 * Is, seg_off, seg_pad, 1, Tpad, da_sT, Tpad, s, true));
  MOE_TRY_HIP(moe::launch_seg_transpose(xb, D, D, seg_off, seg_pad, 1, Tpad, x_T, Tpad, s, true));
  auto one_group = [&](const uint16_t* A, int64_t M, int64_t a_rows, int64_t a0, const uint16_t* B, int N, void* C,
                       int64_t ldc) {
    moe::GemmArgs a = dense_args(A + a0 * moe::kTileK, Tpad, M, B, Tpad, N, 0, C, ldc);
    a.a_plane = a_rows;
    a.a_bytes = (a_rows * Tpad - a0 * moe::kTileK) * 2;
    a.b_plane = N;
    a.k_groups = seg_kg;
    a.n_groups = 1;
    return a;
  };
  MOE_TRY_HIP(moe::launch_gemm(one_group(doutT, D, D, 0, h_sT, Is, g->dws_down, Is), moe::kEpiBF16, s));
  MOE_TRY_HIP(moe::launch_gemm(one_group(da_sT, Is, 2 * Is, 0, x_T, D, g->dws_gate, D), moe::kEpiBF16, s));
  MOE_TRY_HIP(moe::launch_gemm(one_group(da_sT, Is, 2 * Is, Is, x_T, D, g->dws_up, D), moe::kEpiBF16, s));

  // ---- router: gate gradients, the selected logits' gradient, its two products ----
  float* dg = at<float>(ws, L.dg);
  uint16_t* dl = at<uint16_t>(ws, L.dl);
  uint16_t* dlT = at<uint16_t>(ws, L.dlT);
  float* dx_r = at<float>(ws, L.dx_r);
  MOE_TRY_HIP(moe::launch_route_grad(dob, static_cast<const uint16_t*>(y_routes), P, D, k, dg, s));
  MOE_TRY_HIP(moe::launch_gate_grad(topk_gate, dg, topk_idx, T, E, static_cast<int>(Ep), k, dl, s));
  MOE_TRY_HIP(moe::launch_gemm(dense_args(dl, Ep, T, bw->w_router_t, 0, D, static_cast<int>(Ep), dx_r, D),
                               moe::kEpiF32, s));
  MOE_TRY_HIP(moe::launch_seg_transpose(dl, Ep, static_cast<int>(Ep), seg_off, seg_pad, 1, Tpad, dlT, Tpad, s, true));
  MOE_TRY_HIP(moe::launch_gemm(one_group(dlT, E, Ep, 0, x_T, D, g->dw_router, D), moe::kEpiF32, s));

  // ---- dx, in a fixed order ----
  return hip_status(moe::launch_dx_assemble(dx_s, dx_r, dx_ring, route_dst, T, D, k, P, g->dx, dev_error, s));
}

}  // extern "C"
