/*
 * moe.h - C ABI of the MI355X (gfx950) MoE-layer library, libmoe.so.
 *
 * The library computes the forward pass of one DeepSeek-V3-style MoE layer on
 * one GPU's share of the work (MoK paper "Mixture-of-Kittens: MoE Megakernel
 * for NVL72s", §2.1, MoE equation):
 *
 *   MoE(x) = f_shared(x) + sum_{i in E} g_i f_i(x),   g_i = s_i / sum_{j in E} s_j
 *   f_i(x) = W_down^(i) ( SiLU(W_gate^(i) x) * W_up^(i) x )
 *
 * in three calls, in stream order:
 *   moe_route     router projection, top-k selection and normalised gates;
 *   moe_schedule  the dispatch schedule of Algorithm 1 (per-expert counts,
 *                 prefix sums, the position -> source-route table and its
 *                 inverse);
 *   moe_forward   shared expert, then per minibatch of b routed rows: gather
 *                 into the ring buffer, grouped up/gate GEMM with SwiGLU,
 *                 grouped down GEMM; then the fixed-order gate-weighted combine.
 * and, for training on one GPU, the backward pass of such a forward
 * (moe_backward_prepare once per weight set, then moe_backward).
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers, allocated and owned by the caller;
 *     all tensors are dense row-major.  bf16 data are raw IEEE bfloat16 bit
 *     patterns (uint16_t), e4m3 data raw OCP E4M3FN bytes, scales raw E8M0
 *     bytes.
 *   - The library never allocates, frees or synchronises device memory, and
 *     never reads device memory on the host.  All work is enqueued on `stream`
 *     (a hipStream_t; NULL is the default stream).  Calls on distinct
 *     workspaces are independent; calls sharing a workspace must be ordered by
 *     the caller (stream order does that).
 *   - Shapes are validated on the host from `moe_shape` alone, before any
 *     launch; violations return MOE_ERR_INVALID_ARG / MOE_ERR_UNSUPPORTED.
 *     Every GEMM operand must stay below 2^31 bytes (x: T*D*2; the ring:
 *     C*D*e; h: b*I*e; the shared h: T*I_shared*e; one routed or the shared
 *     weight matrix: I*D*e, I_shared*D*e; e = 2 in bf16, 1 in MXFP8);
 *     larger shapes return MOE_ERR_UNSUPPORTED.
 *   - Data errors found on the device (an expert id out of range, more routed
 *     rows than `max_rows`, a non-finite router logit) set bits of a sticky
 *     word in the workspace and never cause an out-of-bounds access; read it
 *     with moe_get_device_error().  Tokens are never dropped silently.
 *   - Results are bitwise identical from run to run, and for every minibatch
 *     size b and ring size C: no floating-point atomics, no split-K, and the
 *     combine sums the k routed rows in slot order (MoK paper §3.4,
 *     "Determinism").
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 8

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null pointer, inconsistent sizes, bad tunable */
  MOE_ERR_UNSUPPORTED = -2, /* valid request the library does not implement */
  MOE_ERR_WORKSPACE = -3,   /* workspace smaller than moe_workspace_bytes() */
  MOE_ERR_HIP = -4          /* a HIP launch or runtime call failed */
} moe_status;

/* Arithmetic of the routed experts (MoK paper §3.4, "MXFP8 Support": the shared
 * expert always stays bf16). */
typedef enum { MOE_BF16 = 0, MOE_MXFP8 = 1 } moe_precision;

/* Device error bits, OR-ed into the workspace's sticky error word. */
#define MOE_DEVERR_EXPERT_RANGE 0x1 /* a route names an expert outside [0, E_total) */
#define MOE_DEVERR_ROW_OVERFLOW 0x2 /* routed rows exceed max_rows; extra rows skipped */
#define MOE_DEVERR_NONFINITE 0x4    /* a router logit is NaN or infinite */
#define MOE_DEVERR_PIPELINE 0x8     /* a persistent-kernel wait gave up (about 1 s):
                                       its workgroups were not all resident */

/*
 * Sizes and tunables.  On one GPU: num_src_ranks = 1, rank = 0,
 * experts_per_rank = E_total, tokens_per_src_rank = T, max_rows = T*k.
 * The (R, c, L, N) fields are those of Algorithm 1 (MoK paper §3.1): R source
 * ranks with N tokens each, this is rank c, which holds local experts
 * c*L .. c*L+L-1; they let one GPU build and run its share of an
 * expert-parallel layer from an all-gathered route matrix.
 */
typedef struct {
  int64_t T;                   /* tokens of this rank (rows of x_local, gates) */
  int64_t D;                   /* hidden width; multiple of 64 */
  int64_t I;                   /* routed expert intermediate width; multiple of 64 */
  int64_t I_shared;            /* shared expert intermediate width; multiple of 64 */
  int64_t E_total;             /* router width (all routed experts); <= 1024 */
  int64_t k;                   /* experts per token; 1 <= k <= min(E_total, 16) */
  int64_t num_src_ranks;       /* R */
  int64_t rank;                /* c */
  int64_t experts_per_rank;    /* L; R*L == E_total; L <= 1024 */
  int64_t tokens_per_src_rank; /* N; == T when R == 1 */
  int64_t max_rows;            /* bound on routed rows P received; T*k when R == 1 */
  int64_t minibatch_rows;      /* b: rows per gather/GEMM step (granularity), >= 1 */
  int64_t ring_rows;           /* C: ring buffer capacity, a positive multiple of b */
  int32_t precision;           /* moe_precision of the routed experts */
  int32_t shared_precision;    /* moe_precision of the shared expert: MOE_BF16, as
                                  the MoK paper keeps it (§3.4, "MXFP8 Support"),
                                  or MOE_MXFP8 as an option (D and I_shared then
                                  multiples of 128) */
  int32_t pipeline;            /* 0: the routed minibatch loop as stream-ordered
                                  launches (gather, up/gate, down per minibatch);
                                  1: as one persistent kernel whose workgroups
                                  wait on device-side counters (MoK paper §3.2,
                                  "Maximally Deferred Synchronization", "Kernel
                                  Fusion"); up/gate runs up to H - 1 minibatches
                                  ahead of down, H = C/b clamped to 2 .. 4 (H h
                                  buffers of [b, I] in the workspace); routed
                                  precision MOE_BF16 only */
  int32_t mem_workgroups;      /* pipeline == 1: workgroups of the persistent
                                  kernel that gather minibatches C/b and later
                                  (MoK paper §3.4, "Computation-Communication SM
                                  Tuning"); a multiple of 8, at least 8 when
                                  the ring holds fewer than all minibatches,
                                  and leaving at least 8 for the GEMMs; unused
                                  (every workgroup runs GEMM items) when the
                                  ring holds all minibatches */
  int32_t weights_tiled;       /* 0: the routed weights w_gate, w_up, w_down
                                  row-major as described under moe_weights;
                                  1: K-tiled, as moe_tile_bf16 writes them:
                                  each expert's [N, K] matrix as [K/64, N, 64]
                                  in bf16 (planes of 64 K columns, each
                                  holding all N rows), or its E4M3 bytes as
                                  [K/128, N, 128] in MXFP8 (moe_tile_bf16 on
                                  the bytes taken as 2-byte units; the scales
                                  stay as described under moe_weights), so
                                  that one K stage of the expert GEMMs reads
                                  one contiguous plane.  Values and results
                                  are the same either way */
} moe_shape;

/* Expert weights, all K-contiguous (each output row is a contiguous K vector):
 *   routed  w_gate, w_up [L, I, D]; w_down [L, D, I]   (bf16, or e4m3 for MXFP8;
 *           with moe_shape.weights_tiled, bf16 [L, D/64, I, 64] and
 *           [L, I/64, D, 64], e4m3 [L, D/128, I, 128] and [L, I/128, D, 128])
 *           s_gate, s_up [L, D/128, I, 4]; s_down [L, I/128, D, 4]   (E8M0,
 *           MXFP8 only): stage-major scales, as moe_mxfp8_pack_scales writes
 *           them from the row-major [L, N, K/32] of moe_quantize_mxfp8
 *   shared  ws_gate, ws_up [I_shared, D]; ws_down [D, I_shared]   (bf16, or
 *           e4m3 when shared_precision is MOE_MXFP8)
 *           ss_gate, ss_up [D/128, I_shared, 4]; ss_down [I_shared/128, D, 4]
 *           (E8M0, shared_precision MOE_MXFP8 only, else NULL): stage-major
 *           scales, as moe_mxfp8_pack_scales writes them with groups = 1
 * In MXFP8 the activations follow the weights: x (routed: in the gather;
 * shared: in its own pass) and h are quantised along their K axis. */
typedef struct {
  const void *w_gate, *w_up, *w_down;
  const uint8_t *s_gate, *s_up, *s_down;
  const void *ws_gate, *ws_up, *ws_down;
  const uint8_t *ss_gate, *ss_up, *ss_down;
} moe_weights;

/* Bytes of device workspace the three calls below need for `shape` (one
 * workspace serves all of them; it also holds the sticky error word).
 * Returns MOE_ERR_INVALID_ARG / MOE_ERR_UNSUPPORTED for a bad shape. */
moe_status moe_workspace_bytes(const moe_shape* shape, size_t* bytes);

/* Clear the workspace's sticky error word (one small kernel on `stream`). */
moe_status moe_workspace_init(const moe_shape* shape, void* ws, size_t ws_bytes, void* stream);

/*
 * Router projection, top-k selection and gates (MoK paper §2.1: the router
 * projection picks each token's k routed experts and gives each one a weight;
 * the weights are normalised over the chosen experts, g_i = s_i / sum_{j in E}
 * s_j in the MoK blog's notation, with s the softmax of the logits).
 *
 *   x         [T, D] bf16, or NULL: then `logits` is an INPUT (given logits,
 *             as in the MoK paper's §4.1 benchmark protocol)
 *   w_router  [E_total, D] bf16 (ignored when x is NULL)
 *   logits    [T, E_total] fp32: output of x @ w_router^T (fp32 accumulation),
 *             or input when x is NULL
 *   topk_idx  [T, k] int32 out: slot s of token t holds the expert with the
 *             s-th largest logit; ties go to the lower expert id; -0.0 == +0.0
 *   topk_gate [T, k] fp32 out: exp(l_s - l_0) / sum_{s'} exp(l_s' - l_0)
 * A non-finite logit sets MOE_DEVERR_NONFINITE (NaN then ranks last).
 */
moe_status moe_route(const moe_shape* shape, const void* x, const void* w_router, float* logits,
                     int32_t* topk_idx, float* topk_gate, void* ws, size_t ws_bytes, void* stream);

/*
 * Dispatch schedule (MoK paper §3.1, "Scheduling", and its Algorithm 1).
 * routes A [R, N*k] holds global expert ids (topk_idx is A when R == 1);
 * route j of source rank r goes to local expert l = A[r][j] - c*L when that
 * lies in [0, L).  The received routes are laid out expert by expert: local
 * expert l owns positions offsets[l] .. offsets[l+1]-1.  Inside that region
 * the routes are ordered by their ordinal o (the number of earlier routes of
 * the same rank to the same expert) and then by source rank, so the ranks
 * take turns.  Each route's position is computed on its own in closed form,
 * from the per-(rank, expert) counts and o, with no sort.
 * Outputs: expert_counts [L] routes per local expert; expert_offsets [L+1]
 * (exclusive prefix sum, [L] = P); sched_src [max_rows]: sched_src[p] =
 * r*N*k + j for the route at position p (the table row is the buffer
 * position; entries >= P untouched); route_dst [R*N*k]: the inverse, the
 * position of each route, or -1 for a route to a non-local expert.  Integer
 * only; deterministic (no order-dependent atomics).  Bit-exact with the
 * ordering above.
 */
moe_status moe_schedule(const moe_shape* shape, const int32_t* routes, int32_t* expert_counts,
                        int32_t* expert_offsets, int32_t* sched_src, int32_t* route_dst, void* ws,
                        size_t ws_bytes, void* stream);

/*
 * moe_schedule for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  It
 * computes exactly what moe_schedule computes, with the same outputs, but
 * takes no workspace.  Its scratch (per-route ordinals, per-chunk histograms
 * and the per-(rank, expert) counts: 4*(R*N*k + R*ceil(N*k/1024)*L + R*L)
 * bytes, each piece rounded up to 256) lives in a fixed device array of the
 * library, MOE_SCHEDULE_STATIC_SCRATCH_BYTES bytes on each GPU, which the
 * GPU holds until the process ends; shapes that need more return
 * MOE_ERR_UNSUPPORTED before any device work.
 *   dev_error  device int32, caller-owned: the kernels OR MOE_DEVERR_* bits
 *              into it (clear it first for a fresh reading); never NULL
 * The call runs on the current device (the stream's); its first call on a
 * device looks up that device's copy of the array (a host query, no
 * allocation, no synchronisation).  Every call on one GPU shares that GPU's
 * array and leaves its contents behind: calls that overlap in time on one GPU
 * (streams not ordered against each other) race and must not be issued;
 * calls ordered on one stream are safe.  The same rule holds for graph
 * replays.
 */
#define MOE_SCHEDULE_STATIC_SCRATCH_BYTES (16u << 20)
moe_status moe_schedule_static(const moe_shape* shape, const int32_t* routes, int32_t* expert_counts,
                               int32_t* expert_offsets, int32_t* sched_src, int32_t* route_dst, int32_t* dev_error,
                               void* stream);

/*
 * The layer forward from a schedule (MoK paper §2.1 MoE equation; §3.3 ring
 * buffer; §3.4 "Shared Expert", "Determinism").
 *
 *   x_src      [R*N, D] bf16: source token rows; route r*N*k + j reads row
 *              r*N + j/k (x_src == x_local when R == 1)
 *   x_local    [T, D] bf16: this rank's tokens, input of the shared expert
 *   topk_gate  [T, k] fp32 gates of this rank's routes (from moe_route)
 *   expert_offsets, sched_src, route_dst: from moe_schedule
 *   out        [T, D] bf16 out: RNE of out32
 *   out32      [T, D] fp32 out, or NULL: the pre-cast result
 *
 * Per minibatch m (rows m*b .. m*b+b-1 of the schedule, in ascending order):
 * rows are gathered into ring slots (p mod C) with no other local copy; the
 * up/gate GEMM + SwiGLU writes h (bf16); the down GEMM writes each routed
 * output row (bf16) to the route it came from (R == 1: slot sched_src[p],
 * reusing the table for the combine as in §3.1) or to outbox row p (R > 1).
 * The combine then forms, for each local token t, in this fixed order and fp32:
 *   acc = 0; for s in 0..k-1: acc = fma(g[t,s], y[t,s], acc); out32[t] = acc + shared[t]
 * where y[t,s] is the row of route t*k+s, or 0 for a route to a remote expert
 * (R > 1: its row comes back from another rank, outside this library).
 * The first call in a process asks the runtime for the current device's
 * compute-unit count and the down kernels' occupancy (host queries only: no
 * allocation, no synchronisation) and keeps them; the call can be captured in
 * a HIP graph.
 */
moe_status moe_forward(const moe_shape* shape, const moe_weights* weights, const void* x_src,
                       const void* x_local, const float* topk_gate, const int32_t* expert_offsets,
                       const int32_t* sched_src, const int32_t* route_dst, void* out, float* out32,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * ---- Backward pass (one GPU: num_src_ranks == 1; bf16 routed and shared) ----
 *
 * The gradients of the layer for an output gradient dout (MoK paper §2.1 MoE
 * equation; §3.1: the dispatch table read in reverse; §3.3 "Ring-Aware
 * Forward Replay": the up/gate projections are recomputed, not kept; §3.4
 * "Router Weight Gradient Computation": the gate gradients <dout, y> from the
 * routed rows the forward stored).  With g the renormalised gates:
 *   dg_s = <dout, y_s>,  dy_s = g_s dout,  dl_s = g_s (dg_s - sum g dg)
 *   per expert: a_g = W_gate x, a_u = W_up x (replayed, stored bf16),
 *     dh = W_down^T dy, da_g = dh a_u SiLU'(a_g), da_u = dh SiLU(a_g) (bf16),
 *     dx += W_gate^T da_g + W_up^T da_u, dW_down += dy h^T,
 *     dW_gate += da_g x^T, dW_up += da_u x^T   (h = SiLU(a_g) a_u, bf16)
 *   the shared expert the same with dy = dout; the router: dx += W_r^T dl,
 *   dW_r = dl x^T (dl stored bf16 for these two products).
 * Every sum runs in a fixed order: results are bitwise repeatable.
 */

/* The weights rearranged for the backward (caller-allocated device memory,
 * filled once per weight set by moe_backward_prepare; bf16):
 *   w_gu: W_gate and W_up of each expert stacked ([2I, D], the replay's
 *     operand); w_gu_t: [W_gate^T | W_up^T] ([D, 2I]); w_down_t: W_down^T
 *     ([I, D]); each expert's matrix K-tiled as under moe_shape.weights_tiled
 *     ([D/64, 2I, 64], [2I/64, D, 64], [D/64, I, 64]; sizes unchanged);
 *   ws_gu [2I_s, D], ws_gu_t [D, 2I_s], ws_down_t [I_s, D]: the shared expert;
 *   w_router_t [D, Ep]: W_r^T with Ep = E_total rounded up to 64 (zero past
 *     E_total). */
typedef struct {
  void *w_gu, *w_gu_t, *w_down_t;
  void *ws_gu, *ws_gu_t, *ws_down_t;
  void* w_router_t;
} moe_bwd_weights;

/* Gradient outputs (caller-allocated device memory): dx [T, D] fp32;
 * dw_gate, dw_up [L, I, D], dw_down [L, D, I] bf16; dws_gate, dws_up
 * [I_s, D], dws_down [D, I_s] bf16; dw_router [E_total, D] fp32. */
typedef struct {
  float* dx;
  void *dw_gate, *dw_up, *dw_down;
  void *dws_gate, *dws_up, *dws_down;
  float* dw_router;
} moe_grads;

/* Fill `bw` from the forward's weights and the router weights (transposes and
 * copies on `stream`, run once per weight set).  MOE_ERR_UNSUPPORTED unless
 * num_src_ranks == 1, both precisions are MOE_BF16 and the routed weights are
 * row-major (weights_tiled == 0); the same holds for moe_backward and
 * moe_backward_workspace_bytes. */
moe_status moe_backward_prepare(const moe_shape* shape, const moe_weights* weights, const void* w_router,
                                const moe_bwd_weights* bw, void* stream);

/* Bytes of device workspace moe_backward needs (a separate allocation from
 * the forward's; 10.0 GB at the DeepSeek-V3 shape, mostly the routed rows'
 * intermediates and their transposed copies). */
moe_status moe_backward_workspace_bytes(const moe_shape* shape, size_t* bytes);

/*
 * The backward pass, for the tokens of one moe_route + moe_schedule +
 * moe_forward (R == 1).
 *   x          [T, D] bf16, the forward's input
 *   topk_idx, topk_gate, expert_offsets, sched_src, route_dst: as moe_route
 *              and moe_schedule produced them for that forward
 *   y_routes   [T*k, D] bf16: the forward's routed rows (moe_routed_rows of
 *              its workspace)
 *   dout       [T, D] bf16: the output gradient
 *   grads      the outputs (every one written)
 *   dev_error  device int32, caller-owned: MOE_DEVERR_* bits are OR-ed in
 * Shapes are validated before any launch, as for the forward; every GEMM
 * operand of the backward must stay below 2^31 bytes (MOE_ERR_UNSUPPORTED).
 * x, y_routes and dout must be 16-byte aligned (MOE_ERR_INVALID_ARG).
 */
moe_status moe_backward(const moe_shape* shape, const moe_bwd_weights* bw, const void* x, const int32_t* topk_idx,
                        const float* topk_gate, const int32_t* expert_offsets, const int32_t* sched_src,
                        const int32_t* route_dst, const void* y_routes, const void* dout, const moe_grads* grads,
                        int32_t* dev_error, void* ws, size_t ws_bytes, void* stream);

/*
 * Where moe_forward leaves the routed output rows inside the workspace (bf16,
 * row stride D): with R == 1, [T*k, D] indexed by route t*k + s; with R > 1,
 * the outbox [max_rows, D] indexed by schedule position p (rows >= P are not
 * written): the rows this rank returns to their source ranks, where the
 * table read as {dst_rank, dst_index} places them (MoK paper §3.1).  *rows
 * receives the device address, *n_rows the row count.  Host-only arithmetic
 * on ws: no device access, no synchronisation.  The rows are valid after
 * moe_forward and until the next call that uses the same workspace.
 */
moe_status moe_routed_rows(const moe_shape* shape, const void* ws, size_t ws_bytes, const void** rows,
                           int64_t* n_rows);

/*
 * K-tiling of bf16 matrices (the routed weights' moe_shape.weights_tiled
 * layout; the weights are prepared once, ahead of the layer, as in MoK paper
 * §3.4, "MXFP8 Support").  src [groups, rows, K] row-major -> dst [groups,
 * K/64, rows, 64]: element (g, r, k) lands at ((g*(K/64) + k/64)*rows + r)*64
 * + k%64.  K must be a positive multiple of 64, both pointers 16-byte aligned
 * and the buffers distinct (MOE_ERR_INVALID_ARG otherwise).  Byte moves only
 * (bit-exact).  Device memory, caller-owned; one launch on `stream`.
 */
moe_status moe_tile_bf16(const void* src, int64_t groups, int64_t rows, int64_t K, void* dst, void* stream);

/*
 * MX quantisation along rows (MoK paper §3.4, "MXFP8 Support": weights are
 * pre-quantised by a dedicated kernel).  src [rows, K] bf16, K a multiple of
 * 32 -> q [rows, K] E4M3FN and scale [rows, K/32] E8M0: per block of 32,
 * X = floor(log2(amax)) - 8 clamped to [-127, 127] (all-zero block: X = -127),
 * scale byte X + 127, elements RNE(v / 2^X) saturated to +-448.
 */
moe_status moe_quantize_mxfp8(const void* src, int64_t rows, int64_t K, uint8_t* q, uint8_t* scale,
                              void* stream);

/*
 * MX scales into the layout moe_forward reads (the same scales, moved; MoK
 * paper §3.4, "MXFP8 Support": the weights are prepared once, ahead of the
 * layer).  scale [groups, rows, K/32] row-major (moe_quantize_mxfp8's layout)
 * -> packed [groups, K/128, rows, 4]: the byte of row r, 32-wide K block j of
 * group g lands at ((g*(K/128) + j/4)*rows + r)*4 + j%4, so that the scale
 * words of consecutive rows for one 128-wide K stage are adjacent.  K must be
 * a multiple of 128; both pointers 4-byte aligned and not the same buffer.
 * Byte moves only (bit-exact).
 */
moe_status moe_mxfp8_pack_scales(const uint8_t* scale, int64_t groups, int64_t rows, int64_t K, uint8_t* packed,
                                 void* stream);

/* Read the sticky device error word (MOE_DEVERR_* bits).  SYNCHRONISES the
 * stream: diagnostics only, never on the hot path. */
moe_status moe_get_device_error(const moe_shape* shape, const void* ws, size_t ws_bytes,
                                void* stream, int32_t* host_code);

/*
 * Benchmark instrumentation, not part of the layer.  While a probe is active,
 * every launch of kernel `kernel_id` (one of moe_kernel_id) made by the calls
 * above is bracketed by a pair of HIP events recorded on the launch stream,
 * for up to `max_launches` launches.  moe_probe_end() SYNCHRONISES the device,
 * returns the summed event time in ms and the number of timed launches, and
 * releases the events.  One probe per process; not thread-safe.
 */
typedef enum {
  MOE_K_ROUTER_GEMM = 0, /* moe_route: logits = x W_r^T */
  MOE_K_TOPK = 1,        /* moe_route: top-k + gates */
  MOE_K_SCHEDULE = 2,    /* moe_schedule: all three schedule kernels, as one interval */
  MOE_K_TILES = 3,       /* moe_forward: per-minibatch tile lists */
  MOE_K_SHARED_UP = 4,   /* shared expert up/gate + SwiGLU */
  MOE_K_SHARED_DOWN = 5, /* shared expert down projection */
  MOE_K_GATHER = 6,      /* routed rows into the ring */
  MOE_K_UP_GATE = 7,     /* routed grouped up/gate + SwiGLU */
  MOE_K_DOWN = 8,        /* routed grouped down projection */
  MOE_K_COMBINE = 9,     /* gate-weighted combine */
  MOE_K_PIPELINE = 10,   /* pipeline == 1: the persistent routed kernel (gathers
                            of minibatches C/b and later, up/gate, down) */
  MOE_K_BWD_REPLAY = 11, /* moe_backward: up/gate replay of the routed rows */
  MOE_K_BWD_DGRAD = 12,  /* moe_backward: the routed data-gradient GEMMs (dh, dx) */
  MOE_K_BWD_WGRAD = 13,  /* moe_backward: the routed weight-gradient GEMMs */
  MOE_K_COUNT = 14
} moe_kernel_id;

moe_status moe_probe_begin(int32_t kernel_id, int32_t max_launches);
moe_status moe_probe_end(double* total_ms, int32_t* launches);

/*
 * Measurement, not part of the layer: the operand stream of the routed
 * expert GEMMs' K loop with the arithmetic taken out, to locate the floor of
 * their load pipeline on the device.  `items` workgroups (8 waves each, cut
 * into 8 contiguous per-XCD runs as the GEMMs cut their work items) each walk
 * row_bytes / 128 stages; at each stage a workgroup moves 128 bytes of each
 * of a_rows activation-like rows and b_rows weight-like rows into LDS rings of
 * slots_a and slots_b stages with direct buffer->LDS loads, one barrier per
 * stage, refilling a slot right after the barrier that frees it (the GEMMs'
 * protocol).  Item i reads activation block i / a_share of `act` and weight
 * block i of `wts`:
 *   act  [ceil(items / a_share)][a_rows][row_bytes]  device, caller-owned
 *   wts  [items][b_rows][row_bytes]                  device, caller-owned
 * Nothing is written to device memory.  Supported (a_rows, b_rows, slots_a,
 * slots_b): (320, 256, 2, 2) and (320, 0, 2, 2), the bf16 up/gate stage;
 * (256, 256, 2, 3) and (256, 0, 2, 3), the MXFP8 up/gate stage, and (256, 256,
 * 2, 2), the same with two weight slots; (0, 256, n, n)
 * for n = 2 .. 5 and (0, 256, 2, 3).  Other combinations: MOE_ERR_UNSUPPORTED;
 * row_bytes not a positive multiple of 128, items or a_share < 1, or a NULL
 * buffer that a nonzero row count needs: MOE_ERR_INVALID_ARG.  One launch on
 * `stream`; no synchronisation.
 */
typedef struct {
  const void* act;
  const void* wts;
  int64_t row_bytes;
  int32_t items, a_share;
  int32_t a_rows, b_rows;
  int32_t slots_a, slots_b;
} moe_stream_probe_args;
moe_status moe_stream_probe(const moe_stream_probe_args* args, void* stream);

/* Static string for a status code. */
const char* moe_status_str(moe_status status);

/* MOE_ABI_VERSION of the built library. */
int32_t moe_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
