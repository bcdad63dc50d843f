#!/usr/bin/env python3
"""MoE-layer forward benchmark on one MI355X.

One step = the whole hot path on one batch: moe_route (router GEMM from x,
top-k, gates) + moe_schedule (Algorithm 1) + moe_forward (shared expert,
gather into the ring, grouped up/gate + SwiGLU, grouped down, combine).

Workloads (synthetic seeded inputs and random weights, resident in HBM):
  dsv3  DeepSeek-V3 layer shape, all experts on one GPU: T=8192, D=7168,
        I=2048, 256 routed experts, top-8, one shared expert (I=2048), bf16
        (the default, and the headline line)
  mx    the same with 384 routed experts in MXFP8 (E4M3 + E8M0 per 32 along K)
  ep64  one rank's share at expert parallelism 64: 4 local experts receiving
        32,768 routed rows of 64 source ranks with Zipf(1.2)-skewed counts,
        the shared expert on the rank's 4,096 tokens
  mid, tiny  small shapes

Prints ONE JSON line.  value = local tokens/s; also TFLOP/s by the
expert-FFN count 6*(routed rows + tokens)*D*I (MoK paper §4.1; 6*T*(k+1)*D*I
when every expert is local) and its fraction of the dense MFMA peak of the
routed precision, a roofline of the dominant kernel (up/gate + SwiGLU) timed
with HIP events inside the timed region, a per-kernel breakdown with each
kernel's algorithmic bytes and FLOP, and the CPU oracle timed on a sample.
The bf16 workloads also time the persistent routed kernel at minibatches of
512, 2048 and 8192 rows (a ring of four) under "granularity_sweep".
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer fwd tokens/sec + TFLOP/s (% MFMA peak), DSV3 shape, 1 MI355X"
PEAK_BF16 = 2516.6e12   # MI355X dense bf16 MFMA, FLOP/s
PEAK_FP8 = 5033.2e12    # MI355X dense fp8 MFMA, FLOP/s
PEAK_HBM = 8.0e12       # MI355X HBM3E, bytes/s


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dsv3", choices=["tiny", "mid", "dsv3", "mx", "ep64"])
    ap.add_argument("--precision", default=None, choices=["bf16", "mxfp8"],
                    help="routed-expert precision (default: mxfp8 for the mx workload, else bf16)")
    ap.add_argument("--shared-precision", default="bf16", choices=["bf16", "mxfp8"],
                    help="shared-expert precision (bf16 as the pages keep it; mxfp8 is an option)")
    ap.add_argument("--minibatch", type=int, default=0, help="rows per minibatch b (0: all routed rows)")
    ap.add_argument("--ring", type=int, default=0, help="ring rows C (0: b)")
    ap.add_argument("--weights", default="tiled", choices=["tiled", "row-major"],
                    help="layout of the routed weights: K-tiled (prepared once with tile_bf16 / tile_mxfp8, "
                         "outside the timed region) or row-major; --backward always runs row-major")
    ap.add_argument("--pipeline", action="store_true",
                    help="run the routed minibatch loop as one persistent kernel (bf16 routed experts)")
    ap.add_argument("--mem-workgroups", type=int, default=16,
                    help="with --pipeline: workgroups that gather the minibatches past the ring (multiple of 8)")
    ap.add_argument("--routing", default="x", choices=["x", "gaussian", "zipf"],
                    help="x: router projection from x; gaussian/zipf: given fp32 logits")
    ap.add_argument("--cpu-fraction", type=float, default=-1.0,
                    help="fraction of the layer's expert work in the oracle's timed CPU sample (0: skip; default "
                         "the whole layer (or rank share), 1/4 in MXFP8)")
    ap.add_argument("--no-breakdown", action="store_true", help="skip the per-kernel timing passes")
    ap.add_argument("--backward", action="store_true",
                    help="also time moe_backward on the step's routes and a seeded output gradient (bf16, R = 1)")
    ap.add_argument("--sweep", default="", metavar="[p]B[:C[:M]],...",
                    help="after the main run, time the step at these minibatch sizes b (ring C, default b; a 'p' "
                         "prefix, or --pipeline, runs the persistent routed kernel with M memory workgroups, default "
                         "--mem-workgroups) and report them under 'granularity_sweep'; by default the bf16 "
                         "workloads sweep the persistent kernel at b = 512, 2048 and 8192 with C = 4b")
    ap.add_argument("--no-granularity", action="store_true", help="skip the default granularity sweep")
    ap.add_argument("--graph", action="store_true",
                    help="in the sweep, also time the step captured once in a HIP graph and replayed "
                         "(launch overhead removed)")
    ap.add_argument("--floor", action="store_true",
                    help="instead of the layer, measure the expert GEMMs' load floor: stream probes of the routed "
                         "up/gate K loop without arithmetic (moe_stream_probe), and hipBLASLt (torch.bmm) on the "
                         "uniform stand-in of the expert GEMMs; prints one JSON line")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="after the run, copy a MIB-MiB buffer 3 times with a plain device copy (a known-size "
                         "reference for hardware byte counters)")
    return ap.parse_args()


def src_digest(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "mixture_experts_layer_counts_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# sources an expert GEMM kernel is compiled from, and the tile-list builder
# that sets its work order: stored counter readings apply only while none of
# them has changed
GEMM_SOURCES = {False: ("gemm.hip", "gemm_common.h", "common.h", "kernels.h", "schedule.hip"),
                True: ("gemm_mx.hip", "gemm_common.h", "common.h", "kernels.h", "mx.h", "schedule.hip")}


def gemm_digest(mx):
    return src_digest(*GEMM_SOURCES[bool(mx)])


class Job:
    """One benchmark configuration: its layer, inputs and step function."""

    def __init__(self, **kw):
        self.__dict__.update(kw)


def time_weight_quantize(torch, inp, quantize_mxfp8, pack_mxfp8_scales):
    """One more pass of the ahead-of-time MX weight preparation (moe_quantize_mxfp8
    on every routed weight tensor, then moe_mxfp8_pack_scales on its scales),
    timed with its outputs freshly allocated before the clock starts.
    Algorithmic bytes: bf16 read (2 B per element), E4M3 written (1 B), scales
    written (1/32 B), then read and written once more by the packing."""
    srcs = [inp["w_" + n] for n in ("gate", "up", "down")]
    for s in srcs:  # warm the allocator with the outputs' sizes
        q, sc = quantize_mxfp8(s)
        del q, sc
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    keep = []
    for s in srcs:
        q, sc = quantize_mxfp8(s)
        keep.append((q, pack_mxfp8_scales(sc)))
    torch.cuda.synchronize()
    t = time.perf_counter() - t0
    n = sum(s.numel() for s in srcs)
    nbytes = n * (2 + 1 + 1 / 32) + 2 * n / 32
    del keep
    return {"ms": round(t * 1e3, 3), "elements": n, "alg_bytes": int(nbytes),
            "GB_per_s": round(nbytes / t / 1e9, 1), "hbm_frac": round(nbytes / t / PEAK_HBM, 4)}


def tile_weights(args, precision):
    """Whether the routed weights run K-tiled: never for the backward, which
    prepares its own copies from row-major weights."""
    return args.weights == "tiled" and not args.backward


def tile_routed(weights, precision):
    """The routed weights K-tiled: bf16 w_* by tile_bf16, E4M3 q_* by tile_mxfp8."""
    from mixture_experts_layer_counts_amd import tile_bf16, tile_mxfp8
    if precision == "bf16":
        return dict(weights, **{n: tile_bf16(weights[n]) for n in ("w_gate", "w_up", "w_down")})
    return dict(weights, **{n: tile_mxfp8(weights[n]) for n in ("q_gate", "q_up", "q_down")})


def setup_single(args, torch, synth, MoELayer, shape_for, quantize_mxfp8):
    """All experts on one GPU (R = 1)."""
    w = synth.workload(args.workload, routing=args.routing)
    precision = args.precision or ("mxfp8" if args.workload == "mx" else "bf16")
    P = w.T * w.k
    b = args.minibatch or P
    C = args.ring or b
    log(f"workload {w.name}: T={w.T} D={w.D} I={w.I} E={w.E} k={w.k} I_shared={w.I_shared}; b={b} C={C}; "
        f"routing={args.routing}; {precision}; drawing inputs on {torch.cuda.get_device_name(0)}")
    t0 = time.time()
    inp = synth.make_inputs(w, device="cuda")
    weights = inp
    wq = None
    if precision == "mxfp8":  # routed weights quantised ahead of time (MoK paper §3.4), outside the timed region
        from mixture_experts_layer_counts_amd import pack_mxfp8_scales
        weights = {n: inp[n] for n in ("ws_gate", "ws_up", "ws_down")}
        for n in ("gate", "up", "down"):
            q, sc = quantize_mxfp8(inp["w_" + n])
            weights["q_" + n], weights["s_" + n] = q, pack_mxfp8_scales(sc)
        wq = time_weight_quantize(torch, inp, quantize_mxfp8, pack_mxfp8_scales)
    tiled = tile_weights(args, precision)
    if tiled:  # routed weights K-tiled ahead of time, outside the timed region
        weights = tile_routed(weights, precision)
    if args.shared_precision == "mxfp8":  # the shared weights too, ahead of time
        from mixture_experts_layer_counts_amd import pack_mxfp8_scales
        weights = dict(weights)
        for n in ("gate", "up", "down"):
            q, sc = quantize_mxfp8(inp["ws_" + n])
            weights["qs_" + n], weights["ss_" + n] = q, pack_mxfp8_scales(sc.unsqueeze(0))[0]
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f}s")
    dev = torch.device("cuda", 0)
    x, wr, logits_in = inp["x"], inp["w_router"], inp.get("logits")
    out = torch.empty((w.T, w.D), dtype=torch.bfloat16, device=dev)

    def make(b, C, mem=None, pipeline=None):
        layer = MoELayer(shape_for(w.T, w.D, w.I, w.E, w.k, I_shared=w.I_shared, minibatch_rows=b, ring_rows=C,
                                   precision=precision, shared_precision=args.shared_precision,
                                   pipeline=args.pipeline if pipeline is None else pipeline,
                                   mem_workgroups=args.mem_workgroups if mem is None else mem,
                                   weights_tiled=tiled), device=dev)

        def step():
            if logits_in is not None:
                _, idx, gate = layer.route(None, None, logits_in)
            else:
                _, idx, gate = layer.route(x, wr)
            sched = layer.schedule(idx)
            layer.forward(weights, x, x, gate, sched, out32=False, out=out)
            return sched
        return layer, step

    layer, step = make(b, C)
    return Job(name=w.name, w=w, R=1, c=0, T=w.T, E_route=w.E, P=P, b=b, C=C, precision=precision, layer=layer,
               inp=inp, step=step, make=make, routed_from_x=logits_in is None, weight_quantize=wq,
               shared_precision=args.shared_precision, routing=args.routing,
               config={"workload": f"{w.name}: T={w.T} D={w.D} I={w.I} E={w.E} top-{w.k} + 1 shared "
                                   f"(I={w.I_shared})", "minibatch_rows": b, "ring_rows": C,
                       "shared_precision": args.shared_precision,
                       "routed_weights": "K-tiled" if tiled else "row-major",
                       "routing": "router projection from x" if logits_in is None else f"given {args.routing} logits"})


def setup_ep64(args, torch, synth, MoELayer, shape_for, quantize_mxfp8):
    """One rank's share at EP = 64 (DeepSeek-V3 expert shape)."""
    import numpy as np
    if args.shared_precision != "bf16":
        raise SystemExit("--shared-precision mxfp8 is for the single-GPU workloads")
    R, N, k, L, c, E_total = 64, 4096, 8, 4, 0, 256
    counts = synth.zipf_counts(32768, L, 1.2)
    P = int(sum(counts))
    precision = args.precision or "bf16"
    w = synth.Workload("ep64", T=R * N, D=7168, I=2048, E=L, k=k, I_shared=2048, seed=50)
    b = args.minibatch or P
    C = args.ring or b
    log(f"workload ep64: R={R} source ranks x N={N} tokens, top-{k} of {E_total}; rank {c} holds {L} experts "
        f"receiving {P} rows (Zipf 1.2 counts {counts}); D={w.D} I={w.I}; b={b} C={C}; {precision}")
    t0 = time.time()
    inp = synth.make_inputs(w, device="cuda")  # x: the pooled token rows of all 64 ranks
    A = torch.from_numpy(synth.ep_share_routes(R, N, k, E_total, c, L, counts, seed=50)).to("cuda")
    wr = synth.make_inputs(synth.Workload("ep64-router", T=1, D=w.D, I=64, E=E_total, k=k, I_shared=64, seed=51),
                           device="cuda", with_weights=False)["w_router"]
    weights = inp
    if precision == "mxfp8":
        from mixture_experts_layer_counts_amd import pack_mxfp8_scales
        weights = {n: inp[n] for n in ("ws_gate", "ws_up", "ws_down")}
        for n in ("gate", "up", "down"):
            q, sc = quantize_mxfp8(inp["w_" + n])
            weights["q_" + n], weights["s_" + n] = q, pack_mxfp8_scales(sc)
    tiled = tile_weights(args, precision)
    if tiled:  # routed weights K-tiled ahead of time, outside the timed region
        weights = tile_routed(weights, precision)
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f}s")
    dev = torch.device("cuda", 0)
    # routing of this rank's own tokens (router width E_total); the routes of
    # all 64 ranks, this one's included, come from the Zipf-share generator
    router = MoELayer(shape_for(N, w.D, w.I, E_total, k, I_shared=w.I_shared, minibatch_rows=1, ring_rows=1),
                      device=dev)
    x_pool = inp["x"]
    x_local = x_pool[c * N:(c + 1) * N]
    out = torch.empty((N, w.D), dtype=torch.bfloat16, device=dev)

    def make(b, C, mem=None, pipeline=None):
        layer = MoELayer(shape_for(N, w.D, w.I, E_total, k, I_shared=w.I_shared, minibatch_rows=b, ring_rows=C,
                                   precision=precision, R=R, rank=c, max_rows=P,
                                   pipeline=args.pipeline if pipeline is None else pipeline,
                                   mem_workgroups=args.mem_workgroups if mem is None else mem,
                                   weights_tiled=tiled), device=dev)

        def step():
            _, _, gate = router.route(x_local, wr)
            sched = layer.schedule(A)
            layer.forward(weights, x_pool, x_local, gate, sched, out32=False, out=out)
            return sched
        return layer, step

    layer, step = make(b, C)
    return Job(name="ep64", w=w, R=R, T=N, E_route=E_total, P=P, b=b, C=C, precision=precision, layer=layer,
               inp=inp, step=step, make=make, routed_from_x=True, A=A, c=c, L=L, wr=wr, router=router, routing="x",
               config={"workload": f"ep64: one rank of 64 (4 local experts D={w.D} I={w.I}, {P} routed rows, "
                                   f"Zipf(1.2) counts {counts}; shared expert on {N} tokens)",
                       "minibatch_rows": b, "ring_rows": C, "routed_weights": "K-tiled" if tiled else "row-major",
                       "routing": "router projection from x (local tokens); routes of all ranks synthetic"})


def kernel_model(job, offsets, sched_src):
    """Algorithmic HBM bytes and FLOP of each kernel per step: every operand
    read once and every result written once."""
    import numpy as np
    w, T, P, E = job.w, job.T, job.P, job.E_route
    D, I, Is, k = w.D, w.I, w.I_shared, w.k
    mx = job.precision == "mxfp8"
    wb = 1.0 + 1.0 / 32 if mx else 2.0  # bytes per routed weight / activation element
    smx = getattr(job, "shared_precision", "bf16") == "mxfp8"
    sb = 1.0 + 1.0 / 32 if smx else 2.0  # the same for the shared expert
    counts = np.diff(offsets)
    touched = int(np.count_nonzero(counts))
    unique_src = len(np.unique(sched_src[:P] // k)) if P else 0
    local_routes = int(np.count_nonzero(job.route_dst_local >= 0))
    m = {
        "router_gemm": (T * D * 2 + E * D * 2 + T * E * 4, 2.0 * T * E * D),
        "topk": (T * E * 4 + T * k * 8, 0.0),
        "schedule": (job.R * T * k * 8 + P * 4 + len(offsets) * 8, 0.0),
        "tiles": (len(offsets) * 4, 0.0),
        # MX shared expert: x read once in bf16, written and read again in MX
        "shared_up": (T * D * 2 + (2 * T * D * sb if smx else 0) + 2 * Is * D * sb + T * Is * sb, 4.0 * T * Is * D),
        "shared_down": (T * Is * sb + D * Is * sb + T * D * 4, 2.0 * T * D * Is),
        "gather": (unique_src * D * 2 + P * D * wb, 0.0),
        "up_gate": (touched * 2 * I * D * wb + P * D * wb + P * I * wb, 4.0 * P * I * D),
        "down": (touched * D * I * wb + P * I * wb + P * D * 2, 2.0 * P * D * I),
        "combine": (local_routes * D * 2 + T * D * 4 + T * D * 2 + T * k * 8, 0.0),
    }
    # the persistent routed kernel: up/gate and down, plus the gathers of the
    # minibatches past the ring (read and written once in the kernel)
    in_kernel = max(0, P - min(job.C // job.b, -(-P // job.b)) * job.b)
    m["pipeline"] = (m["up_gate"][0] + m["down"][0] + in_kernel * D * 2 * 2, m["up_gate"][1] + m["down"][1])
    return m


def time_launches(torch, fn, reps=5, warm=2):
    """Mean ms of fn() over reps launches on the current stream (HIP events), after warm untimed ones."""
    for _ in range(warm):
        fn()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        fn()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / reps


def run_floor(torch, _lib):
    """The load floor of the routed expert GEMMs, and a library reference point.

    Stream probes (moe_stream_probe): the routed up/gate's K-loop loads, with
    the GEMM's LDS rings and slot protocol and no arithmetic, at the bf16
    DeepSeek-V3 work (4,096 items of 320 activation and 256 weight rows,
    K = 7,168 bf16) and the MXFP8 layer's (6,144 items of 256 + 256 rows,
    K = 7,168 bytes); each stream alone and both together; then the weight
    stream alone at 1 to 4 stages in flight; then the down projections'
    stages (K = I = 2,048; 28 N blocks share a row tile), both streams and
    weight rows alone.  16 consecutive items share their
    activation rows, as the 16 N blocks of one row tile do.  Reference:
    hipBLASLt (torch.bmm) on the uniform stand-in of the expert GEMMs, 256
    experts of 256 rows each, the weights a contiguous right operand.  Also
    torch's own kernels on the access patterns of the gather and the combine
    (pure reads, pure writes, copy, k rows in and 1 out, 1 in and k out), for
    the rates such mixed streams reach on the device.
    """
    lib = _lib.load()
    stream = torch.cuda.current_stream().cuda_stream
    out = {"mode": "floor", "device": torch.cuda.get_device_name(0), "probes": [], "hipblaslt": []}

    def probe(name, items, row_bytes, a_rows, b_rows, slots_a, slots_b, share=16):
        blocks = (items + share - 1) // share
        act = torch.empty(max(blocks * a_rows * row_bytes, 1), dtype=torch.uint8, device="cuda")
        wts = torch.empty(max(items * b_rows * row_bytes, 1), dtype=torch.uint8, device="cuda")
        a = _lib.MoeStreamProbeArgs(act.data_ptr(), wts.data_ptr(), row_bytes, items, share, a_rows, b_rows,
                                    slots_a, slots_b)

        def launch():
            _lib.check("moe_stream_probe", lib.moe_stream_probe(ctypes.byref(a), ctypes.c_void_p(stream)))

        ms = time_launches(torch, launch)
        w_bytes, a_bytes = items * b_rows * row_bytes, blocks * a_rows * row_bytes
        lds_bytes = items * (a_rows + b_rows) * row_bytes
        rec = {"probe": name, "items": items, "row_bytes": row_bytes, "a_rows": a_rows, "b_rows": b_rows,
               "slots": [slots_a, slots_b], "ms": round(ms, 4),
               "weight_GB": round(w_bytes / 1e9, 3), "act_unique_GB": round(a_bytes / 1e9, 3),
               "lds_fill_GB": round(lds_bytes / 1e9, 3),
               "weight_TB_per_s": round(w_bytes / ms / 1e9, 3) if w_bytes else None,
               "lds_fill_TB_per_s": round(lds_bytes / ms / 1e9, 3)}
        log("floor", json.dumps(rec))
        out["probes"].append(rec)
        del act, wts
        torch.cuda.empty_cache()

    # bf16 up/gate at the DeepSeek-V3 shape: 256 experts x 16 N blocks, 320-row tiles
    for a_rows, b_rows, tag in ((320, 256, "bf16 up/gate: both streams"), (320, 0, "bf16 up/gate: activation rows"),
                                (0, 256, "bf16 up/gate: weight rows")):
        probe(tag, 4096, 7168 * 2, a_rows, b_rows, 2, 2)
    # MXFP8 up/gate: 384 experts x 16 N blocks, 256-row tiles, weight ring one slot deeper
    for a_rows, b_rows, tag in ((256, 256, "mxfp8 up/gate: both streams"), (256, 0, "mxfp8 up/gate: activation rows"),
                                (0, 256, "mxfp8 up/gate: weight rows")):
        probe(tag, 6144, 7168, a_rows, b_rows, 2, 3)
    probe("mxfp8 up/gate: both streams, two weight slots", 6144, 7168, 256, 256, 2, 2)
    for n in (2, 3, 4, 5):
        probe(f"weight rows, {n - 1} stage(s) of 32 KB in flight per workgroup", 6144, 7168, 0, 256, n, n)
    # down projections: h rows against W_down, K = I = 2048, 28 N blocks of 256 share a row tile
    probe("bf16 down: both streams", 256 * 28, 2048 * 2, 320, 256, 2, 2, share=28)
    probe("bf16 down: weight rows", 256 * 28, 2048 * 2, 0, 256, 2, 2, share=28)
    probe("mxfp8 down: both streams", 384 * 28, 2048, 256, 256, 2, 3, share=28)
    probe("mxfp8 down: weight rows", 384 * 28, 2048, 0, 256, 2, 3, share=28)
    probe("mxfp8 down: both streams, two weight slots", 384 * 28, 2048, 256, 256, 2, 2, share=28)

    # hipBLASLt on the uniform stand-in (fresh N(0,1) bf16 operands)
    for name, K, N in (("up/gate (gate and up as one 2I-wide operand)", 7168, 4096), ("down", 2048, 7168)):
        a = torch.randn(256, 256, K, device="cuda", dtype=torch.bfloat16)
        w = torch.randn(256, K, N, device="cuda", dtype=torch.bfloat16)
        c = torch.empty(256, 256, N, device="cuda", dtype=torch.bfloat16)
        ms = time_launches(torch, lambda: torch.bmm(a, w, out=c))
        flops = 2.0 * 256 * 256 * K * N
        rec = {"gemm": name, "experts": 256, "rows": 256, "K": K, "N": N, "ms": round(ms, 4),
               "TFLOP_per_s": round(flops / ms / 1e9, 1), "weight_TB_per_s": round(256 * K * N * 2 / ms / 1e9, 3)}
        log("floor", json.dumps(rec))
        out["hipblaslt"].append(rec)
        del a, w, c
        torch.cuda.empty_cache()
    # library kernels with the access patterns of the gather and the combine,
    # at the DeepSeek-V3 shape (T = 8192 tokens, k = 8, D = 7168, bf16)
    out["streams"] = []
    T, k, D = 8192, 8, 7168
    x = torch.randn(T * k, D, device="cuda", dtype=torch.bfloat16)
    y = torch.empty_like(x)
    xs = x[:T]
    z = torch.empty(T, D, device="cuda", dtype=torch.bfloat16)
    r32 = torch.empty((), device="cuda", dtype=torch.float32)
    row = T * D * 2
    for name, fn, nbytes in (
            ("pure reads (torch.sum over T*k rows)",
             lambda: torch.sum(x, dim=(0, 1), dtype=torch.float32, out=r32), k * row),
            ("pure writes (fill_ of T*k rows)", lambda: y.fill_(1.0), k * row),
            ("copy (T*k rows)", lambda: y.copy_(x), 2 * k * row),
            ("k rows in, 1 out (sum over k, the combine's pattern)",
             lambda: torch.sum(x.view(T, k, D), dim=1, out=z), (k + 1) * row),
            ("1 row in, k out (broadcast copy, the gather's pattern)",
             lambda: y.view(T, k, D).copy_(xs.unsqueeze(1).expand(T, k, D)), (k + 1) * row)):
        ms = time_launches(torch, fn)
        rec = {"pattern": name, "ms": round(ms, 4), "GB": round(nbytes / 1e9, 3),
               "TB_per_s": round(nbytes / ms / 1e9, 3)}
        log("floor", json.dumps(rec))
        out["streams"].append(rec)
    del x, y, z
    torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (expert parallelism across GPUs is "
              "designed, not built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.floor:
        from mixture_experts_layer_counts_amd import _lib
        run_floor(torch, _lib)
        return

    import synth
    from mixture_experts_layer_counts_amd import MoELayer, _lib, quantize_mxfp8, shape_for

    lib = _lib.load()  # fails loudly when the HIP library is not built
    setup = setup_ep64 if args.workload == "ep64" else setup_single
    job = setup(args, torch, synth, MoELayer, shape_for, quantize_mxfp8)
    mx = job.precision == "mxfp8"
    peak_mma = PEAK_FP8 if mx else PEAK_BF16

    for _ in range(args.warmup):
        sched = job.step()
    torch.cuda.synchronize()
    if job.layer.device_error():
        raise RuntimeError(f"device error word {job.layer.device_error():#x}")
    offsets = sched["offsets"].cpu().numpy().astype(np.int64)
    sched_src = sched["sched"].cpu().numpy().astype(np.int64)
    rd = sched["route_dst"].cpu().numpy()
    job.route_dst_local = rd[job.c * job.T * job.w.k:(job.c + 1) * job.T * job.w.k] if job.R > 1 else rd
    log(f"warmup done ({args.warmup} steps); per-expert rows min/max = "
        f"{int(np.diff(offsets).min())}/{int(np.diff(offsets).max())}")

    # timed region, with the dominant kernel bracketed by HIP events on its stream
    dominant = "pipeline" if args.pipeline else "up_gate"
    n_launch_per_step = 1 if args.pipeline else (job.P + job.b - 1) // job.b
    if args.pipeline:
        job.config["pipeline"] = {"persistent_routed_kernel": True, "mem_workgroups": args.mem_workgroups}
    _lib.check("moe_probe_begin", lib.moe_probe_begin(_lib.KERNELS[dominant], args.steps * n_launch_per_step))
    # one event pair per step on the stream the library launches on (torch's
    # current stream), for the per-step median the MoK paper's protocol reports
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        evs[i][0].record()
        job.step()
        evs[i][1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    med_ms = statistics.median(a.elapsed_time(b) for a, b in evs)
    tot, n = ctypes.c_double(), ctypes.c_int32()
    _lib.check("moe_probe_end", lib.moe_probe_end(ctypes.byref(tot), ctypes.byref(n)))
    ms = (t1 - t0) * 1e3 / args.steps
    dom_ms = tot.value / max(n.value, 1)
    log(f"timed {args.steps} steps: {ms:.3f} ms/step; {dominant}: {n.value} launches, {dom_ms:.3f} ms each")

    # per-kernel breakdown (separate untimed passes, one probe per kernel)
    model = kernel_model(job, offsets, sched_src)
    kernels = {}
    if not args.no_breakdown:
        reps = max(3, min(args.steps, 10))
        for name, kid in _lib.KERNELS.items():
            _lib.check("moe_probe_begin", lib.moe_probe_begin(kid, reps * max(n_launch_per_step, 1) + 4))
            for _ in range(reps):
                job.step()
            _lib.check("moe_probe_end", lib.moe_probe_end(ctypes.byref(tot), ctypes.byref(n)))
            if not n.value:
                continue
            t = tot.value / reps * 1e-3
            nbytes, flops = model[name]
            shared_mx = name.startswith("shared") and getattr(job, "shared_precision", "bf16") == "mxfp8"
            peak_k = peak_mma if name in ("up_gate", "down") else (PEAK_FP8 if shared_mx else PEAK_BF16)
            e = {"ms_per_step": round(t * 1e3, 4), "launches_per_step": n.value // reps,
                 "alg_bytes": int(nbytes), "GB_per_s": round(nbytes / t / 1e9, 1),
                 "hbm_frac": round(nbytes / t / PEAK_HBM, 4)}
            if flops:
                e.update({"alg_flop": flops, "TFLOP_per_s": round(flops / t / 1e12, 1),
                          "mfma_frac": round(flops / t / peak_k, 4)})
            e["bound"] = "mfma" if flops / peak_k > nbytes / PEAK_HBM else "hbm"
            kernels[name] = e
        log("breakdown:", json.dumps(kernels))

    # roofline of the dominant kernel per launch: the gate and up rows of every
    # expert the minibatch touches, its ring rows read once and its h rows
    # written once (bf16, or E4M3 bytes plus one scale byte per 32 in MXFP8)
    w = job.w
    counts = np.diff(offsets)
    wb = 1.0 + 1.0 / 32 if mx else 2.0
    launches = []
    for m in range((job.P + job.b - 1) // job.b):
        lo, hi = m * job.b, min((m + 1) * job.b, job.P)
        touched = int(np.count_nonzero((offsets[:-1] < hi) & (offsets[1:] > lo) & (counts > 0)))
        rows = hi - lo
        launches.append((touched * 2 * w.I * w.D * wb + rows * w.D * wb + rows * w.I * wb,
                         2.0 * rows * 2 * w.I * w.D))
    if args.pipeline:  # one launch holds every minibatch's up/gate and down, and the in-kernel gathers
        alg_bytes, alg_flops = model["pipeline"]
    else:
        alg_bytes = float(np.mean([l[0] for l in launches]))
        alg_flops = float(np.mean([l[1] for l in launches]))
    t_dom = dom_ms * 1e-3
    bound = "hbm" if alg_bytes / PEAK_HBM >= alg_flops / peak_mma else "mfma"
    if bound == "hbm":
        achieved, peak, unit = alg_bytes / t_dom / 1e9, PEAK_HBM / 1e9, "GB/s"
    else:
        achieved, peak, unit = alg_flops / t_dom / 1e12, peak_mma / 1e12, "TFLOP/s"
    # counters taken on the same workload, routing, minibatch, precision,
    # routed-weight layout and GEMM sources
    traffic = None
    suffix = "" if job.routing == "x" else "_" + job.routing
    tr_path = os.path.join(ROOT, "profiles", f"traffic_{dominant}_{job.name}{suffix}.json")
    if os.path.exists(tr_path):
        tr = json.load(open(tr_path))
        if tr.get("src_digest") == gemm_digest(mx) and tr.get("minibatch_rows") == job.b and \
                tr.get("precision", "bf16") == job.precision and tr.get("routing", "x") == job.routing and \
                tr.get("routed_weights", "row-major") == job.config.get("routed_weights", "row-major"):
            traffic = tr.get("hbm_bytes_per_launch")
    roofline = {"kernel": dominant, "bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": traffic,
                "alg_bytes_per_launch": alg_bytes, "alg_flops_per_launch": alg_flops,
                "ms_per_launch": round(dom_ms, 4),
                "mfma_frac": round(alg_flops / t_dom / peak_mma, 4),
                "hbm_frac": round(alg_bytes / t_dom / PEAK_HBM, 4)}

    flops = 6.0 * (job.P + job.T) * w.D * w.I
    result = {
        "metric": METRIC,
        "value": round(job.T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_median": round(med_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8 (e4m3 + e8m0/32) routed, bf16 shared" if mx else "bf16",
        "data": "synthetic (seeded N(0,1) tokens, N(0,1/fan_in) bf16 weights drawn on the GPU)",
        "config": job.config,
        "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
        "mfma_peak_frac": round(flops / (ms * 1e-3) / peak_mma, 4),
        "routed_rows_per_s": round(job.P / (ms * 1e-3), 1),
        "roofline": roofline,
        "kernels": kernels,
    }
    if "router_gemm" in kernels or "topk" in kernels:
        # the MoK paper times the layer from given router logits: the step
        # without the router projection and top-k
        route_ms = sum(kernels[n]["ms_per_step"] for n in ("router_gemm", "topk") if n in kernels)
        result["ms_per_step_excl_route"] = round(ms - route_ms, 4)

    if args.backward:
        result["backward"] = backward_leg(job, args, torch, offsets)

    if getattr(job, "weight_quantize", None):
        result["weight_quantize"] = job.weight_quantize  # ahead of time, not part of the step
    if not args.sweep and not args.no_granularity and job.precision == "bf16" and job.P > 8192:
        # the persistent routed kernel at small minibatches, a ring of four
        args.sweep = "p512:2048,p2048:8192,p8192:32768"
    if args.sweep:
        result["granularity_sweep"] = sweep(job, args, torch)

    if args.calibrate_copy > 0:
        nb = args.calibrate_copy << 20
        src_t = torch.empty(nb, dtype=torch.uint8, device="cuda").fill_(1)
        dst_t = torch.empty_like(src_t)
        for _ in range(3):
            dst_t.copy_(src_t)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = nb
        del src_t, dst_t

    frac = args.cpu_fraction if args.cpu_fraction >= 0 else (0.25 if mx else 1.0)
    if frac > 0:
        log(f"timing the CPU oracle on {frac:g} of the layer's work")
        result["cpu_baseline"] = (cpu_baseline_ep(job, max(1, int(round(job.T * frac)))) if job.name == "ep64"
                                  else cpu_baseline(job, frac))
    print(json.dumps(result), flush=True)


def backward_model(job, offsets):
    """Algorithmic HBM bytes and FLOP of the backward's three timed groups:
    every operand read once and every result written once.  The routed rows
    replay up/gate (4 P D I), take dh = dY W_down and dx = da [W_gate; W_up]
    (6 P D I) and the weight gradients dW = dY^T h, da^T x (6 P D I); the
    transposed copies that feed the weight-gradient GEMMs are counted as one
    read and one write of each operand."""
    import numpy as np
    w, P = job.w, job.P
    D, I = w.D, w.I
    touched = int(np.count_nonzero(np.diff(offsets)))
    wexp = touched * I * D * 2  # one bf16 expert matrix of I x D, over the touched experts
    return {
        "bwd_replay": (P * D * 2 + 2 * wexp + P * 2 * I * 2, 4.0 * P * D * I),
        # dh GEMM, SwiGLU backward, dx GEMM
        "bwd_dgrad": ((P * D * 2 + wexp + P * I * 4) + (P * 2 * I * 2 + P * I * 4 + P * I * 2 + P * 2 * I * 2) +
                      (P * 2 * I * 2 + 2 * wexp + P * D * 4), 6.0 * P * D * I),
        # transposes of dY, h, da, x (read + write), then the three GEMMs
        "bwd_wgrad": (2 * (P * D * 2 + P * I * 2 + P * 2 * I * 2 + P * D * 2) +
                      (P * D * 2 + P * I * 2 + P * 2 * I * 2 + P * D * 2 + 3 * wexp), 6.0 * P * D * I),
    }


def backward_leg(job, args, torch, offsets):
    """moe_backward after the forward: the routes, schedule and routed rows of
    the step just timed, a seeded N(0,1) bf16 output gradient.  Timed like the
    forward (warmup, then K calls between synchronisations, with a per-call
    event median), then once more per group with the library's probes.
    FLOP: executed 16 (P + T I_s / I) D I + 4 T E D (routed and shared:
    replay 4, data gradients 6, weight gradients 6; router 2 + 2), of which
    the replay's 4 is recomputation; the usual training count leaves it out."""
    from mixture_experts_layer_counts_amd import MoEBackward, _lib, prepare_backward
    if job.R != 1 or job.precision != "bf16" or getattr(job, "shared_precision", "bf16") != "bf16":
        raise SystemExit("--backward is for the bf16 single-GPU workloads")
    w, inp, layer = job.w, job.inp, job.layer
    lib = _lib.load()
    x, wr, logits_in = inp["x"], inp["w_router"], inp.get("logits")
    if logits_in is not None:
        _, idx, gate = layer.route(None, None, logits_in)
    else:
        _, idx, gate = layer.route(x, wr)
    sched = layer.schedule(idx)
    out = torch.empty((w.T, w.D), dtype=torch.bfloat16, device=x.device)
    layer.forward(inp, x, x, gate, sched, out32=False, out=out)
    y = layer.routed_rows()
    t0 = time.perf_counter()
    bw = prepare_backward(layer.shape, inp, wr)
    torch.cuda.synchronize()
    prep_ms = (time.perf_counter() - t0) * 1e3
    b = MoEBackward(layer.shape, device=x.device)
    dout = torch.randn((w.T, w.D), generator=torch.Generator(device=x.device).manual_seed(w.seed + 5),
                       device=x.device).to(torch.bfloat16)
    grads = None
    for _ in range(max(1, args.warmup)):
        grads = b(bw, x, idx, gate, sched, y, dout, grads)
    torch.cuda.synchronize()
    if b.device_error():
        raise RuntimeError(f"backward device error word {b.device_error():#x}")
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        evs[i][0].record()
        b(bw, x, idx, gate, sched, y, dout, grads)
        evs[i][1].record()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    med = statistics.median(a.elapsed_time(c) for a, c in evs)
    model = backward_model(job, offsets)
    groups = {}
    tot, n = ctypes.c_double(), ctypes.c_int32()
    reps = max(3, min(args.steps, 10))
    for name, (nbytes, flops) in model.items():
        _lib.check("moe_probe_begin", lib.moe_probe_begin(_lib.KERNELS[name], reps + 2))
        for _ in range(reps):
            b(bw, x, idx, gate, sched, y, dout, grads)
        _lib.check("moe_probe_end", lib.moe_probe_end(ctypes.byref(tot), ctypes.byref(n)))
        t = tot.value / max(n.value, 1) * 1e-3
        groups[name] = {"ms": round(t * 1e3, 4), "alg_bytes": int(nbytes), "GB_per_s": round(nbytes / t / 1e9, 1),
                        "hbm_frac": round(nbytes / t / PEAK_HBM, 4), "alg_flop": flops,
                        "TFLOP_per_s": round(flops / t / 1e12, 1), "mfma_frac": round(flops / t / PEAK_BF16, 4)}
    D, I, Is, T, P, E = w.D, w.I, w.I_shared, w.T, job.P, w.E
    executed = 16.0 * (P * I + T * Is) * D + 4.0 * T * E * D
    useful = 12.0 * (P * I + T * Is) * D + 4.0 * T * E * D
    r = {"ms_per_call": round(ms, 4), "ms_per_call_median": round(med, 4), "calls": args.steps,
         "tokens_per_s": round(T / (ms * 1e-3), 1),
         "flop_executed": executed, "flop_without_replay": useful,
         "tflops_executed": round(executed / (ms * 1e-3) / 1e12, 2),
         "mfma_peak_frac_executed": round(executed / (ms * 1e-3) / PEAK_BF16, 4),
         "prepare_ms": round(prep_ms, 2), "workspace_bytes": b.ws_bytes, "groups": groups}
    log("backward:", json.dumps(r))
    del b, bw, grads
    torch.cuda.empty_cache()
    return r


def sweep(job, args, torch):
    """Step time at other minibatch sizes b and ring sizes C (MoK paper §3.2:
    finer minibatches overlap better but pay per-minibatch overheads)."""
    out = []
    job.layer = None  # release the main workspace first
    for item in args.sweep.split(","):
        persistent = args.pipeline or item.startswith("p")
        parts = item.lstrip("p").split(":")
        b = min(int(parts[0]), job.P)
        C = min(int(parts[1]), -(-job.P // b) * b) if len(parts) > 1 and parts[1] else b
        mem = int(parts[2]) if len(parts) > 2 else args.mem_workgroups
        layer, step = job.make(b, C, mem, pipeline=persistent)
        for _ in range(2):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        n = max(3, args.steps // 2)
        for _ in range(n):
            step()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / n
        if layer.device_error():
            raise RuntimeError(f"device error word {layer.device_error():#x} at b={b} C={C}")
        e = {"minibatch_rows": b, "ring_rows": C, "minibatches": (job.P + b - 1) // b,
             "ms_per_step": round(ms, 4), "tokens_per_s": round(job.T / (ms * 1e-3), 1),
             "persistent": persistent}
        if persistent:
            e["mem_workgroups"] = mem
        if args.graph:
            # the same step captured once (the library allocates nothing and
            # never synchronises, so it can be captured) and replayed
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                step()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step()
            g.replay()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(n):
                g.replay()
            torch.cuda.synchronize()
            e["graph_ms_per_step"] = round((time.perf_counter() - t0) * 1e3 / n, 4)
            if layer.device_error():
                raise RuntimeError(f"device error word {layer.device_error():#x} at b={b} C={C} (graph)")
            del g
        out.append(e)
        log(f"sweep b={b} C={C}" + (f" persistent mem={mem}" if persistent else "") + f": {ms:.3f} ms/step" +
            (f", graph {e['graph_ms_per_step']:.3f}" if args.graph else ""))
        del layer, step
        torch.cuda.empty_cache()
    return out


def _threads():
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threadpool_limits(os.cpu_count())
        return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: numpy's default pool
        return os.cpu_count()


def _oracle_mx(host, experts):
    """The oracle's own MX quantisation of the given experts (not timed: the
    method quantises weights ahead of time)."""
    from concurrent.futures import ThreadPoolExecutor

    from oracle import bf16 as obf16
    from oracle import mx as omx
    jobs = [(n, int(e)) for n in ("gate", "up", "down") for e in experts]
    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        res = dict(zip(jobs, ex.map(lambda j: omx.quantize(obf16.to_f64(host["w_" + j[0]][j[1]])), jobs)))
    for n in ("gate", "up", "down"):
        host["q_" + n] = _ExpertTable({int(e): res[(n, int(e))][0] for e in experts})
        host["s_" + n] = _ExpertTable({int(e): res[(n, int(e))][1] for e in experts})


def cpu_baseline(job, frac):
    """The oracle, as it stands, on a fixed fraction of the layer's work.

    The sample is the first ``frac`` of the routed experts with every route
    they receive, so each sampled expert sees its whole batch of rows and the
    widening of its weights is spread over those rows as in the full layer;
    plus the router projection, top-k and gates of all T tokens, and the
    shared expert and the combine on the first frac*T tokens.  That is a
    fraction frac of the layer's expert work (a little more of its routing),
    reported as frac*T tokens."""
    import numpy as np

    import synth
    from oracle import moe as ref

    w, inp = job.w, job.inp
    threads = _threads()
    n_exp = max(1, int(round(w.E * frac)))
    n_tok = max(1, int(round(w.T * frac)))
    experts = np.arange(n_exp)
    xb = synth.bits(inp["x"])
    wrb = synth.bits(inp["w_router"])
    logits_given = inp.get("logits")
    # host copies of the sampled experts' weights (copy time not counted)
    host = {"ws_gate": synth.bits(inp["ws_gate"]), "ws_up": synth.bits(inp["ws_up"]),
            "ws_down": synth.bits(inp["ws_down"])}
    for n in ("w_gate", "w_up", "w_down"):
        host[n] = _ExpertTable({int(e): synth.bits(inp[n][int(e)]) for e in experts})
    if job.precision == "mxfp8":
        _oracle_mx(host, experts)
    sp = getattr(job, "shared_precision", "bf16")
    if sp == "mxfp8":  # the oracle's own MX quantisation of the shared weights (ahead of time, not timed)
        host = ref.quantize_shared_mx(host)
    t0 = time.perf_counter()
    lg = ref.router_logits(xb, wrb).astype(np.float32) if logits_given is None else synth.host_f32(logits_given)
    idx = ref.topk(lg, w.k)
    g = ref.gates(lg, idx)
    tok_routed = np.nonzero((idx < n_exp).any(axis=1))[0]
    Y = ref.routed_outputs(xb, host, idx, job.precision, tokens=tok_routed, experts=experts)
    tok = np.arange(n_tok)
    sh = ref.shared_output(xb, host, tokens=tok, precision=sp)
    pos = np.searchsorted(tok_routed, tok)
    hit = (pos < len(tok_routed)) & (tok_routed[np.minimum(pos, len(tok_routed) - 1)] == tok)
    Yt = np.zeros((n_tok,) + Y.shape[1:])
    Yt[hit] = Y[pos[hit]]
    ref.combine(sh, g[tok], Yt)
    secs = time.perf_counter() - t0
    rows = int(np.count_nonzero(idx < n_exp))
    return {"value": round(n_tok / secs, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{frac:g} of the {w.name} layer's expert work: experts 0..{n_exp - 1} of {w.E} with all "
                      f"{rows} routes they receive (each expert its whole batch), the router projection, top-k and "
                      f"gates of all {w.T} tokens, the shared expert and combine on {n_tok} tokens; counted as "
                      f"{n_tok} tokens; numpy fp64 on {platform.processor() or platform.machine()}, "
                      f"os.cpu_count()={os.cpu_count()}; {secs:.1f}s"}


def cpu_baseline_ep(job, n_tok):
    """The oracle's EP share on n_tok local tokens' worth of work: their router
    projection, their output, and P/T routed rows per token (the first rows of
    the schedule), so that tokens/s compares with the GPU's local tokens/s."""
    import numpy as np

    import synth
    from oracle import moe as ref

    w, inp = job.w, job.inp
    threads = _threads()
    k, T, c = w.k, job.T, job.c
    n_rows = int(round(n_tok * job.P / T))
    A = job.A.cpu().numpy()
    host = {n: synth.bits(inp[n]) for n in ("w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")}
    x_pool = synth.bits(inp["x"])
    g = np.full((T, k), 1.0 / k)
    t0 = time.perf_counter()
    ref.router_logits(x_pool[c * T:c * T + n_tok], synth.bits(job.wr))
    ref.ep_share_forward(x_pool, host, A, c, job.L, k, g, positions=np.arange(n_rows), tokens=np.arange(n_tok))
    secs = time.perf_counter() - t0
    return {"value": round(n_tok / secs, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n_tok} local tokens of the ep64 share (their router projection and output, plus the "
                      f"first {n_rows} of the {job.P} routed rows), numpy fp64 on "
                      f"{platform.processor() or platform.machine()}, os.cpu_count()={os.cpu_count()}; {secs:.1f}s"}


class _ExpertTable:
    """Expert-indexed view of the host copies of the experts a sample uses."""

    def __init__(self, d):
        self.d = d

    def __getitem__(self, e):
        return self.d[int(e)]


if __name__ == "__main__":
    main()
