#!/usr/bin/env python3
"""MoE-layer forward benchmark on one MI355X.

One step = the whole hot path on one batch: moe_route (router GEMM from x,
top-k, gates) + moe_schedule (Algorithm 1) + moe_forward (shared expert,
gather into the ring, grouped up/gate + SwiGLU, grouped down, combine), on the
DeepSeek-V3 layer shape by default (T=8192 tokens, D=7168, I=2048, 256 routed
experts, top-8, one shared expert with I=2048; bf16; synthetic seeded inputs
and random weights already resident in HBM).

Prints ONE JSON line.  value = tokens/s; also TFLOP/s by the expert-FFN count
6*T*(k+1)*D*I (MoK paper §4.1) and its fraction of the bf16 dense MFMA peak.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import platform
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
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dsv3", choices=["tiny", "mid", "dsv3", "mx"])
    ap.add_argument("--precision", default=None, choices=["bf16", "mxfp8"],
                    help="routed-expert precision (default: mxfp8 for the mx workload, else bf16)")
    ap.add_argument("--minibatch", type=int, default=0, help="rows per minibatch b (0: all routed rows)")
    ap.add_argument("--ring", type=int, default=0, help="ring rows C (0: b)")
    ap.add_argument("--routing", default="x", choices=["x", "gaussian", "zipf"],
                    help="x: router projection from x; gaussian/zipf: given fp32 logits")
    ap.add_argument("--cpu-sample", type=int, default=-1,
                    help="tokens of the oracle's timed CPU sample (0: skip; default 48, 4 in MXFP8)")
    ap.add_argument("--no-breakdown", action="store_true", help="skip the per-kernel timing passes")
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


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (expert parallelism across GPUs is "
              "designed, not built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    from mixture_experts_layer_counts_amd import MoELayer, _lib, shape_for

    if not os.path.exists(_lib.LIB_PATH):
        from mixture_experts_layer_counts_amd import build
        build.build()
    lib = _lib.load()
    dev = torch.device("cuda", 0)
    w = synth.workload(args.workload, routing=args.routing)
    precision = args.precision or ("mxfp8" if args.workload == "mx" else "bf16")
    mx = precision == "mxfp8"
    P = w.T * w.k
    b = args.minibatch or P
    C = args.ring or b
    log(f"workload {w.name}: T={w.T} D={w.D} I={w.I} E={w.E} k={w.k} I_shared={w.I_shared}; b={b} C={C}; "
        f"routing={args.routing}; {precision}; drawing inputs on {torch.cuda.get_device_name(0)}")
    t0 = time.time()
    inp = synth.make_inputs(w, device="cuda")
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f}s")
    weights = inp
    if mx:  # routed weights quantised ahead of time (MoK paper §3.4), outside the timed region
        from mixture_experts_layer_counts_amd import quantize_mxfp8
        weights = {n: inp[n] for n in ("ws_gate", "ws_up", "ws_down")}
        for n in ("gate", "up", "down"):
            weights["q_" + n], weights["s_" + n] = quantize_mxfp8(inp["w_" + n])
        torch.cuda.synchronize()
    layer = MoELayer(shape_for(w.T, w.D, w.I, w.E, w.k, I_shared=w.I_shared, minibatch_rows=b, ring_rows=C,
                               precision=precision), device=dev)
    x, wr, logits_in = inp["x"], inp["w_router"], inp.get("logits")
    out = torch.empty((w.T, w.D), dtype=torch.bfloat16, device=dev)

    def step():
        if logits_in is not None:
            _, idx, gate = layer.route(None, None, logits_in)
        else:
            _, idx, gate = layer.route(x, wr)
        sched = layer.schedule(idx)
        layer.forward(weights, x, x, gate, sched, out32=False, out=out)
        return sched

    for _ in range(args.warmup):
        sched = step()
    torch.cuda.synchronize()
    if layer.device_error():
        raise RuntimeError(f"device error word {layer.device_error():#x}")
    offsets = sched["offsets"].cpu().numpy().astype(np.int64)
    log(f"warmup done ({args.warmup} steps); per-expert rows min/max = "
        f"{int(np.diff(offsets).min())}/{int(np.diff(offsets).max())}")

    # timed region, with the dominant kernel bracketed by HIP events on its stream
    dominant = "up_gate"
    n_launch_per_step = (P + b - 1) // b
    _lib.check("moe_probe_begin", lib.moe_probe_begin(_lib.KERNELS[dominant], args.steps * n_launch_per_step))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    tot, n = ctypes.c_double(), ctypes.c_int32()
    _lib.check("moe_probe_end", lib.moe_probe_end(ctypes.byref(tot), ctypes.byref(n)))
    ms = (t1 - t0) * 1e3 / args.steps
    dom_ms = tot.value / max(n.value, 1)
    log(f"timed {args.steps} steps: {ms:.3f} ms/step; {dominant}: {n.value} launches, {dom_ms:.3f} ms each")

    # per-kernel breakdown (separate untimed passes, one probe per kernel)
    kernels = {}
    if not args.no_breakdown:
        reps = max(3, min(args.steps, 10))
        for name, kid in _lib.KERNELS.items():
            if name == "router_gemm" and logits_in is not None:
                continue
            _lib.check("moe_probe_begin", lib.moe_probe_begin(kid, reps * max(n_launch_per_step, 1) + 4))
            for _ in range(reps):
                step()
            _lib.check("moe_probe_end", lib.moe_probe_end(ctypes.byref(tot), ctypes.byref(n)))
            if n.value:
                kernels[name] = {"ms_per_step": round(tot.value / reps, 4), "launches_per_step": n.value // reps}
        log("breakdown:", json.dumps(kernels))

    # roofline of the dominant kernel: algorithmic bytes and flops per launch.
    # Per launch: the gate and up rows of every expert the minibatch touches,
    # the minibatch's ring rows read once and its h rows written once (bf16,
    # or E4M3 bytes plus one scale byte per 32 in MXFP8).
    counts = np.diff(offsets)
    if mx:
        w_bytes_expert = 2 * w.I * (w.D + w.D // 32)
        a_row, h_row, peak_mma = w.D + w.D // 32, w.I + w.I // 32, PEAK_FP8
    else:
        w_bytes_expert = 2 * w.I * w.D * 2
        a_row, h_row, peak_mma = w.D * 2, w.I * 2, PEAK_BF16
    launches = []
    for m in range(n_launch_per_step):
        lo, hi = m * b, min((m + 1) * b, P)
        touched = int(np.count_nonzero((offsets[:-1] < hi) & (offsets[1:] > lo) & (counts > 0)))
        rows = hi - lo
        launches.append((touched * w_bytes_expert + rows * a_row + rows * h_row, 2.0 * rows * 2 * w.I * w.D))
    alg_bytes = float(np.mean([l[0] for l in launches]))
    alg_flops = float(np.mean([l[1] for l in launches]))
    t_dom = dom_ms * 1e-3
    bound = "hbm" if alg_bytes / PEAK_HBM >= alg_flops / peak_mma else "mfma"
    if bound == "hbm":
        achieved, peak, unit = alg_bytes / t_dom / 1e9, PEAK_HBM / 1e9, "GB/s"
    else:
        achieved, peak, unit = alg_flops / t_dom / 1e12, peak_mma / 1e12, "TFLOP/s"
    traffic = None
    tr_path = os.path.join(ROOT, "profiles", f"traffic_{dominant}_{w.name}.json")
    if os.path.exists(tr_path):
        tr = json.load(open(tr_path))
        src = "gemm_mx.hip" if mx else "gemm.hip"
        if tr.get("src_digest") == src_digest(src) and tr.get("minibatch_rows") == b and \
                tr.get("precision", "bf16") == precision:
            traffic = tr.get("hbm_bytes_per_launch")
    roofline = {"kernel": dominant, "bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": traffic,
                "alg_bytes_per_launch": alg_bytes, "alg_flops_per_launch": alg_flops,
                "ms_per_launch": round(dom_ms, 4),
                "mfma_frac": round(alg_flops / t_dom / peak_mma, 4),
                "hbm_frac": round(alg_bytes / t_dom / PEAK_HBM, 4)}

    flops = w.flops()
    result = {
        "metric": METRIC,
        "value": round(w.T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if not mx else "mxfp8 (e4m3 + e8m0/32) routed, bf16 shared",
        "data": "synthetic (seeded N(0,1) tokens, N(0,1/fan_in) bf16 weights drawn on the GPU)",
        "config": {"workload": f"{w.name}: T={w.T} D={w.D} I={w.I} E={w.E} top-{w.k} + 1 shared (I={w.I_shared})",
                   "minibatch_rows": b, "ring_rows": C,
                   "routing": "router projection from x" if logits_in is None else f"given {args.routing} logits"},
        "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
        "mfma_peak_frac": round(flops / (ms * 1e-3) / (PEAK_FP8 if mx else PEAK_BF16), 4),
        "roofline": roofline,
        "kernels": kernels,
    }

    if args.calibrate_copy > 0:
        n = args.calibrate_copy << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = n
        del src, dst

    n_cpu = args.cpu_sample if args.cpu_sample >= 0 else (4 if mx else 48)
    if n_cpu > 0:
        result["cpu_baseline"] = cpu_baseline(w, inp, n_cpu, precision)
    print(json.dumps(result), flush=True)


def cpu_baseline(w, inp, n_tok, precision="bf16"):
    """The oracle, as it stands, on the first n_tok tokens of the same workload.

    In MXFP8 the oracle's own quantisation of the touched experts' weights is
    done beforehand and not timed (the method quantises weights ahead of time).
    """
    import numpy as np
    import torch

    import synth
    from oracle import moe as ref

    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threadpool_limits(os.cpu_count())
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: numpy's default pool
        threads = os.cpu_count()
    tok = np.arange(n_tok)
    xb = synth.bits(inp["x"][:n_tok])
    wrb = synth.bits(inp["w_router"])
    logits_given = inp.get("logits")
    t0 = time.perf_counter()
    if logits_given is None:
        lg = ref.router_logits(xb, wrb).astype(np.float32)
    else:
        lg = synth.host_f32(logits_given[:n_tok])
    t_route = time.perf_counter() - t0
    idx = ref.topk(lg, w.k)
    experts = np.unique(idx)
    # host copies of the weights the sample touches (copy time not counted)
    host = {"ws_gate": synth.bits(inp["ws_gate"]), "ws_up": synth.bits(inp["ws_up"]),
            "ws_down": synth.bits(inp["ws_down"])}
    for n in ("w_gate", "w_up", "w_down"):
        sub = synth.bits(inp[n][torch.as_tensor(experts, device=inp[n].device)])
        arr = {int(e): sub[i] for i, e in enumerate(experts)}
        host[n] = _ExpertTable(arr)
    if precision == "mxfp8":
        from concurrent.futures import ThreadPoolExecutor

        from oracle import bf16 as obf16
        from oracle import mx as omx
        jobs = [(n, int(e)) for n in ("gate", "up", "down") for e in experts]
        with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
            res = dict(zip(jobs, ex.map(lambda j: omx.quantize(obf16.to_f64(host["w_" + j[0]][j[1]])), jobs)))
        for n in ("gate", "up", "down"):
            host["q_" + n] = _ExpertTable({int(e): res[(n, int(e))][0] for e in experts})
            host["s_" + n] = _ExpertTable({int(e): res[(n, int(e))][1] for e in experts})
    t0 = time.perf_counter()
    ref.forward(xb, host, lg, w.k, precision=precision, tokens=tok)
    t_fwd = time.perf_counter() - t0
    secs = t_route + t_fwd
    return {"value": round(n_tok / secs, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n_tok} tokens of the {w.name} workload ({len(experts)} distinct routed experts + "
                      f"the shared expert), numpy fp64 on {platform.processor() or platform.machine()}, "
                      f"os.cpu_count()={os.cpu_count()}; {secs:.1f}s"}


class _ExpertTable:
    """Expert-indexed view of the host copies of the experts a sample uses."""

    def __init__(self, d):
        self.d = d

    def __getitem__(self, e):
        return self.d[int(e)]


if __name__ == "__main__":
    main()
