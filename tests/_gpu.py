"""Helpers shared by the GPU parity tests (not collected by pytest)."""

from __future__ import annotations

import os
import sys

import numpy as np
import pytest
import torch

import synth
from oracle import moe as ref


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from mixture_experts_layer_counts_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):  # the HIP path has no fallback: a missing build is a failure
        pytest.fail(f"{_lib.LIB_PATH} not built")
    return torch.device("cuda", 0)


def say(*msg):
    print("[gpu-case]", *msg, file=sys.stderr, flush=True)


def host_weights(inp):
    return {n: synth.bits(t) for n, t in inp.items() if t.dtype == torch.bfloat16}


def to_dev(inp, dev):
    return {n: t.to(dev) for n, t in inp.items()}


def layer(w: synth.Workload, dev, b=None, C=None, R=1, precision="bf16", shared_precision="bf16"):
    from mixture_experts_layer_counts_amd import MoELayer, shape_for
    return MoELayer(shape_for(w.T, w.D, w.I, w.E, w.k, I_shared=w.I_shared, minibatch_rows=b, ring_rows=C,
                              precision=precision, shared_precision=shared_precision), device=dev)


def mx_shared_weights_dev(inp_dev):
    """The shared expert's weights MX-quantised on the GPU (moe_quantize_mxfp8)
    with their scales packed stage-major (moe_mxfp8_pack_scales, one group)."""
    from mixture_experts_layer_counts_amd import pack_mxfp8_scales, quantize_mxfp8
    out = {}
    for n in ("gate", "up", "down"):
        q, s = quantize_mxfp8(inp_dev["ws_" + n])
        out["qs_" + n], out["ss_" + n] = q, pack_mxfp8_scales(s.unsqueeze(0))[0]
    return out


def mx_weights_dev(inp_dev):
    """Routed weights MX-quantised on the GPU by moe_quantize_mxfp8, scales
    packed by moe_mxfp8_pack_scales (the product's own preprocessing); the
    shared expert stays bf16."""
    from mixture_experts_layer_counts_amd import pack_mxfp8_scales, quantize_mxfp8
    out = {n: inp_dev[n] for n in ("ws_gate", "ws_up", "ws_down")}
    for n in ("gate", "up", "down"):
        q, s = quantize_mxfp8(inp_dev["w_" + n])
        out["q_" + n], out["s_" + n] = q, pack_mxfp8_scales(s)
    return out


def oracle_mx_weights(inp, experts=None):
    """The oracle's own MX quantisation of the bf16 routed weights (of the
    given experts only, keyed by expert id, when ``experts`` is given), and
    the bf16 shared weights.  Experts are quantised in a thread pool: numpy
    releases the GIL, and each expert's arithmetic is the oracle's as is."""
    from concurrent.futures import ThreadPoolExecutor
    from oracle import bf16, mx
    host = {n: synth.bits(inp[n]) for n in ("ws_gate", "ws_up", "ws_down")}
    ids = list(range(inp["w_gate"].shape[0])) if experts is None else [int(e) for e in experts]
    jobs = [(n, e) for n in ("gate", "up", "down") for e in ids]
    rows = {(n, e): synth.bits(inp["w_" + n][e]) for n, e in jobs}
    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        res = dict(zip(jobs, ex.map(lambda j: mx.quantize(bf16.to_f64(rows[j])), jobs)))
    for n in ("gate", "up", "down"):
        if experts is None:
            host["q_" + n] = np.stack([res[(n, e)][0] for e in ids])
            host["s_" + n] = np.stack([res[(n, e)][1] for e in ids])
        else:
            host["q_" + n] = {e: res[(n, e)][0] for e in ids}
            host["s_" + n] = {e: res[(n, e)][1] for e in ids}
    return host


def rel_err(got, want):
    """max|got - want| / RMS(want)."""
    want = np.asarray(want, dtype=np.float64)
    return float(np.max(np.abs(np.asarray(got, dtype=np.float64) - want)) / np.sqrt(np.mean(want ** 2)))


def bf16_stats(got, want, tol):
    """For a gradient stored in bf16: (RMS of the error / RMS(want), share of
    the elements beyond tol * RMS(want) plus one bf16 step of their own value,
    max|err| / RMS(want))."""
    want = np.asarray(want, dtype=np.float64)
    err = np.abs(np.asarray(got, dtype=np.float64) - want)
    rms = np.sqrt(np.mean(want ** 2))
    out = err > 2.0 ** -7 * np.abs(want) + tol * rms
    return float(np.sqrt(np.mean(err ** 2)) / rms), float(np.mean(out)), float(err.max() / rms)


def bf16_grad_ok(got, want, name=""):
    """The bound for bf16-stored gradients (see test_gpu_backward): RMS(err)
    <= 2e-3 RMS, at most 1e-5 of the elements beyond 1e-2 RMS plus one bf16
    step, max|err| <= 1e-1 RMS."""
    rms_err, share, mx = bf16_stats(got, want, 1e-2)
    say("  ", name, "RMS(err)/RMS =", rms_err, "share beyond =", share, "max|err|/RMS =", mx)
    return rms_err <= 2e-3 and share <= 1e-5 and mx <= 1e-1


class DeviceExperts:
    """expert id -> the bf16 bits of that expert's matrix of a device weight
    tensor [E, ...], copied to the host when asked for."""

    def __init__(self, t):
        self.t = t

    def __getitem__(self, e):
        return synth.bits(self.t[int(e)])


def gate_tolerance(logits_sel: np.ndarray, k: int) -> np.ndarray:
    """Relative bound on a gate computed in fp32 from fp32 logits:
    u * (2 * max_s |l_s - l_0| + k + 8), u = 2^-24 (the subtraction, the
    exponential's few-ulp error, the k-term sum and the division)."""
    d = np.abs(logits_sel - logits_sel[:, :1]).max(axis=1, keepdims=True)
    return 2.0 ** -24 * (2.0 * d + k + 8)


def oracle_layer(w: synth.Workload, inp, logits_np, tokens=None):
    return ref.forward(synth.bits(inp["x"]), host_weights(inp), logits_np, w.k, tokens=tokens)


def cover_tokens(idx: np.ndarray, n: int, seed: int, sched=None, offsets=None, k=None) -> np.ndarray:
    """Token ids for a full-shape parity sample: a seeded draw of n tokens,
    one more token for every expert the draw leaves without a route, and,
    given the schedule (sched_src, offsets, k), the tokens whose routes sit
    at the first and the last position of every expert's region (the tile
    edges of that expert's rows)."""
    idx = np.asarray(idx)
    T = idx.shape[0]
    rng = np.random.default_rng(seed)
    tok = set(rng.choice(T, size=min(n, T), replace=False).tolist())
    seen = set(idx[sorted(tok)].ravel().tolist())
    for e in np.unique(idx):
        if int(e) not in seen:
            t = int(np.nonzero((idx == e).any(axis=1))[0][0])
            tok.add(t)
            seen.update(idx[t].tolist())
    if sched is not None:
        for e in range(len(offsets) - 1):
            if offsets[e + 1] > offsets[e]:
                tok.add(int(sched[offsets[e]]) // k)
                tok.add(int(sched[offsets[e + 1] - 1]) // k)
    return np.array(sorted(tok), dtype=np.int64)


def _expert_groups(experts, per_job):
    experts = np.asarray(sorted(set(int(e) for e in experts)), dtype=np.int64)
    return [experts[i:i + per_job] for i in range(0, len(experts), per_job)]


def oracle_routed_pooled(x_bits, fetch, cases, precision="bf16", per_job=2, workers=16):
    """The oracle's routed outputs for several (idx, tokens) cases over the
    same expert weights, evaluated expert group by expert group in a thread
    pool (numpy releases the GIL in the arithmetic).

    fetch(experts) returns the oracle's weights dict for those experts
    (keyed by expert id: "w_*" bf16 bits, or "q_*"/"s_*" MX codes and
    row-major scales).  Each job runs ref.routed_outputs on the tokens that
    route to its experts, with ``experts`` set, so the jobs' results are
    disjoint and are placed into Y [len(tokens), k, D] per case.  Returns one
    Y per case."""
    from concurrent.futures import ThreadPoolExecutor
    ys = [np.zeros((len(tok), idx.shape[1], x_bits.shape[1]), dtype=np.float64) for idx, tok in cases]
    used = set()
    for idx, tok in cases:
        used.update(np.unique(np.asarray(idx)[tok]).tolist())

    def job(group):
        wts = fetch(group)
        res = []
        for idx, tok in cases:
            sel = np.asarray(idx)[tok]
            rows = np.nonzero(np.isin(sel, group).any(axis=1))[0]
            res.append((rows, ref.routed_outputs(x_bits, wts, idx, precision, tok[rows], experts=group)
                        if len(rows) else None))
        return res

    groups = _expert_groups(used, per_job)
    with ThreadPoolExecutor(max_workers=min(workers, os.cpu_count() or 1)) as ex:
        for n, res in enumerate(ex.map(job, groups), 1):
            for y, (rows, part) in zip(ys, res):
                if part is not None:
                    y[rows] += part
            if n % max(1, len(groups) // 10) == 0:
                say(f"  oracle: {n}/{len(groups)} expert groups done")
    return ys


def fetch_bf16(inp):
    """fetch() for oracle_routed_pooled: the bf16 bits of some experts, copied
    from the (device) weight tensors."""
    def fetch(group):
        return {n: {int(e): synth.bits(inp[n][int(e)]) for e in group} for n in ("w_gate", "w_up", "w_down")}
    return fetch


def fetch_mx(inp):
    """fetch() for oracle_routed_pooled: the oracle's own MX quantisation of
    some experts' bf16 weights (codes and row-major scales along K)."""
    from oracle import bf16, mx

    def fetch(group):
        out = {}
        for n in ("gate", "up", "down"):
            q, s = {}, {}
            for e in group:
                q[int(e)], s[int(e)] = mx.quantize(bf16.to_f64(synth.bits(inp["w_" + n][int(e)])))
            out["q_" + n], out["s_" + n] = q, s
        return out
    return fetch
