"""GPU parity of moe_route: router GEMM, top-k selection and gates."""

import numpy as np
import pytest
import torch

import synth
from oracle import moe as ref
from tests._gpu import gate_tolerance, layer, need_gpu, say

pytestmark = pytest.mark.gpu

ROUTE_CASES = [
    # the router GEMM's K ranges (planes the top-k adds in order): 4 for up to
    # 128 output tiles of 128 x 128, 2 for up to 256, 1 beyond; logits per
    # lane of the top-k from 1 (E <= 64) to 16 (E = 1000)
    synth.workload("tiny"),
    synth.Workload("ragged", T=333, D=320, I=64, E=24, k=5, I_shared=64, seed=11),
    synth.Workload("wide", T=130, D=256, I=64, E=384, k=8, I_shared=64, seed=12),
    synth.Workload("e1k", T=70, D=128, I=64, E=1000, k=16, I_shared=64, seed=13),
    synth.Workload("e100", T=1000, D=512, I=64, E=100, k=6, I_shared=64, seed=23),
    synth.Workload("e512", T=700, D=256, I=64, E=512, k=16, I_shared=64, seed=24),
    synth.Workload("d7168", T=2000, D=7168, I=64, E=256, k=8, I_shared=64, seed=25),
    synth.Workload("k2ranges", T=5632, D=128, I=64, E=384, k=8, I_shared=64, seed=17),
    synth.Workload("k2ranges-e64", T=16512, D=128, I=64, E=64, k=6, I_shared=64, seed=19),
    synth.Workload("k1range", T=11008, D=128, I=64, E=384, k=8, I_shared=64, seed=18),
    synth.Workload("k1range-e64", T=33024, D=128, I=64, E=64, k=6, I_shared=64, seed=20),
]


@pytest.mark.parametrize("w", ROUTE_CASES, ids=lambda w: w.name)
def test_route_from_x(w):
    dev = need_gpu()
    say("route_from_x", w)
    inp = synth.make_inputs(w, with_weights=False)
    m = layer(w, dev)
    logits, idx, gate = m.route(inp["x"].to(dev), inp["w_router"].to(dev))
    torch.cuda.synchronize()
    xb, wb = synth.bits(inp["x"]), synth.bits(inp["w_router"])
    L64 = ref.router_logits(xb, wb)
    bound = ref.logit_bound(xb, wb)
    lg32 = logits.cpu().numpy()
    lg = lg32.astype(np.float64)
    assert np.all(np.abs(lg - L64) <= bound), "router logits outside the fp32 summation bound"
    # given its own fp32 logits, the selection is the oracle's on every token,
    # and the gates are within the fp32 gate bound of the oracle's
    gi32 = idx.cpu().numpy()
    assert np.array_equal(ref.topk(lg32, w.k), gi32)
    g32, gref32 = gate.cpu().numpy().astype(np.float64), ref.gates(lg32, gi32)
    sel32 = np.take_along_axis(lg, gi32.astype(np.int64), 1)
    assert np.all(np.abs(g32 - gref32) <= gate_tolerance(sel32, w.k) * gref32)
    # selection: where the fp64 logits leave no doubt the choice must be the
    # oracle's; everywhere it must be a valid top-k under the error bound
    gi = idx.cpu().numpy().astype(np.int64)
    oi = ref.topk(L64.astype(np.float32), w.k).astype(np.int64)
    srt = np.sort(L64, axis=1)[:, ::-1]
    gap = srt[:, w.k - 1] - srt[:, w.k] if w.k < w.E else np.full(w.T, np.inf)
    clear = gap > 2 * bound.max(axis=1)
    assert np.array_equal(np.sort(gi[clear], 1), np.sort(oi[clear], 1))
    for t in range(w.T):
        sel = set(gi[t].tolist())
        assert len(sel) == w.k and all(0 <= e < w.E for e in sel)
        lo = min(L64[t, e] + bound[t, e] for e in sel)
        hi = max((L64[t, f] - bound[t, f] for f in range(w.E) if f not in sel), default=-np.inf)
        assert lo >= hi
    # gates on the tokens with an unambiguous selection, against fp64 gates
    # of the fp64 logits (the logit error enters twice through the exponent)
    g = gate.cpu().numpy().astype(np.float64)
    gref = ref.gates(L64, oi)
    sel_l = np.take_along_axis(L64, oi, 1)
    tol = gate_tolerance(sel_l, w.k) + 4 * bound.max(axis=1, keepdims=True)
    ok = clear & np.all(gi == oi, axis=1)
    assert np.all(np.abs(g[ok] - gref[ok]) <= tol[ok] * gref[ok])


LOGIT_CASES = [
    ("gaussian", synth.workload("tiny", routing="gaussian")),
    ("gaussian-mid", synth.workload("mid", routing="gaussian", T=1024)),
    ("zipf", synth.Workload("zipf", T=2048, D=128, I=64, E=256, k=8, I_shared=64, seed=21, routing="zipf")),
    ("zipf384", synth.Workload("zipf384", T=512, D=128, I=64, E=384, k=8, I_shared=64, seed=22, routing="zipf")),
]


@pytest.mark.parametrize("name,w", LOGIT_CASES, ids=[c[0] for c in LOGIT_CASES])
def test_route_given_logits_bit_exact(name, w):
    dev = need_gpu()
    say("route_given_logits", name, w)
    logits = synth.make_logits(w)
    m = layer(w, dev)
    _, idx, gate = m.route(None, None, logits.to(dev))
    torch.cuda.synchronize()
    l = logits.numpy()
    oi = ref.topk(l, w.k)
    assert np.array_equal(idx.cpu().numpy(), oi)
    g = gate.cpu().numpy().astype(np.float64)
    gref = ref.gates(l, oi)
    tol = gate_tolerance(np.take_along_axis(l.astype(np.float64), oi.astype(np.int64), 1), w.k)
    assert np.all(np.abs(g - gref) <= tol * gref)
    assert m.device_error() == 0


def test_route_ties_and_signed_zero():
    dev = need_gpu()
    w = synth.Workload("ties", T=200, D=64, I=64, E=40, k=7, I_shared=64, seed=5)
    l = synth.ties_logits(w.T, w.E, seed=9)
    say("route_ties", w)
    m = layer(w, dev)
    _, idx, gate = m.route(None, None, l.to(dev))
    assert np.array_equal(idx.cpu().numpy(), ref.topk(l.numpy(), w.k))


def test_route_k_equals_e_and_k1():
    dev = need_gpu()
    for E, k in ((8, 8), (64, 1), (65, 16), (16, 16)):
        w = synth.Workload("kE", T=50, D=64, I=64, E=E, k=k, I_shared=64, seed=E + k, routing="gaussian")
        say("route_kE", w)
        l = synth.make_logits(w)
        m = layer(w, dev)
        _, idx, gate = m.route(None, None, l.to(dev))
        assert np.array_equal(idx.cpu().numpy(), ref.topk(l.numpy(), k))
        if k == 1:
            assert torch.all(gate == 1.0)


def test_route_nonfinite_sets_error_bit():
    dev = need_gpu()
    w = synth.Workload("nan", T=8, D=64, I=64, E=16, k=2, I_shared=64, seed=1, routing="gaussian")
    l = synth.make_logits(w)
    l[3, 5] = float("nan")
    say("route_nonfinite", w)
    m = layer(w, dev)
    _, idx, _ = m.route(None, None, l.to(dev))
    from mixture_experts_layer_counts_amd import _lib
    assert m.device_error() & _lib.DEVERR_NONFINITE
    # NaN ranks last: the other tokens are untouched and token 3 never picks 5
    rows = [t for t in range(w.T) if t != 3]
    assert np.array_equal(idx.cpu().numpy()[rows], ref.topk(l.numpy()[rows], w.k))
    assert 5 not in idx.cpu().numpy()[3]


def test_route_from_x_nonfinite_sets_error_bit():
    # an infinite entry of x makes its token's logits non-finite (the router
    # GEMM's 4 K-range planes, summed by the top-k); the error bit is set and
    # the other tokens' selections are the oracle's top-k of the GPU's logits
    dev = need_gpu()
    w = synth.Workload("inf-x", T=600, D=256, I=64, E=128, k=4, I_shared=64, seed=26)
    inp = synth.make_inputs(w, with_weights=False)
    x = inp["x"].clone()
    x[257, 3] = float("inf")
    say("route_from_x nonfinite", w)
    m = layer(w, dev)
    logits, idx, _ = m.route(x.to(dev), inp["w_router"].to(dev))
    from mixture_experts_layer_counts_amd import _lib
    assert m.device_error() & _lib.DEVERR_NONFINITE
    lg = logits.cpu().numpy()
    assert not np.all(np.isfinite(lg[257]))
    rows = [t for t in range(w.T) if t != 257]
    assert np.all(np.isfinite(lg[rows]))
    assert np.array_equal(idx.cpu().numpy()[rows], ref.topk(lg[rows], w.k))
