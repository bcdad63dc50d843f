"""Pins of the oracle's backward pass (oracle/backward.py).

Against: torch float64 autograd of the same layer written in torch (a library
differentiation, independent of the oracle's hand-written gradient formulas),
on several shapes; central finite differences of the oracle's own forward
pieces on single weight and input entries; and exact invariants (the softmax
gradient sums to zero, k = 1 leaves the logits without gradient, a zero
output gradient gives zero everywhere).  The bf16 storage mode is checked to
stay within a bounded distance of the exact gradients.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
from oracle import backward as bwd
from oracle import bf16
from oracle import moe


def case(T=24, D=64, I=32, E=6, k=2, Is=32, seed=0):
    w = synth.Workload("b", T=T, D=D, I=I, E=E, k=k, I_shared=Is, seed=seed)
    inp = synth.make_inputs(w)
    host = {n: synth.bits(t) for n, t in inp.items() if t.dtype == torch.bfloat16}
    g = torch.Generator().manual_seed(seed + 100)
    dout = torch.randn((T, D), generator=g).to(torch.bfloat16)
    L64 = moe.router_logits(host["x"], host["w_router"])
    return w, inp, host, synth.bits(dout), L64


def torch_grads(inp, dout_bits, L64, k):
    """dLoss/d(everything) by torch float64 autograd of the layer with the
    selection held fixed (taken on the fp32 logits, as the oracle takes it)."""
    t = {n: v.double().clone().requires_grad_(True) for n, v in inp.items() if v.dtype == torch.bfloat16}
    dout = torch.from_numpy(bf16.to_f64(dout_bits))
    idx = torch.from_numpy(moe.topk(L64.astype(np.float32), k).astype(np.int64))
    logits = t["x"] @ t["w_router"].T
    g = torch.softmax(torch.gather(logits, 1, idx), dim=1)

    def ffn(x, wg, wu, wd):
        return F.linear(F.silu(F.linear(x, wg)) * F.linear(x, wu), wd)

    out = ffn(t["x"], t["ws_gate"], t["ws_up"], t["ws_down"])
    for s in range(k):
        rows = [ffn(t["x"][i:i + 1], t["w_gate"][e], t["w_up"][e], t["w_down"][e]) for i, e in
                enumerate(idx[:, s].tolist())]
        out = out + g[:, s:s + 1] * torch.cat(rows)
    (out * dout).sum().backward()
    return {n: v.grad.numpy() for n, v in t.items()}


@pytest.mark.parametrize("shape", [dict(), dict(T=40, D=128, I=64, E=8, k=3, Is=48, seed=3),
                                   dict(T=17, D=64, I=96, E=5, k=5, Is=32, seed=4)])
def test_exact_backward_matches_torch_autograd(shape):
    w, inp, host, dout, L64 = case(**shape)
    got = bwd.backward(host["x"], host, L64, w.k, dout, w_router_bits=host["w_router"], exact=True)
    want = torch_grads(inp, dout, L64, w.k)
    for mine, theirs in (("dx", "x"), ("dW_gate", "w_gate"), ("dW_up", "w_up"), ("dW_down", "w_down"),
                         ("dWs_gate", "ws_gate"), ("dWs_up", "ws_up"), ("dWs_down", "ws_down"),
                         ("dW_router", "w_router")):
        ref = want[theirs]
        assert np.allclose(got[mine], ref, rtol=1e-9, atol=1e-11 * np.abs(ref).max()), mine


def test_exact_backward_matches_finite_differences():
    # the loss sum(out * dout) of the oracle's own exact forward pieces, with
    # single entries of x and of the weights moved by +-eps; the selection is
    # held fixed (eps is far below every logit gap of this case)
    w, inp, host, dout_bits, L64 = case(T=6, D=32, I=16, E=4, k=2, Is=16, seed=7)
    V = {n: bf16.to_f64(b) for n, b in host.items()}
    dout = bf16.to_f64(dout_bits)
    idx = moe.topk(L64.astype(np.float32), w.k)

    def loss(V):
        logits = V["x"] @ V["w_router"].T
        g = np.exp(np.take_along_axis(logits, idx.astype(np.int64), 1))
        g = g / g.sum(axis=1, keepdims=True)
        out = moe.ffn(V["x"], V["ws_gate"], V["ws_up"], V["ws_down"], h_store=None, y_store=None)
        for t in range(w.T):
            for s in range(w.k):
                e = idx[t, s]
                out[t] += g[t, s] * moe.ffn(V["x"][t:t + 1], V["w_gate"][e], V["w_up"][e], V["w_down"][e],
                                            h_store=None, y_store=None)[0]
        return float(np.sum(out * dout))

    got = bwd.backward(host["x"], host, L64, w.k, dout_bits, w_router_bits=host["w_router"], exact=True)
    grad_of = {"x": "dx", "w_gate": "dW_gate", "w_up": "dW_up", "w_down": "dW_down", "ws_gate": "dWs_gate",
               "ws_up": "dWs_up", "ws_down": "dWs_down", "w_router": "dW_router"}
    e0 = int(idx[0, 0])
    probes = [("x", (2, 5)), ("x", (0, 31)), ("w_gate", (e0, 3, 7)), ("w_up", (e0, 11, 2)),
              ("w_down", (e0, 4, 9)), ("ws_gate", (5, 6)), ("ws_up", (0, 0)), ("ws_down", (30, 15)),
              ("w_router", (e0, 12)), ("w_router", (int(idx[3, 1]), 1))]
    eps = 1e-6
    for name, pos in probes:
        Vp = {n: v.copy() for n, v in V.items()}
        Vm = {n: v.copy() for n, v in V.items()}
        Vp[name][pos] += eps
        Vm[name][pos] -= eps
        fd = (loss(Vp) - loss(Vm)) / (2 * eps)
        an = got[grad_of[name]][pos]
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, pos, fd, an)


def test_softmax_gradient_sums_to_zero_and_k1_has_none():
    w, inp, host, dout, L64 = case(k=3)
    got = bwd.backward(host["x"], host, L64, 3, dout, exact=True)
    assert np.allclose(got["dlogits"].sum(axis=1), 0.0, atol=1e-12 * np.abs(got["dlogits"]).max())
    # off the selection the logits have no gradient
    mask = np.zeros_like(got["dlogits"], dtype=bool)
    np.put_along_axis(mask, got["idx"].astype(np.int64), True, axis=1)
    assert np.all(got["dlogits"][~mask] == 0)
    one = bwd.backward(host["x"], host, L64, 1, dout, exact=True)
    assert np.all(one["dlogits"] == 0)


def test_zero_output_gradient_gives_zero_gradients():
    w, inp, host, dout, L64 = case()
    zero = np.zeros_like(dout)
    got = bwd.backward(host["x"], host, L64, w.k, zero, w_router_bits=host["w_router"])
    for n in ("dx", "dW_gate", "dW_up", "dW_down", "dWs_gate", "dWs_up", "dWs_down", "dW_router"):
        assert np.all(got[n] == 0), n


def test_storage_rounding_is_present_and_bounded():
    # the bf16 storage of g * dout, the replayed a_g and a_u, da and the weight
    # gradients moves the gradients by at most a few percent of their RMS
    # (measured here: dW_gate 0.066, the largest; for one expert of 24 rows
    # 0.009 from a_g/a_u, 0.009 from da, 0.015 from g * dout); the GPU
    # comparison mirrors these roundings, so only rounding-boundary flips
    # between fp32 and fp64 values remain there
    w, inp, host, dout, L64 = case(T=64, D=128, I=64, E=8, k=4, Is=64, seed=9)
    a = bwd.backward(host["x"], host, L64.astype(np.float32), w.k, dout, w_router_bits=host["w_router"])
    b = bwd.backward(host["x"], host, L64.astype(np.float32), w.k, dout, w_router_bits=host["w_router"],
                     exact=True)
    for n in ("dx", "dW_gate", "dW_up", "dW_down", "dWs_gate", "dWs_down", "dW_router"):
        rel = np.max(np.abs(a[n] - b[n])) / np.sqrt(np.mean(b[n] ** 2))
        assert 0 < rel < 1e-1, (n, rel)


def test_sampled_pieces_equal_the_whole_layer():
    # the per-token, per-expert and per-column pieces used on samples of a
    # large layer give the rows of the whole-layer result (bf16 storage mode)
    w, inp, host, dout, L64 = case(T=48, D=64, I=32, E=7, k=3, Is=40, seed=11)
    lg = L64.astype(np.float32)
    full = bwd.backward(host["x"], host, lg, w.k, dout, w_router_bits=host["w_router"])
    idx, g = full["idx"], full["gates"]

    def close(a, b):
        return np.allclose(a, b, rtol=1e-12, atol=1e-12 * np.abs(b).max())

    for e in (0, 3, 6):
        ti, b = bwd.expert_backward(host["x"], host, idx, g, dout, e)
        assert np.array_equal(np.sort(np.unique(ti)), np.nonzero((idx == e).any(axis=1))[0])
        for n in ("dW_gate", "dW_up", "dW_down"):
            assert close(b[n], full[n][e]), (e, n)
    tok = np.array([0, 5, 17, 47])
    Y = moe.routed_outputs(host["x"], host, idx, tokens=tok)
    dx = bwd.token_dx(host["x"], host, lg, w.k, dout, tok, Y, host["w_router"])
    assert close(dx, full["dx"][tok])
    assert close(bwd.logit_grad_rows(lg, w.k, dout, Y, tok), full["dlogits"][tok])
    cols = np.array([1, 8, 39])
    sh = bwd.shared_columns_backward(host["x"], host, dout, cols)
    assert close(sh["dWs_gate"], full["dWs_gate"][cols]) and close(sh["dWs_up"], full["dWs_up"][cols])
    assert close(sh["dWs_down"], full["dWs_down"][:, cols])
    ex = np.array([2, 4])
    every = np.nonzero(np.isin(idx, ex).any(axis=1))[0]
    Ye = moe.routed_outputs(host["x"], host, idx, tokens=every)
    assert close(bwd.router_weight_rows(host["x"], lg, w.k, dout, Ye, every, ex), full["dW_router"][ex])
    with pytest.raises(ValueError):
        bwd.router_weight_rows(host["x"], lg, w.k, dout, Ye[:-1], every[:-1], ex)
