"""Pins of the oracle's layer computation (expert FFNs, shared expert, combine).

Against: torch float64 library routines (F.linear, F.silu) for a dense SwiGLU
FFN; the identity "one expert, top-1 plus the shared expert = one dense SwiGLU
FFN over the concatenated intermediate axis"; a scalar pure-Python evaluation
of the MoE equation on a tiny case; exact invariants (zero input, power-of-two
scaling, token permutation).
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
from oracle import bf16, moe, mx


def small(T=24, D=64, I=32, E=6, k=2, Is=32, seed=0):
    w = synth.Workload("t", T=T, D=D, I=I, E=E, k=k, I_shared=Is, seed=seed, routing="gaussian")
    inp = synth.make_inputs(w)
    host = {n: synth.bits(t) for n, t in inp.items() if t.dtype == torch.bfloat16}
    return w, inp, host, inp["logits"].numpy()


def torch_swiglu(x, wg, wu, wd):
    return F.linear(F.silu(F.linear(x, wg)) * F.linear(x, wu), wd)


def test_ffn_matches_torch_float64():
    w, inp, host, _ = small()
    x = inp["x"].double()
    ref = torch_swiglu(x, inp["w_gate"][3].double(), inp["w_up"][3].double(), inp["w_down"][3].double())
    got = moe.ffn(bf16.to_f64(host["x"]), bf16.to_f64(host["w_gate"][3]), bf16.to_f64(host["w_up"][3]),
                  bf16.to_f64(host["w_down"][3]), h_store=None, y_store=None)
    assert np.allclose(got, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_one_expert_top1_plus_shared_is_dense_ffn():
    # E = 1, k = 1: gate = 1, so MoE(x) = f_shared(x) + f_0(x), which is one
    # SwiGLU FFN whose intermediate axis is the two experts' axes side by side.
    w, inp, host, logits = small(E=1, k=1, I=48, Is=16)
    wg = torch.cat([inp["ws_gate"], inp["w_gate"][0]]).double()
    wu = torch.cat([inp["ws_up"], inp["w_up"][0]]).double()
    wd = torch.cat([inp["ws_down"], inp["w_down"][0]], dim=1).double()
    dense = torch_swiglu(inp["x"].double(), wg, wu, wd).numpy()
    exact = moe.forward(host["x"], host, logits, 1, exact=True)
    assert np.all(exact["gates"] == 1.0)
    assert np.allclose(exact["out"], dense, rtol=1e-12, atol=1e-12)
    # with the storage rounding of h and Y the result stays within their bounds
    stored = moe.forward(host["x"], host, logits, 1)
    assert np.max(np.abs(stored["out"] - dense)) < 2e-2 * np.sqrt(np.mean(dense ** 2))


def scalar_moe(x, W, logits, k):
    """MoE equation token by token with scalar Python arithmetic (tiny sizes)."""
    T, D = len(x), len(x[0])
    E, I = len(W["w_gate"]), len(W["w_gate"][0])
    Is = len(W["ws_gate"])

    def f(xv, wg, wu, wd, n_int):
        h = []
        for i in range(n_int):
            a = sum(wg[i][d] * xv[d] for d in range(D))
            b = sum(wu[i][d] * xv[d] for d in range(D))
            h.append(a / (1.0 + math.exp(-a)) * b)
        return [sum(wd[o][i] * h[i] for i in range(n_int)) for o in range(D)]

    out = []
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(logits[t][e]), e))[:k]
        z = [math.exp(float(logits[t][e]) - max(float(logits[t][q]) for q in order)) for e in order]
        g = [v / sum(z) for v in z]
        acc = f(x[t], W["ws_gate"], W["ws_up"], W["ws_down"], Is)
        for s, e in enumerate(order):
            y = f(x[t], W["w_gate"][e], W["w_up"][e], W["w_down"][e], I)
            acc = [acc[d] + g[s] * y[d] for d in range(D)]
        out.append(acc)
    return np.array(out)


def test_forward_matches_scalar_python_moe():
    w, inp, host, logits = small(T=5, D=12, I=6, E=5, k=3, Is=4, seed=3)
    W = {n: bf16.to_f64(host[n]).tolist() for n in ("w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")}
    ref = scalar_moe(bf16.to_f64(host["x"]).tolist(), W, logits.tolist(), 3)
    got = moe.forward(host["x"], host, logits, 3, exact=True)["out"]
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_zero_input_gives_zero_output():
    w, inp, host, logits = small()
    host = dict(host)
    host["x"] = np.zeros_like(host["x"])
    assert np.all(moe.forward(host["x"], host, logits, w.k)["out"] == 0.0)


def test_power_of_two_scaling_of_down_projection():
    # doubling every W_down doubles Y and the shared output exactly (rounding
    # to bf16 commutes with multiplication by 2)
    w, inp, host, logits = small()
    a = moe.forward(host["x"], host, logits, w.k)
    h2 = dict(host)
    for n in ("w_down", "ws_down"):
        h2[n] = bf16.from_f64(2.0 * bf16.to_f64(host[n]))
    b = moe.forward(host["x"], h2, logits, w.k)
    assert np.array_equal(b["out"], 2.0 * a["out"])


def test_token_permutation_equivariance():
    w, inp, host, logits = small(T=32)
    perm = np.random.default_rng(0).permutation(32)
    a = moe.forward(host["x"], host, logits, w.k)["out"]
    h2 = dict(host)
    h2["x"] = host["x"][perm]
    b = moe.forward(h2["x"], h2, logits[perm], w.k)["out"]
    assert np.allclose(b, a[perm], rtol=1e-13, atol=1e-13)


def test_sampled_tokens_equal_full_layer():
    w, inp, host, logits = small(T=40)
    full = moe.forward(host["x"], host, logits, w.k)["out"]
    tok = np.array([3, 17, 39, 0])
    part = moe.forward(host["x"], host, logits, w.k, tokens=tok)["out"]
    assert np.allclose(part, full[tok], rtol=1e-13, atol=1e-13)


def test_routed_outputs_over_disjoint_expert_sets_add_up():
    # evaluating the routes expert set by expert set (as the full-shape GPU
    # tests do in a thread pool) gives the full routed outputs, bit for bit
    w, inp, host, l = small(T=40, E=8, k=3, seed=5)
    idx = moe.topk(l, w.k)
    full = moe.routed_outputs(host["x"], host, idx)
    parts = [moe.routed_outputs(host["x"], host, idx, experts=g) for g in ([0, 3, 5], [1, 2], [4, 6, 7])]
    assert np.array_equal(parts[0] + parts[1] + parts[2], full)
    for g, p in zip(([0, 3, 5], [1, 2], [4, 6, 7]), parts):  # rows of other experts stay zero
        assert np.all(p[~np.isin(idx, g)] == 0)


def test_mx_mode_is_lossless_on_grid_inputs():
    # weights and x chosen on the MX grid: quantisation is then the identity,
    # so the MXFP8 layer equals the bf16 layer when h is left unrounded
    w, inp, host, logits = small(D=64, I=32)
    rng = np.random.default_rng(2)

    def grid(shape):
        codes = rng.integers(0x30, 0x50, shape).astype(np.uint8)  # |v| in [2^-1, 2^3]
        codes[..., ::32] = 0x7E
        codes |= (rng.integers(0, 2, shape) * 0x80).astype(np.uint8)
        return mx.dequantize(codes, np.full(shape[:-1] + (shape[-1] // 32,), 127 - 9, dtype=np.uint8))

    h2 = dict(host)
    for n in ("w_gate", "w_up", "w_down"):
        h2[n] = bf16.from_f64(grid(host[n].shape))  # grid values need <= 4 bits: exact in bf16
    h2["x"] = bf16.from_f64(grid(host["x"].shape))
    q = moe.quantize_weights_mx(h2)
    for n, qn, sn in (("w_gate", "q_gate", "s_gate"), ("w_down", "q_down", "s_down")):
        assert np.array_equal(mx.dequantize(q[qn], q[sn]), bf16.to_f64(h2[n]))
    a = moe.forward(h2["x"], q, logits, w.k, precision="mxfp8", exact=True)["out"]
    b = moe.forward(h2["x"], h2, logits, w.k, precision="bf16", exact=True)["out"]
    assert np.allclose(a, b, rtol=1e-13, atol=1e-13)


def test_mx_shared_expert_is_lossless_on_grid_inputs():
    # the MXFP8 shared expert on x and weights chosen on the MX grid equals the
    # bf16 shared expert when h is left unrounded (a swapped gate/up, a wrong
    # operand or a missed dequantisation would break the equality)
    w, inp, host, logits = small(D=64, I=32, Is=64)
    rng = np.random.default_rng(3)

    def grid(shape):
        codes = rng.integers(0x30, 0x50, shape).astype(np.uint8)  # |v| in [2^-1, 2^3]
        codes[..., ::32] = 0x7E
        codes |= (rng.integers(0, 2, shape) * 0x80).astype(np.uint8)
        return mx.dequantize(codes, np.full(shape[:-1] + (shape[-1] // 32,), 127 - 9, dtype=np.uint8))

    h2 = dict(host)
    for n in ("ws_gate", "ws_up", "ws_down", "x"):
        h2[n] = bf16.from_f64(grid(host[n].shape))
    q = moe.quantize_shared_mx(h2)
    for n in ("gate", "up", "down"):
        assert np.array_equal(mx.dequantize(q["qs_" + n], q["ss_" + n]), bf16.to_f64(h2["ws_" + n]))
    a = moe.shared_output(h2["x"], q, exact=True, precision="mxfp8")
    b = moe.shared_output(h2["x"], h2, exact=True, precision="bf16")
    assert np.allclose(a, b, rtol=1e-13, atol=1e-13)
    # stored: h in MX along I_shared moves the output by a bounded amount
    s = moe.shared_output(h2["x"], q, precision="mxfp8")
    rms = np.sqrt(np.mean(b ** 2))
    assert 1e-4 < np.max(np.abs(s - b)) / rms < 0.3
    # the whole layer with the MX shared expert changes only the shared term
    f1 = moe.forward(h2["x"], q, logits, w.k, shared_precision="mxfp8")
    f0 = moe.forward(h2["x"], h2, logits, w.k)
    assert np.array_equal(f1["Y"], f0["Y"])
    assert np.allclose(f1["out"] - f1["shared"], f0["out"] - f0["shared"], rtol=0, atol=1e-12)


def test_storage_rounding_is_present_and_bounded():
    # Rounding h and each routed output row to bf16 moves the layer output by
    # about 1e-2 RMS: the same size as the bf16 parity tolerance.  This is why
    # the oracle rounds the stored intermediates exactly as the method stores
    # them instead of comparing against the unrounded formula.
    w, inp, host, logits = small(T=64, D=128, I=64, E=8, k=2, Is=64, seed=5)
    exact = moe.forward(host["x"], host, logits, 2, exact=True)
    stored = moe.forward(host["x"], host, logits, 2)
    rms = np.sqrt(np.mean(exact["out"] ** 2))
    dev = np.max(np.abs(stored["out"] - exact["out"])) / rms
    assert 1e-3 < dev < 4e-2
    # the stored routed rows are bf16 values
    assert np.array_equal(bf16.round_f64(stored["Y"]), stored["Y"])
    q = moe.quantize_weights_mx(host)
    m = moe.forward(host["x"], q, logits, 2, precision="mxfp8")["out"]
    assert np.max(np.abs(m - exact["out"])) < 0.3 * rms  # MX moves weights and x by up to 2^-4 relative
