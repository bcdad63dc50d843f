"""Pins of the oracle's router: logits, top-k selection and normalised gates."""

import math

import numpy as np
import pytest
import torch

import synth
from oracle import moe


def brute_topk(l, k):
    """Rank counting with an explicit comparator, pure Python: expert e is in
    slot s when exactly s experts precede it (larger logit, or equal logit and
    lower id)."""
    T, E = l.shape
    out = np.full((T, k), -1, dtype=np.int64)
    for t in range(T):
        for e in range(E):
            before = 0
            for f in range(E):
                if l[t, f] > l[t, e] or (l[t, f] == l[t, e] and f < e):
                    before += 1
            if before < k:
                out[t, before] = e
    return out


@pytest.mark.parametrize("T,E,k", [(40, 8, 2), (17, 33, 5), (9, 64, 8), (5, 7, 7), (6, 12, 1)])
def test_topk_matches_brute_force(T, E, k):
    l = torch.randn(T, E, generator=torch.Generator().manual_seed(T * E + k)).numpy()
    assert np.array_equal(moe.topk(l, k), brute_topk(l, k))


def test_topk_ties_and_signed_zero():
    l = synth.ties_logits(50, 16, seed=3).numpy()
    assert np.any(np.signbit(l) & (l == 0))  # -0.0 is present
    for k in (1, 4, 16):
        assert np.array_equal(moe.topk(l, k), brute_topk(l, k))
    # -0.0 and +0.0 tie: the lower id wins whichever sign it carries
    l2 = np.array([[-0.0, 0.0, -1.0], [0.0, -0.0, -1.0]], dtype=np.float32)
    assert np.array_equal(moe.topk(l2, 1), [[0], [0]])


def test_topk_rejects_non_finite():
    l = np.zeros((2, 4), dtype=np.float32)
    l[1, 2] = np.nan
    with pytest.raises(ValueError):
        moe.topk(l, 2)


def test_gates_against_short_form_scalar_python():
    # g_s = exp(l_s - l_max) / sum_{s'} exp(l_s' - l_max) over the selected
    # experts only: the same numbers as s_i / sum_j s_j with s the softmax over
    # all experts, computed here with scalar math.exp.
    l = torch.randn(30, 24, generator=torch.Generator().manual_seed(2)).numpy()
    k = 6
    idx = moe.topk(l, k)
    g = moe.gates(l, idx)
    for t in range(30):
        sel = [float(l[t, e]) for e in idx[t]]
        m = max(sel)
        z = [math.exp(v - m) for v in sel]
        ref = [v / sum(z) for v in z]
        assert np.allclose(g[t], ref, rtol=1e-14, atol=0)


def test_gates_invariants():
    l = torch.randn(50, 16, generator=torch.Generator().manual_seed(4)).numpy()
    idx = moe.topk(l, 4)
    g = moe.gates(l, idx)
    assert np.allclose(g.sum(-1), 1.0, rtol=0, atol=1e-15)
    assert np.all(np.diff(g, axis=-1) <= 0)  # slot order is logit order
    # k = 1 -> the single gate is exactly 1
    assert np.all(moe.gates(l, moe.topk(l, 1)) == 1.0)
    # equal selected logits -> 1/k each
    eq = np.zeros((3, 8), dtype=np.float32)
    assert np.allclose(moe.gates(eq, moe.topk(eq, 4)), 0.25, rtol=0, atol=1e-16)
    # shifting all logits by a constant changes nothing
    g2 = moe.gates(l.astype(np.float64) + 3.0, idx)  # exact shift in fp64
    assert np.allclose(g, g2, rtol=1e-12, atol=0)


def test_gates_match_torch_softmax_renormalised():
    l = torch.randn(20, 10, generator=torch.Generator().manual_seed(6), dtype=torch.float32)
    idx = moe.topk(l.numpy(), 3)
    s = torch.softmax(l.double(), dim=-1)
    sel = torch.gather(s, 1, torch.from_numpy(idx).long())
    ref = (sel / sel.sum(-1, keepdim=True)).numpy()
    assert np.allclose(moe.gates(l.numpy(), idx), ref, rtol=1e-13, atol=0)


def test_router_logits_and_bound_against_torch_fp32():
    w = synth.workload("tiny")
    inp = synth.make_inputs(w, with_weights=False)
    xb, wb = synth.bits(inp["x"]), synth.bits(inp["w_router"])
    L64 = moe.router_logits(xb, wb)
    # torch's float64 matmul of the same values (a library routine)
    ref = (inp["x"].double() @ inp["w_router"].double().T).numpy()
    assert np.allclose(L64, ref, rtol=1e-13, atol=1e-13)
    # torch's fp32 matmul lies inside the summation bound
    l32 = (inp["x"].float() @ inp["w_router"].float().T).numpy()
    assert np.all(np.abs(l32 - L64) <= moe.logit_bound(xb, wb))
    # and the bound is not vacuous: well below the logits' spread
    assert moe.logit_bound(xb, wb).max() < 1e-3 * np.std(L64)
