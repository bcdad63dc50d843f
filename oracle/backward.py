"""The MoE-layer backward pass, written out plainly in fp64 (numpy).

Test infrastructure: only the tests, the smoke check and the benchmark's
CPU-baseline leg use this module.

What is differentiated (MoK paper "Mixture-of-Kittens: MoE Megakernel for
NVL72s", §2.1 MoE equation; backward in §3.3 "Ring-Aware Forward Replay" and
§3.4 "Router Weight Gradient Computation"):

    out = f_shared(x) + sum_s g_s f_{e_s}(x),   g = softmax of the k selected logits
    f(x) = W_down ( SiLU(W_gate x) * (W_up x) ),  logits = W_r x

Given dout = dLoss/dout, for each token (the selection itself is piecewise
constant and has no gradient):

    dg_s      = <dout, y_s>                          y_s the stored routed row
    dy_s      = g_s dout
    per expert FFN with input x and output gradient dy:
      a_g = W_gate x,  a_u = W_up x,  h = SiLU(a_g) a_u
      dh  = W_down^T dy
      da_g = dh * a_u * SiLU'(a_g),  SiLU'(a) = s(a) (1 + a (1 - s(a))),  s = sigmoid
      da_u = dh * SiLU(a_g)
      dx  += W_gate^T da_g + W_up^T da_u
      dW_down += dy h^T,  dW_gate += da_g x^T,  dW_up += da_u x^T
    the shared expert the same, with dy = dout
    dl_s      = g_s (dg_s - sum_s' g_s' dg_s')        (softmax over the selected logits)
    dx       += W_r^T dl,  dW_r += dl x^T             (dl zero off the selection)

Readings (listed in the design doc), mirrored from what the GPU path stores:
* the storage roundings of the forward (h and y in bf16) pass the gradient
  through unchanged;
* a_g and a_u are recomputed ("replayed") and stored in bf16; the backward's
  h is SiLU(a_g) a_u of those stored values, stored in bf16;
* g_s dout is stored in bf16 (the down projection's data-gradient operand);
  dout itself arrives in bf16 and feeds the shared expert directly;
* da_g and da_u are stored in bf16; dh, dx and the router-weight gradient
  stay fp32 (here fp64);
* the router-logit gradient is stored in bf16 for its two GEMMs;
* the expert weight gradients are stored in bf16.
``exact=True`` evaluates the same formulas with no rounding at all.
"""

from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from . import bf16 as _bf16
from . import moe as _moe


def _round(exact: bool):
    return (lambda v: v) if exact else _bf16.round_f64


def silu_grad(a: np.ndarray) -> np.ndarray:
    """d SiLU(a) / da = s(a) (1 + a (1 - s(a))), s the logistic sigmoid."""
    s = 1.0 / (1.0 + np.exp(-a))
    return s * (1.0 + a * (1.0 - s))


def ffn_backward(x: np.ndarray, dy: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray,
                 exact: bool = False) -> Dict[str, np.ndarray]:
    """Backward of f(x) = W_down (SiLU(W_gate x) * W_up x) for rows x [n, D]
    with output gradients dy [n, D] (fp64 values).  w_gate, w_up [I, D],
    w_down [D, I].  Returns dx [n, D] and dW_gate, dW_up [I, D], dW_down
    [D, I], summed over the rows."""
    r = _round(exact)
    a_g = r(x @ w_gate.T)  # replayed, stored
    a_u = r(x @ w_up.T)
    silu = _moe.silu(a_g)
    h = r(silu * a_u)
    dh = dy @ w_down
    da_g = r(dh * a_u * silu_grad(a_g))
    da_u = r(dh * silu)
    return {"dx": da_g @ w_gate + da_u @ w_up,
            "dW_gate": r(da_g.T @ x), "dW_up": r(da_u.T @ x), "dW_down": r(dy.T @ h)}


def gate_logit_grad(g: np.ndarray, dg: np.ndarray) -> np.ndarray:
    """Gradient with respect to the selected logits of g = softmax(selected
    logits): dl_s = g_s (dg_s - sum_s' g_s' dg_s')."""
    return g * (dg - np.sum(g * dg, axis=-1, keepdims=True))


def backward(x_bits: np.ndarray, weights: Dict[str, np.ndarray], logits: np.ndarray, k: int,
             dout_bits: np.ndarray, w_router_bits: Optional[np.ndarray] = None,
             exact: bool = False) -> Dict[str, np.ndarray]:
    """The layer's gradients for all tokens (bf16 mode of the forward).

    x_bits [T, D], dout_bits [T, D] bf16; weights holds the bf16 expert
    weights (w_*, ws_*); logits [T, E] are the router logits the selection and
    the gates are taken on (fp32, or fp64 values in the exact checks).  With
    w_router_bits the router-weight gradient and the router's share of dx are
    included.  Returns dx [T, D], dW_gate/dW_up [E, I, D], dW_down [E, D, I],
    dWs_gate/dWs_up [I_s, D], dWs_down [D, I_s], dlogits [T, E] (fp32 values
    before the bf16 storage), dW_router [E, D] and, per token, dg [T, k].
    """
    r = _round(exact)
    x = _bf16.to_f64(x_bits)
    dout = _bf16.to_f64(dout_bits)
    T, D = x.shape
    E, I = weights["w_gate"].shape[0], weights["w_gate"].shape[1]
    idx = _moe.topk(logits, k)
    g = _moe.gates(logits, idx)

    # the shared expert, with the output gradient as it arrives
    sh = ffn_backward(x, dout, _bf16.to_f64(weights["ws_gate"]), _bf16.to_f64(weights["ws_up"]),
                      _bf16.to_f64(weights["ws_down"]), exact)
    dx = sh["dx"].copy()

    # gate gradients from the stored routed rows of the forward
    Y = _moe.routed_outputs(x_bits, weights, idx, exact=exact)
    dg = np.einsum("td,tkd->tk", dout, Y)

    # routed experts: the routes of each expert together
    dW = {n: np.zeros(weights[w].shape, dtype=np.float64)
          for n, w in (("dW_gate", "w_gate"), ("dW_up", "w_up"), ("dW_down", "w_down"))}
    for e in np.unique(idx):
        ti, si = np.nonzero(idx == e)
        dy = r(g[ti, si][:, None] * dout[ti])
        b = ffn_backward(x[ti], dy, _bf16.to_f64(weights["w_gate"][e]), _bf16.to_f64(weights["w_up"][e]),
                         _bf16.to_f64(weights["w_down"][e]), exact)
        np.add.at(dx, ti, b["dx"])
        for n in dW:
            dW[n][e] = b[n]

    # router: the gradient of the selected logits, zero elsewhere
    dl_sel = gate_logit_grad(g, dg)
    dlogits = np.zeros((T, np.asarray(logits).shape[1]), dtype=np.float64)
    np.put_along_axis(dlogits, idx.astype(np.int64), dl_sel, axis=1)
    out = {"dx": dx, "dWs_gate": sh["dW_gate"], "dWs_up": sh["dW_up"], "dWs_down": sh["dW_down"],
           "dlogits": dlogits, "dg": dg, "idx": idx, "gates": g, **dW}
    if w_router_bits is not None:
        dlb = r(dlogits)
        out["dx"] = dx + dlb @ _bf16.to_f64(w_router_bits)
        out["dW_router"] = dlb.T @ x
    return out
