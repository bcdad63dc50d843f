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
        ti, b = expert_backward(x_bits, weights, idx, g, dout_bits, int(e), exact=exact)
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


# ---- pieces of the same computation, for samples of a large layer ----
# Every token's dx depends on that token alone, every expert's weight gradient
# on the routes to that expert alone, and every intermediate column i of the
# shared expert on column i alone (SwiGLU is elementwise in i), so these give
# the rows of backward()'s results without evaluating the whole layer.

def expert_backward(x_bits: np.ndarray, weights: Dict[str, np.ndarray], idx: np.ndarray, g: np.ndarray,
                    dout_bits: np.ndarray, e: int, tokens: Optional[np.ndarray] = None, exact: bool = False):
    """The routes to expert e (of the given tokens, else of all): returns the
    token id of each route and ffn_backward of those rows, i.e. each route's
    dx contribution [n, D] and the weight gradients of e summed over exactly
    those routes.  idx [T, k] the selection, g [T, k] the gates."""
    r = _round(exact)
    idx = np.asarray(idx)
    pool = np.arange(idx.shape[0]) if tokens is None else np.asarray(tokens)
    ti, si = np.nonzero(idx[pool] == e)
    ti = pool[ti]
    dy = r(np.asarray(g)[ti, si][:, None] * _bf16.to_f64(dout_bits[ti]))
    b = ffn_backward(_bf16.to_f64(x_bits[ti]), dy, _bf16.to_f64(weights["w_gate"][e]),
                     _bf16.to_f64(weights["w_up"][e]), _bf16.to_f64(weights["w_down"][e]), exact)
    return ti, b


def logit_grad_rows(logits: np.ndarray, k: int, dout_bits: np.ndarray, Y: np.ndarray,
                    tokens: np.ndarray) -> np.ndarray:
    """dlogits rows [n, E] of the given tokens, from their stored routed rows
    Y [n, k, D] (the forward's rows, as moe.routed_outputs gives them)."""
    lg = np.asarray(logits)[tokens]
    sel = _moe.topk(lg, k)
    g = _moe.gates(lg, sel)
    dg = np.einsum("td,tkd->tk", _bf16.to_f64(dout_bits[tokens]), Y)
    out = np.zeros(lg.shape, dtype=np.float64)
    np.put_along_axis(out, sel.astype(np.int64), gate_logit_grad(g, dg), axis=1)
    return out


def token_dx(x_bits: np.ndarray, weights: Dict[str, np.ndarray], logits: np.ndarray, k: int,
             dout_bits: np.ndarray, tokens: np.ndarray, Y: np.ndarray, w_router_bits: np.ndarray,
             exact: bool = False, map_fn=map) -> np.ndarray:
    """Rows ``tokens`` of backward()'s dx [n, D]: the shared expert's share,
    every route's share, and the router's share r(dlogits) W_r.  Y [n, k, D]
    the tokens' stored routed rows; map_fn maps the per-expert evaluations
    (the builtin map, or a thread pool's)."""
    r = _round(exact)
    tokens = np.asarray(tokens)
    idx = _moe.topk(logits, k)
    g = _moe.gates(logits, idx)
    sh = ffn_backward(_bf16.to_f64(x_bits[tokens]), _bf16.to_f64(dout_bits[tokens]),
                      _bf16.to_f64(weights["ws_gate"]), _bf16.to_f64(weights["ws_up"]),
                      _bf16.to_f64(weights["ws_down"]), exact)
    dx = sh["dx"].copy()
    where = {int(t): n for n, t in enumerate(tokens)}
    experts = [int(e) for e in np.unique(idx[tokens])]
    for ti, b in map_fn(lambda e: expert_backward(x_bits, weights, idx, g, dout_bits, e, tokens, exact), experts):
        np.add.at(dx, [where[int(t)] for t in ti], b["dx"])
    dl = logit_grad_rows(logits, k, dout_bits, Y, tokens)
    return dx + r(dl) @ _bf16.to_f64(w_router_bits)


def shared_columns_backward(x_bits: np.ndarray, weights: Dict[str, np.ndarray], dout_bits: np.ndarray,
                            cols: np.ndarray, exact: bool = False) -> Dict[str, np.ndarray]:
    """Rows ``cols`` of dWs_gate and dWs_up and columns ``cols`` of dWs_down,
    over all tokens: the shared expert restricted to those intermediate
    columns."""
    cols = np.asarray(cols)
    b = ffn_backward(_bf16.to_f64(x_bits), _bf16.to_f64(dout_bits), _bf16.to_f64(weights["ws_gate"][cols]),
                     _bf16.to_f64(weights["ws_up"][cols]), _bf16.to_f64(weights["ws_down"][:, cols]), exact)
    return {"dWs_gate": b["dW_gate"], "dWs_up": b["dW_up"], "dWs_down": b["dW_down"]}


def router_weight_rows(x_bits: np.ndarray, logits: np.ndarray, k: int, dout_bits: np.ndarray, Y: np.ndarray,
                       tokens: np.ndarray, experts: np.ndarray, exact: bool = False) -> np.ndarray:
    """Rows ``experts`` of backward()'s dW_router [len(experts), D]; ``tokens``
    must hold every token that selects one of them (the other tokens' logit
    gradients are zero in those columns), Y [n, k, D] their routed rows."""
    r = _round(exact)
    tokens, experts = np.asarray(tokens), np.asarray(experts)
    every = np.nonzero(np.isin(_moe.topk(logits, k), experts).any(axis=1))[0]
    if not np.all(np.isin(every, tokens)):
        raise ValueError("tokens must include every token that selects the given experts")
    dl = r(logit_grad_rows(logits, k, dout_bits, Y, tokens))
    return dl[:, experts].T @ _bf16.to_f64(x_bits[tokens])
