"""The MoE-layer forward pass, written out plainly in fp64 (numpy).

What is computed (MoK paper "Mixture-of-Kittens: MoE Megakernel for NVL72s",
§2.1, MoE equation; MoK blog repost, section "Overlapping computation and
communication in MoE"):

    MoE(x, s) = f_shared(x) + sum_{i in E} g_i f_i(x),   g_i = s_i / sum_{j in E} s_j
    f_i(x)    = W_down^(i) ( SiLU(W_gate^(i) x) * W_up^(i) x ),  SiLU(a) = a * sigmoid(a)

with E the k experts selected by the router projection (§2.1), and the
dispatch schedule of Algorithm 1 (§3.1) placing the routed rows in
expert-contiguous buffer positions.

Readings where the pages are silent (listed in the design doc):
* router scores s are the softmax of fp32 router logits over all experts; the
  selection is the k largest fp32 logits, ties to the lower expert id, with
  -0.0 equal to +0.0; slot s of token t is its s-th selection in that order and
  route j = t*k + s;
* the intermediate h is stored in bf16 (MX along I in MXFP8 mode) and each
  routed expert's output row is stored in bf16; the shared expert's output and
  the gate-weighted sum stay at full precision;
* in MXFP8 mode the routed experts see MX-quantised activations and weights
  (§3.4 "MXFP8 Support"); the shared expert and the router stay bf16.  The
  shared expert may be taken to MXFP8 too, as an option beside the pages'
  choice: then it sees MX-quantised x and weights and stores h in MX along
  I_shared, like a routed expert, and its output stays at full precision.
"""

from __future__ import annotations

from typing import Dict, Optional, Tuple

import numpy as np

from . import bf16 as _bf16
from . import mx as _mx


# ----------------------------------------------------------------------------
# Router projection, top-k selection and normalised gates (§2.1)
# ----------------------------------------------------------------------------

def router_logits(x_bits: np.ndarray, w_router_bits: np.ndarray) -> np.ndarray:
    """logits[t, e] = sum_d x[t, d] * W_r[e, d], in fp64 from the bf16 inputs."""
    return _bf16.to_f64(x_bits) @ _bf16.to_f64(w_router_bits).T


def topk(logits_f32: np.ndarray, k: int) -> np.ndarray:
    """The k selected experts of each token, in slot order.

    The decision is taken on the fp32 logits themselves.  Experts are ordered by
    (larger logit first, then lower id); -0.0 and +0.0 are the same logit.
    Returns int32 [T, k]: entry (t, s) is the expert in slot s of token t.
    """
    l = np.asarray(logits_f32, dtype=np.float32)
    if not np.all(np.isfinite(l)):
        raise ValueError("non-finite router logit")
    T, E = l.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    lv = l.astype(np.float64) + 0.0  # -0.0 + 0.0 == +0.0
    ids = np.broadcast_to(np.arange(E), (T, E))
    # lexsort sorts by the last key first: primary key -logit, secondary key id
    order = np.lexsort((ids, -lv), axis=-1)
    return order[:, :k].astype(np.int32)


def router_scores(logits_f32: np.ndarray) -> np.ndarray:
    """s = softmax of the logits over all experts (reading of "router weights")."""
    l = np.asarray(logits_f32, dtype=np.float64)
    z = np.exp(l - l.max(axis=-1, keepdims=True))
    return z / z.sum(axis=-1, keepdims=True)


def gates(logits_f32: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """g_i = s_i / sum_{j in E} s_j over the selected experts E (fp64, [T, k])."""
    s = router_scores(logits_f32)
    sel = np.take_along_axis(s, np.asarray(idx, dtype=np.int64), axis=-1)
    return sel / sel.sum(axis=-1, keepdims=True)


# ----------------------------------------------------------------------------
# Dispatch schedule (Algorithm 1, §3.1 "Scheduling")
# ----------------------------------------------------------------------------

def schedule(A: np.ndarray, c: int, L: int) -> Dict[str, np.ndarray]:
    """The dispatch schedule of the MoK paper, §3.1 "Scheduling".

    A [R, N*K]: A[r, j] is the global expert of route j on source rank r.
    c: this rank; local expert l is global expert c*L + l.

    The routes this rank receives are laid out expert by expert, each local
    expert's routes in one contiguous region.  Inside a region a route is
    keyed by its ordinal o (how many earlier routes of the same source rank
    went to the same expert) and then by its source rank r, so the ranks take
    turns.  The table is therefore the local routes sorted by the key
    (l, o, r); no two routes share a key.  Algorithm 1 of §3.1 computes the
    same positions in closed form; the tests check that form against this
    table.

    Returns
      M        [R, L]  routes per (source rank, local expert)
      counts   [L]     rows received per local expert (sum over r of M)
      offsets  [L+1]   start of each expert's region; offsets[L] = P
      sched    [P]     position p receives route (r, j), stored as r*N*K + j
      route_dst [R*N*K] position of each route on this rank, -1 if not local
    """
    A = np.asarray(A, dtype=np.int64)
    R, NK = A.shape
    local = (A >= c * L) & (A < c * L + L)
    r, j = np.nonzero(local)  # the local routes, by rank and then by route id
    l = A[r, j] - c * L
    M = np.zeros((R, L), dtype=np.int64)
    np.add.at(M, (r, l), 1)
    counts = M.sum(axis=0)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    # ordinal: the routes of one (rank, expert) pair, in route order, are 0, 1, 2, ...
    o = np.zeros(len(r), dtype=np.int64)
    for pair in np.unique(r * L + l):
        mine = np.nonzero(r * L + l == pair)[0]  # ascending route id j
        o[mine] = np.arange(len(mine))
    # the table: local routes sorted by (l, o, r)
    order = np.lexsort((r, o, l))
    sched = (r[order] * NK + j[order]).astype(np.int64)
    route_dst = np.full(R * NK, -1, dtype=np.int64)
    route_dst[sched] = np.arange(len(sched))
    return {"M": M, "counts": counts, "offsets": offsets, "sched": sched, "route_dst": route_dst}


# ----------------------------------------------------------------------------
# Expert feed-forward networks (§2.1; SiLU gate from the blog's notation)
# ----------------------------------------------------------------------------

def silu(a: np.ndarray) -> np.ndarray:
    return a / (1.0 + np.exp(-a))


def ffn(x: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray,
        h_store: str = "bf16", y_store: Optional[str] = "bf16") -> np.ndarray:
    """f(x) = W_down (SiLU(W_gate x) * W_up x) for rows x [n, D], fp64.

    w_gate, w_up: [I, D]; w_down: [D, I] (all fp64 values).  h is rounded the
    way it is stored ("bf16", "mx" along I, or None), and so is the output row
    ("bf16" or None).
    """
    a_g = x @ w_gate.T
    a_u = x @ w_up.T
    h = silu(a_g) * a_u
    if h_store == "bf16":
        h = _bf16.round_f64(h)
    elif h_store == "mx":
        h = _mx.round_f64(h)
    elif h_store is not None:
        raise ValueError(h_store)
    y = h @ w_down.T
    if y_store == "bf16":
        y = _bf16.round_f64(y)
    elif y_store is not None:
        raise ValueError(y_store)
    return y


def _expert_weights(weights: Dict[str, np.ndarray], e: int, precision: str):
    """fp64 values of expert e's weights as the routed FFN sees them."""
    if precision == "bf16":
        return (_bf16.to_f64(weights["w_gate"][e]), _bf16.to_f64(weights["w_up"][e]),
                _bf16.to_f64(weights["w_down"][e]))
    if precision == "mxfp8":
        return (_mx.dequantize(weights["q_gate"][e], weights["s_gate"][e]),
                _mx.dequantize(weights["q_up"][e], weights["s_up"][e]),
                _mx.dequantize(weights["q_down"][e], weights["s_down"][e]))
    raise ValueError(precision)


def routed_outputs(x_bits: np.ndarray, weights: Dict[str, np.ndarray], idx: np.ndarray,
                   precision: str = "bf16", tokens: Optional[np.ndarray] = None,
                   exact: bool = False, experts: Optional[np.ndarray] = None) -> np.ndarray:
    """Y[t, s] = f_{idx[t,s]}(x_t) for every route, fp64 [len(tokens), k, D].

    The routes of one expert are evaluated together (a matmul per expert); each
    route's row is independent of the others.  In MXFP8 mode x is MX-quantised
    along D before the projections (§3.4: activation quantisation in dispatch).
    ``exact`` skips the storage rounding of h and of the output rows.  With
    ``experts`` given, only the routes to those experts are evaluated and the
    other rows of Y stay zero (so that disjoint expert sets can be evaluated
    apart and their results added).
    """
    idx = np.asarray(idx, dtype=np.int64)
    tokens = np.arange(idx.shape[0]) if tokens is None else np.asarray(tokens)
    x = _bf16.to_f64(x_bits[tokens])
    if precision == "mxfp8":
        x = _mx.round_f64(x)
    sel = idx[tokens]
    n, k = sel.shape
    Y = np.zeros((n, k, x.shape[1]), dtype=np.float64)
    h_store = None if exact else ("bf16" if precision == "bf16" else "mx")
    y_store = None if exact else "bf16"
    keep = None if experts is None else {int(e) for e in experts}
    for e in np.unique(sel):
        if keep is not None and int(e) not in keep:
            continue
        ti, si = np.nonzero(sel == e)
        wg, wu, wd = _expert_weights(weights, int(e), precision)
        Y[ti, si] = ffn(x[ti], wg, wu, wd, h_store=h_store, y_store=y_store)
    return Y


def shared_output(x_bits: np.ndarray, weights: Dict[str, np.ndarray],
                  tokens: Optional[np.ndarray] = None, exact: bool = False,
                  precision: str = "bf16") -> np.ndarray:
    """f_shared(x) in fp64, output unrounded.  bf16: bf16 weights, h stored in
    bf16.  mxfp8: x MX-quantised along D, the MX weights "qs_*"/"ss_*"
    (row-major scales [N, K/32]) dequantised, h stored in MX along I_shared."""
    x = _bf16.to_f64(x_bits if tokens is None else x_bits[tokens])
    if precision == "bf16":
        return ffn(x, _bf16.to_f64(weights["ws_gate"]), _bf16.to_f64(weights["ws_up"]),
                   _bf16.to_f64(weights["ws_down"]), h_store=None if exact else "bf16", y_store=None)
    if precision == "mxfp8":
        return ffn(_mx.round_f64(x), _mx.dequantize(weights["qs_gate"], weights["ss_gate"]),
                   _mx.dequantize(weights["qs_up"], weights["ss_up"]),
                   _mx.dequantize(weights["qs_down"], weights["ss_down"]),
                   h_store=None if exact else "mx", y_store=None)
    raise ValueError(precision)


def combine(shared: np.ndarray, g: np.ndarray, Y: np.ndarray) -> np.ndarray:
    """MoE(x) = f_shared(x) + sum_s g_s * Y_s (the router-weighted sum)."""
    return shared + np.einsum("tk,tkd->td", g, Y)


def forward(x_bits: np.ndarray, weights: Dict[str, np.ndarray], logits_f32: np.ndarray, k: int,
            precision: str = "bf16", tokens: Optional[np.ndarray] = None,
            exact: bool = False, shared_precision: str = "bf16") -> Dict[str, np.ndarray]:
    """The whole layer for the given (or all) tokens from fp32 router logits.

    The selection and the gates are taken on the given fp32 logits (the same
    values the GPU path routes on).  Returns idx, gates, Y and out (fp64).
    ``exact`` evaluates the formula with no storage rounding of intermediates.
    """
    idx = topk(logits_f32, k)
    g = gates(logits_f32, idx)
    tok = np.arange(idx.shape[0]) if tokens is None else np.asarray(tokens)
    Y = routed_outputs(x_bits, weights, idx, precision, tok, exact=exact)
    sh = shared_output(x_bits, weights, tok, exact=exact, precision=shared_precision)
    return {"idx": idx, "gates": g, "Y": Y, "shared": sh, "out": combine(sh, g[tok], Y)}


# ----------------------------------------------------------------------------
# One rank's share under expert parallelism (§2.1, Fig. 2; §3.1)
# ----------------------------------------------------------------------------

def _expert_rows(x: np.ndarray, weights: Dict[str, np.ndarray], experts: np.ndarray,
                 precision: str) -> np.ndarray:
    """f_{experts[i]}(x[i]) for rows x (fp64, already MX-rounded in MXFP8
    mode), with h and the output row stored as the method stores them."""
    out = np.zeros_like(x)
    h_store = "bf16" if precision == "bf16" else "mx"
    for e in np.unique(experts):
        rows = np.nonzero(experts == e)[0]
        wg, wu, wd = _expert_weights(weights, int(e), precision)
        out[rows] = ffn(x[rows], wg, wu, wd, h_store=h_store, y_store="bf16")
    return out


def ep_share_forward(x_src_bits: np.ndarray, weights: Dict[str, np.ndarray], A: np.ndarray, c: int, L: int,
                     k: int, gates_local: np.ndarray, precision: str = "bf16",
                     positions: Optional[np.ndarray] = None,
                     tokens: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Rank c's part of the layer when the routed experts are spread over R
    ranks, L per rank (rank c holds global experts c*L .. c*L+L-1).

    x_src_bits [R*N, D]: token rows of every source rank (rank r's token t is
      row r*N + t); rank c's own tokens are rows c*N .. c*N+N-1.
    weights: rank c's experts, indexed by local expert l = global - c*L, and
      the shared expert.
    A [R, N*k]: the global expert of each route (route j of rank r is slot
      j % k of token j // k); gates_local [N, k]: the gates of rank c's tokens.

    Returns the schedule of the routes rank c receives (Algorithm 1) and
      rows [len(positions), D]: at schedule position p, the output of the route
        (r, j) it holds, f_{A[r,j]}(x_src[r*N + j//k]) stored in bf16: what
        rank c sends back to rank r, where route_dst read as a destination
        index places it (§3.1 table reuse);
      out [len(tokens), D]: for rank c's own token t, f_shared(x_t) plus the
        gate-weighted rows of its slots whose expert lives on rank c (the rows
        of the other slots are added where they arrive).
    """
    A = np.asarray(A, dtype=np.int64)
    R, NK = A.shape
    N = NK // k
    sch = schedule(A, c, L)
    P = int(sch["offsets"][-1])
    pos = np.arange(P) if positions is None else np.asarray(positions, dtype=np.int64)
    route = sch["sched"][pos]
    r, j = route // NK, route % NK
    x_rows = _bf16.to_f64(x_src_bits[r * N + j // k])
    if precision == "mxfp8":
        x_rows = _mx.round_f64(x_rows)
    rows = _expert_rows(x_rows, weights, A[r, j] - c * L, precision)

    tok = np.arange(N) if tokens is None else np.asarray(tokens, dtype=np.int64)
    x_local = x_src_bits[c * N:(c + 1) * N]
    sh = shared_output(x_local, weights, tok)
    sel = A[c].reshape(N, k)[tok]
    ti, si = np.nonzero((sel >= c * L) & (sel < c * L + L))
    xl = _bf16.to_f64(x_local[tok[ti]])
    if precision == "mxfp8":
        xl = _mx.round_f64(xl)
    Y = np.zeros((len(tok), k, x_src_bits.shape[1]), dtype=np.float64)
    Y[ti, si] = _expert_rows(xl, weights, sel[ti, si] - c * L, precision)
    out = combine(sh, np.asarray(gates_local, dtype=np.float64)[tok], Y)
    return {**sch, "positions": pos, "rows": rows, "out": out}


def layer_flops(T: int, D: int, I: int, k: int) -> float:
    """Expert-FFN FLOP of one forward, 6*T*(k+1)*D*I (§4.1)."""
    return 6.0 * T * (k + 1) * D * I


def quantize_weights_mx(weights: Dict[str, np.ndarray]) -> Dict[str, np.ndarray]:
    """MX-quantise the routed expert weights along their K axis (D for gate and
    up, I for down) from their bf16 values."""
    out = dict(weights)
    for name, q, s in (("w_gate", "q_gate", "s_gate"), ("w_up", "q_up", "s_up"),
                       ("w_down", "q_down", "s_down")):
        out[q], out[s] = _mx.quantize(_bf16.to_f64(weights[name]))
    return out


def quantize_shared_mx(weights: Dict[str, np.ndarray]) -> Dict[str, np.ndarray]:
    """MX-quantise the shared expert's weights along their K axis (D for gate
    and up, I_shared for down) from their bf16 values: "qs_*" codes and "ss_*"
    row-major scales [N, K/32]."""
    out = dict(weights)
    for name, q, s in (("ws_gate", "qs_gate", "ss_gate"), ("ws_up", "qs_up", "ss_up"),
                       ("ws_down", "qs_down", "ss_down")):
        out[q], out[s] = _mx.quantize(_bf16.to_f64(weights[name]))
    return out


def logit_bound(x_bits: np.ndarray, w_router_bits: np.ndarray) -> np.ndarray:
    """Bound on |fl32(logit) - logit| for any fp32 summation order.

    bf16 x bf16 products are exact in fp32, so only the D-1 additions round:
    |err| <= gamma_D * sum_d |x_d w_{e,d}| with gamma_D = D u / (1 - D u)
    (Higham, "Accuracy and Stability of Numerical Algorithms", §3.1), taken
    here with u = 2^-23 so that it also holds if the hardware adder truncates.
    """
    x = np.abs(_bf16.to_f64(x_bits))
    w = np.abs(_bf16.to_f64(w_router_bits))
    D = x.shape[1]
    u = 2.0 ** -23  # twice the round-to-nearest unit: also covers truncating adders
    return (D * u / (1 - D * u)) * (x @ w.T)
