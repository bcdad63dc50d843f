"""Seeded synthetic inputs for the MoE-layer forward.

This module is shared by the tests, the benchmark and the smoke check, and it is
the only thing the GPU path and the CPU oracle have in common.  It holds random
draws and the bf16 storage rounding of those draws, and none of the layer's own
arithmetic (no projection, selection, schedule, activation or reduction).

Recipe (also stated in the design doc):

* every tensor is drawn in fp32 from its own ``torch.Generator`` whose seed is
  derived from (workload seed, tensor name, expert index), so a tensor does not
  depend on which other tensors were drawn or in which order;
* ``x ~ N(0, 1)``; every weight ``~ N(0, 1/fan_in)`` (std ``1/sqrt(fan_in)``,
  fan_in = D for the router, gate and up projections, I for the down
  projection), then rounded to bf16 with round-to-nearest-even;
* "gaussian" logits (the routing the benchmark uses when it starts from logits,
  as in Mixture-of-Kittens §4.1: router logits drawn from a standard normal)
  are N(0, 1) fp32; "zipf" logits are ``log((e+1)^-s) + Gumbel(0, 1)``, whose
  top-k is a draw of k experts without replacement with Zipf(s) weights.

Small workloads are drawn on the CPU; large ones may be drawn directly on a GPU
(``device="cuda"``), in which case the oracle gets host copies of the very same
bits.  The two devices give different streams for the same seed, so the device
is part of the recipe.
"""

from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Dict, Optional

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    """Sizes of one MoE layer on one GPU (notation of Mixture-of-Kittens §2.1).

    T tokens of width D; E routed experts with intermediate width I, top-k;
    one shared expert with intermediate width I_shared.
    """

    name: str
    T: int
    D: int
    I: int
    E: int
    k: int
    I_shared: int
    seed: int
    routing: str = "x"  # "x": logits from the router projection; "gaussian"/"zipf": given logits
    zipf_s: float = 1.2

    @property
    def P(self) -> int:
        """Routed rows (every token is sent to k experts)."""
        return self.T * self.k

    def flops(self) -> float:
        """Expert-FFN FLOP of the forward pass, 6·T·(k+1)·D·I (Mixture-of-Kittens §4.1)."""
        return 6.0 * self.T * (self.k + 1) * self.D * self.I


WORKLOADS: Dict[str, Workload] = {
    # T=64, D=128, I=64, 8 routed experts, top-2, one shared expert (I=64).
    "tiny": Workload("tiny", T=64, D=128, I=64, E=8, k=2, I_shared=64, seed=0),
    # T=4096, D=2048, I=768, 128 routed experts, top-8, one shared expert.
    "mid": Workload("mid", T=4096, D=2048, I=768, E=128, k=8, I_shared=768, seed=1),
    # DeepSeek-V3 layer shape with all 256 experts on one GPU.
    "dsv3": Workload("dsv3", T=8192, D=7168, I=2048, E=256, k=8, I_shared=2048, seed=2),
    # Kimi-K2.7 shape (384 experts) used for the MXFP8 variant.
    "mx": Workload("mx", T=8192, D=7168, I=2048, E=384, k=8, I_shared=2048, seed=4),
}


def workload(name: str, **overrides) -> Workload:
    base = WORKLOADS[name]
    return dataclasses.replace(base, **overrides) if overrides else base


def _seed(base: int, *parts) -> int:
    h = hashlib.sha256(repr((base,) + parts).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device: str, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal_bf16(shape, std: float, device: str, seed: int) -> torch.Tensor:
    t = torch.randn(shape, generator=_gen(device, seed), device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(torch.bfloat16)


def make_inputs(w: Workload, device: str = "cpu", with_weights: bool = True) -> Dict[str, torch.Tensor]:
    """Draw every input of one layer forward on ``device``.

    Returns bf16 tensors ``x [T,D]``, ``w_router [E,D]``, ``w_gate``/``w_up
    [E,I,D]``, ``w_down [E,D,I]``, ``ws_gate``/``ws_up [I_s,D]``, ``ws_down
    [D,I_s]`` and, when ``w.routing`` is not "x", fp32 ``logits [T,E]``.
    Expert weights are drawn expert by expert so that the fp32 staging buffer
    stays one expert large.
    """
    T, D, I, E, Is = w.T, w.D, w.I, w.E, w.I_shared
    out: Dict[str, torch.Tensor] = {}
    out["x"] = _normal_bf16((T, D), 1.0, device, _seed(w.seed, "x"))
    out["w_router"] = _normal_bf16((E, D), 1.0 / math.sqrt(D), device, _seed(w.seed, "w_router"))
    if with_weights:
        for name, shape, fan_in in (("w_gate", (I, D), D), ("w_up", (I, D), D), ("w_down", (D, I), I)):
            buf = torch.empty((E,) + shape, dtype=torch.bfloat16, device=device)
            for e in range(E):
                buf[e] = _normal_bf16(shape, 1.0 / math.sqrt(fan_in), device, _seed(w.seed, name, e))
            out[name] = buf
        out["ws_gate"] = _normal_bf16((Is, D), 1.0 / math.sqrt(D), device, _seed(w.seed, "ws_gate"))
        out["ws_up"] = _normal_bf16((Is, D), 1.0 / math.sqrt(D), device, _seed(w.seed, "ws_up"))
        out["ws_down"] = _normal_bf16((D, Is), 1.0 / math.sqrt(Is), device, _seed(w.seed, "ws_down"))
    if w.routing != "x":
        out["logits"] = make_logits(w, device)
    return out


def make_logits(w: Workload, device: str = "cpu", kind: Optional[str] = None) -> torch.Tensor:
    """fp32 router logits [T, E] for runs that start from given logits."""
    kind = kind or (w.routing if w.routing != "x" else "gaussian")
    g = _gen(device, _seed(w.seed, "logits", kind))
    if kind == "gaussian":
        return torch.randn((w.T, w.E), generator=g, device=device, dtype=torch.float32)
    if kind == "zipf":
        u = torch.rand((w.T, w.E), generator=g, device=device, dtype=torch.float64)
        u = u.clamp_(min=1e-300)
        gumbel = -torch.log(-torch.log(u))
        ranks = torch.arange(1, w.E + 1, device=device, dtype=torch.float64)
        return (-w.zipf_s * torch.log(ranks) + gumbel).to(torch.float32)
    raise ValueError(f"unknown logits kind {kind!r}")


def bits(t: torch.Tensor) -> np.ndarray:
    """Host copy of a bf16 tensor's bit patterns as uint16 (what the oracle takes)."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_f32(t: torch.Tensor) -> np.ndarray:
    assert t.dtype == torch.float32
    return t.detach().contiguous().cpu().numpy()


def ties_logits(T: int, E: int, seed: int, levels: int = 3) -> torch.Tensor:
    """Logits drawn from a few values only (with +0.0 and -0.0 among them), so
    that many experts tie; used to test the tie rule of the top-k selection."""
    g = _gen("cpu", _seed(seed, "ties"))
    vals = torch.tensor([0.0, -0.0, 1.5, -2.0, 0.25][: max(2, levels)], dtype=torch.float32)
    idx = torch.randint(0, vals.numel(), (T, E), generator=g)
    return vals[idx]


def ep_share_routes(R: int, N: int, k: int, E_total: int, rank: int, L: int,
                    counts, seed: int) -> np.ndarray:
    """Route matrix A [R, N*k] (global expert ids) for one rank's share under
    expert parallelism, with prescribed numbers of routes to each local expert.

    For each local expert l, ``counts[l]`` distinct (source rank, token) pairs
    are drawn without replacement, and l is put in a free slot of that token;
    every other slot holds a distinct non-local expert.  Only the random layout
    is drawn here; the schedule is built by the code under test.
    """
    rng = np.random.default_rng(_seed(seed, "ep_routes"))
    local = np.arange(rank * L, rank * L + L)
    nonlocal_ids = np.setdiff1d(np.arange(E_total), local)
    A = np.full((R, N, k), -1, dtype=np.int64)
    for l, n_l in enumerate(counts):
        free = np.nonzero((A < 0).sum(axis=2).reshape(-1) > 0)[0]
        pick = rng.choice(free, size=int(n_l), replace=False)
        for flat in pick:
            r, t = divmod(int(flat), N)
            slots = np.nonzero(A[r, t] < 0)[0]
            A[r, t, rng.choice(slots)] = local[l]
    for r in range(R):
        for t in range(N):
            row = A[r, t]
            holes = np.nonzero(row < 0)[0]
            if holes.size:
                row[holes] = rng.choice(nonlocal_ids, size=holes.size, replace=False)
    return A.reshape(R, N * k).astype(np.int32)


def zipf_counts(total: int, L: int, s: float) -> list:
    """Largest-remainder split of ``total`` rows over L experts with weights (l+1)^-s."""
    w = np.array([(l + 1) ** (-s) for l in range(L)])
    q = total * w / w.sum()
    base = np.floor(q).astype(int)
    rem = total - base.sum()
    order = np.argsort(-(q - base), kind="stable")
    base[order[:rem]] += 1
    return base.tolist()


def random_routes(R: int, N: int, K: int, E_total: int, seed: int, skew: Optional[float] = None) -> np.ndarray:
    """Route matrix A [R, N*K]: each token draws K distinct experts, uniformly
    or with Zipf(skew) weights (expert e has weight (e+1)^-skew)."""
    rng = np.random.default_rng(_seed(seed, "routes", R, N, K, E_total, skew))
    p = None
    if skew is not None:
        p = np.arange(1, E_total + 1, dtype=np.float64) ** (-skew)
        p /= p.sum()
    A = np.empty((R, N * K), dtype=np.int32)
    for r in range(R):
        for t in range(N):
            A[r, t * K:(t + 1) * K] = rng.choice(E_total, size=K, replace=False, p=p)
    return A
