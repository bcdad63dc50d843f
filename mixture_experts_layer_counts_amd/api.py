"""Thin torch binding of libmoe.so: argument checks and marshalling only.

Torch supplies device memory and the current HIP stream; the C calls do all
of the work.  Names follow include/moe.h: ``route``, ``schedule``,
``forward``, ``quantize_mxfp8`` and ``pack_mxfp8_scales``.
"""

from __future__ import annotations

import ctypes
from typing import Dict, Optional, Tuple

import torch

from . import _lib


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _need(t: torch.Tensor, name: str, dtype, shape, device: torch.device) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def shape_for(T: int, D: int, I: int, E: int, k: int, I_shared: Optional[int] = None,
              minibatch_rows: Optional[int] = None, ring_rows: Optional[int] = None,
              precision: str = "bf16", R: int = 1, rank: int = 0, max_rows: Optional[int] = None,
              shared_precision: str = "bf16", pipeline: bool = False, mem_workgroups: int = 0,
              weights_tiled: bool = False) -> _lib.MoeShape:
    """A moe_shape for one GPU (R = 1) or for rank ``rank`` of R source ranks.
    ``precision`` is that of the routed experts, ``shared_precision`` that of
    the shared expert (bf16 unless MXFP8 is asked for).  ``pipeline`` runs the
    routed minibatch loop as one persistent kernel, ``mem_workgroups`` of
    whose workgroups gather the minibatches the ring does not hold at once.
    ``weights_tiled``: the routed bf16 weights come K-tiled (``tile_bf16``)."""
    L = E // R
    max_rows = T * k if max_rows is None else max_rows
    b = minibatch_rows or max(max_rows, 1)
    C = ring_rows or b
    s = _lib.MoeShape()
    s.T, s.D, s.I, s.I_shared, s.E_total, s.k = T, D, I, I if I_shared is None else I_shared, E, k
    s.num_src_ranks, s.rank, s.experts_per_rank, s.tokens_per_src_rank = R, rank, L, T
    s.max_rows, s.minibatch_rows, s.ring_rows = max_rows, b, C
    s.precision = {"bf16": _lib.MOE_BF16, "mxfp8": _lib.MOE_MXFP8}[precision]
    s.shared_precision = {"bf16": _lib.MOE_BF16, "mxfp8": _lib.MOE_MXFP8}[shared_precision]
    s.pipeline, s.mem_workgroups = int(bool(pipeline)), mem_workgroups
    s.weights_tiled = int(bool(weights_tiled))
    return s


class MoELayer:
    """One layer's shape plus its device workspace, on ``device``."""

    def __init__(self, shape: _lib.MoeShape, device="cuda"):
        self.lib = _lib.load()
        self.shape = shape
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        nbytes = ctypes.c_size_t(0)
        _lib.check("moe_workspace_bytes", self.lib.moe_workspace_bytes(ctypes.byref(shape), ctypes.byref(nbytes)))
        self.ws_bytes = nbytes.value
        # the caching allocator hands out 512-byte aligned blocks
        self.ws = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device=self.device)
        _lib.check("moe_workspace_init",
                   self.lib.moe_workspace_init(ctypes.byref(shape), _ptr(self.ws), self.ws_bytes, _stream()))

    # -- sizes -------------------------------------------------------------
    @property
    def T(self):
        return self.shape.T

    @property
    def k(self):
        return self.shape.k

    # -- moe_route ---------------------------------------------------------
    def route(self, x: Optional[torch.Tensor], w_router: Optional[torch.Tensor],
              logits: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
        s, dev = self.shape, self.device
        if x is None:
            if logits is None:
                raise ValueError("given-logits mode needs logits")
            _need(logits, "logits", torch.float32, (s.T, s.E_total), dev)
        else:
            _need(x, "x", torch.bfloat16, (s.T, s.D), dev)
            _need(w_router, "w_router", torch.bfloat16, (s.E_total, s.D), dev)
            logits = torch.empty((s.T, s.E_total), dtype=torch.float32, device=dev)
        idx = torch.empty((s.T, s.k), dtype=torch.int32, device=dev)
        gate = torch.empty((s.T, s.k), dtype=torch.float32, device=dev)
        _lib.check("moe_route", self.lib.moe_route(ctypes.byref(s), _ptr(x), _ptr(w_router), _ptr(logits),
                                                   _ptr(idx), _ptr(gate), _ptr(self.ws), self.ws_bytes, _stream()))
        return logits, idx, gate

    # -- moe_schedule ------------------------------------------------------
    def schedule(self, routes: torch.Tensor) -> Dict[str, torch.Tensor]:
        s, dev = self.shape, self.device
        NK = s.T * s.k
        routes = routes.reshape(s.num_src_ranks, NK)
        _need(routes, "routes", torch.int32, (s.num_src_ranks, NK), dev)
        L = s.experts_per_rank
        out = {
            "counts": torch.empty(L, dtype=torch.int32, device=dev),
            "offsets": torch.empty(L + 1, dtype=torch.int32, device=dev),
            "sched": torch.empty((max(s.max_rows, 1),), dtype=torch.int32, device=dev),
            "route_dst": torch.empty(s.num_src_ranks * NK, dtype=torch.int32, device=dev),
        }
        _lib.check("moe_schedule", self.lib.moe_schedule(
            ctypes.byref(s), _ptr(routes), _ptr(out["counts"]), _ptr(out["offsets"]), _ptr(out["sched"]),
            _ptr(out["route_dst"]), _ptr(self.ws), self.ws_bytes, _stream()))
        return out

    # -- moe_forward -------------------------------------------------------
    def forward(self, weights: Dict[str, torch.Tensor], x_src: torch.Tensor, x_local: torch.Tensor,
                gate: torch.Tensor, sched: Dict[str, torch.Tensor], out32: bool = True,
                out: Optional[torch.Tensor] = None, out_f32: Optional[torch.Tensor] = None):
        s, dev = self.shape, self.device
        L, D, I, Is = s.experts_per_rank, s.D, s.I, s.I_shared
        _need(x_local, "x_local", torch.bfloat16, (s.T, D), dev)
        _need(x_src, "x_src", torch.bfloat16, (s.num_src_ranks * s.T, D), dev)
        _need(gate, "gate", torch.float32, (s.T, s.k), dev)
        w = _lib.MoeWeights()
        if s.precision == _lib.MOE_BF16:
            for n, (N, K) in (("w_gate", (I, D)), ("w_up", (I, D)), ("w_down", (D, I))):
                # row-major [L, N, K], or K-tiled [L, K/64, N, 64] (tile_bf16)
                _need(weights[n], n, torch.bfloat16, (L, K // 64, N, 64) if s.weights_tiled else (L, N, K), dev)
                setattr(w, n, _ptr(weights[n]))
        else:
            for n, qn, sn, shp in (("w_gate", "q_gate", "s_gate", (L, I, D)), ("w_up", "q_up", "s_up", (L, I, D)),
                                   ("w_down", "q_down", "s_down", (L, D, I))):
                # row-major [L, N, K] bytes, or K-tiled [L, K/128, N, 128] (tile_mxfp8)
                _need(weights[qn], qn, torch.uint8,
                      (L, shp[2] // 128, shp[1], 128) if s.weights_tiled else shp, dev)
                _need(weights[sn], sn, torch.uint8, (L, shp[2] // 128, shp[1], 4), dev)
                setattr(w, n, _ptr(weights[qn]))
                setattr(w, sn, _ptr(weights[sn]))
        if s.shared_precision == _lib.MOE_BF16:
            for n, shp in (("ws_gate", (Is, D)), ("ws_up", (Is, D)), ("ws_down", (D, Is))):
                _need(weights[n], n, torch.bfloat16, shp, dev)
                setattr(w, n, _ptr(weights[n]))
        else:  # E4M3 bytes "qs_*" and packed scales "ss_*" (quantize_mxfp8, pack_mxfp8_scales)
            for n, qn, sn, shp in (("ws_gate", "qs_gate", "ss_gate", (Is, D)), ("ws_up", "qs_up", "ss_up", (Is, D)),
                                   ("ws_down", "qs_down", "ss_down", (D, Is))):
                _need(weights[qn], qn, torch.uint8, shp, dev)
                _need(weights[sn], sn, torch.uint8, (shp[1] // 128, shp[0], 4), dev)
                setattr(w, n, _ptr(weights[qn]))
                setattr(w, sn, _ptr(weights[sn]))
        if out is None:
            out = torch.empty((s.T, D), dtype=torch.bfloat16, device=dev)
        _need(out, "out", torch.bfloat16, (s.T, D), dev)
        if out32 and out_f32 is None:
            out_f32 = torch.empty((s.T, D), dtype=torch.float32, device=dev)
        if out_f32 is not None:
            _need(out_f32, "out32", torch.float32, (s.T, D), dev)
        _lib.check("moe_forward", self.lib.moe_forward(
            ctypes.byref(s), ctypes.byref(w), _ptr(x_src), _ptr(x_local), _ptr(gate), _ptr(sched["offsets"]),
            _ptr(sched["sched"]), _ptr(sched["route_dst"]), _ptr(out), _ptr(out_f32), _ptr(self.ws), self.ws_bytes,
            _stream()))
        return out, out_f32

    # -- whole layer -------------------------------------------------------
    def __call__(self, x: torch.Tensor, w_router: Optional[torch.Tensor], weights: Dict[str, torch.Tensor],
                 logits: Optional[torch.Tensor] = None):
        """route + schedule + forward for R = 1 (from x, or from given logits)."""
        lg, idx, gate = self.route(None if logits is not None else x, w_router, logits)
        sched = self.schedule(idx)
        out, out32 = self.forward(weights, x, x, gate, sched)
        return {"logits": lg, "idx": idx, "gate": gate, "out": out, "out32": out32, **sched}

    def routed_rows(self) -> torch.Tensor:
        """The routed output rows moe_forward left in the workspace (a view,
        bf16 [n, D]): by route t*k+s when R == 1, by schedule position when R > 1."""
        addr, n = ctypes.c_void_p(), ctypes.c_int64()
        _lib.check("moe_routed_rows", self.lib.moe_routed_rows(ctypes.byref(self.shape), _ptr(self.ws), self.ws_bytes,
                                                               ctypes.byref(addr), ctypes.byref(n)))
        off, D = addr.value - self.ws.data_ptr(), self.shape.D
        return self.ws[off:off + n.value * D * 2].view(torch.bfloat16).view(n.value, D)

    def device_error(self) -> int:
        code = ctypes.c_int32(0)
        _lib.check("moe_get_device_error", self.lib.moe_get_device_error(
            ctypes.byref(self.shape), _ptr(self.ws), self.ws_bytes, _stream(), ctypes.byref(code)))
        return code.value


def schedule_static(shape: _lib.MoeShape, routes: torch.Tensor, dev_error: torch.Tensor) -> Dict[str, torch.Tensor]:
    """moe_schedule_static: the schedule of ``routes`` [R, N*k] int32 with no
    workspace (the library's fixed scratch array); device error bits are
    OR-ed into ``dev_error`` (one int32 on the same device)."""
    lib = _lib.load()
    dev = routes.device
    NK = shape.T * shape.k
    routes = routes.reshape(shape.num_src_ranks, NK)
    _need(routes, "routes", torch.int32, (shape.num_src_ranks, NK), dev)
    _need(dev_error, "dev_error", torch.int32, (1,), dev)
    L = shape.experts_per_rank
    out = {
        "counts": torch.empty(L, dtype=torch.int32, device=dev),
        "offsets": torch.empty(L + 1, dtype=torch.int32, device=dev),
        "sched": torch.empty((max(shape.max_rows, 1),), dtype=torch.int32, device=dev),
        "route_dst": torch.empty(shape.num_src_ranks * NK, dtype=torch.int32, device=dev),
    }
    _lib.check("moe_schedule_static", lib.moe_schedule_static(
        ctypes.byref(shape), _ptr(routes), _ptr(out["counts"]), _ptr(out["offsets"]), _ptr(out["sched"]),
        _ptr(out["route_dst"]), _ptr(dev_error), _stream()))
    return out


def _weights_struct(shape: _lib.MoeShape, weights: Dict[str, torch.Tensor], dev) -> _lib.MoeWeights:
    L, D, I, Is = shape.experts_per_rank, shape.D, shape.I, shape.I_shared
    w = _lib.MoeWeights()
    for n, shp in (("w_gate", (L, I, D)), ("w_up", (L, I, D)), ("w_down", (L, D, I)), ("ws_gate", (Is, D)),
                   ("ws_up", (Is, D)), ("ws_down", (D, Is))):
        _need(weights[n], n, torch.bfloat16, shp, dev)
        setattr(w, n, _ptr(weights[n]))
    return w


def prepare_backward(shape: _lib.MoeShape, weights: Dict[str, torch.Tensor], w_router: torch.Tensor
                     ) -> Dict[str, torch.Tensor]:
    """The weights rearranged for moe_backward (moe_backward_prepare), once per
    weight set: w_gu, w_gu_t, w_down_t, ws_gu, ws_gu_t, ws_down_t, w_router_t."""
    lib = _lib.load()
    dev = w_router.device
    L, D, I, Is, E = shape.experts_per_rank, shape.D, shape.I, shape.I_shared, shape.E_total
    Ep = (E + 63) // 64 * 64
    w = _weights_struct(shape, weights, dev)
    _need(w_router, "w_router", torch.bfloat16, (E, D), dev)
    out = {"w_gu": (L, 2 * I, D), "w_gu_t": (L, D, 2 * I), "w_down_t": (L, I, D), "ws_gu": (2 * Is, D),
           "ws_gu_t": (D, 2 * Is), "ws_down_t": (Is, D), "w_router_t": (D, Ep)}
    out = {n: torch.empty(shp, dtype=torch.bfloat16, device=dev) for n, shp in out.items()}
    bw = _lib.MoeBwdWeights(*[_ptr(out[n]) for n, _ in _lib.MoeBwdWeights._fields_])
    _lib.check("moe_backward_prepare", lib.moe_backward_prepare(ctypes.byref(shape), ctypes.byref(w), _ptr(w_router),
                                                                ctypes.byref(bw), _stream()))
    return out


class MoEBackward:
    """The workspace of moe_backward for one layer shape, on ``device``."""

    def __init__(self, shape: _lib.MoeShape, device="cuda"):
        self.lib = _lib.load()
        self.shape = shape
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        nbytes = ctypes.c_size_t(0)
        _lib.check("moe_backward_workspace_bytes",
                   self.lib.moe_backward_workspace_bytes(ctypes.byref(shape), ctypes.byref(nbytes)))
        self.ws_bytes = nbytes.value
        self.ws = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device=self.device)
        self.err = torch.zeros(1, dtype=torch.int32, device=self.device)

    def __call__(self, bw: Dict[str, torch.Tensor], x: torch.Tensor, idx: torch.Tensor, gate: torch.Tensor,
                 sched: Dict[str, torch.Tensor], y_routes: torch.Tensor, dout: torch.Tensor,
                 grads: Optional[Dict[str, torch.Tensor]] = None) -> Dict[str, torch.Tensor]:
        s, dev = self.shape, self.device
        T, D, I, Is, E, k, L = s.T, s.D, s.I, s.I_shared, s.E_total, s.k, s.experts_per_rank
        _need(x, "x", torch.bfloat16, (T, D), dev)
        _need(dout, "dout", torch.bfloat16, (T, D), dev)
        _need(idx, "idx", torch.int32, (T, k), dev)
        _need(gate, "gate", torch.float32, (T, k), dev)
        _need(y_routes, "y_routes", torch.bfloat16, (T * k, D), dev)
        shapes = {"dx": ((T, D), torch.float32), "dw_gate": ((L, I, D), torch.bfloat16),
                  "dw_up": ((L, I, D), torch.bfloat16), "dw_down": ((L, D, I), torch.bfloat16),
                  "dws_gate": ((Is, D), torch.bfloat16), "dws_up": ((Is, D), torch.bfloat16),
                  "dws_down": ((D, Is), torch.bfloat16), "dw_router": ((E, D), torch.float32)}
        if grads is None:
            grads = {n: torch.empty(shp, dtype=dt, device=dev) for n, (shp, dt) in shapes.items()}
        for n, (shp, dt) in shapes.items():
            _need(grads[n], n, dt, shp, dev)
        g = _lib.MoeGrads(*[_ptr(grads[n]) for n, _ in _lib.MoeGrads._fields_])
        b = _lib.MoeBwdWeights(*[_ptr(bw[n]) for n, _ in _lib.MoeBwdWeights._fields_])
        _lib.check("moe_backward", self.lib.moe_backward(
            ctypes.byref(s), ctypes.byref(b), _ptr(x), _ptr(idx), _ptr(gate), _ptr(sched["offsets"]),
            _ptr(sched["sched"]), _ptr(sched["route_dst"]), _ptr(y_routes), _ptr(dout), ctypes.byref(g),
            _ptr(self.err), _ptr(self.ws), self.ws_bytes, _stream()))
        return grads

    def device_error(self) -> int:
        torch.cuda.current_stream().synchronize()
        return int(self.err.item())


def quantize_mxfp8(src: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """MX-quantise a bf16 tensor along its last axis (moe_quantize_mxfp8)."""
    lib = _lib.load()
    if src.dtype != torch.bfloat16 or not src.is_contiguous() or src.device.type != "cuda":
        raise ValueError("src must be a contiguous bf16 device tensor")
    K = src.shape[-1]
    rows = src.numel() // max(K, 1)
    q = torch.empty(src.shape, dtype=torch.uint8, device=src.device)
    sc = torch.empty(src.shape[:-1] + (K // 32,), dtype=torch.uint8, device=src.device)
    _lib.check("moe_quantize_mxfp8", lib.moe_quantize_mxfp8(_ptr(src), rows, K, _ptr(q), _ptr(sc), _stream()))
    return q, sc


def tile_bf16(w: torch.Tensor) -> torch.Tensor:
    """Row-major bf16 matrices [G, N, K] -> the K-tiled [G, K/64, N, 64]
    that ``forward`` reads with ``weights_tiled`` (moe_tile_bf16)."""
    lib = _lib.load()
    if w.dtype != torch.bfloat16 or not w.is_contiguous() or w.device.type != "cuda" or w.dim() != 3:
        raise ValueError("w must be a contiguous bf16 [G, N, K] device tensor")
    G, N, K = w.shape
    if K % 64:
        raise ValueError("K must be a multiple of 64")
    out = torch.empty((G, K // 64, N, 64), dtype=torch.bfloat16, device=w.device)
    _lib.check("moe_tile_bf16", lib.moe_tile_bf16(_ptr(w), G, N, K, _ptr(out), _stream()))
    return out


def tile_mxfp8(q: torch.Tensor) -> torch.Tensor:
    """Row-major E4M3 bytes [G, N, K] -> the K-tiled [G, K/128, N, 128] that
    ``forward`` reads with ``weights_tiled`` (moe_tile_bf16 on the bytes taken
    as 2-byte units)."""
    if q.dtype != torch.uint8 or not q.is_contiguous() or q.dim() != 3 or q.shape[2] % 128:
        raise ValueError("q must be contiguous uint8 [G, N, K] with K a multiple of 128")
    G, N, K = q.shape
    return tile_bf16(q.view(torch.bfloat16)).view(torch.uint8).view(G, K // 128, N, 128)


def pack_mxfp8_scales(scale: torch.Tensor) -> torch.Tensor:
    """Row-major MX scales [G, N, K/32] -> the stage-major [G, K/128, N, 4]
    that ``forward`` reads (moe_mxfp8_pack_scales)."""
    lib = _lib.load()
    if scale.dtype != torch.uint8 or not scale.is_contiguous() or scale.device.type != "cuda" or scale.dim() != 3:
        raise ValueError("scale must be a contiguous uint8 [G, N, K/32] device tensor")
    G, N, KS = scale.shape
    if KS % 4:
        raise ValueError("K must be a multiple of 128")
    packed = torch.empty((G, KS // 4, N, 4), dtype=torch.uint8, device=scale.device)
    _lib.check("moe_mxfp8_pack_scales", lib.moe_mxfp8_pack_scales(_ptr(scale), G, N, KS * 32, _ptr(packed),
                                                                  _stream()))
    return packed
