"""ctypes view of libmoe.so (the C ABI declared in include/moe.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation of any step.
"""

from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "moe.h")

MOE_OK = 0
STATUS = {0: "MOE_OK", -1: "MOE_ERR_INVALID_ARG", -2: "MOE_ERR_UNSUPPORTED", -3: "MOE_ERR_WORKSPACE",
          -4: "MOE_ERR_HIP"}
MOE_BF16, MOE_MXFP8 = 0, 1
DEVERR_EXPERT_RANGE, DEVERR_ROW_OVERFLOW, DEVERR_NONFINITE, DEVERR_PIPELINE = 0x1, 0x2, 0x4, 0x8
KERNELS = {"router_gemm": 0, "topk": 1, "schedule": 2, "tiles": 3, "shared_up": 4, "shared_down": 5, "gather": 6,
           "up_gate": 7, "down": 8, "combine": 9, "pipeline": 10, "bwd_replay": 11, "bwd_dgrad": 12,
           "bwd_wgrad": 13}


class MoeShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "T", "D", "I", "I_shared", "E_total", "k", "num_src_ranks", "rank", "experts_per_rank",
        "tokens_per_src_rank", "max_rows", "minibatch_rows", "ring_rows")] + [
        ("precision", ctypes.c_int32), ("shared_precision", ctypes.c_int32), ("pipeline", ctypes.c_int32),
        ("mem_workgroups", ctypes.c_int32), ("weights_tiled", ctypes.c_int32)]


class MoeWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down", "ws_gate", "ws_up", "ws_down", "ss_gate", "ss_up",
        "ss_down")]


class MoeBwdWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w_gu", "w_gu_t", "w_down_t", "ws_gu", "ws_gu_t", "ws_down_t",
                                              "w_router_t")]


class MoeGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("dx", "dw_gate", "dw_up", "dw_down", "dws_gate", "dws_up", "dws_down",
                                              "dw_router")]


class MoeStreamProbeArgs(ctypes.Structure):
    _fields_ = [("act", ctypes.c_void_p), ("wts", ctypes.c_void_p), ("row_bytes", ctypes.c_int64),
                ("items", ctypes.c_int32), ("a_share", ctypes.c_int32), ("a_rows", ctypes.c_int32),
                ("b_rows", ctypes.c_int32), ("slots_a", ctypes.c_int32), ("slots_b", ctypes.c_int32)]


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}")
        self.status = status


_lib = None

_P = ctypes.c_void_p
_SIGS = {
    "moe_workspace_bytes": (ctypes.c_int, [ctypes.POINTER(MoeShape), ctypes.POINTER(ctypes.c_size_t)]),
    "moe_workspace_init": (ctypes.c_int, [ctypes.POINTER(MoeShape), _P, ctypes.c_size_t, _P]),
    "moe_route": (ctypes.c_int, [ctypes.POINTER(MoeShape), _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_schedule": (ctypes.c_int, [ctypes.POINTER(MoeShape), _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_schedule_static": (ctypes.c_int, [ctypes.POINTER(MoeShape), _P, _P, _P, _P, _P, _P, _P]),
    "moe_forward": (ctypes.c_int, [ctypes.POINTER(MoeShape), ctypes.POINTER(MoeWeights), _P, _P, _P, _P, _P, _P,
                                   _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_routed_rows": (ctypes.c_int, [ctypes.POINTER(MoeShape), _P, ctypes.c_size_t, ctypes.POINTER(_P),
                                       ctypes.POINTER(ctypes.c_int64)]),
    "moe_quantize_mxfp8": (ctypes.c_int, [_P, ctypes.c_int64, ctypes.c_int64, _P, _P, _P]),
    "moe_mxfp8_pack_scales": (ctypes.c_int, [_P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _P, _P]),
    "moe_tile_bf16": (ctypes.c_int, [_P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _P, _P]),
    "moe_get_device_error": (ctypes.c_int, [ctypes.POINTER(MoeShape), _P, ctypes.c_size_t, _P,
                                            ctypes.POINTER(ctypes.c_int32)]),
    "moe_backward_prepare": (ctypes.c_int, [ctypes.POINTER(MoeShape), ctypes.POINTER(MoeWeights), _P,
                                            ctypes.POINTER(MoeBwdWeights), _P]),
    "moe_backward_workspace_bytes": (ctypes.c_int, [ctypes.POINTER(MoeShape), ctypes.POINTER(ctypes.c_size_t)]),
    "moe_backward": (ctypes.c_int, [ctypes.POINTER(MoeShape), ctypes.POINTER(MoeBwdWeights), _P, _P, _P, _P, _P, _P,
                                    _P, _P, ctypes.POINTER(MoeGrads), _P, _P, ctypes.c_size_t, _P]),
    "moe_probe_begin": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32]),
    "moe_probe_end": (ctypes.c_int, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int32)]),
    "moe_stream_probe": (ctypes.c_int, [ctypes.POINTER(MoeStreamProbeArgs), _P]),
    "moe_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_abi_version": (ctypes.c_int32, []),
}


def header_functions(path: str = HEADER) -> list:
    """Names of the functions include/moe.h declares."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(moe_\w+)\s*\(", text, flags=re.M)))


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m mixture_experts_layer_counts_amd.build`"
                           " (the HIP library has no fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(fn: str, status: int) -> None:
    if status != MOE_OK:
        raise MoeError(fn, status)
