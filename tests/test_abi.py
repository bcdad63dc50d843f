"""The C ABI on the CPU: libmoe.so loads, exports every function include/moe.h
declares, and its host-side validation answers without touching a GPU."""

import ctypes
import os
import re

import pytest

from mixture_experts_layer_counts_amd import _lib, shape_for


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from mixture_experts_layer_counts_amd import build
        build.build()
    return _lib.load()


def test_exports_every_declared_function(lib):
    names = _lib.header_functions()
    assert {"moe_route", "moe_schedule", "moe_forward", "moe_workspace_bytes"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    # and the binding declares a signature for each
    assert set(names) == set(_lib._SIGS)


def test_abi_version_matches_header(lib):
    v = int(re.search(r"#define MOE_ABI_VERSION (\d+)", open(_lib.HEADER).read()).group(1))
    assert lib.moe_abi_version() == v


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4):
        assert lib.moe_status_str(code)
    assert lib.moe_status_str(-99) == b"unknown status"


def ws_bytes(lib, s):
    n = ctypes.c_size_t(0)
    st = lib.moe_workspace_bytes(ctypes.byref(s), ctypes.byref(n))
    return st, n.value


def test_workspace_sizes(lib):
    s = shape_for(T=8192, D=7168, I=2048, E=256, k=8, minibatch_rows=8192, ring_rows=8192)
    st, n = ws_bytes(lib, s)
    assert st == 0
    # at least ring + h + routed outputs + shared h + shared fp32 output
    need = 8192 * 7168 * 2 + 8192 * 2048 * 2 + 65536 * 7168 * 2 + 8192 * 2048 * 2 + 8192 * 7168 * 4
    assert need <= n < need * 1.05
    # a larger ring needs more
    s2 = shape_for(T=8192, D=7168, I=2048, E=256, k=8, minibatch_rows=8192, ring_rows=16384)
    assert ws_bytes(lib, s2)[1] > n


@pytest.mark.parametrize("field,value,code", [
    ("D", 100, -2),             # not a multiple of 64
    ("I", 96, -2),
    ("k", 0, -1),
    ({"k": 17, "max_rows": 64 * 17}, None, -2),  # more than 16 routes per token
    ("E_total", 2000, -1),      # R * L != E_total
    ("minibatch_rows", 0, -1),
    ("ring_rows", 1000, -1),    # not a multiple of b
    ("max_rows", 5, -1),        # R == 1 needs T*k
    ("precision", 7, -1),
    ("shared_precision", 7, -1),
    ("tokens_per_src_rank", 3, -1),
])
def test_invalid_shapes_are_rejected(lib, field, value, code):
    s = shape_for(T=64, D=128, I=64, E=32, k=2, minibatch_rows=32, ring_rows=64)
    assert ws_bytes(lib, s)[0] == 0
    for f, v in (field.items() if isinstance(field, dict) else [(field, value)]):
        setattr(s, f, v)
    assert ws_bytes(lib, s)[0] == code


def test_mxfp8_shapes(lib):
    # MX GEMM stages are 128 elements of K wide: D and I must be multiples of 128
    for D, I, code in ((128, 128, 0), (7168, 2048, 0), (128, 64, -2), (192, 128, -2)):
        s = shape_for(T=64, D=D, I=I, E=8, k=2, I_shared=64, precision="mxfp8")
        assert ws_bytes(lib, s)[0] == code
    # the MX ring and h are E4M3 bytes plus one scale byte per 32
    sb = shape_for(T=8192, D=7168, I=2048, E=384, k=8, minibatch_rows=65536, ring_rows=65536)
    sm = shape_for(T=8192, D=7168, I=2048, E=384, k=8, minibatch_rows=65536, ring_rows=65536, precision="mxfp8")
    saved = 65536 * 7168 * 2 - 65536 * (7168 + 224) + 65536 * 2048 * 2 - 65536 * (2048 + 64)
    assert abs((ws_bytes(lib, sb)[1] - ws_bytes(lib, sm)[1]) - saved) < 4096


def test_mxfp8_shared_shapes(lib):
    # the MX shared expert's GEMMs take 128-wide K stages over D and I_shared
    for D, Is, code in ((128, 128, 0), (7168, 2048, 0), (128, 64, -2), (192, 128, -2)):
        s = shape_for(T=64, D=D, I=64, E=8, k=2, I_shared=Is, shared_precision="mxfp8")
        assert ws_bytes(lib, s)[0] == code
    # its activations take E4M3 bytes plus stage-major scales in the workspace
    sb = shape_for(T=8192, D=7168, I=2048, E=384, k=8)
    sm = shape_for(T=8192, D=7168, I=2048, E=384, k=8, shared_precision="mxfp8")
    assert ws_bytes(lib, sm)[1] > ws_bytes(lib, sb)[1]


def test_mxfp8_shared_forward_needs_scales(lib):
    s = shape_for(T=64, D=128, I=128, E=8, k=2, I_shared=128, shared_precision="mxfp8")
    st, n = ws_bytes(lib, s)
    fake = ctypes.c_void_p(4096)  # never dereferenced: the call returns first
    w = _lib.MoeWeights()
    for f in ("w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down"):
        setattr(w, f, 4096)
    assert lib.moe_forward(ctypes.byref(s), ctypes.byref(w), fake, fake, fake, fake, fake, fake, fake, None, fake,
                           n, None) == -1


def test_mxfp8_forward_needs_scales(lib):
    s = shape_for(T=64, D=128, I=128, E=8, k=2, I_shared=64, precision="mxfp8")
    st, n = ws_bytes(lib, s)
    fake = ctypes.c_void_p(4096)  # never dereferenced: the call returns first
    w = _lib.MoeWeights()
    for f in ("w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down"):
        setattr(w, f, 4096)
    assert lib.moe_forward(ctypes.byref(s), ctypes.byref(w), fake, fake, fake, fake, fake, fake, fake, None, fake,
                           n, None) == -1


def test_calls_validate_before_launching(lib):
    s = shape_for(T=64, D=128, I=64, E=8, k=2)
    st, n = ws_bytes(lib, s)
    fake = ctypes.c_void_p(4096)  # never dereferenced: every call below returns first
    # workspace too small
    assert lib.moe_route(ctypes.byref(s), fake, fake, fake, fake, fake, fake, n - 1, None) == -3
    # misaligned workspace
    assert lib.moe_schedule(ctypes.byref(s), fake, fake, fake, fake, fake, ctypes.c_void_p(4097), n, None) == -1
    # null outputs
    assert lib.moe_route(ctypes.byref(s), fake, fake, None, fake, fake, fake, n, None) == -1
    w = _lib.MoeWeights()
    assert lib.moe_forward(ctypes.byref(s), ctypes.byref(w), fake, fake, fake, fake, fake, fake, fake, None, fake,
                           n, None) == -1
    # null shape
    assert lib.moe_workspace_bytes(None, ctypes.byref(ctypes.c_size_t())) == -1


def test_pack_scales_validates_before_launching(lib):
    a, b = ctypes.c_void_p(4096), ctypes.c_void_p(8192)  # never dereferenced
    assert lib.moe_mxfp8_pack_scales(a, 2, 8, 96, b, None) == -1      # K not a multiple of 128
    assert lib.moe_mxfp8_pack_scales(a, 2, 8, 128, a, None) == -1     # in place
    assert lib.moe_mxfp8_pack_scales(ctypes.c_void_p(4097), 2, 8, 128, b, None) == -1  # misaligned
    assert lib.moe_mxfp8_pack_scales(None, 2, 8, 128, b, None) == -1
    assert lib.moe_mxfp8_pack_scales(a, -1, 8, 128, b, None) == -1
    assert lib.moe_mxfp8_pack_scales(a, 0, 8, 128, b, None) == 0      # nothing to move: no launch


def test_tile_bf16_validates_before_launching(lib):
    a, b = ctypes.c_void_p(4096), ctypes.c_void_p(8192)  # never dereferenced
    assert lib.moe_tile_bf16(a, 2, 8, 96, b, None) == -1             # K not a multiple of 64
    assert lib.moe_tile_bf16(a, 2, 8, 128, a, None) == -1            # in place
    assert lib.moe_tile_bf16(ctypes.c_void_p(4104), 2, 8, 128, b, None) == -1  # misaligned
    assert lib.moe_tile_bf16(None, 2, 8, 128, b, None) == -1
    assert lib.moe_tile_bf16(a, 2, -1, 128, b, None) == -1
    assert lib.moe_tile_bf16(a, 0, 8, 128, b, None) == 0             # nothing to move: no launch


def test_tiled_weights_flag(lib):
    # the routed weights K-tiled (bf16 or E4M3); the backward prepares its
    # own copies from row-major weights
    assert ws_bytes(lib, shape_for(T=64, D=128, I=128, E=8, k=2, weights_tiled=True))[0] == 0
    bad = shape_for(T=64, D=128, I=128, E=8, k=2)
    bad.weights_tiled = 2
    assert ws_bytes(lib, bad)[0] == -1
    assert ws_bytes(lib, shape_for(T=64, D=128, I=128, E=8, k=2, precision="mxfp8", weights_tiled=True))[0] == 0
    n = ctypes.c_size_t()
    s = shape_for(T=64, D=128, I=128, E=8, k=2, weights_tiled=True)
    assert lib.moe_backward_workspace_bytes(ctypes.byref(s), ctypes.byref(n)) == -2


# Each case breaks exactly one buffer-resource limit of the GEMM operands
# (fewer than 2^31 bytes each) while every other operand stays small; the
# second set of sizes is the same shape brought just under that limit.
@pytest.mark.parametrize("name,kw,ok", [
    ("x T*D*2", dict(T=16384, D=65536, I=64, E=8, k=1, minibatch_rows=64, ring_rows=64), dict(T=16383)),
    ("ring C*D*2", dict(T=64, D=7168, I=64, E=8, k=2, minibatch_rows=150016, ring_rows=150016),
     dict(minibatch_rows=149760, ring_rows=149760)),
    ("h b*I*2", dict(T=64, D=64, I=65536, E=8, k=2, I_shared=64, minibatch_rows=16384, ring_rows=16384),
     dict(minibatch_rows=16320, ring_rows=16320)),
    ("shared h T*Is*2", dict(T=16384, D=64, I=64, E=8, k=1, I_shared=65536, minibatch_rows=64, ring_rows=64),
     dict(T=16383)),
    ("routed weights I*D*2", dict(T=64, D=32768, I=32768, E=8, k=2, I_shared=64, minibatch_rows=64, ring_rows=64),
     dict(I=32704)),
    ("shared weights Is*D*2", dict(T=64, D=32768, I=64, E=8, k=2, I_shared=32768, minibatch_rows=64,
                                   ring_rows=64), dict(I_shared=32704)),
])
def test_operand_byte_limits_are_refused_before_any_launch(lib, name, kw, ok):
    s = shape_for(**kw)
    assert ws_bytes(lib, s)[0] == -2, name
    fake = ctypes.c_void_p(4096)  # never dereferenced: every call below returns first
    w = _lib.MoeWeights()
    for f in ("w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down"):
        setattr(w, f, 4096)
    assert lib.moe_forward(ctypes.byref(s), ctypes.byref(w), fake, fake, fake, fake, fake, fake, fake, None, fake,
                           1 << 40, None) == -2, name
    assert lib.moe_route(ctypes.byref(s), fake, fake, fake, fake, fake, fake, 1 << 40, None) == -2, name
    assert lib.moe_schedule(ctypes.byref(s), fake, fake, fake, fake, fake, fake, 1 << 40, None) == -2, name
    assert ws_bytes(lib, shape_for(**{**kw, **ok}))[0] == 0, name


def test_mxfp8_operands_are_one_byte_per_element(lib):
    # the MX ring holds E4M3 bytes: a ring that is too large in bf16 fits in MXFP8
    kw = dict(T=64, D=7168, I=128, E=8, k=2, I_shared=128, minibatch_rows=150016, ring_rows=150016)
    assert ws_bytes(lib, shape_for(**kw))[0] == -2
    assert ws_bytes(lib, shape_for(**kw, precision="mxfp8"))[0] == 0


def test_schedule_static_validates_before_any_device_work(lib):
    fake = ctypes.c_void_p(4096)  # never dereferenced: every call below returns first
    s = shape_for(T=64, D=128, I=64, E=8, k=2)
    # a null error word or null outputs
    assert lib.moe_schedule_static(ctypes.byref(s), fake, fake, fake, fake, fake, None, None) == -1
    assert lib.moe_schedule_static(ctypes.byref(s), fake, None, fake, fake, fake, fake, None) == -1
    # a bad shape
    bad = shape_for(T=64, D=128, I=64, E=8, k=2)
    bad.k = 0
    assert lib.moe_schedule_static(ctypes.byref(bad), fake, fake, fake, fake, fake, fake, None) == -1
    # more scratch than the library's fixed array holds: 4 bytes per route
    # alone exceed it past 4 Mi routes
    big = shape_for(T=16384, D=128, I=64, E=256, k=8, R=64, max_rows=65536)
    assert 64 * 16384 * 8 * 4 > (16 << 20)
    assert lib.moe_schedule_static(ctypes.byref(big), fake, fake, fake, fake, fake, fake, None) == -2


def test_pipeline_shape_fields(lib):
    # the persistent routed kernel: memory workgroups in multiples of 8, bf16 routed experts only
    ok = shape_for(T=64, D=128, I=64, E=8, k=2, minibatch_rows=32, ring_rows=64, pipeline=True, mem_workgroups=8)
    assert ws_bytes(lib, ok)[0] == 0
    assert ws_bytes(lib, shape_for(T=64, D=128, I=64, E=8, k=2, pipeline=True, mem_workgroups=12))[0] == -1
    assert ws_bytes(lib, shape_for(T=64, D=128, I=64, E=8, k=2, pipeline=True, mem_workgroups=-8))[0] == -1
    bad = shape_for(T=64, D=128, I=64, E=8, k=2)
    bad.pipeline = 2
    assert ws_bytes(lib, bad)[0] == -1
    assert ws_bytes(lib, shape_for(T=64, D=128, I=128, E=8, k=2, I_shared=128, precision="mxfp8",
                                   pipeline=True))[0] == -2
    # it keeps H = C/b (2 .. 4) h buffers and per-minibatch counters in the workspace
    plain = shape_for(T=64, D=128, I=64, E=8, k=2, minibatch_rows=32, ring_rows=64)
    assert ws_bytes(lib, ok)[1] >= ws_bytes(lib, plain)[1] + 32 * 64 * 2 + 3 * 4 * 4
    for C, H in ((32, 2), (96, 3), (128, 4), (256, 4)):
        deep = shape_for(T=64, D=128, I=64, E=8, k=2, minibatch_rows=32, ring_rows=C, pipeline=True,
                         mem_workgroups=8)
        flat = shape_for(T=64, D=128, I=64, E=8, k=2, minibatch_rows=32, ring_rows=C)
        assert ws_bytes(lib, deep)[1] >= ws_bytes(lib, flat)[1] + (H - 1) * 32 * 64 * 2 + 3 * 4 * 4, C


def test_backward_validates_before_any_launch(lib):
    s = shape_for(T=64, D=128, I=64, E=8, k=2)
    n = ctypes.c_size_t(0)
    assert lib.moe_backward_workspace_bytes(ctypes.byref(s), ctypes.byref(n)) == 0 and n.value > 0
    # the backward is for one GPU's bf16 layer: R > 1 and MXFP8 are refused
    ep = shape_for(T=64, D=128, I=64, E=16, k=2, R=2, rank=0, max_rows=256)
    mx = shape_for(T=64, D=128, I=128, E=8, k=2, I_shared=128, precision="mxfp8")
    for bad in (ep, mx):
        assert lib.moe_backward_workspace_bytes(ctypes.byref(bad), ctypes.byref(ctypes.c_size_t())) == -2
    # the transposed routed rows, D x (T k + 64 E) bf16, past 2^31 bytes at a
    # shape whose forward operands all fit (the ring: 2,146,959,360 bytes)
    big = shape_for(T=18720, D=7168, I=2048, E=256, k=8)
    assert ws_bytes(lib, big)[0] == 0
    assert lib.moe_backward_workspace_bytes(ctypes.byref(big), ctypes.byref(ctypes.c_size_t())) == -2
    fake = ctypes.c_void_p(4096)  # never dereferenced: every call below returns first
    bw = _lib.MoeBwdWeights(*([fake.value] * len(_lib.MoeBwdWeights._fields_)))
    g = _lib.MoeGrads(*([fake.value] * len(_lib.MoeGrads._fields_)))

    def call(x=fake, y=fake, dout=fake, ws=fake, nbytes=n.value, grads=g, weights=bw):
        return lib.moe_backward(ctypes.byref(s), ctypes.byref(weights), x, fake, fake, fake, fake, fake, y, dout,
                                ctypes.byref(grads), fake, ws, nbytes, None)

    assert call(nbytes=n.value - 1) == -3                        # workspace too small
    assert call(ws=ctypes.c_void_p(4096 + 64)) == -1              # workspace not 256-byte aligned
    for kw in ("x", "y", "dout"):                                 # rows read in 16-byte pieces
        assert call(**{kw: ctypes.c_void_p(4096 + 8)}) == -1, kw
        assert call(**{kw: None}) == -1, kw
    assert call(grads=_lib.MoeGrads()) == -1                      # null gradient outputs
    assert call(weights=_lib.MoeBwdWeights()) == -1               # weights not prepared
    w = _lib.MoeWeights()
    assert lib.moe_backward_prepare(ctypes.byref(s), ctypes.byref(w), fake, ctypes.byref(bw), None) == -1


def test_stream_probe_validates_before_any_launch(lib):
    # the measurement probe answers unsupported or invalid arguments on the host
    def call(**kw):
        f = dict(act=4096, wts=4096, row_bytes=7168, items=64, a_share=16, a_rows=256, b_rows=256, slots_a=2,
                 slots_b=3)
        f.update(kw)
        a = _lib.MoeStreamProbeArgs(f["act"], f["wts"], f["row_bytes"], f["items"], f["a_share"], f["a_rows"],
                                    f["b_rows"], f["slots_a"], f["slots_b"])
        return lib.moe_stream_probe(ctypes.byref(a), None)

    assert lib.moe_stream_probe(None, None) == -1
    assert call(row_bytes=7000) == -1          # not a multiple of 128
    assert call(items=0) == -1
    assert call(a_share=0) == -1
    assert call(act=None) == -1                # activation rows asked, no buffer
    assert call(wts=None) == -1
    assert call(slots_b=4) == -2               # the MXFP8 stage runs 2 + 3 or 2 + 2 slots
    assert call(a_rows=128) == -2
    assert call(a_rows=0, b_rows=256, slots_a=6, slots_b=6) == -2
    assert call(row_bytes=128 << 20) == -2     # one item's rows past 2^31 bytes
