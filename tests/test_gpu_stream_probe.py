"""The operand-stream probe (moe_stream_probe) runs through the C ABI at each
supported ring configuration on small buffers and leaves device memory as it
was: it only moves rows into LDS."""

import ctypes

import pytest
import torch

from mixture_experts_layer_counts_amd import _lib
from tests._gpu import need_gpu, say

pytestmark = pytest.mark.gpu

CONFIGS = [(320, 256, 2, 2), (320, 0, 2, 2), (256, 256, 2, 3), (256, 0, 2, 3), (256, 256, 2, 2), (0, 256, 2, 3)] + \
          [(0, 256, n, n) for n in (2, 3, 4, 5)]


@pytest.mark.parametrize("a_rows,b_rows,sa,sb", CONFIGS)
def test_stream_probe_runs(a_rows, b_rows, sa, sb):
    dev = need_gpu()
    say("stream_probe", a_rows, b_rows, sa, sb)
    lib = _lib.load()
    items, share, row_bytes = 37, 16, 1152  # a ragged last XCD run and block; 9 stages
    blocks = (items + share - 1) // share
    g = torch.Generator(device=dev).manual_seed(3)
    act = torch.randint(0, 256, (max(blocks * a_rows * row_bytes, 1),), dtype=torch.uint8, device=dev, generator=g)
    wts = torch.randint(0, 256, (max(items * b_rows * row_bytes, 1),), dtype=torch.uint8, device=dev, generator=g)
    act0, wts0 = act.clone(), wts.clone()
    a = _lib.MoeStreamProbeArgs(act.data_ptr(), wts.data_ptr(), row_bytes, items, share, a_rows, b_rows, sa, sb)
    st = lib.moe_stream_probe(ctypes.byref(a), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, _lib.STATUS.get(st, st)
    torch.cuda.synchronize()
    assert torch.equal(act, act0) and torch.equal(wts, wts0)
