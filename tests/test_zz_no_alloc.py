"""moe_schedule_static, the schedule entry point that allocates nothing,
against moe_schedule (the workspace entry point) through the C ABI: the
same tables bit for bit and the same device error bits, on calls in a row
that share the library's scratch array (each later call smaller than the
one before, so a stale entry from a larger call would show)."""

import numpy as np
import pytest
import torch

import synth
from mixture_experts_layer_counts_amd import MoELayer, shape_for
from mixture_experts_layer_counts_amd.api import schedule_static
from tests._gpu import need_gpu, say

pytestmark = pytest.mark.gpu

CASES = [  # name, R, N, k, E, c, L, routes
    ("ep64", 64, 4096, 8, 256, 0, 4, "ep"),       # 2,097,152 routes: 8 MiB of ordinals
    ("dsv3", 1, 8192, 8, 256, 0, 256, "topk"),
    ("ep8-zipf", 8, 700, 6, 64, 3, 8, "zipf"),
    ("tiny", 1, 64, 2, 8, 0, 8, "topk"),
]


def routes_for(name, R, N, k, E, c, L, kind):
    if kind == "ep":
        return synth.ep_share_routes(R, N, k, E, c, L, synth.zipf_counts(32768, L, 1.2), seed=3)
    if kind == "zipf":
        return synth.random_routes(R, N, k, E, seed=R + N, skew=1.2)
    return synth.random_routes(R, N, k, E, seed=N)


def test_schedule_static_matches_workspace_schedule():
    dev = need_gpu()
    for name, R, N, k, E, c, L, kind in CASES:
        A = torch.from_numpy(routes_for(name, R, N, k, E, c, L, kind)).to(dev)
        shape = shape_for(N, 128, 64, E, k, R=R, rank=c, max_rows=R * N * k)
        say("schedule_static", name, "R", R, "N", N, "k", k, "E", E, "c", c)
        want = MoELayer(shape, device=dev).schedule(A)
        err = torch.zeros(1, dtype=torch.int32, device=dev)
        got = schedule_static(shape, A, err)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        P = int(want["offsets"][-1].item())
        for n in ("counts", "offsets", "route_dst"):
            assert torch.equal(got[n], want[n]), (name, n)
        assert torch.equal(got["sched"][:P], want["sched"][:P]), name


def test_schedule_static_reports_device_errors():
    dev = need_gpu()
    A = synth.random_routes(1, 100, 2, 8, seed=1)
    A[0, 7] = 9  # an expert outside [0, E_total)
    shape = shape_for(100, 128, 64, 8, 2)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    schedule_static(shape, torch.from_numpy(A).to(dev), err)
    torch.cuda.synchronize()
    assert int(err.item()) & 0x1
