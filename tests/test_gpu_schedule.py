"""GPU parity of moe_schedule (Algorithm 1): every table bit-exact."""

import numpy as np
import pytest
import torch

import synth
from oracle import moe as ref
from tests._gpu import need_gpu, say

pytestmark = pytest.mark.gpu


def run_schedule(dev, A, T, k, E_total, R, c, max_rows=None):
    from mixture_experts_layer_counts_amd import MoELayer, shape_for
    L = E_total // R
    max_rows = T * k if (R == 1 or max_rows is None) else max_rows
    m = MoELayer(shape_for(T, 64, 64, E_total, k, I_shared=64, R=R, rank=c, max_rows=max_rows), device=dev)
    out = m.schedule(torch.from_numpy(np.ascontiguousarray(A, dtype=np.int32)).to(dev))
    torch.cuda.synchronize()
    return m, {n: t.cpu().numpy() for n, t in out.items()}


def check_tables(got, want, P):
    assert np.array_equal(got["counts"], want["counts"])
    assert np.array_equal(got["offsets"], want["offsets"])
    assert np.array_equal(got["sched"][:P], want["sched"])
    assert np.array_equal(got["route_dst"], want["route_dst"])


CASES = [  # name, R, N, k, E_total, c, skew
    ("tiny", 1, 64, 2, 8, 0, None),
    ("ragged", 1, 1001, 3, 24, 0, 1.2),
    ("dsv3-routes", 1, 8192, 8, 256, 0, None),
    ("skewed384", 1, 3000, 8, 384, 0, 1.2),
    ("e1024", 1, 700, 4, 1024, 0, None),
    ("ep4", 4, 500, 4, 32, 1, None),
    ("ep8-zipf", 8, 2100, 8, 64, 3, 1.2),
    ("ep64", 64, 300, 8, 256, 0, None),
]


@pytest.mark.parametrize("name,R,N,k,E,c,skew", CASES, ids=[c[0] for c in CASES])
def test_schedule_bit_exact(name, R, N, k, E, c, skew):
    dev = need_gpu()
    A = synth.random_routes(R, N, k, E, seed=len(name), skew=skew)
    want = ref.schedule(A, c, E // R)
    P = int(want["offsets"][-1])
    say("schedule", name, R, N, k, E, c, "P=", P)
    m, got = run_schedule(dev, A, N, k, E, R, c, max_rows=max(P, 1))
    check_tables(got, want, P)
    assert m.device_error() == 0


def test_schedule_from_topk_of_given_logits():
    dev = need_gpu()
    w = synth.workload("mid", routing="gaussian")
    l = synth.make_logits(w).numpy()
    A = ref.topk(l, w.k).reshape(1, -1)
    want = ref.schedule(A, 0, w.E)
    say("schedule_from_topk", w)
    _, got = run_schedule(dev, A, w.T, w.k, w.E, 1, 0)
    check_tables(got, want, w.T * w.k)


def test_schedule_empty_and_all_to_one():
    dev = need_gpu()
    A = np.zeros((1, 40 * 2), dtype=np.int32)
    A[0, 1::2] = 5  # two experts take everything, the rest are empty
    want = ref.schedule(A, 0, 8)
    say("schedule_all_to_two")
    _, got = run_schedule(dev, A, 40, 2, 8, 1, 0)
    check_tables(got, want, 80)
    # rank with no local route at all
    A2 = synth.random_routes(4, 50, 2, 16, seed=3)
    A2[A2 // 4 == 2] = 0
    want2 = ref.schedule(A2, 2, 4)
    assert want2["offsets"][-1] == 0
    _, got2 = run_schedule(dev, A2, 50, 2, 16, 4, 2, max_rows=1)
    check_tables(got2, want2, 0)


def test_schedule_expert_out_of_range_sets_error():
    dev = need_gpu()
    from mixture_experts_layer_counts_amd import _lib
    A = synth.random_routes(1, 100, 2, 8, seed=4)
    A[0, 17] = 8  # outside [0, E_total)
    A[0, 30] = -1
    say("schedule_out_of_range")
    m, got = run_schedule(dev, A, 100, 2, 8, 1, 0)
    assert m.device_error() & _lib.DEVERR_EXPERT_RANGE
    # the remaining routes are placed as the definition says for them alone
    keep = np.ones(A.shape[1], bool)
    keep[[17, 30]] = False
    valid = got["route_dst"][keep]
    assert np.all(valid >= 0) and np.all(got["route_dst"][~keep] == -1)


def test_schedule_row_overflow_sets_error_and_stays_in_bounds():
    dev = need_gpu()
    from mixture_experts_layer_counts_amd import _lib
    A = synth.random_routes(4, 100, 4, 16, seed=6)
    want = ref.schedule(A, 0, 4)
    P = int(want["offsets"][-1])
    say("schedule_overflow P=", P)
    m, got = run_schedule(dev, A, 100, 4, 16, 4, 0, max_rows=P // 2)
    assert m.device_error() & _lib.DEVERR_ROW_OVERFLOW
    rd = got["route_dst"]
    assert rd.max() < P // 2
    placed = rd >= 0
    assert np.array_equal(rd[placed], want["route_dst"][placed])
