"""Pins of the oracle's dispatch schedule (MoK paper §3.1, "Scheduling").

The oracle builds the table as the definition of §3.1 states it: the local
routes sorted by (local expert, per-rank ordinal, source rank).  Algorithm 1
of the same section gives each position in closed form instead; the first
test derives that form by counting and checks the table against it.  On top
of that: library routines (bincount, stable argsort) and the properties the
table must have (a bijection onto expert-contiguous regions, source ranks
interleaved round-robin inside a region).
"""

import numpy as np
import pytest

import synth
from oracle import moe


def random_routes(R, N, K, E_total, seed, skew=None):
    return synth.random_routes(R, N, K, E_total, seed, skew).astype(np.int64)


CASES = [  # R, N, K, L, c, E_total, skew
    (1, 50, 2, 8, 0, 8, None),
    (1, 200, 8, 16, 0, 16, 1.2),
    (4, 30, 3, 5, 2, 20, None),
    (8, 40, 4, 4, 0, 32, 1.2),
    (3, 25, 2, 6, 1, 18, 2.0),
]


def closed_form_position(A, c, L, r, j):
    """Where route j of source rank r lands, counted directly.

    In the region of its local expert l the route follows every route with a
    smaller ordinal (each rank r' contributes min(M[r', l], o) of those) and
    the routes with the same ordinal from lower ranks (each rank r' < r that
    sent more than o routes to l contributes one).  That count, plus the
    region start, is the closed form of Algorithm 1 (MoK paper §3.1).
    """
    l = int(A[r, j]) - c * L
    o = int(np.count_nonzero(A[r, :j] == A[r, j]))
    M_l = np.array([np.count_nonzero(A[q] == c * L + l) for q in range(A.shape[0])])
    start = sum(np.count_nonzero(A == c * L + e) for e in range(l))
    return start + int(np.minimum(M_l, o).sum()) + int(np.count_nonzero(M_l[:r] > o))


@pytest.mark.parametrize("R,N,K,L,c,E_total,skew", CASES)
def test_table_matches_closed_form(R, N, K, L, c, E_total, skew):
    A = random_routes(R, N, K, E_total, seed=R * 100 + N, skew=skew)
    s = moe.schedule(A, c, L)
    for r in range(R):
        for j in range(N * K):
            if c * L <= A[r, j] < (c + 1) * L:
                p = closed_form_position(A, c, L, r, j)
                assert s["sched"][p] == r * N * K + j
                assert s["route_dst"][r * N * K + j] == p


@pytest.mark.parametrize("R,N,K,L,c,E_total,skew", CASES)
def test_table_properties(R, N, K, L, c, E_total, skew):
    A = random_routes(R, N, K, E_total, seed=R * 7 + N, skew=skew)
    s = moe.schedule(A, c, L)
    M, counts, S, sched, dst = s["M"], s["counts"], s["offsets"], s["sched"], s["route_dst"]
    local = (A >= c * L) & (A < (c + 1) * L)
    # counts are per-(rank, expert) histograms
    for r in range(R):
        assert np.array_equal(M[r], np.bincount(A[r][local[r]] - c * L, minlength=L))
    assert np.array_equal(S, np.concatenate([[0], np.cumsum(counts)]))
    # bijection between local routes and positions; route_dst is the inverse
    flat_local = np.nonzero(local.reshape(-1))[0]
    assert np.array_equal(np.sort(sched), flat_local)
    assert np.array_equal(dst[sched], np.arange(S[-1]))
    assert np.all(dst[~local.reshape(-1)] == -1)
    # expert-contiguous regions of the right length
    expert_of = A.reshape(-1)[sched] - c * L
    for l in range(L):
        assert np.all(expert_of[S[l]:S[l + 1]] == l)
    # within a region: per source rank, routes keep their original order, and
    # the first min_r M[r, l] rounds cycle through the ranks round-robin
    for l in range(L):
        reg = sched[S[l]:S[l + 1]]
        ranks, js = reg // (N * K), reg % (N * K)
        for r in range(R):
            assert np.all(np.diff(js[ranks == r]) > 0)
        present = [r for r in range(R) if M[r, l] > 0]
        rounds = min(M[r, l] for r in present) if present else 0
        head = ranks[: rounds * len(present)]
        assert np.array_equal(head, np.tile(present, rounds))


def test_single_rank_is_stable_counting_sort():
    A = random_routes(1, 300, 8, 32, seed=11, skew=1.2)
    s = moe.schedule(A, 0, 32)
    assert np.array_equal(s["sched"], np.argsort(A[0], kind="stable"))


def test_empty_experts_and_all_to_one():
    A = np.zeros((1, 40), dtype=np.int64)  # every route to expert 0
    s = moe.schedule(A, 0, 4)
    assert list(s["counts"]) == [40, 0, 0, 0]
    assert list(s["offsets"]) == [0, 40, 40, 40, 40]
    assert np.array_equal(s["sched"], np.arange(40))
    # no local route at all
    s2 = moe.schedule(A + 8, 0, 4)
    assert s2["offsets"][-1] == 0 and s2["sched"].size == 0 and np.all(s2["route_dst"] == -1)


def test_ep_share_generator_counts():
    counts = synth.zipf_counts(600, 4, 1.2)
    assert sum(counts) == 600 and counts == sorted(counts, reverse=True)
    A = synth.ep_share_routes(R=8, N=100, k=4, E_total=32, rank=0, L=4, counts=counts, seed=1)
    s = moe.schedule(A, 0, 4)
    assert list(s["counts"]) == counts
    # each token holds distinct experts
    tok = A.reshape(8, 100, 4)
    assert all(len(set(tok[r, t])) == 4 for r in range(8) for t in range(100))
