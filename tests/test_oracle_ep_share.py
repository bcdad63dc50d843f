"""Pins of the oracle's expert-parallel share (one rank of R).

* With R = 1 the share is the whole layer: equal to the oracle's forward.
* With R > 1 the rows every rank returns, placed by the owner's route_dst
  (the schedule table read as {dst_rank, dst_index}, MoK paper §3.1) and
  summed with the gates, rebuild the whole layer over all R*N tokens and all
  R*L experts: the oracle's forward.
* With every route of a rank on another rank, its own output is the shared
  expert alone.
"""

import numpy as np
import torch

import synth
from oracle import moe


def setup(R, N, D, I, L, k, seed, Is=32):
    E = R * L
    w = synth.Workload("ep", T=R * N, D=D, I=I, E=E, k=k, I_shared=Is, seed=seed, routing="gaussian")
    inp = synth.make_inputs(w)
    host = {n: synth.bits(t) for n, t in inp.items() if t.dtype == torch.bfloat16}
    logits = inp["logits"].numpy()
    idx = moe.topk(logits, k)
    g = moe.gates(logits, idx)
    return w, host, logits, idx.reshape(R, N * k), g


def rank_weights(host, c, L):
    out = {n: host[n] for n in ("ws_gate", "ws_up", "ws_down")}
    for n in ("w_gate", "w_up", "w_down"):
        out[n] = host[n][c * L:(c + 1) * L]
    return out


def test_single_rank_share_is_the_layer():
    w, host, logits, A, g = setup(R=1, N=40, D=64, I=32, L=6, k=2, seed=1)
    share = moe.ep_share_forward(host["x"], host, A, 0, 6, 2, g)
    full = moe.forward(host["x"], host, logits, 2)
    assert np.allclose(share["out"], full["out"], rtol=0, atol=1e-12)
    # R = 1: the outbox row at position p is the route sched[p]'s output
    Y = full["Y"].reshape(-1, w.D)
    assert np.allclose(share["rows"], Y[share["sched"]], rtol=0, atol=1e-12)


def test_rank_shares_rebuild_the_layer():
    R, N, L, k = 4, 12, 2, 3
    w, host, logits, A, g = setup(R=R, N=N, D=64, I=32, L=L, k=k, seed=2)
    full = moe.forward(host["x"], host, logits, k)
    shares = [moe.ep_share_forward(host["x"], rank_weights(host, c, L), A, c, L, k, g[c * N:(c + 1) * N])
              for c in range(R)]
    NK = N * k
    for c in range(R):
        xb = host["x"][c * N:(c + 1) * N]
        sh = moe.shared_output(xb, host)
        rebuilt = sh.copy()
        for t in range(N):
            for s in range(k):
                e = int(A[c, t * k + s])
                owner = e // L
                p = int(shares[owner]["route_dst"][c * NK + t * k + s])
                assert p >= 0
                rebuilt[t] += g[c * N + t, s] * shares[owner]["rows"][p]
        assert np.allclose(rebuilt, full["out"][c * N:(c + 1) * N], rtol=0, atol=1e-12)
        # a rank's own out holds exactly its locally served slots
        local_part = sh.copy()
        for t in range(N):
            for s in range(k):
                e = int(A[c, t * k + s])
                if e // L == c:
                    local_part[t] += g[c * N + t, s] * shares[c]["rows"][int(shares[c]["route_dst"][c * NK + t * k + s])]
        assert np.allclose(shares[c]["out"], local_part, rtol=0, atol=1e-12)


def test_rank_with_no_local_route_outputs_the_shared_expert():
    R, N, L, k = 2, 10, 3, 2
    w, host, logits, A, g = setup(R=R, N=N, D=64, I=32, L=L, k=k, seed=3)
    A = A.copy()
    A[0] = np.where(A[0] < L, A[0] + L, A[0])  # rank 0's routes all go to rank 1 (duplicates are fine here)
    share = moe.ep_share_forward(host["x"], rank_weights(host, 0, L), A, 0, L, k, g[:N])
    assert np.array_equal(share["out"], moe.shared_output(host["x"][:N], host))


def test_positions_and_tokens_subsets():
    R, N, L, k = 3, 16, 2, 2
    w, host, logits, A, g = setup(R=R, N=N, D=64, I=32, L=L, k=k, seed=4)
    wts = rank_weights(host, 1, L)
    full = moe.ep_share_forward(host["x"], wts, A, 1, L, k, g[N:2 * N])
    pos = np.array([0, 3, len(full["sched"]) - 1])
    tok = np.array([2, 7, 15])
    sub = moe.ep_share_forward(host["x"], wts, A, 1, L, k, g[N:2 * N], positions=pos, tokens=tok)
    assert np.allclose(sub["rows"], full["rows"][pos], rtol=0, atol=1e-12)
    assert np.allclose(sub["out"], full["out"][tok], rtol=0, atol=1e-12)
