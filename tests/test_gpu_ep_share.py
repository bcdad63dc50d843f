"""GPU parity of one rank's share under expert parallelism (R source ranks,
L local experts): moe_schedule on the routes of all R ranks, moe_forward on
the pooled source rows; the outbox rows (moe_routed_rows) and this rank's
output against the oracle's ep_share_forward.

The last case is the DeepSeek-V3 one-rank share at EP = 64 in the launch
configuration the benchmark times: 4 local experts (D=7168, I=2048)
receiving 32,768 routed rows with Zipf(1.2)-skewed counts, the shared expert
on the rank's 4,096 tokens, b = C = 32,768.  The oracle checks every region
and row-tile edge plus 512 seeded rows of the outbox, and 512 seeded local
tokens; ring mode (b = 4,096, C = 8,192) must give the same bits.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import moe as ref
from tests._gpu import mx_weights_dev, need_gpu, oracle_mx_weights, rel_err, say

pytestmark = pytest.mark.gpu


def rows_ok(got, want, tol):
    """Outbox rows are stored in bf16 on both sides, so besides the layer's
    budget (tol * RMS) a row element may differ by one bf16 rounding step
    where the fp32 and fp64 values straddle a rounding boundary: at most
    2^-7 |y| (8 significant bits)."""
    want = np.asarray(want, dtype=np.float64)
    rms = np.sqrt(np.mean(want ** 2))
    excess = np.abs(np.asarray(got, dtype=np.float64) - want) - (2.0 ** -7 * np.abs(want) + tol * rms)
    return float(excess.max()) <= 0.0


def local_gates(N, k, seed):
    g = torch.rand((N, k), generator=torch.Generator().manual_seed(seed), dtype=torch.float32) + 0.05
    return g / g.sum(dim=1, keepdim=True)


def run_share(w, inp_dev, A, c, R, L, g, b, C, max_rows, weights):
    from mixture_experts_layer_counts_amd import MoELayer, shape_for
    N = w.T // R
    precision = "mxfp8" if "q_gate" in weights else "bf16"
    m = MoELayer(shape_for(N, w.D, w.I, R * L, w.k, I_shared=w.I_shared, minibatch_rows=b, ring_rows=C,
                           precision=precision, R=R, rank=c, max_rows=max_rows), device=inp_dev["x"].device)
    sched = m.schedule(torch.from_numpy(A).to(inp_dev["x"].device))
    x_local = inp_dev["x"][c * N:(c + 1) * N]
    out, out32 = m.forward(weights, inp_dev["x"], x_local, g.to(inp_dev["x"].device), sched)
    torch.cuda.synchronize()
    assert m.device_error() == 0
    return m, sched, out, out32


def local_weights(inp, c, L):
    out = {n: inp[n] for n in ("ws_gate", "ws_up", "ws_down")}
    for n in ("w_gate", "w_up", "w_down"):
        out[n] = inp[n][c * L:(c + 1) * L].contiguous()
    return out


CASES = [  # name, R, N, k, L, c, D, I, Is, counts or None, [(b, C)], precision
    ("ep4", 4, 64, 4, 4, 1, 256, 128, 128, None, [(None, None), (64, 128)], "bf16"),
    ("ep8-zipf", 8, 100, 8, 4, 3, 384, 256, 128, [180, 90, 60, 40], [(None, None), (100, 300)], "bf16"),
    ("ep8-zipf-mx", 8, 100, 8, 4, 3, 384, 256, 128, [180, 90, 60, 40], [(None, None), (128, 256)], "mxfp8"),
    ("ep16-ragged", 16, 37, 6, 2, 15, 192, 192, 64, [101, 7], [(None, None), (50, 100)], "bf16"),
]


@pytest.mark.parametrize("name,R,N,k,L,c,D,I,Is,counts,bcs,prec", CASES, ids=[x[0] for x in CASES])
def test_ep_share_parity(name, R, N, k, L, c, D, I, Is, counts, bcs, prec):
    dev = need_gpu()
    E = R * L
    w = synth.Workload(name, T=R * N, D=D, I=I, E=E, k=k, I_shared=Is, seed=40 + R)
    inp = synth.make_inputs(w)
    if counts is None:
        A = synth.random_routes(R, N, k, E, seed=R)
    else:
        A = synth.ep_share_routes(R, N, k, E, c, L, counts, seed=R)
    g = local_gates(N, k, seed=R)
    host = {n: synth.bits(t) for n, t in inp.items() if t.dtype == torch.bfloat16}
    if prec == "mxfp8":
        wts = oracle_mx_weights({n: inp[n][c * L:(c + 1) * L] if n.startswith("w_") else inp[n] for n in inp})
    else:
        wts = {n: (host[n][c * L:(c + 1) * L] if n in ("w_gate", "w_up", "w_down") else host[n]) for n in host}
    want = ref.ep_share_forward(host["x"], wts, A, c, L, k, g.numpy().astype(np.float64), precision=prec)
    P = int(want["offsets"][-1])
    say("ep_share", name, "R", R, "N", N, "k", k, "L", L, "c", c, prec, "P =", P)
    inp_dev = {n: t.to(dev) for n, t in inp.items()}
    lw = local_weights(inp_dev, c, L)
    if prec == "mxfp8":
        lw = mx_weights_dev(lw)
    first = None
    tol = 1e-2 if prec == "bf16" else 5e-2
    for b, C in bcs:
        m, sched, out, out32 = run_share(w, inp_dev, A, c, R, L, g, b, C, P + 5, lw)
        assert np.array_equal(sched["offsets"].cpu().numpy(), want["offsets"])
        assert np.array_equal(sched["sched"].cpu().numpy()[:P], want["sched"])
        assert np.array_equal(sched["route_dst"].cpu().numpy(), want["route_dst"])
        rows = m.routed_rows()[:P].float().cpu().numpy()
        e_rows, e_out = rel_err(rows, want["rows"]), rel_err(out32.cpu().numpy(), want["out"])
        say("  b, C =", b, C, "rows max|err|/RMS =", e_rows, "out =", e_out)
        assert rows_ok(rows, want["rows"], tol) and e_out <= tol
        assert torch.equal(out.cpu().view(torch.int16), out32.cpu().to(torch.bfloat16).view(torch.int16))
        if first is None:
            first = (rows, out32.cpu())
        else:
            assert np.array_equal(first[0], rows) and torch.equal(first[1].view(torch.int32), out32.cpu().view(torch.int32))


def tile_edges(offsets, heights=(256, 320)):
    """First and last schedule position of every expert region and of every
    row tile in it, for the routed tile heights (a region of n rows is cut
    into ceil(n / BM) tiles of equal height, rounded up to 32 rows)."""
    pos = set()
    for a, b in zip(offsets[:-1], offsets[1:]):
        n = int(b - a)
        if n == 0:
            continue
        for bm in heights:
            tiles = -(-n // bm)
            h = -(-(-(-n // tiles)) // 32) * 32
            for i in range(tiles):
                lo, hi = a + i * h, min(a + (i + 1) * h, b)
                if lo < b:
                    pos.update((int(lo), int(hi) - 1))
    return pos


@pytest.mark.timeout(600)
def test_ep64_dsv3_share_every_edge():
    dev = need_gpu()
    R, N, k, L, c = 64, 4096, 8, 4, 0
    counts = synth.zipf_counts(32768, L, 1.2)
    w = synth.Workload("ep64", T=R * N, D=7168, I=2048, E=L, k=k, I_shared=2048, seed=50)
    say("ep64: drawing the 64-rank token pool (3.8 GB) and 4 local experts on the GPU")
    inp = synth.make_inputs(w, device="cuda")
    A = synth.ep_share_routes(R, N, k, R * L, c, L, counts, seed=50)
    g = local_gates(N, k, seed=50)
    P = sum(counts)
    say("ep64: b = C =", P)
    m, sched, out, out32 = run_share(w, inp, A, c, R, L, g, P, P, P, local_weights(inp, c, L))
    offsets = sched["offsets"].cpu().numpy()
    assert offsets.tolist() == [0] + np.cumsum(counts).tolist()
    rows_all = m.routed_rows()[:P].cpu().view(torch.int16).numpy()
    out32_all = out32.cpu().numpy()
    # ring mode: minibatches of 4,096 rows cycling an 8,192-row ring give the same bits
    say("ep64: ring mode, b = 4096, C = 8192")
    m2, sched2, out_2, out32_2 = run_share(w, inp, A, c, R, L, g, 4096, 8192, P, local_weights(inp, c, L))
    assert np.array_equal(m2.routed_rows()[:P].cpu().view(torch.int16).numpy(), rows_all)
    assert np.array_equal(out32_2.cpu().numpy().view(np.int32), out32_all.view(np.int32))
    del m2, out_2, out32_2
    # every region and tile edge, plus 512 seeded rows; 512 seeded local tokens
    rng = np.random.default_rng(50)
    pos = np.array(sorted(tile_edges(offsets) | set(rng.choice(P, 512, replace=False).tolist())))
    tok = np.sort(rng.choice(N, 512, replace=False))
    host_x = synth.bits(inp["x"])
    wts = {n: synth.bits(inp[n]) for n in ("w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")}
    say("ep64: oracle on", len(pos), "rows and", len(tok), "tokens")
    want = ref.ep_share_forward(host_x, wts, A, c, L, k, g.numpy().astype(np.float64), positions=pos, tokens=tok)
    assert np.array_equal(sched["sched"].cpu().numpy()[:P], want["sched"])
    assert np.array_equal(sched["route_dst"].cpu().numpy(), want["route_dst"])
    rows = torch.from_numpy(rows_all[pos]).view(torch.bfloat16).float().numpy()
    e_rows = rel_err(rows, want["rows"])
    e_out = rel_err(out32_all[tok], want["out"])
    say("ep64 rows max|err|/RMS =", e_rows, "over", len(pos), "rows; out =", e_out, "over", len(tok), "tokens")
    assert rows_ok(rows, want["rows"], 1e-2) and e_out <= 1e-2
    assert np.array_equal(out.cpu().view(torch.int16).numpy(),
                          torch.from_numpy(out32_all).to(torch.bfloat16).view(torch.int16).numpy())
    del inp, m
    torch.cuda.empty_cache()
