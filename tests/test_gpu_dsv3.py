"""Parity at the full DeepSeek-V3 layer shape (T=8192, D=7168, I=2048, 256
experts, top-8, shared I=2048), in the launch configuration bench.py times
(one minibatch of all 65,536 routed rows, ring of the same size), and in ring
mode (minibatches of 2,048 rows cycling a 4,096-row ring).

* routing and schedule from given fp32 logits: bit-exact over all tokens;
* the full path from x, over all tokens:
  - router logits within the fp32 summation bound of the fp64 logits;
  - the selection equal to the oracle's top-k of the GPU's own fp32 logits
    (identical fp32 logits must give identical indices), and the gates
    within the fp32 gate bound of the oracle's;
  - the schedule tables equal to the oracle's for that selection;
  - bf16 output = RNE(out32);
* the layer output against the oracle, fed the same fp32 logits, on a sample
  of over 512 tokens that together route to every one of the 256 experts and
  include the first and last row of every expert's region;
* ring mode: bitwise equal to the single-minibatch run;
* the persistent routed kernel at b = 512, 2,048 and 8,192 (rings of four
  minibatches): bitwise equal to the single-minibatch run;
* the backward (moe_backward after the forward from x, seeded N(0,1) bf16
  output gradient) against the backward oracle's sampled pieces: dx of 16
  seeded tokens, every weight gradient of four experts (the first, the last,
  the most and the least loaded), eight intermediate columns of the shared
  expert's weight gradients over all tokens, and the router-weight gradient
  row of the least loaded expert (all tokens that select it), under the
  bounds of the smaller backward cases.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import moe as ref
from tests._gpu import (DeviceExperts, bf16_grad_ok, cover_tokens, fetch_bf16, gate_tolerance, layer, need_gpu,
                        oracle_routed_pooled, rel_err, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsv3():
    dev = need_gpu()
    w = synth.workload("dsv3")
    say("dsv3: drawing 22.5 GB of weights on the GPU")
    inp = synth.make_inputs(w, device="cuda")
    torch.cuda.synchronize()
    yield w, inp, dev
    del inp
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def dsv3_run(dsv3):
    """The layer from x at b = C = P, the configuration the benchmark times."""
    w, inp, dev = dsv3
    P = w.T * w.k
    m = layer(w, dev, P, P)
    say("dsv3 full layer from x, b = C =", P)
    r = m(inp["x"], inp["w_router"], inp)
    torch.cuda.synchronize()
    assert m.device_error() == 0
    # bf16 tensors are kept as their int16 bit patterns (numpy has no bf16)
    host = {n: (v.cpu().view(torch.int16) if v.dtype == torch.bfloat16 else v.cpu()).numpy() for n, v in r.items()}
    del m, r
    torch.cuda.empty_cache()
    return host


def check_schedule_properties(sched, idx, E, P):
    counts, offsets = sched["counts"], sched["offsets"]
    src, dst = sched["sched"][:P], sched["route_dst"]
    flat = idx.reshape(-1)
    assert offsets[0] == 0 and offsets[-1] == P
    assert np.array_equal(np.diff(offsets), counts)
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert np.array_equal(np.sort(src), np.arange(P))
    assert np.array_equal(dst[src], np.arange(P))
    ex = flat[src]
    assert np.all(np.diff(ex) >= 0)
    for e in range(E):  # stable inside each expert region
        assert np.all(np.diff(src[offsets[e]:offsets[e + 1]]) > 0)


def test_dsv3_given_logits_route_and_schedule_bit_exact(dsv3):
    w, inp, dev = dsv3
    logits = synth.make_logits(w)  # N(0,1) fp32, as in the MoK paper's benchmark protocol
    m = layer(w, dev)
    say("dsv3 route (given logits) + schedule")
    _, idx, gate = m.route(None, None, logits.to(dev))
    sched = m.schedule(idx)
    torch.cuda.synchronize()
    l = logits.numpy()
    oi = ref.topk(l, w.k)
    assert np.array_equal(idx.cpu().numpy(), oi)
    g = gate.cpu().numpy().astype(np.float64)
    gref = ref.gates(l, oi)
    assert np.all(np.abs(g - gref) <= gate_tolerance(np.take_along_axis(l, oi, 1).astype(np.float64), w.k) * gref)
    want = ref.schedule(oi.reshape(1, -1), 0, w.E)
    assert np.array_equal(sched["counts"].cpu().numpy(), want["counts"])
    assert np.array_equal(sched["offsets"].cpu().numpy(), want["offsets"])
    assert np.array_equal(sched["sched"].cpu().numpy(), want["sched"])
    assert np.array_equal(sched["route_dst"].cpu().numpy(), want["route_dst"])


def test_dsv3_from_x_route_and_schedule_all_tokens(dsv3, dsv3_run):
    w, inp, dev = dsv3
    r = dsv3_run
    P = w.T * w.k
    xb, wrb = synth.bits(inp["x"]), synth.bits(inp["w_router"])
    say("dsv3 fp64 router logits and their fp32 bound over all tokens")
    L64 = ref.router_logits(xb, wrb)
    bound = ref.logit_bound(xb, wrb)
    lg = r["logits"]
    assert np.all(np.abs(lg.astype(np.float64) - L64) <= bound), "router logits outside the fp32 summation bound"
    gi = r["idx"]
    assert np.array_equal(ref.topk(lg, w.k), gi), "top-k differs from the oracle's on the same fp32 logits"
    g, gref = r["gate"].astype(np.float64), ref.gates(lg, gi)
    tol = gate_tolerance(np.take_along_axis(lg, gi.astype(np.int64), 1).astype(np.float64), w.k)
    assert np.all(np.abs(g - gref) <= tol * gref)
    want = ref.schedule(gi.reshape(1, -1), 0, w.E)
    for n in ("counts", "offsets", "route_dst"):
        assert np.array_equal(r[n], want[n]), n
    assert np.array_equal(r["sched"][:P], want["sched"])
    check_schedule_properties(r, gi, w.E, P)
    out32 = torch.from_numpy(r["out32"])
    assert np.array_equal(r["out"], out32.to(torch.bfloat16).view(torch.int16).numpy())


def test_dsv3_output_every_expert(dsv3, dsv3_run):
    w, inp, dev = dsv3
    r = dsv3_run
    gi, lg = r["idx"], r["logits"]
    tok = cover_tokens(gi, 512, seed=2, sched=r["sched"], offsets=r["offsets"], k=w.k)
    assert len(tok) >= 512 and len(np.unique(gi[tok])) == w.E
    say("dsv3 oracle on", len(tok), "tokens covering all", w.E, "experts (thread pool)")
    xb = synth.bits(inp["x"])
    Y = oracle_routed_pooled(xb, fetch_bf16(inp), [(gi, tok)])[0]
    shared = {n: synth.bits(inp[n]) for n in ("ws_gate", "ws_up", "ws_down")}
    want = ref.combine(ref.shared_output(xb, shared, tok), ref.gates(lg, gi)[tok], Y)
    err = rel_err(r["out32"][tok], want)
    say("dsv3 max|err|/RMS over", len(tok), "tokens =", err)
    assert err <= 1e-2


@pytest.mark.parametrize("b,C", [(2048, 4096), (8192, 32768)])
def test_dsv3_ring_mode_bitwise_equal(dsv3, dsv3_run, b, C):
    # minibatches of b rows cycling a ring of C rows give the bits of the
    # single-minibatch run (table-order gather, 256-row tiles at b = 2048)
    w, inp, dev = dsv3
    m = layer(w, dev, b, C)
    say("dsv3 ring mode from x, b =", b, "C =", C)
    r = m(inp["x"], inp["w_router"], inp)
    torch.cuda.synchronize()
    assert m.device_error() == 0
    assert np.array_equal(r["idx"].cpu().numpy(), dsv3_run["idx"])
    assert np.array_equal(r["out32"].cpu().numpy().view(np.int32), dsv3_run["out32"].view(np.int32))
    assert np.array_equal(r["out"].cpu().view(torch.int16).numpy(), dsv3_run["out"])
    del m, r
    torch.cuda.empty_cache()


@pytest.mark.parametrize("b,C", [(512, 2048), (2048, 8192), (8192, 32768)])
def test_dsv3_persistent_kernel_bitwise_equal(dsv3, dsv3_run, b, C):
    # the persistent routed kernel at the minibatch sizes the benchmark's
    # granularity sweep times (a ring of four minibatches, 16 gathering
    # workgroups) gives the bits of the single-minibatch stream-ordered run
    from mixture_experts_layer_counts_amd import MoELayer, shape_for
    w, inp, dev = dsv3
    m = MoELayer(shape_for(w.T, w.D, w.I, w.E, w.k, I_shared=w.I_shared, minibatch_rows=b, ring_rows=C,
                           pipeline=True, mem_workgroups=16), device=dev)
    say("dsv3 persistent kernel from x, b =", b, "C =", C)
    r = m(inp["x"], inp["w_router"], inp)
    torch.cuda.synchronize()
    assert m.device_error() == 0
    assert np.array_equal(r["out32"].cpu().numpy().view(np.int32), dsv3_run["out32"].view(np.int32))
    assert np.array_equal(r["out"].cpu().view(torch.int16).numpy(), dsv3_run["out"])
    del m, r
    torch.cuda.empty_cache()


def test_dsv3_backward_sampled(dsv3):
    import os
    from concurrent.futures import ThreadPoolExecutor

    from mixture_experts_layer_counts_amd import MoEBackward, prepare_backward
    from oracle import backward as bwd
    w, inp, dev = dsv3
    P = w.T * w.k
    m = layer(w, dev, P, P)
    say("dsv3 backward: forward from x at b = C = P, then moe_backward")
    r = m(inp["x"], inp["w_router"], inp)
    bw = prepare_backward(m.shape, inp, inp["w_router"])
    b = MoEBackward(m.shape, device=dev)
    dout = torch.randn((w.T, w.D), generator=torch.Generator().manual_seed(w.seed + 5)).to(torch.bfloat16)
    g = b(bw, inp["x"], r["idx"], r["gate"], r, m.routed_rows(), dout.to(dev))
    torch.cuda.synchronize()
    assert m.device_error() == 0 and b.device_error() == 0
    lg, gi = r["logits"].cpu().numpy(), r["idx"].cpu().numpy()
    counts = np.bincount(gi.ravel(), minlength=w.E)
    live = np.nonzero(counts)[0]
    rare = int(live[np.argmin(counts[live])])
    experts = sorted({0, w.E - 1, int(np.argmax(counts)), rare})
    tok_dx = np.sort(np.random.default_rng(5).choice(w.T, size=16, replace=False))
    tok_r = np.nonzero((gi == rare).any(axis=1))[0]
    rng = np.random.default_rng(6)
    cols = np.unique(np.concatenate([[0, 1, w.I_shared // 2, w.I_shared - 1], rng.choice(w.I_shared, 4)]))
    got = {"dx": g["dx"][torch.from_numpy(tok_dx).to(dev)].cpu().numpy(),
           "dw_router": g["dw_router"][rare].cpu().numpy()}
    for n in ("dw_gate", "dw_up", "dw_down"):
        got[n] = {e: g[n][e].float().cpu().numpy() for e in experts}
    c_dev = torch.from_numpy(cols).to(dev)
    got["dws_gate"] = g["dws_gate"][c_dev].float().cpu().numpy()
    got["dws_up"] = g["dws_up"][c_dev].float().cpu().numpy()
    got["dws_down"] = g["dws_down"][:, c_dev].float().cpu().numpy()
    del g, b, bw, m, r
    torch.cuda.empty_cache()

    xb, db, wrb = synth.bits(inp["x"]), synth.bits(dout), synth.bits(inp["w_router"])
    wts = {n: DeviceExperts(inp[n]) for n in ("w_gate", "w_up", "w_down")}
    wts.update({n: synth.bits(inp[n]) for n in ("ws_gate", "ws_up", "ws_down")})
    gates = ref.gates(lg, gi)
    for e in experts:
        say("dsv3 backward: expert", e, "with", int(counts[e]), "routes")
        _, want = bwd.expert_backward(xb, wts, gi, gates, db, e)
        for gpu, n in (("dw_gate", "dW_gate"), ("dw_up", "dW_up"), ("dw_down", "dW_down")):
            assert bf16_grad_ok(got[gpu][e], want[n], f"{gpu}[{e}]"), (gpu, e)
    say("dsv3 backward: shared columns", cols.tolist(), "over all tokens")
    want = bwd.shared_columns_backward(xb, wts, db, cols)
    for gpu, n in (("dws_gate", "dWs_gate"), ("dws_up", "dWs_up"), ("dws_down", "dWs_down")):
        assert bf16_grad_ok(got[gpu], want[n], gpu), gpu
    tok = np.union1d(tok_dx, tok_r)
    say("dsv3 backward: routed rows of", len(tok), "tokens (thread pool)")
    Y = oracle_routed_pooled(xb, fetch_bf16(inp), [(gi, tok)])[0]
    say("dsv3 backward: dx of", len(tok_dx), "tokens")
    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        want_dx = bwd.token_dx(xb, wts, lg, w.k, db, tok_dx, Y[np.searchsorted(tok, tok_dx)], wrb, map_fn=ex.map)
    err = rel_err(got["dx"], want_dx)
    say("   dx max|err|/RMS =", err)
    assert err <= 1e-2
    want_r = bwd.router_weight_rows(xb, lg, w.k, db, Y[np.searchsorted(tok, tok_r)], tok_r, [rare])[0]
    err = rel_err(got["dw_router"], want_r)
    say("   dw_router[%d] (%d tokens) max|err|/RMS =" % (rare, len(tok_r)), err)
    assert err <= 1e-2
