"""Parity of the MXFP8 layer at its full shape (T=8192, D=7168, I=2048, 384
routed experts, top-8, one shared expert with I=2048) in the launch
configuration the benchmark times (one minibatch of all 65,536 routed rows,
ring of the same size), from given fp32 logits with both routings the
benchmark runs: N(0,1) logits (near-uniform expert load) and Zipf(1.2)-skewed
logits (experts receive from a few rows to several thousand).

* routing and schedule tables: bit-exact over all tokens;
* layer output: a sample of over 512 tokens per routing that together route
  to every one of the 384 experts and include the first and last row of every
  expert's region, against the oracle with its own MX quantisation of every
  expert's weights (done once, in a thread pool, for both routings);
* ring mode (minibatches of 8,192 rows cycling a 16,384-row ring, the
  table-order MX gather): bitwise equal to the single-minibatch run.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import moe as ref
from tests._gpu import (cover_tokens, fetch_mx, gate_tolerance, layer, mx_weights_dev, need_gpu,
                        oracle_routed_pooled, rel_err, say)

pytestmark = pytest.mark.gpu


def host_run(r):
    return {n: (v.cpu().view(torch.int16) if v.dtype == torch.bfloat16 else v.cpu()).numpy() for n, v in r.items()}


@pytest.mark.timeout(1100)
def test_mx_shape_uniform_and_zipf_every_expert():
    dev = need_gpu()
    w = synth.workload("mx", routing="gaussian")
    say("mx shape: drawing 33.8 GB of bf16 weights on the GPU")
    inp = synth.make_inputs(w, device="cuda")
    say("mx shape: quantising the routed weights on the GPU")
    wq = mx_weights_dev(inp)
    P = w.T * w.k
    runs = {}
    for kind in ("gaussian", "zipf"):
        logits = synth.make_logits(w, device="cuda", kind=kind)
        m = layer(w, dev, P, P, precision="mxfp8")
        say("mx shape:", kind, "logits, layer forward, b = C =", P)
        r = m(inp["x"], inp["w_router"], wq, logits=logits)
        torch.cuda.synchronize()
        assert m.device_error() == 0
        runs[kind] = host_run(r)
        if kind == "gaussian":  # ring mode, table-order MX gather
            m2 = layer(w, dev, 8192, 16384, precision="mxfp8")
            say("mx shape: ring mode, b = 8192, C = 16384")
            r2 = m2(inp["x"], inp["w_router"], wq, logits=logits)
            torch.cuda.synchronize()
            assert m2.device_error() == 0
            h2 = host_run(r2)
            assert np.array_equal(h2["out32"].view(np.int32), runs[kind]["out32"].view(np.int32))
            assert np.array_equal(h2["out"], runs[kind]["out"])
            del m2, r2
        del m, r
        torch.cuda.empty_cache()
    del wq
    torch.cuda.empty_cache()

    cases = []
    for kind, r in runs.items():
        l, gi = r["logits"], r["idx"]
        oi = ref.topk(l, w.k)
        assert np.array_equal(gi, oi), kind
        g, gref = r["gate"].astype(np.float64), ref.gates(l, oi)
        assert np.all(np.abs(g - gref) <= gate_tolerance(np.take_along_axis(l, oi.astype(np.int64), 1)
                                                         .astype(np.float64), w.k) * gref), kind
        want_s = ref.schedule(oi.reshape(1, -1), 0, w.E)
        for n in ("counts", "offsets", "route_dst"):
            assert np.array_equal(r[n], want_s[n]), (kind, n)
        assert np.array_equal(r["sched"][:P], want_s["sched"]), kind
        assert np.array_equal(r["out"], torch.from_numpy(r["out32"]).to(torch.bfloat16).view(torch.int16).numpy())
        tok = cover_tokens(oi, 512, seed=4, sched=r["sched"], offsets=r["offsets"], k=w.k)
        assert len(tok) >= 512 and len(np.unique(oi[tok])) == w.E, kind
        say("mx shape:", kind, "counts per expert", int(r["counts"].min()), "..", int(r["counts"].max()),
            "; sample of", len(tok), "tokens")
        cases.append((oi, tok))

    say("mx shape: oracle MX quantisation of all", w.E, "experts and both samples (thread pool)")
    xb = synth.bits(inp["x"])
    ys = oracle_routed_pooled(xb, fetch_mx(inp), cases, precision="mxfp8")
    shared = {n: synth.bits(inp[n]) for n in ("ws_gate", "ws_up", "ws_down")}
    for (kind, r), (oi, tok), Y in zip(runs.items(), cases, ys):
        want = ref.combine(ref.shared_output(xb, shared, tok), ref.gates(r["logits"], oi)[tok], Y)
        err = rel_err(r["out32"][tok], want)
        say("mx shape:", kind, "max|err|/RMS over", len(tok), "tokens =", err)
        assert err <= 5e-2, kind
    del inp
    torch.cuda.empty_cache()
