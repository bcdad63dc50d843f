"""Parity at the full DeepSeek-V3 layer shape (T=8192, D=7168, I=2048, 256
experts, top-8, shared I=2048), in the launch configuration bench.py times
(one minibatch of all 65,536 routed rows, ring of the same size).

The oracle cannot run the whole layer here in seconds, so:
* routing and schedule from given fp32 logits: bit-exact over all tokens;
* the full path from x: sampled tokens, evaluated one by one by the oracle
  (router logits within the fp32 bound, selection, output within tolerance);
* schedule tables: properties that hold at any size.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import moe as ref
from tests._gpu import layer, need_gpu, rel_err, say

pytestmark = pytest.mark.gpu

SAMPLE = [0, 1, 511, 1024, 2047, 3000, 4096, 5000, 6000, 7000, 8000, 8191]


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


def check_schedule_properties(sched, idx, E, P):
    counts, offsets = sched["counts"].cpu().numpy(), sched["offsets"].cpu().numpy()
    src, dst = sched["sched"].cpu().numpy()[:P], sched["route_dst"].cpu().numpy()
    flat = idx.cpu().numpy().reshape(-1)
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
    want = ref.schedule(oi.reshape(1, -1), 0, w.E)
    assert np.array_equal(sched["counts"].cpu().numpy(), want["counts"])
    assert np.array_equal(sched["offsets"].cpu().numpy(), want["offsets"])
    assert np.array_equal(sched["sched"].cpu().numpy(), want["sched"])
    assert np.array_equal(sched["route_dst"].cpu().numpy(), want["route_dst"])


def test_dsv3_full_path_sampled_tokens(dsv3):
    w, inp, dev = dsv3
    P = w.T * w.k
    m = layer(w, dev, P, P)
    say("dsv3 full layer from x, b = C =", P)
    r = m(inp["x"], inp["w_router"], inp)
    torch.cuda.synchronize()
    assert m.device_error() == 0
    check_schedule_properties(r, r["idx"], w.E, P)
    tok = np.array(SAMPLE)
    xb = synth.bits(inp["x"][torch.as_tensor(tok, device=dev)])
    wrb = synth.bits(inp["w_router"])
    L64 = ref.router_logits(xb, wrb)
    bound = ref.logit_bound(xb, wrb)
    lg = r["logits"][torch.as_tensor(tok, device=dev)].cpu().numpy().astype(np.float64)
    assert np.all(np.abs(lg - L64) <= bound)
    # the selection must be valid under the worst-case bound for every token,
    # and equal the oracle's where the gap beats the probabilistic bound
    gi = r["idx"].cpu().numpy()[tok]
    for i in range(len(tok)):
        sel = set(gi[i].tolist())
        lo = min(L64[i, e] + bound[i, e] for e in sel)
        hi = max(L64[i, f] - bound[i, f] for f in range(w.E) if f not in sel)
        assert lo >= hi
    pb = ref.logit_bound_probabilistic(xb, wrb)
    srt = np.sort(L64, axis=1)[:, ::-1]
    clear = srt[:, w.k - 1] - srt[:, w.k] > 2 * pb.max(axis=1)
    oi = ref.topk(L64.astype(np.float32), w.k)
    assert np.array_equal(np.sort(gi[clear], 1), np.sort(oi[clear], 1))
    keep = np.nonzero(clear)[0]
    say("dsv3 unambiguous sampled tokens:", len(keep), "of", len(tok))
    assert len(keep) >= len(tok) // 2
    # host copies of the experts the kept tokens use, and the oracle per token
    experts = np.unique(oi[keep])
    say("dsv3 oracle on", len(keep), "tokens,", len(experts), "experts")
    host = {n: synth.bits(inp[n]) for n in ("ws_gate", "ws_up", "ws_down")}
    for n in ("w_gate", "w_up", "w_down"):
        sub = synth.bits(inp[n][torch.as_tensor(experts, device=dev)])
        host[n] = {int(e): sub[i] for i, e in enumerate(experts)}
    want = ref.forward(xb[keep], host, L64[keep].astype(np.float32), w.k)
    got = r["out32"].cpu().numpy()[tok[keep]]
    err = rel_err(got, want["out"])
    say("dsv3 sampled max|err|/RMS =", err)
    assert err <= 1e-2
    assert torch.equal(r["out"][torch.as_tensor(tok, device=dev)].cpu().view(torch.int16),
                       r["out32"][torch.as_tensor(tok, device=dev)].cpu().to(torch.bfloat16).view(torch.int16))
