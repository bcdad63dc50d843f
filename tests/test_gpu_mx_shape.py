"""Parity of the MXFP8 layer at its full shape (T=8192, D=7168, I=2048, 384
routed experts, top-8, one shared expert with I=2048) in the launch
configuration the benchmark times (one minibatch of all 65,536 routed rows,
ring of the same size), from given N(0,1) fp32 logits.

* routing and schedule tables: bit-exact over all tokens;
* layer output: sampled tokens, evaluated by the oracle one by one.  The
  sampled tokens' logits are lifted on one common set of 8 experts, so that
  the oracle quantises only those 8 experts' weights (the other 8184 tokens
  keep their Gaussian routing).
"""

import numpy as np
import pytest
import torch

import synth
from oracle import moe as ref
from tests._gpu import layer, mx_weights_dev, need_gpu, oracle_mx_weights, rel_err, say

pytestmark = pytest.mark.gpu

SAMPLE = [0, 1, 777, 2048, 4095, 5000, 6666, 8191]
HOT = [3, 50, 101, 177, 200, 255, 300, 383]


def test_mx_shape_route_schedule_and_sampled_tokens():
    dev = need_gpu()
    w = synth.workload("mx", routing="gaussian")
    say("mx shape: drawing 33.8 GB of bf16 weights on the GPU")
    inp = synth.make_inputs(w, device="cuda")
    tok = torch.as_tensor(SAMPLE, device=dev)
    logits = inp["logits"]
    logits[tok[:, None], torch.as_tensor(HOT, device=dev)[None, :]] += 8.0
    say("mx shape: quantising the routed weights on the GPU")
    wq = mx_weights_dev(inp)
    P = w.T * w.k
    m = layer(w, dev, P, P, precision="mxfp8")
    say("mx shape: layer forward, b = C =", P)
    r = m(inp["x"], inp["w_router"], wq, logits=logits)
    torch.cuda.synchronize()
    assert m.device_error() == 0

    l = logits.cpu().numpy()
    oi = ref.topk(l, w.k)
    assert np.array_equal(r["idx"].cpu().numpy(), oi)
    want_s = ref.schedule(oi.reshape(1, -1), 0, w.E)
    for n in ("counts", "offsets", "sched", "route_dst"):
        assert np.array_equal(r[n].cpu().numpy(), want_s[n])
    assert set(oi[SAMPLE].ravel().tolist()) == set(HOT)

    say("mx shape: oracle on", len(SAMPLE), "tokens and", len(HOT), "experts")
    weights = oracle_mx_weights(inp, HOT)
    xb = synth.bits(inp["x"][tok])
    want = ref.forward(xb, weights, l[SAMPLE], w.k, precision="mxfp8")
    got = r["out32"][tok].cpu().numpy()
    err = rel_err(got, want["out"])
    say("mx shape sampled max|err|/RMS =", err)
    assert err <= 5e-2
    assert torch.equal(r["out"][tok].cpu().view(torch.int16), r["out32"][tok].cpu().to(torch.bfloat16).view(torch.int16))
    del inp, wq, r, m
    torch.cuda.empty_cache()
