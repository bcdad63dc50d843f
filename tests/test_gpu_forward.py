"""GPU parity of the whole layer (moe_route + moe_schedule + moe_forward).

Layer outputs are compared as the fp32 pre-cast result against the fp64
oracle, which stores h and the routed output rows in bf16 exactly as the
method does: max|out32 - ref| <= 1e-2 * RMS(ref).  The bf16 output must be
the round-to-nearest-even of out32, bit for bit.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import moe as ref
from tests._gpu import host_weights, layer, need_gpu, rel_err, say, to_dev

pytestmark = pytest.mark.gpu

TOL_BF16 = 1e-2

CASES = [
    # name, workload, [(b, C), ...]
    ("tiny", synth.workload("tiny", routing="gaussian"), [(None, None), (16, 32), (32, 32), (128, 128)]),
    ("ragged", synth.Workload("ragged", T=300, D=256, I=192, E=16, k=4, I_shared=128, seed=7, routing="gaussian"),
     [(None, None), (100, 300), (256, 512)]),
    ("skewed", synth.Workload("skewed", T=257, D=192, I=128, E=24, k=6, I_shared=320, seed=8, routing="zipf"),
     [(None, None), (200, 400)]),
    # all rows at once take 320-row routed tiles (>= 192 rows per expert and
    # >= 128 up/gate work items); minibatches of 512-4096 rows, whose few
    # expert segments leave most CUs idle with 256-row tiles, take 128-row
    # tiles with up/gate items 64 columns wide and down items 64, 128 and 256
    # wide
    ("mid", synth.workload("mid", routing="gaussian"),
     [(4096, 8192), (None, None), (512, 1024), (1024, 1024), (2048, 4096)]),
    # 320-row tiles with Zipf routing: experts of one to four such tiles and
    # of a few rows, in one minibatch and in two
    ("skewed320", synth.Workload("skewed320", T=1024, D=256, I=1024, E=24, k=6, I_shared=128, seed=9,
                                 routing="zipf"), [(None, None), (5120, 5120)]),
    # limits: the most routes per token, the most experts, a single token
    ("k16", synth.Workload("k16", T=33, D=128, I=64, E=64, k=16, I_shared=64, seed=14, routing="gaussian"),
     [(None, None), (64, 128)]),
    ("e1024", synth.Workload("e1024", T=40, D=128, I=64, E=1024, k=8, I_shared=64, seed=15, routing="gaussian"),
     [(None, None), (100, 200)]),
    ("t1", synth.Workload("t1", T=1, D=128, I=64, E=8, k=2, I_shared=64, seed=16, routing="gaussian"),
     [(None, None), (1, 1)]),
]


def run_layer(w, inp_dev, b, C):
    m = layer(w, inp_dev["x"].device, b, C)
    r = m(inp_dev["x"], inp_dev["w_router"], inp_dev, logits=inp_dev.get("logits"))
    torch.cuda.synchronize()
    assert m.device_error() == 0
    return r


@pytest.mark.parametrize("name,w,bcs", CASES, ids=[c[0] for c in CASES])
def test_layer_parity_given_logits(name, w, bcs):
    dev = need_gpu()
    inp = synth.make_inputs(w)
    inp_dev = to_dev(inp, dev)
    say("layer_parity", name, w)
    want = ref.forward(synth.bits(inp["x"]), host_weights(inp), inp["logits"].numpy(), w.k)
    first = None
    for b, C in bcs:
        say("  b, C =", b, C)
        r = run_layer(w, inp_dev, b, C)
        assert np.array_equal(r["idx"].cpu().numpy(), want["idx"])
        out32 = r["out32"].cpu()
        err = rel_err(out32.numpy(), want["out"])
        say("  max|err|/RMS =", err)
        assert err <= TOL_BF16
        # bf16 output = RNE(out32), bit for bit
        assert torch.equal(r["out"].cpu().view(torch.int16), out32.to(torch.bfloat16).view(torch.int16))
        # every minibatch size and ring size gives the same bits
        if first is None:
            first = out32
        else:
            assert torch.equal(first.view(torch.int32), out32.view(torch.int32))


def test_layer_run_to_run_bitwise():
    dev = need_gpu()
    w = synth.Workload("det", T=512, D=256, I=128, E=32, k=8, I_shared=128, seed=9, routing="gaussian")
    inp_dev = to_dev(synth.make_inputs(w), dev)
    say("layer_determinism", w)
    outs = [run_layer(w, inp_dev, 512, 1024)["out32"].cpu() for _ in range(3)]
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int32), outs[0].view(torch.int32))


def test_layer_token_permutation_equivariant():
    dev = need_gpu()
    w = synth.Workload("perm", T=256, D=128, I=128, E=16, k=4, I_shared=64, seed=10, routing="gaussian")
    inp = synth.make_inputs(w)
    perm = torch.randperm(w.T, generator=torch.Generator().manual_seed(0))
    a = run_layer(w, to_dev(inp, dev), 256, 512)["out32"].cpu()
    inp2 = dict(inp)
    inp2["x"], inp2["logits"] = inp["x"][perm], inp["logits"][perm]
    say("layer_permutation", w)
    b = run_layer(w, to_dev(inp2, dev), 256, 512)["out32"].cpu()
    assert torch.equal(b.view(torch.int32), a[perm].view(torch.int32))


def test_layer_zero_input_and_single_expert():
    dev = need_gpu()
    w = synth.Workload("zero", T=96, D=128, I=64, E=4, k=2, I_shared=64, seed=3, routing="gaussian")
    inp = synth.make_inputs(w)
    inp["x"] = torch.zeros_like(inp["x"])
    say("layer_zero", w)
    r = run_layer(w, to_dev(inp, dev), None, None)
    assert torch.all(r["out32"] == 0)
    # one expert, top-1: the oracle's own identity case, on the GPU
    w1 = synth.Workload("one", T=80, D=128, I=64, E=1, k=1, I_shared=64, seed=4, routing="gaussian")
    inp1 = synth.make_inputs(w1)
    want = ref.forward(synth.bits(inp1["x"]), host_weights(inp1), inp1["logits"].numpy(), 1)
    r1 = run_layer(w1, to_dev(inp1, dev), None, None)
    assert rel_err(r1["out32"].cpu().numpy(), want["out"]) <= TOL_BF16


def test_layer_from_x_every_token():
    # full path from x: the router GEMM decides the routing.  The selection
    # must equal the oracle's top-k of the GPU's own fp32 logits on every
    # token, and the output the oracle's from those logits; where the fp64
    # logits leave no doubt, the selection is also the fp64 one.
    dev = need_gpu()
    w = synth.Workload("fromx", T=400, D=256, I=128, E=16, k=4, I_shared=128, seed=12)
    inp = synth.make_inputs(w)
    say("layer_from_x", w)
    r = run_layer(w, to_dev(inp, dev), 600, 1200)
    xb, wb = synth.bits(inp["x"]), synth.bits(inp["w_router"])
    lg = r["logits"].cpu().numpy()
    want = ref.forward(xb, host_weights(inp), lg, w.k)
    assert np.array_equal(r["idx"].cpu().numpy(), want["idx"])
    assert rel_err(r["out32"].cpu().numpy(), want["out"]) <= TOL_BF16
    L64 = ref.router_logits(xb, wb)
    bound = ref.logit_bound(xb, wb).max(axis=1)
    srt = np.sort(L64, axis=1)[:, ::-1]
    clear = np.nonzero(srt[:, w.k - 1] - srt[:, w.k] > 2 * bound)[0]
    assert len(clear) > 0.9 * w.T
    o64 = ref.topk(L64.astype(np.float32), w.k)
    assert np.array_equal(np.sort(want["idx"][clear], 1), np.sort(o64[clear], 1))
