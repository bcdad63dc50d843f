"""GPU parity of the layer with the shared expert in MXFP8 (an option beside
the pages' bf16 shared expert): x is MX-quantised along D for it, h along
I_shared, and its fp32 output enters the combine.  Against the oracle's layer
with its own MX quantisation of the same bf16 weights, within 5e-2 * RMS, and
bitwise the same for every minibatch and ring size."""

import numpy as np
import pytest
import torch

import synth
from oracle import moe as ref
from tests._gpu import (host_weights, layer, mx_shared_weights_dev, mx_weights_dev, need_gpu, oracle_mx_weights,
                        rel_err, say, to_dev)

pytestmark = pytest.mark.gpu

TOL_MX = 5e-2

CASES = [
    # name, workload, routed precision, [(b, C), ...]
    ("tiny", synth.Workload("tiny-mxs", T=64, D=128, I=128, E=8, k=2, I_shared=128, seed=40, routing="gaussian"),
     "mxfp8", [(None, None), (32, 64)]),
    # T = 300: two shared tiles of 160 and 140 rows
    ("ragged", synth.Workload("ragged-mxs", T=300, D=384, I=256, E=16, k=4, I_shared=256, seed=41,
                              routing="gaussian"), "mxfp8", [(None, None), (256, 512)]),
    ("wide", synth.Workload("wide-mxs", T=1024, D=1024, I=512, E=48, k=8, I_shared=512, seed=42, routing="zipf"),
     "mxfp8", [(None, None)]),
    # one token: a single shared tile of one row
    ("t1", synth.Workload("t1-mxs", T=1, D=128, I=128, E=8, k=2, I_shared=128, seed=46, routing="gaussian"),
     "mxfp8", [(None, None), (1, 2)]),
    # routed experts in bf16, shared expert in MXFP8
    ("bf16-routed", synth.Workload("bf16r-mxs", T=257, D=256, I=192, E=24, k=6, I_shared=384, seed=43,
                                   routing="gaussian"), "bf16", [(None, None), (200, 400)]),
]


@pytest.mark.parametrize("name,w,prec,bcs", CASES, ids=[c[0] for c in CASES])
def test_mx_shared_layer_parity(name, w, prec, bcs):
    dev = need_gpu()
    inp = synth.make_inputs(w)
    inp_dev = to_dev(inp, dev)
    say("mx_shared_layer_parity", name, prec, w)
    weights = dict(mx_weights_dev(inp_dev) if prec == "mxfp8" else inp_dev)
    weights.update(mx_shared_weights_dev(inp_dev))
    host = oracle_mx_weights(inp) if prec == "mxfp8" else host_weights(inp)
    host = ref.quantize_shared_mx({**host, **{n: synth.bits(inp[n]) for n in ("ws_gate", "ws_up", "ws_down")}})
    want = ref.forward(synth.bits(inp["x"]), host, inp["logits"].numpy(), w.k, precision=prec,
                       shared_precision="mxfp8")
    first = None
    for b, C in bcs:
        say("  b, C =", b, C)
        m = layer(w, dev, b, C, precision=prec, shared_precision="mxfp8")
        r = m(inp_dev["x"], inp_dev["w_router"], weights, logits=inp_dev["logits"])
        torch.cuda.synchronize()
        assert m.device_error() == 0
        assert np.array_equal(r["idx"].cpu().numpy(), want["idx"])
        out32 = r["out32"].cpu()
        err = rel_err(out32.numpy(), want["out"])
        say("  max|err|/RMS =", err)
        assert err <= TOL_MX
        assert torch.equal(r["out"].cpu().view(torch.int16), out32.to(torch.bfloat16).view(torch.int16))
        if first is None:
            first = out32
        else:  # minibatch and ring sizes do not change a bit
            assert torch.equal(first.view(torch.int32), out32.view(torch.int32))


def test_mx_shared_expert_alone_matches_oracle_shared_term():
    # one routed expert whose gate is 1 and whose weights are zero: the layer
    # output is the shared expert's output alone
    dev = need_gpu()
    w = synth.Workload("shared-only", T=200, D=256, I=128, E=1, k=1, I_shared=256, seed=44, routing="gaussian")
    inp = synth.make_inputs(w)
    for n in ("w_gate", "w_up", "w_down"):
        inp[n].zero_()
    inp_dev = to_dev(inp, dev)
    say("mx_shared_alone")
    weights = dict(inp_dev)
    weights.update(mx_shared_weights_dev(inp_dev))
    host = ref.quantize_shared_mx({n: synth.bits(inp[n]) for n in ("ws_gate", "ws_up", "ws_down")})
    want = ref.shared_output(synth.bits(inp["x"]), host, precision="mxfp8")
    m = layer(w, dev, shared_precision="mxfp8")
    r = m(inp_dev["x"], inp_dev["w_router"], weights, logits=inp_dev["logits"])
    torch.cuda.synchronize()
    assert m.device_error() == 0
    err = rel_err(r["out32"].cpu().numpy(), want)
    say("  max|err|/RMS =", err)
    assert err <= TOL_MX


def test_mx_shared_expert_full_size_sampled():
    # the shared expert at the DeepSeek-V3 layer shape (8192 tokens, D = 7168,
    # I_shared = 2048): 32 dense tiles, the fp32 epilogue over N = 7168.  Two
    # routed experts with zero weights and top-1 keep the routed term at zero,
    # so the output is the shared term; sampled tokens against the oracle.
    dev = need_gpu()
    w = synth.Workload("dsv3-shared", T=8192, D=7168, I=2048, E=2, k=1, I_shared=2048, seed=45, routing="gaussian")
    say("mx_shared_full: drawing inputs on the GPU")
    inp = synth.make_inputs(w, device="cuda")
    for n in ("w_gate", "w_up", "w_down"):
        inp[n].zero_()
    weights = dict(inp)
    weights.update(mx_shared_weights_dev(inp))
    m = layer(w, dev, shared_precision="mxfp8")
    r = m(inp["x"], inp["w_router"], weights, logits=inp["logits"])
    torch.cuda.synchronize()
    assert m.device_error() == 0
    tok = np.array([0, 1, 255, 256, 4095, 7679, 7680, 8000, 8191])  # tile edges of 256-row tiles
    host = ref.quantize_shared_mx({n: synth.bits(inp[n].cpu()) for n in ("ws_gate", "ws_up", "ws_down")})
    want = ref.shared_output(synth.bits(inp["x"][torch.as_tensor(tok, device=dev)].cpu()), host, precision="mxfp8")
    got = r["out32"][torch.as_tensor(tok, device=dev)].cpu().numpy()
    err = rel_err(got, want)
    say("  max|err|/RMS =", err)
    assert err <= TOL_MX
