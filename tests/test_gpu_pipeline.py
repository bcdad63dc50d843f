"""The routed minibatch loop as one persistent kernel (moe_shape.pipeline = 1)
against the stream-ordered launches (pipeline = 0) through the C ABI.

The persistent kernel runs the stream-ordered path's own work items, so its
results must be the same bits: the layer output, and for an EP share the
outbox rows, at every minibatch size, ring size and split of the workgroups
between gathers and GEMMs.  Each case also meets the oracle, and the device
error word must stay clear (a wait that gave up would set
MOE_DEVERR_PIPELINE).
"""

import numpy as np
import pytest
import torch

import synth
from mixture_experts_layer_counts_amd import MoELayer, shape_for
from oracle import moe as ref
from tests._gpu import host_weights, need_gpu, rel_err, say, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    # name, workload, [(b, C, memory workgroups)]; tilings: 128-row tiles
    # (small b), 256-row (tiny minibatch counts) and 320-row (skewed320, all
    # rows at once); rings of C/b = 3, 4 and 8 minibatches keep H = 3 and 4 h
    # buffers, up/gate running 2 and 3 minibatches ahead of down
    ("tiny", synth.workload("tiny", routing="gaussian"),
     [(16, 32, 8), (16, 16, 8), (32, 64, 16), (128, 128, 0), (16, 48, 8), (16, 128, 8)]),
    ("ragged", synth.Workload("ragged", T=300, D=256, I=192, E=16, k=4, I_shared=128, seed=7, routing="gaussian"),
     [(100, 300, 8), (100, 100, 24), (256, 512, 8), (1200, 1200, 0), (64, 192, 8), (100, 400, 16)]),
    ("mid", synth.workload("mid", routing="gaussian"),
     [(512, 1024, 16), (512, 512, 32), (2048, 2048, 8), (4096, 8192, 16), (32768, 32768, 0), (512, 4096, 8),
      (1024, 3072, 8)]),
    ("skewed320", synth.Workload("skewed320", T=1024, D=256, I=1024, E=24, k=6, I_shared=128, seed=9,
                                 routing="zipf"), [(6144, 6144, 0), (3072, 3072, 8)]),
    # 2048-row minibatches of ~256-row segments with I = 2048: 256-row tiles
    ("wideI", synth.Workload("wideI", T=2048, D=256, I=2048, E=32, k=4, I_shared=128, seed=19, routing="gaussian"),
     [(2048, 4096, 8), (2048, 2048, 16), (1024, 4096, 8)]),
]


def run(w, inp_dev, b, C, pipeline, mem):
    m = MoELayer(shape_for(w.T, w.D, w.I, w.E, w.k, I_shared=w.I_shared, minibatch_rows=b, ring_rows=C,
                           pipeline=pipeline, mem_workgroups=mem), device=inp_dev["x"].device)
    r = m(inp_dev["x"], inp_dev["w_router"], inp_dev, logits=inp_dev.get("logits"))
    torch.cuda.synchronize()
    assert m.device_error() == 0
    return r


@pytest.mark.parametrize("name,w,bcs", CASES, ids=[c[0] for c in CASES])
def test_pipeline_bitwise_equal_to_stream_ordered(name, w, bcs):
    dev = need_gpu()
    inp = synth.make_inputs(w)
    inp_dev = to_dev(inp, dev)
    want = ref.forward(synth.bits(inp["x"]), host_weights(inp), inp["logits"].numpy(), w.k)
    for b, C, mem in bcs:
        say("pipeline", name, "b, C =", b, C, "memory workgroups =", mem)
        a = run(w, inp_dev, b, C, False, 0)
        p = run(w, inp_dev, b, C, True, mem)
        assert torch.equal(a["out32"].view(torch.int32), p["out32"].view(torch.int32))
        assert torch.equal(a["out"].view(torch.int16), p["out"].view(torch.int16))
        err = rel_err(p["out32"].cpu().numpy(), want["out"])
        say("  max|err|/RMS =", err)
        assert err <= 1e-2


def test_pipeline_ep_share_outbox_bitwise():
    # an EP share (R = 8 source ranks, 4 local experts of 32, Zipf counts):
    # the outbox rows and the rank's output, persistent against stream-ordered
    dev = need_gpu()
    R, N, k, L, c = 8, 200, 8, 4, 3
    w = synth.Workload("ep8", T=R * N, D=384, I=256, E=R * L, k=k, I_shared=128, seed=61)
    inp = synth.make_inputs(w)
    A = torch.from_numpy(synth.ep_share_routes(R, N, k, R * L, c, L, [400, 200, 120, 80], seed=61)).to(dev)
    g = torch.rand((N, k), generator=torch.Generator().manual_seed(3)) + 0.05
    g = (g / g.sum(dim=1, keepdim=True)).to(dev)
    inp_dev = to_dev(inp, dev)
    weights = {n: inp_dev[n] for n in ("ws_gate", "ws_up", "ws_down")}
    for n in ("w_gate", "w_up", "w_down"):
        weights[n] = inp_dev[n][c * L:(c + 1) * L].contiguous()
    x_local = inp_dev["x"][c * N:(c + 1) * N]
    got = []
    for pipeline, mem in ((False, 0), (True, 8), (True, 16)):
        m = MoELayer(shape_for(N, w.D, w.I, R * L, k, I_shared=w.I_shared, minibatch_rows=256, ring_rows=512,
                               R=R, rank=c, max_rows=800, pipeline=pipeline, mem_workgroups=mem), device=dev)
        sched = m.schedule(A)
        out, out32 = m.forward(weights, inp_dev["x"], x_local, g, sched)
        torch.cuda.synchronize()
        assert m.device_error() == 0
        got.append((m.routed_rows()[:800].cpu().view(torch.int16), out32.cpu().view(torch.int32)))
    for rows, o in got[1:]:
        assert torch.equal(rows, got[0][0]) and torch.equal(o, got[0][1])


def test_pipeline_refuses_bad_splits():
    # moe_forward refuses these before any of its launches: minibatches past
    # the ring with no memory workgroups to gather them, and a split that
    # leaves fewer than 8 workgroups for the GEMMs (the grid is every
    # workgroup the chip holds at once)
    from mixture_experts_layer_counts_amd import _lib
    dev = need_gpu()
    w = synth.workload("tiny", routing="gaussian")
    inp_dev = to_dev(synth.make_inputs(w), dev)

    def forward(mem):
        m = MoELayer(shape_for(w.T, w.D, w.I, w.E, w.k, minibatch_rows=16, ring_rows=16, pipeline=True,
                               mem_workgroups=mem), device=dev)
        return m(inp_dev["x"], inp_dev["w_router"], inp_dev, logits=inp_dev["logits"])

    for mem in (0, 1 << 20):
        with pytest.raises(_lib.MoeError) as e:
            forward(mem)
        assert e.value.status == -1
    torch.cuda.synchronize()
