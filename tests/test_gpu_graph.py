"""The whole layer (moe_route from x + moe_schedule + moe_forward), also with
the persistent routed kernel, and the backward (moe_backward), each captured
in a HIP graph and replayed.

The library allocates nothing, reads no device data on the host and clears
its scratch words with kernels, so a caller may capture a step and replay it.
Each replay must give the eager step's results bit for bit, also with other
eager work and synchronisations between the replays.
"""

import pytest
import torch

import synth
from tests._gpu import layer, need_gpu, say, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    # one minibatch (source-side gather; the down projection's resident
    # workgroups walk several items each), and several minibatches through a
    # ring smaller than the routed rows
    ("ragged-one", synth.Workload("ragged", T=300, D=256, I=192, E=16, k=4, I_shared=128, seed=7), None, None, False),
    ("ragged-ring", synth.Workload("ragged", T=300, D=256, I=192, E=16, k=4, I_shared=128, seed=7), 256, 512,
     False),
    ("mid-one", synth.workload("mid", T=1024), None, None, False),
    # the persistent routed kernel: its counters and queues are cleared by a
    # fill kernel in the captured sequence, and its memory workgroups gather
    # the minibatches past the ring
    ("mid-persistent", synth.workload("mid", T=1024), 512, 2048, True),
]


def make_layer(w, dev, b, C, pipeline):
    if not pipeline:
        return layer(w, dev, b, C)
    from mixture_experts_layer_counts_amd import MoELayer, shape_for
    return MoELayer(shape_for(w.T, w.D, w.I, w.E, w.k, I_shared=w.I_shared, minibatch_rows=b, ring_rows=C,
                              pipeline=True, mem_workgroups=16), device=dev)


@pytest.mark.parametrize("name,w,b,C,pipeline", CASES, ids=[c[0] for c in CASES])
def test_layer_graph_replay_bitwise(name, w, b, C, pipeline):
    dev = need_gpu()
    say("graph_replay", name, w, b, C, "persistent" if pipeline else "")
    inp_dev = to_dev(synth.make_inputs(w), dev)
    m = make_layer(w, dev, b, C, pipeline)
    keys = ("logits", "idx", "gate", "offsets", "sched", "route_dst", "out", "out32")

    eager = m(inp_dev["x"], inp_dev["w_router"], inp_dev)
    torch.cuda.synchronize()
    want = {k: eager[k].clone() for k in keys}

    # a second layer object supplies eager work between the replays
    other = make_layer(w, dev, b, C, pipeline)
    noise = torch.randn_like(inp_dev["x"], dtype=torch.float32).to(torch.bfloat16)

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        m(inp_dev["x"], inp_dev["w_router"], inp_dev)  # warm-up on the capturing stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        got = m(inp_dev["x"], inp_dev["w_router"], inp_dev)
    for rep in range(3):
        for k in ("out", "out32", "logits"):
            got[k].fill_(0)
        g.replay()
        torch.cuda.synchronize()
        for k in keys:
            assert torch.equal(got[k], want[k]), f"replay {rep}: {k} differs from the eager step"
        # eager work on other inputs, then a synchronisation, before the next replay
        other(noise, inp_dev["w_router"], inp_dev)
        torch.cuda.synchronize()
    assert m.device_error() == 0


def test_backward_graph_replay_bitwise():
    # moe_backward is launches only (no allocation, no host read, no memset),
    # so a caller may capture it too; each replay gives the eager gradients bit
    # for bit, with other eager backward work between the replays
    from mixture_experts_layer_counts_amd import MoEBackward, prepare_backward
    dev = need_gpu()
    w = synth.Workload("ragged", T=300, D=256, I=192, E=16, k=4, I_shared=128, seed=7, routing="gaussian")
    say("graph_replay backward", w)
    inp_dev = to_dev(synth.make_inputs(w), dev)
    m = layer(w, dev)
    r = m(inp_dev["x"], inp_dev["w_router"], inp_dev, logits=inp_dev["logits"])
    y = m.routed_rows()
    bw = prepare_backward(m.shape, inp_dev, inp_dev["w_router"])
    b = MoEBackward(m.shape, device=dev)
    dout = torch.randn((w.T, w.D), generator=torch.Generator().manual_seed(4)).to(torch.bfloat16).to(dev)
    grads = b(bw, inp_dev["x"], r["idx"], r["gate"], r, y, dout)
    torch.cuda.synchronize()
    want = {n: v.clone() for n, v in grads.items()}

    other = MoEBackward(m.shape, device=dev)
    noise = torch.randn_like(dout, dtype=torch.float32).to(torch.bfloat16)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        b(bw, inp_dev["x"], r["idx"], r["gate"], r, y, dout, grads)  # warm-up on the capturing stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        b(bw, inp_dev["x"], r["idx"], r["gate"], r, y, dout, grads)
    for rep in range(3):
        for v in grads.values():
            v.zero_()
        g.replay()
        torch.cuda.synchronize()
        for n in want:
            assert torch.equal(grads[n], want[n]), f"replay {rep}: {n} differs from the eager backward"
        other(bw, inp_dev["x"], r["idx"], r["gate"], r, y, noise)
        torch.cuda.synchronize()
    assert b.device_error() == 0 and other.device_error() == 0
