"""The whole layer (moe_route from x + moe_schedule + moe_forward) captured in
a HIP graph and replayed.

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
    ("ragged-one", synth.Workload("ragged", T=300, D=256, I=192, E=16, k=4, I_shared=128, seed=7), None, None),
    ("ragged-ring", synth.Workload("ragged", T=300, D=256, I=192, E=16, k=4, I_shared=128, seed=7), 256, 512),
    ("mid-one", synth.workload("mid", T=1024), None, None),
]


@pytest.mark.parametrize("name,w,b,C", CASES, ids=[c[0] for c in CASES])
def test_layer_graph_replay_bitwise(name, w, b, C):
    dev = need_gpu()
    say("graph_replay", name, w, b, C)
    inp_dev = to_dev(synth.make_inputs(w), dev)
    m = layer(w, dev, b, C)
    keys = ("logits", "idx", "gate", "offsets", "sched", "route_dst", "out", "out32")

    eager = m(inp_dev["x"], inp_dev["w_router"], inp_dev)
    torch.cuda.synchronize()
    want = {k: eager[k].clone() for k in keys}

    # a second layer object supplies eager work between the replays
    other = layer(w, dev, b, C)
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
