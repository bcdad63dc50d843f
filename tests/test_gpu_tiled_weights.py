"""The routed weights in the K-tiled layout (moe_shape.weights_tiled):
moe_tile_bf16 moves every element to ((g*(K/64) + k/64)*N + n)*64 + k%64, and
the layer gives bitwise the same output as with row-major weights, through
the C ABI: bf16 at several shapes, minibatch and ring sizes, stream-ordered
and persistent; MXFP8 with the E4M3 bytes tiled in 128-byte planes."""

import pytest
import torch

import synth
from tests._gpu import need_gpu, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("G,N,K", [(1, 1, 64), (3, 37, 192), (4, 2048, 7168)])
def test_tile_bf16_bit_exact(G, N, K):
    dev = need_gpu()
    from mixture_experts_layer_counts_amd import tile_bf16
    say("tile_bf16", (G, N, K))
    w = torch.randint(-32768, 32768, (G, N, K), dtype=torch.int16,
                      generator=torch.Generator().manual_seed(G * N + K)).view(torch.bfloat16)
    got = tile_bf16(w.to(dev)).cpu()
    torch.cuda.synchronize()
    want = w.view(G, N, K // 64, 64).permute(0, 2, 1, 3).contiguous()
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))


CASES = [
    (synth.Workload("tiny", T=64, D=128, I=128, E=8, k=2, I_shared=64, seed=50, routing="gaussian"),
     [(None, None, False, 0), (16, 32, False, 0), (16, 64, True, 8)]),
    (synth.Workload("ragged", T=300, D=384, I=256, E=16, k=4, I_shared=128, seed=51, routing="gaussian"),
     [(None, None, False, 0), (100, 300, False, 0), (128, 256, True, 8)]),
    (synth.Workload("skewed", T=257, D=256, I=384, E=24, k=6, I_shared=192, seed=52, routing="zipf"),
     [(None, None, False, 0), (None, None, True, 0), (200, 400, False, 0)]),
    (synth.Workload("mid", T=2048, D=1024, I=512, E=32, k=8, I_shared=512, seed=53, routing="gaussian"),
     [(None, None, False, 0), (512, 2048, False, 0), (512, 1024, True, 8), (2048, 4096, True, 16)]),
    (synth.Workload("wide", T=2048, D=7168, I=2048, E=16, k=8, I_shared=2048, seed=54, routing="zipf"),
     [(None, None, False, 0), (4096, 8192, True, 16)]),
]


@pytest.mark.parametrize("w,bcs", CASES, ids=[c[0].name for c in CASES])
def test_tiled_weights_bitwise_equal(w, bcs):
    dev = need_gpu()
    from mixture_experts_layer_counts_amd import MoELayer, shape_for, tile_bf16
    inp_dev = to_dev(synth.make_inputs(w), dev)
    tiled = dict(inp_dev, **{n: tile_bf16(inp_dev[n]) for n in ("w_gate", "w_up", "w_down")})
    for b, C, pipeline, mem in bcs:
        say("tiled weights", w.name, "b, C =", b, C, "pipeline", pipeline, mem)
        outs = []
        for wt, weights in ((False, inp_dev), (True, tiled)):
            m = MoELayer(shape_for(w.T, w.D, w.I, w.E, w.k, I_shared=w.I_shared, minibatch_rows=b, ring_rows=C,
                                   pipeline=pipeline, mem_workgroups=mem, weights_tiled=wt), device=dev)
            r = m(inp_dev["x"], inp_dev["w_router"], weights, logits=inp_dev["logits"])
            torch.cuda.synchronize()
            assert m.device_error() == 0
            outs.append(r["out32"].cpu())
        assert torch.equal(outs[0].view(torch.int32), outs[1].view(torch.int32))


MX_CASES = [
    synth.Workload("tiny-mx", T=64, D=128, I=128, E=8, k=2, I_shared=64, seed=55, routing="gaussian"),
    synth.Workload("ragged-mx", T=300, D=384, I=256, E=16, k=4, I_shared=128, seed=56, routing="zipf"),
    synth.Workload("wide-mx", T=1024, D=7168, I=2048, E=12, k=8, I_shared=2048, seed=57, routing="gaussian"),
]


@pytest.mark.parametrize("w", MX_CASES, ids=[w.name for w in MX_CASES])
def test_tiled_mx_weights_bitwise_equal(w):
    dev = need_gpu()
    from mixture_experts_layer_counts_amd import MoELayer, shape_for, tile_mxfp8
    from tests._gpu import mx_weights_dev
    inp_dev = to_dev(synth.make_inputs(w), dev)
    wq = mx_weights_dev(inp_dev)
    tiled = dict(wq, **{n: tile_mxfp8(wq[n]) for n in ("q_gate", "q_up", "q_down")})
    say("tiled MX weights", w.name)
    outs = []
    for wt, weights in ((False, wq), (True, tiled)):
        m = MoELayer(shape_for(w.T, w.D, w.I, w.E, w.k, I_shared=w.I_shared, precision="mxfp8", weights_tiled=wt),
                     device=dev)
        r = m(inp_dev["x"], inp_dev["w_router"], weights, logits=inp_dev["logits"])
        torch.cuda.synchronize()
        assert m.device_error() == 0
        outs.append(r["out32"].cpu())
    assert torch.equal(outs[0].view(torch.int32), outs[1].view(torch.int32))
