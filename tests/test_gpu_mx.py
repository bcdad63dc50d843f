"""GPU parity of the MXFP8 path: the quantiser is bit-exact with the oracle,
and the layer in MXFP8 is within 5e-2 * RMS of the oracle's MXFP8 layer."""

import numpy as np
import pytest
import torch

import synth
from oracle import bf16, mx
from oracle import moe as ref
from tests._gpu import layer, mx_weights_dev, need_gpu, oracle_mx_weights, rel_err, say, to_dev

pytestmark = pytest.mark.gpu


def edge_rows(K, seed):
    """bf16 rows that reach every branch of the encoder: zero blocks, -0.0,
    bf16 subnormals, ties, saturation at 448, tiny and huge block scales."""
    g = torch.Generator().manual_seed(seed)
    rows = [torch.randn(K, generator=g) * 10.0 ** float(e) for e in (-30, -5, -1, 0, 1, 5, 30)]
    z = torch.zeros(K)
    z[K // 2:] = -0.0
    rows.append(z)
    sub = torch.full((K,), 2.0 ** -130)
    sub[::3] = -(2.0 ** -133)
    rows.append(sub)
    mixed = torch.randn(K, generator=g)
    mixed[::32] = 448.0 * 1.5  # block max well above the others: small elements round to subnormals/zero
    rows.append(mixed)
    ties = torch.tensor([(1 + (2 * (i % 8) + 1) / 16) * 2.0 ** ((i // 8) % 4) for i in range(K)])
    ties[::32] = 448.0  # pins X = 0, so the elements above sit exactly on E4M3 rounding midpoints
    rows.append(ties)
    return torch.stack(rows).to(torch.bfloat16)


@pytest.mark.parametrize("rows,K,seed", [(13, 64, 0), (300, 7168, 1), (1, 32, 2), (2048, 2048, 3)])
def test_quantize_bit_exact(rows, K, seed):
    dev = need_gpu()
    from mixture_experts_layer_counts_amd import quantize_mxfp8
    x = (torch.randn(rows, K, generator=torch.Generator().manual_seed(seed)) *
         torch.exp(torch.randn(rows, 1, generator=torch.Generator().manual_seed(seed + 7)) * 4)).to(torch.bfloat16)
    x = torch.cat([x, edge_rows(K, seed)])
    say("mx quantize", tuple(x.shape))
    q, s = quantize_mxfp8(x.to(dev))
    torch.cuda.synchronize()
    qo, so = mx.quantize(bf16.to_f64(synth.bits(x)))
    assert np.array_equal(s.cpu().numpy(), so)
    assert np.array_equal(q.cpu().numpy(), qo)


@pytest.mark.parametrize("G,N,K", [(1, 1, 128), (3, 37, 384), (4, 2048, 7168)])
def test_pack_scales_bit_exact(G, N, K):
    """moe_mxfp8_pack_scales moves the scale byte of (group g, row r, K block
    j) to ((g*(K/128) + j/4)*N + r)*4 + j%4, and nothing else."""
    dev = need_gpu()
    from mixture_experts_layer_counts_amd import pack_mxfp8_scales
    s = torch.randint(0, 256, (G, N, K // 32), dtype=torch.uint8, generator=torch.Generator().manual_seed(G * N))
    say("mx pack scales", (G, N, K))
    got = pack_mxfp8_scales(s.to(dev)).cpu().numpy().reshape(-1)
    torch.cuda.synchronize()
    src = s.numpy()
    g, r, j = np.meshgrid(np.arange(G), np.arange(N), np.arange(K // 32), indexing="ij")
    dst = ((g * (K // 128) + j // 4) * N + r) * 4 + j % 4
    want = np.empty(G * N * (K // 32), dtype=np.uint8)
    want[dst.reshape(-1)] = src.reshape(-1)
    assert np.array_equal(got, want)


# ---------------------------------------------------------------------------
# The layer in MXFP8 (routed experts MX, shared expert bf16) against the oracle
# at 5e-2 * RMS; MX needs D and I to be multiples of 128.
# ---------------------------------------------------------------------------
TOL_MX = 5e-2

MX_CASES = [
    ("tiny-mx", synth.Workload("tiny-mx", T=64, D=128, I=128, E=8, k=2, I_shared=64, seed=30, routing="gaussian"),
     [(None, None), (16, 32), (128, 128)]),
    ("ragged-mx", synth.Workload("ragged-mx", T=300, D=384, I=256, E=16, k=4, I_shared=128, seed=31,
                                 routing="gaussian"), [(None, None), (100, 300), (256, 512)]),
    ("skewed-mx", synth.Workload("skewed-mx", T=257, D=256, I=384, E=24, k=6, I_shared=192, seed=32, routing="zipf"),
     [(None, None), (200, 400)]),
    ("wide-mx", synth.Workload("wide-mx", T=1024, D=1024, I=512, E=48, k=8, I_shared=512, seed=33,
                               routing="gaussian"), [(8192, 8192), (1000, 3000)]),
    ("k16-mx", synth.Workload("k16-mx", T=40, D=128, I=128, E=64, k=16, I_shared=64, seed=34, routing="gaussian"),
     [(None, None), (128, 256)]),
]


@pytest.mark.parametrize("name,w,bcs", MX_CASES, ids=[c[0] for c in MX_CASES])
def test_mx_layer_parity_given_logits(name, w, bcs):
    dev = need_gpu()
    inp = synth.make_inputs(w)
    inp_dev = to_dev(inp, dev)
    say("mx_layer_parity", name, w)
    wq = mx_weights_dev(inp_dev)
    want = ref.forward(synth.bits(inp["x"]), oracle_mx_weights(inp), inp["logits"].numpy(), w.k, precision="mxfp8")
    first = None
    for b, C in bcs:
        say("  b, C =", b, C)
        m = layer(w, dev, b, C, precision="mxfp8")
        r = m(inp_dev["x"], inp_dev["w_router"], wq, logits=inp_dev["logits"])
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


def test_mx_zero_input_gives_zero():
    dev = need_gpu()
    w = synth.Workload("zero-mx", T=96, D=256, I=128, E=8, k=3, I_shared=64, seed=34, routing="gaussian")
    inp = synth.make_inputs(w)
    inp["x"].zero_()
    inp_dev = to_dev(inp, dev)
    say("mx_zero_input")
    m = layer(w, dev, precision="mxfp8")
    r = m(inp_dev["x"], inp_dev["w_router"], mx_weights_dev(inp_dev), logits=inp_dev["logits"])
    torch.cuda.synchronize()
    assert m.device_error() == 0
    assert torch.all(r["out32"] == 0)

