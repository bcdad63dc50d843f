"""GPU parity of the MXFP8 path: the quantiser is bit-exact with the oracle."""

import numpy as np
import pytest
import torch

import synth
from oracle import bf16, mx
from tests._gpu import need_gpu, say

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
