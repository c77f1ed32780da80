"""GPU parity of the inference pieces around the backbone: classification
head, multi-view probability average, 2D -> 3D inflation (through the C ABI),
against the fp64 oracle on the same seeded inputs.

Bars: the head and the view average accumulate in fp32 from exact inputs, so
their error is fp32 rounding over at most C (head) or K (softmax) terms: the
head within 1e-4 of max|logit|, probabilities within 1e-6.  Inflation by a
power-of-two slot count and the table repetition are exact (bit-exact
compare); by pt = 3 the quotient is rounded once in fp32 (then to bf16), one
unit in the last place at most.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import vswin as ov
import shifted_window_attention_amd as vs

from helpers import dev, host64, say, tdt

pytestmark = pytest.mark.gpu


def _vals(shape, seed, dtype, scale=1.0):
    a = (scale * np.random.default_rng(seed).standard_normal(shape)).astype(np.float32)
    return synth.round_bf16(a) if dtype == "bf16" else a


HEAD_CASES = [
    # name, B, token grid, C, K, dtype
    ("Swin-T stage 4, 400 classes", 2, (8, 7, 7), 768, 400, "bf16"),
    ("Swin-B stage 4, B=3", 3, (8, 7, 7), 1024, 400, "bf16"),
    ("fp32 small", 2, (2, 3, 3), 32, 10, "fp32"),
    ("ragged: one token, C=100, K=33", 1, (1, 1, 1), 100, 33, "bf16"),
    ("K not a multiple of 32, 600 classes", 2, (4, 7, 7), 96, 600, "fp32"),
]


@pytest.mark.parametrize("case", HEAD_CASES, ids=[c[0] for c in HEAD_CASES])
def test_head(case):
    name, B, grid, C, K, dtype = case
    say(f"head {name}")
    x = _vals((B, *grid, C), 1, dtype)
    w = _vals((K, C), 2, dtype, 0.02)
    b = _vals((K,), 3, dtype, 0.02)
    got = vs.vswin_head_fwd(dev(x, dtype), dev(w, dtype), dev(b, dtype))
    torch.cuda.synchronize()
    ref = ov.head(x, w.astype(np.float64), b.astype(np.float64))
    err = np.abs(host64(got) - ref).max()
    assert err <= 1e-4 * np.abs(ref).max() + 1e-7, (name, err, np.abs(ref).max())
    # no bias, and bit-identical on a second call
    got0 = vs.vswin_head_fwd(dev(x, dtype), dev(w, dtype), None)
    got1 = vs.vswin_head_fwd(dev(x, dtype), dev(w, dtype), None)
    torch.cuda.synchronize()
    assert torch.equal(got0, got1)
    ref0 = ov.head(x, w.astype(np.float64), None)
    assert np.abs(host64(got0) - ref0).max() <= 1e-4 * np.abs(ref0).max() + 1e-7


def test_head_empty_batch():
    x = torch.empty((0, 8, 7, 7, 768), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((400, 768), dtype=torch.bfloat16, device="cuda")
    y = vs.vswin_head_fwd(x, w)
    torch.cuda.synchronize()
    assert y.shape == (0, 400)


@pytest.mark.parametrize("B,V,K,scale", [(2, 12, 400, 3.0), (3, 1, 10, 1.0), (1, 50, 8192, 8.0), (4, 4, 257, 30.0),
                                         (1, 300, 700, 2.0)])
def test_multiview_average(B, V, K, scale):
    say(f"multiview B={B} V={V} K={K}")
    z = _vals((B, V, K), 4 + K, "fp32", scale)
    got = vs.vswin_multiview_average(torch.from_numpy(z).cuda())
    torch.cuda.synchronize()
    ref = ov.multiview_average(z)
    assert np.abs(host64(got) - ref).max() <= 1e-6
    np.testing.assert_allclose(host64(got).sum(axis=-1), 1.0, atol=1e-5)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("pt", [2, 4, 3])
def test_inflate_patch_embed(dtype, pt):
    w2 = _vals((96, 3, 4, 4), 5, dtype, 0.02)
    got = host64(vs.vswin_inflate_patch_embed(dev(w2, dtype), pt))
    torch.cuda.synchronize()
    ref = ov.inflate_patch_embed(w2.astype(np.float64), pt)
    assert got.shape == ref.shape == (96, 3, pt, 4, 4)
    if pt in (2, 4):
        assert np.array_equal(got, ref)
    else:
        ulp = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -23
        assert np.all(np.abs(got - ref) <= ulp * np.abs(ref) + 1e-30)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("P,M,heads", [(4, 7, 3), (8, 7, 4), (2, 3, 1)])
def test_inflate_bias_table(dtype, P, M, heads):
    t2 = _vals(((2 * M - 1) ** 2, heads), 6, dtype, 0.02)
    got = host64(vs.vswin_inflate_bias_table(dev(t2, dtype), P))
    torch.cuda.synchronize()
    ref = ov.inflate_bias_table(t2.astype(np.float64), P)
    assert np.array_equal(got, ref)
