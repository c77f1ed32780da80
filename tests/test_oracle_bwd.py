"""Pins of the fp64 backward oracle (CPU only).

The backward oracle is checked against central finite differences of the
forward oracle: for a random direction v of one input (x or a weight),
<grad, v> must equal (L(t + e v) - L(t - e v)) / (2 e) with L = <dy, y>.
The forward oracle itself is pinned elsewhere (closed forms, brute-force
global attention, library special cases), so a wrong sign, a dropped term, a
transposed operand or a mis-indexed table scatter in the backward fails here.
"""
import numpy as np
import pytest

import synth
from oracle import vswin as ov
from oracle import vswin_bwd as ob

NAMES = ["ln1_g", "ln1_b", "qkv_w", "qkv_b", "proj_w", "proj_b", "rpb_table",
         "ln2_g", "ln2_b", "fc1_w", "fc1_b", "fc2_w", "fc2_b"]

CASES = [
    # B, size, C, heads, window, shift, flags
    (1, (4, 4, 6), 8, 2, (2, 2, 3), (1, 1, 1), {}),                      # shifted, no pads
    (1, (4, 4, 6), 8, 2, (2, 2, 3), (0, 0, 0), {}),                      # regular
    (2, (3, 5, 4), 8, 2, (2, 2, 2), (1, 1, 1), {}),                      # pads masked, B = 2
    (1, (3, 5, 4), 8, 1, (2, 2, 2), (1, 1, 1), {"pad_visible": True}),   # pads visible
    (1, (4, 4, 6), 8, 2, (2, 2, 3), (1, 1, 1), {"mask_m100": True}),     # -100 mask
]


def _setup(B, size, C, heads, window, seed):
    rows = ov.table_rows(window)
    p = synth.gen_block_params(C, heads, rows, 4, np.random.SeedSequence(seed), "fp32", "stress")
    p = {k: v.astype(np.float64) for k, v in p.items()}
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, *size, C))
    dy = rng.standard_normal((B, *size, C))
    return x, p, dy


@pytest.mark.parametrize("case", CASES, ids=[str(i) for i in range(len(CASES))])
def test_block_bwd_finite_differences(case):
    B, size, C, heads, window, shift, flags = case
    x, p, dy = _setup(B, size, C, heads, window, 7)
    dx, grads = ob.block_bwd(x, p, heads, window, shift, dy, **flags)
    assert set(grads) == set(NAMES)

    def loss(xx, pp):
        return float((dy * ov.block(xx, pp, heads, window, shift, **flags)[1]).sum())

    rng = np.random.default_rng(11)
    eps = 1e-5
    for name in ["x"] + NAMES:
        base = x if name == "x" else p[name]
        v = rng.standard_normal(base.shape)
        if name == "x":
            lp, lm = loss(x + eps * v, p), loss(x - eps * v, p)
            an = float((dx * v).sum())
        else:
            pp, pm = dict(p), dict(p)
            pp[name] = p[name] + eps * v
            pm[name] = p[name] - eps * v
            lp, lm = loss(x, pp), loss(x, pm)
            an = float((grads[name] * v).sum())
        fd = (lp - lm) / (2 * eps)
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (name, fd, an)


def test_attention_bwd_table_scatter_single_offset():
    """The table gradient lands only on rows some pair's offset uses: rows no
    pair of the window maps to get exactly zero, the offset-0 row (fed by the
    N diagonal pairs alone) does not."""
    B, size, C, heads, window, shift = 1, (2, 2, 2), 4, 1, (2, 2, 2), (0, 0, 0)
    x, p, dy = _setup(B, size, C, heads, window, 3)
    _, grads = ob.block_bwd(x, p, heads, window, shift, dy)
    rel = ov.relative_index(window)
    # rows never used by a pair get exactly zero
    unused = np.setdiff1d(np.arange(ov.table_rows(window)), np.unique(rel))
    assert np.all(grads["rpb_table"][unused] == 0.0)
    # the centre row (offset 0) is used by the N diagonal pairs only
    centre = rel[0, 0]
    assert (rel == centre).sum() == rel.shape[0]
    assert grads["rpb_table"][centre, 0] != 0.0


def test_gelu_and_layernorm_bwd_special_values():
    """GELU'(0) = 1/2; LN's input gradient sums to 0 over the features (output
    invariant to a shift of x) and, without eps and with g = 1, is orthogonal
    to x - mean (invariant to a scale)."""
    assert ob.gelu_bwd(np.array([0.0]), np.array([1.0]))[0] == pytest.approx(0.5)
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 16))
    dy = rng.standard_normal((5, 16))
    dx, dg, db = ob.layer_norm_bwd(x, np.ones(16), dy)
    assert np.abs(dx.sum(axis=1)).max() < 1e-12
    xh = (x - x.mean(1, keepdims=True)) / np.sqrt(x.var(1, keepdims=True) + 1e-5)
    # scale invariance holds exactly only without eps
    dx0, _, _ = ob.layer_norm_bwd(x, np.ones(16), dy, eps=0.0)
    assert np.abs((dx0 * (x - x.mean(1, keepdims=True))).sum(axis=1)).max() < 1e-9
    assert np.allclose(db, dy.sum(0)) and np.allclose(dg, (dy * xh).sum(0))
