"""GPU parity of the backward pass (training) against the fp64 backward oracle.

The HIP backward (through the C ABI) takes bf16 tokens, weights and dy and
accumulates in fp32; the oracle differentiates the forward oracle in fp64 on
the same bf16-representable values.  Gradients have no fixed scale (a weight
gradient sums over every token), so the bar is relative to each tensor's
largest reference entry: max-abs error <= 3e-2 and mean-abs error <= 3e-3 of
max|ref|, the bf16 forward bars applied to the normalised tensor.  The
arithmetic behind it: every backward GEMM operand is rounded to bf16 once
(relative 2^-9 = 2e-3), so a dot product of n terms carries a relative error
of about 2e-3 of its typical term sum, and the attention probabilities are
rounded to bf16 for the dV and dK products as in the forward.
"""
import numpy as np
import pytest
import torch

import synth
import oracle
from oracle import vswin_bwd as ob
import shifted_window_attention_amd as vs

from helpers import dev, dev_params, host64, say

pytestmark = pytest.mark.gpu

REL_MAX, REL_MEAN = 3e-2, 3e-3


def check_rel(got, ref, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite"
    scale = float(np.abs(ref).max())
    err = np.abs(got - ref)
    mx, mean = float(err.max()) / scale, float(err.mean()) / scale
    say(f"  {what}: scale {scale:.3e} max-rel {mx:.3e} mean-rel {mean:.3e}")
    assert mx <= REL_MAX and mean <= REL_MEAN, f"{what}: max {mx:.3e} mean {mean:.3e} (of {scale:.3e})"


def _params(C, heads, window, init, seed):
    rows = (2 * window[0] - 1) * (2 * window[1] - 1) * (2 * window[2] - 1)
    return synth.gen_block_params(C, heads, rows, 4, np.random.SeedSequence(seed), "bf16", init)


def _tok(shape, seed, scale=1.0):
    return synth.round_bf16((scale * np.random.default_rng(seed).standard_normal(shape)).astype(np.float32))


CASES = [
    # name, B, size, C, heads, window, shift, init, flags
    ("shifted", 1, (16, 14, 14), 64, 2, (8, 7, 7), (4, 3, 3), "stress", 0),
    ("regular", 1, (16, 14, 14), 64, 2, (8, 7, 7), (0, 0, 0), "stress", 0),
    ("padded shifted C=96", 1, (16, 12, 13), 96, 3, (8, 7, 7), (4, 3, 3), "stress", 0),
    ("B=2 spec init", 2, (16, 14, 21), 96, 3, (8, 7, 7), (4, 3, 3), "spec", 0),
    ("mask -100 padded", 1, (16, 12, 13), 64, 2, (8, 7, 7), (4, 3, 3), "stress", vs.F_MASK_M100),
    ("window 4 temporal shift 2", 1, (16, 14, 14), 64, 2, (4, 7, 7), (2, 3, 3), "stress", 0),
    ("Swin-B C=128 padded", 1, (16, 12, 13), 128, 4, (8, 7, 7), (4, 3, 3), "stress", 0),
    ("Swin-L C=192", 1, (16, 14, 14), 192, 6, (8, 7, 7), (4, 3, 3), "stress", 0),
    ("window 16 shifted", 1, (16, 14, 14), 96, 3, (16, 7, 7), (8, 3, 3), "stress", 0),
    ("window 4 spatial-only shift", 1, (8, 14, 14), 64, 2, (4, 7, 7), (0, 3, 3), "stress", 0),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_window_msa_bwd(case):
    name, B, size, C, heads, window, shift, init, flags = case
    say(f"window_msa backward {name}")
    p = _params(C, heads, window, init, 41)
    xn = _tok((B, *size, C), 5)
    dy = _tok((B, *size, C), 6)
    dx, g = vs.vswin_window_msa_bwd(dev(xn, "bf16"), dev_params(p, "bf16"), dev(dy, "bf16"), heads, window, shift,
                                    flags=flags)
    torch.cuda.synchronize()
    rdx, rg = ob.window_msa_bwd(xn, p, heads, window, shift, dy, mask_m100=bool(flags & vs.F_MASK_M100))
    check_rel(host64(dx), rdx, f"{name} dx_norm")
    for k in vs.MSA_GRAD_NAMES:
        check_rel(host64(g[k]), rg[k], f"{name} d{k}")


@pytest.mark.parametrize("case", CASES[:9], ids=[c[0] for c in CASES[:9]])
def test_block_bwd(case):
    name, B, size, C, heads, window, shift, init, flags = case
    say(f"block backward {name}")
    p = _params(C, heads, window, init, 43)
    x = _tok((B, *size, C), 7)
    dy = _tok((B, *size, C), 8)
    dx, g = vs.vswin_block_bwd(dev(x, "bf16"), dev_params(p, "bf16"), dev(dy, "bf16"), heads, window, shift,
                               flags=flags)
    torch.cuda.synchronize()
    rdx, rg = ob.block_bwd(x, p, heads, window, shift, dy, mask_m100=bool(flags & vs.F_MASK_M100))
    check_rel(host64(dx), rdx, f"{name} dx")
    for k in vs.GRAD_NAMES:
        check_rel(host64(g[k]), rg[k], f"{name} d{k}")


@pytest.mark.parametrize("shift", [(0, 0, 0), (4, 3, 3)])
def test_block_bwd_stage1_shape(shift):
    """Swin-T stage 1 (1,16,56,56,96), 3 heads, the size the bench times."""
    say(f"block backward, Swin-T stage 1, shift {shift}")
    s = synth.WORKLOADS[2].shape
    x, params = synth.gen_workload(2)
    p = params[0 if shift == (0, 0, 0) else 1]
    dy = _tok(x.shape, 9)
    dx, g = vs.vswin_block_bwd(dev(x, "bf16"), dev_params(p, "bf16"), dev(dy, "bf16"), s.heads, s.window, shift)
    torch.cuda.synchronize()
    rdx, rg = ob.block_bwd(x, p, s.heads, s.window, shift, dy)
    check_rel(host64(dx), rdx, "stage-1 dx")
    for k in vs.GRAD_NAMES:
        check_rel(host64(g[k]), rg[k], f"stage-1 d{k}")


def test_bwd_deterministic_and_empty_batch():
    """Two backward calls give bitwise-identical gradients (no atomics on the
    path), and an empty batch sets every gradient to zero."""
    C, heads, window, shift = 96, 3, (8, 7, 7), (4, 3, 3)
    p = _params(C, heads, window, "stress", 47)
    x = dev(_tok((1, 16, 14, 14, C), 10), "bf16")
    dy = dev(_tok((1, 16, 14, 14, C), 11), "bf16")
    w = dev_params(p, "bf16")
    dx1, g1 = vs.vswin_block_bwd(x, w, dy, heads, window, shift)
    dx2, g2 = vs.vswin_block_bwd(x, w, dy, heads, window, shift)
    torch.cuda.synchronize()
    assert torch.equal(dx1, dx2)
    for k in vs.GRAD_NAMES:
        assert torch.equal(g1[k], g2[k]), k
    e = torch.empty((0, 16, 14, 14, C), dtype=torch.bfloat16, device="cuda")
    filled = {k: torch.full(v.shape, 7.0, device="cuda") for k, v in g1.items()}
    dx0, g0 = vs.vswin_block_bwd(e, w, e, heads, window, shift, grads=filled)
    torch.cuda.synchronize()
    assert dx0.shape == e.shape
    for k in vs.GRAD_NAMES:
        assert torch.count_nonzero(g0[k]) == 0, k
