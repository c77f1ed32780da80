"""Pins of the oracle's backbone composition and of its -100 mask branch
(CPU only).

backbone(): the pages fix the stage structure -- a 2x4x4 patch embedding,
four stages of blocks with no temporal downsampling, spatial halving and
width doubling by patch merging between stages, heads = C / 32 (Video Swin
Transformer, §3.1 and Method steps 1-3; §3.3) -- and that blocks come in
regular-then-shifted pairs (eq. 1).  At stage 4 the 7x7 token grid is no
larger than the 7x7 window, so the window/shift clamp (Pitfalls, "Temporal
window and token count") must leave only the temporal shift.

mask_m100: the published code adds -100 to the logits of pairs from
different regions instead of excluding them (paper-vs-code notes, "Mask
value and padding").  At ordinary logits that is exclusion up to e^-100; on
a hand-built window where one cross-region offset carries a bias of +150 the
weights have a closed form.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
from oracle import vswin as ov

SWIN_T = synth.WORKLOADS[5].backbone


def _record_blocks(monkeypatch):
    """Replace the oracle's block by a recorder (identity on x) and its patch
    merge by a shape-only stand-in, so that backbone()'s call sequence can be
    read without computing the blocks."""
    calls = []

    def fake_block(x, p, heads, window, shift, **kw):
        calls.append(("block", tuple(x.shape), heads, tuple(window), tuple(shift), p))
        return x, x

    def fake_merge(x, m, eps=1e-5):
        calls.append(("merge", tuple(x.shape)))
        B, T, H, W, C = x.shape
        return np.zeros((B, T, (H + 1) // 2, (W + 1) // 2, m["w"].shape[0]))

    monkeypatch.setattr(ov, "block", fake_block)
    monkeypatch.setattr(ov, "patch_merge", fake_merge)
    return calls


def test_backbone_stage_sequence_swin_t(monkeypatch):
    """Swin-T on a 32x224x224 clip: embed to (16,56,56,96); stages of depth
    2,2,6,2 at (16,56,56,96), (16,28,28,192), (16,14,14,384), (16,7,7,768)
    with 3,6,12,24 heads; a merge after each of the first three stages;
    blocks alternate shift 0 and half the window inside every stage."""
    cfg = SWIN_T
    params = synth.gen_backbone_params(cfg, 5, "fp32")
    calls = _record_blocks(monkeypatch)
    video = np.zeros((1, 3, 32, 224, 224))
    out = ov.backbone(video, params, cfg)
    assert out.shape == (1, 16, 7, 7, 768)
    expect = []
    T, H, C = 16, 56, 96
    for i, depth in enumerate((2, 2, 6, 2)):
        for j in range(depth):
            expect.append(("block", (1, T, H, H, C), C // 32, (8, 7, 7), (0, 0, 0) if j % 2 == 0 else (4, 3, 3)))
        if i < 3:
            expect.append(("merge", (1, T, H, H, C)))
            H, C = H // 2, 2 * C            # time is never downsampled
    got = [c[:5] if c[0] == "block" else c for c in calls]
    assert got == expect
    # each block gets its own stage's parameters, in order
    blocks = [c for c in calls if c[0] == "block"]
    flat = [p for st in params["stages"] for p in st]
    assert all(b[5] is p for b, p in zip(blocks, flat)) and len(blocks) == len(flat) == 12


def test_backbone_stage4_clamp():
    """Stage 4 (7x7 tokens, window 8x7x7): the spatial window covers the whole
    grid, so only the temporal shift survives: (8,7,7) / (4,0,0); the first
    three stages keep (4,3,3)."""
    for H, eff in [(56, (4, 3, 3)), (28, (4, 3, 3)), (14, (4, 3, 3)), (7, (4, 0, 0))]:
        win, sh = ov.effective_window((16, H, H), (8, 7, 7), (4, 3, 3))
        assert win == (8, 7, 7) and sh == eff
        g = ov.Geometry(1, (16, H, H), (8, 7, 7), (4, 3, 3))
        assert g.shift == eff and g.nW == 2 * (H // 7) ** 2


def _tiny_cfg():
    return dict(B=1, in_chans=3, frames=8, height=56, width=56, patch=(2, 4, 4), embed_dim=16,
                depths=(2, 2, 2, 2), heads=(1, 1, 2, 2), window=(2, 7, 7), shift=(1, 3, 3), mlp_ratio=4)


def test_backbone_identity_blocks_reduce_to_embed_merges_norm():
    """With every block's linear weights and biases zero, q = k = v = 0 and the
    MLP output is 0, so each block is the identity (eq. 1).  The backbone is
    then Conv3d(k = s = patch) -> three merges -> final LayerNorm, computed
    here with torch's own conv3d, pad, layer_norm and linear (the 7x7 grid of
    the third merge is odd: zero-padded at the end, as the CSDN walk-through's
    PatchMerging pads odd sizes)."""
    cfg = _tiny_cfg()
    params = synth.gen_backbone_params(cfg, 3, "fp32", init="stress")
    for st in params["stages"]:
        for p in st:
            for n in ("qkv_w", "qkv_b", "proj_w", "proj_b", "fc1_w", "fc1_b", "fc2_w", "fc2_b"):
                p[n] = np.zeros_like(p[n])
    video = np.random.default_rng(2).standard_normal((1, 3, 8, 56, 56))
    got = ov.backbone(video, params, cfg)
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    x = F.conv3d(t(video), t(params["embed_w"]), t(params["embed_b"]), stride=(2, 4, 4))
    x = x.permute(0, 2, 3, 4, 1)
    for m in params["merges"]:
        x = F.pad(x, (0, 0, 0, x.shape[3] % 2, 0, x.shape[2] % 2))     # odd H or W: zeros at the end
        x = torch.cat([x[:, :, 0::2, 0::2], x[:, :, 1::2, 0::2], x[:, :, 0::2, 1::2], x[:, :, 1::2, 1::2]], -1)
        x = F.linear(F.layer_norm(x, (x.shape[-1],), t(m["ln_g"]), t(m["ln_b"]), 1e-5), t(m["w"]))
    x = F.layer_norm(x, (x.shape[-1],), t(params["norm_g"]), t(params["norm_b"]), 1e-5)
    assert got.shape == (1, 4, 2, 2, 128)
    assert np.abs(got - x.numpy()).max() <= 1e-12


def test_backbone_rejects_swapped_pair_order(monkeypatch):
    """A backbone whose pairs run shifted-then-regular differs from the
    oracle's beyond the bf16 bar at stress init, so the comparison would
    catch a swapped order."""
    cfg = _tiny_cfg()
    params = synth.gen_backbone_params(cfg, 4, "fp32", init="stress")
    video = np.random.default_rng(3).standard_normal((1, 3, 8, 56, 56))
    ref = ov.backbone(video, params, cfg)
    real_block = ov.block
    half = tuple(w // 2 for w in cfg["window"])

    def swapped(x, p, heads, window, shift, **kw):
        return real_block(x, p, heads, window, half if tuple(shift) == (0, 0, 0) else (0, 0, 0), **kw)

    monkeypatch.setattr(ov, "block", swapped)
    mutant = ov.backbone(video, params, cfg)
    assert np.abs(mutant - ref).max() > 10 * 3e-2


# ----------------------------------------------------------------------------- -100 mask
def test_m100_equals_exclusion_at_ordinary_logits():
    """Logits of order 1: the masked terms carry a factor e^-100 ~ 4e-44, so
    the -100 form equals exclusion to rounding (shifted block with pads)."""
    C, heads, window, shift = 32, 2, (2, 7, 7), (1, 3, 3)
    p = synth.gen_block_params(C, heads, 3 * 13 * 13, 4, np.random.SeedSequence(8), "fp32", "stress")
    x = np.random.default_rng(4).standard_normal((2, 4, 12, 13, C))
    a = ov.window_msa(x, p, heads, window, shift, mask_m100=True)
    b = ov.window_msa(x, p, heads, window, shift)
    assert np.abs(a - b).max() <= 1e-12
    # the geometry really takes the masked path (shifted, with pads)
    g = ov.Geometry(2, (4, 12, 13), window, shift)
    assert g.use_mask and g.has_pad


def test_m100_closed_form_on_built_window():
    """One channel, q = k = 0, v = x, identity projection: logits are the bias
    alone.  Grid (T,H,W) = (1,1,4), window (1,1,2), shift (0,0,1): the rolled
    axis holds original positions 1,2 | 3,0 (roll by -1), so the second
    window straddles the wrap and its two tokens lie in different regions.
    The table has rows for dw = query - key in {-1, 0, +1}; dw = +1 gets +150.
      window (1, 2): token 2 attends to token 1 with logit 150, itself with 0;
                     token 1 sees token 2 with logit 0 (dw = -1);
      window (3, 0): token 0 (the second slot) sees token 3 with 150 - 100,
                     token 3 sees token 0 with 0 - 100 (cross-region).
    """
    x = np.array([0.3, -1.1, 0.7, 2.0]).reshape(1, 1, 1, 4, 1)
    p = {"qkv_w": np.array([[0.0], [0.0], [1.0]]), "qkv_b": np.zeros(3),
         "proj_w": np.array([[1.0]]), "proj_b": np.zeros(1),
         "rpb_table": np.array([[0.0], [0.0], [150.0]])}          # row = dw + 1
    y = ov.window_msa(x, p, 1, (1, 1, 2), (0, 0, 1), mask_m100=True).ravel()
    x0, x1, x2, x3 = x.ravel()
    sig = lambda z: 1.0 / (1.0 + math.exp(-z))
    expect = [
        sig(50.0) * x3 + (1 - sig(50.0)) * x0,          # token 0: 150 - 100 towards token 3
        0.5 * x1 + 0.5 * x2,                             # token 1: logits 0, 0
        sig(150.0) * x1 + (1 - sig(150.0)) * x2,         # token 2: 150 towards token 1
        (1 - sig(-100.0)) * x3 + sig(-100.0) * x0,       # token 3: 0 - 100 towards token 0
    ]
    assert np.abs(y - np.array(expect)).max() <= 1e-15
    # exclusion instead: the straddling window's tokens see only themselves
    y_ex = ov.window_msa(x, p, 1, (1, 1, 2), (0, 0, 1)).ravel()
    assert y_ex[0] == x0 and y_ex[3] == x3
    assert abs(y_ex[2] - expect[2]) <= 1e-15 and abs(y_ex[1] - expect[1]) <= 1e-15
