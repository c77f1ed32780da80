"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

Each test checks the oracle against something other than itself: values the
pages print (tab. 4 / tab. 5 counts, window counts), brute-force global
attention written in original coordinates with no roll or partition,
exact identities, library routines for the special cases, and mutation
sensitivity (a planted mistake in the oracle must be caught).
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import vswin as ov
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")

BACKBONE_T = dict(B=1, in_chans=3, frames=32, height=224, width=224, patch=(2, 4, 4),
                  embed_dim=96, depths=(2, 2, 6, 2), heads=(3, 6, 12, 24),
                  window=(8, 7, 7), shift=(4, 3, 3), mlp_ratio=4)


# ---------------------------------------------------------------- helpers
def _params(C, heads, window, seed=0, init="stress", dtype="fp32"):
    rows = (2 * window[0] - 1) * (2 * window[1] - 1) * (2 * window[2] - 1)
    p = synth.gen_block_params(C, heads, rows, 4, np.random.SeedSequence(seed), dtype, init)
    return {k: v.astype(np.float64) for k, v in p.items()}


def _tokens(B, T, H, W, C, seed=1):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((B, T, H, W, C))


def _cells(n, w, s):
    """Cell id of each original coordinate of one axis: the offset grid
    [0,s), [s,s+w), ..., [np-w+s, np) of the shifted windows (s=0: plain grid)."""
    npad = -(-n // w) * w
    o = np.arange(n)
    if s == 0:
        return o // w
    return np.where(o < s, 0, (o - s) // w + 1)


def _clamp(size, window, shift):
    win, sh = [], []
    for n, w, s in zip(size, window, shift):
        if n <= w:
            win.append(n); sh.append(0)
        else:
            win.append(w); sh.append(s)
    return win, sh


def brute_force_msa(xn, p, heads, window, shift):
    """Global attention over all real tokens of each clip, with an explicit
    block mask in ORIGINAL coordinates: token i sees token j iff they share a
    cell of the (offset) window grid on every axis.  Bias is read for the
    original coordinate offset.  No roll, no pad, no partition."""
    B, T, H, W, C = xn.shape
    win, sh = _clamp((T, H, W), window, shift)
    d = C // heads
    ct, ch, cw = (_cells(n, w, s) for n, w, s in zip((T, H, W), win, sh))
    tt, hh, ww = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    coord = np.stack([tt.ravel(), hh.ravel(), ww.ravel()], 1)
    cell = np.stack([ct[coord[:, 0]], ch[coord[:, 1]], cw[coord[:, 2]]], 1)
    same = (cell[:, None, :] == cell[None, :, :]).all(-1)
    dlt = coord[:, None, :] - coord[None, :, :]
    P0, Mh0, Mw0 = window
    rows = ((dlt[..., 0] + P0 - 1) * (2 * Mh0 - 1) * (2 * Mw0 - 1)
            + (dlt[..., 1] + Mh0 - 1) * (2 * Mw0 - 1) + (dlt[..., 2] + Mw0 - 1))
    rows = np.where(same, rows, 0)          # pairs in different cells are masked anyway
    out = np.zeros_like(xn)
    for b in range(B):
        x = xn[b].reshape(-1, C)
        qkv = x @ p["qkv_w"].T + p["qkv_b"]
        o = np.zeros((x.shape[0], C))
        for h in range(heads):
            q = qkv[:, h * d:(h + 1) * d]
            k = qkv[:, C + h * d:C + (h + 1) * d]
            v = qkv[:, 2 * C + h * d:2 * C + (h + 1) * d]
            s = q @ k.T / math.sqrt(d) + p["rpb_table"][rows, h]
            s = np.where(same, s, -np.inf)
            s -= s.max(1, keepdims=True)
            e = np.exp(s)
            o[:, h * d:(h + 1) * d] = (e / e.sum(1, keepdims=True)) @ v
        out[b] = (o @ p["proj_w"].T + p["proj_b"]).reshape(T, H, W, C)
    return out


# ---------------------------------------------------------------- P-d closed forms
def test_tab5_and_tab4_flops_reproduced():
    g = json.load(open(GOLDEN))
    for row in g["tab5_backbone_gmacs"]:
        cfg = dict(BACKBONE_T, frames=row["frames"], window=(row["temporal_window"], 7, 7))
        gmacs = oracle.backbone_macs(cfg)["total"] / 1e9
        assert round(gmacs) == row["printed_G"], (row, gmacs)
        assert abs(gmacs - row["printed_G"]) < 0.35


def test_tab4_parameter_count():
    g = json.load(open(GOLDEN))["tab4_params_M"]
    n = oracle.backbone_params(BACKBONE_T, num_classes=g["num_classes"]) / 1e6
    assert round(n, 1) == g["printed"]


@pytest.mark.parametrize("i", range(4))
def test_window_counts(i):
    row = json.load(open(GOLDEN))["window_counts"][i]
    assert oracle.num_windows(row["B"], row["size"], row["window"]) == row["count"]
    g = ov.Geometry(row["B"], row["size"], row["window"], [w // 2 for w in row["window"]])
    assert g.nW == row["count"]        # the shifted block keeps the window count (§3.2)


def test_masked_window_count_stage1():
    # shifted block of the Swin-T stage-1 grid: every window that is last along
    # some axis holds two regions; 128 - 1*7*7 = 79 of them
    g = ov.Geometry(1, (16, 56, 56), (8, 7, 7), (4, 3, 3))
    masked = sum(len(set(l.tolist())) > 1 for l in g.win_labels)
    assert masked == 79
    g0 = ov.Geometry(1, (16, 56, 56), (8, 7, 7), (0, 0, 0))
    assert not g0.use_mask


def test_block_macs_split():
    m = oracle.block_macs(1, (16, 56, 56), 96, 3, (8, 7, 7), (0, 0, 0))
    L = 16 * 56 * 56
    assert m["qk"] == m["av"] == 128 * 3 * 392 * 392 * 32
    assert m["total"] == 12 * L * 96 * 96 + 2 * L * 392 * 96
    assert abs(2 * m["total"] / 1e9 - 18.65) < 0.01


# ---------------------------------------------------------------- P-a brute force
CASES = [
    # B, (T,H,W), C, heads, window, shift
    (1, (4, 14, 14), 32, 2, (2, 7, 7), (1, 3, 3)),     # fp32 smoke geometry
    (1, (4, 14, 14), 32, 2, (2, 7, 7), (0, 0, 0)),
    (2, (5, 9, 11), 16, 2, (2, 4, 3), (1, 2, 1)),      # padded on every axis
    (1, (6, 8, 7), 16, 1, (4, 3, 3), (2, 1, 1)),
    (1, (3, 5, 5), 16, 2, (8, 7, 7), (4, 3, 3)),       # clamped to the grid
    (1, (8, 7, 14), 16, 2, (8, 7, 7), (4, 3, 3)),      # equality clamp on T and H
]


@pytest.mark.parametrize("case", CASES)
def test_windowed_equals_bruteforce_global(case):
    B, size, C, heads, window, shift = case
    p = _params(C, heads, window, seed=3)
    xn = _tokens(B, *size, C, seed=4)
    got = oracle.window_msa(xn, p, heads, window, shift)
    ref = brute_force_msa(xn, p, heads, window, shift)
    assert np.max(np.abs(got - ref)) < 1e-12


# ---------------------------------------------------------------- P-b identities
@pytest.mark.parametrize("case", CASES)
def test_partition_roll_pad_identities(case):
    B, size, C, heads, window, shift = case
    g = ov.Geometry(B, size, window, shift)
    x = _tokens(B, *size, 3, seed=5)
    u = ov.pad_end(x, g.padded)
    r = ov.roll3(u, [-s for s in g.shift])
    w = ov.partition(r, g.window)
    assert w.shape == (g.nW, g.N, 3)
    back = ov.crop(ov.roll3(ov.reverse(w, B, g.padded, g.window), g.shift), g.size)
    assert np.array_equal(back, x)
    assert np.array_equal(ov.roll3(ov.roll3(u, g.shift), [-s for s in g.shift]), u)
    m = g.index_map()
    L = B * int(np.prod(size))
    real = m[m >= 0]
    assert np.array_equal(np.sort(real), np.arange(L))            # a permutation of real tokens
    assert (m < 0).sum() == g.nW * g.N - L
    assert np.array_equal(w.reshape(-1, 3)[m.ravel() >= 0], x.reshape(-1, 3)[real])


def test_roll_direction_matches_pages():
    # roll by -s: position r holds original (r + s) mod n (torch/numpy semantics)
    a = np.arange(7)[None, :, None, None, None] * np.ones((1, 7, 1, 1, 1))
    r = ov.roll3(a, (-3, 0, 0))
    assert r[0, 0, 0, 0, 0] == 3 and r[0, 4, 0, 0, 0] == 0


# ---------------------------------------------------------------- P-c mask / locality
def test_cross_region_pairs_have_zero_weight():
    B, size, C, heads, window, shift = 1, (4, 14, 14), 16, 2, (2, 7, 7), (1, 3, 3)
    p = _params(C, heads, window, seed=7)
    x = _tokens(B, *size, C, seed=8)
    g = ov.Geometry(B, size, window, shift)
    m = g.index_map()
    lab = g.win_labels
    # a masked window: last along every axis
    w = [i for i in range(g.nW) if len(set(lab[i].tolist())) > 1][-1]
    i_slot = 0
    j_slot = int(np.nonzero(lab[w] != lab[w][i_slot])[0][0])
    ti, tj = int(m[w, i_slot]), int(m[w, j_slot])
    y0 = oracle.window_msa(x, p, heads, window, shift).reshape(-1, C)
    x2 = x.reshape(-1, C).copy()
    x2[tj] += 10.0
    y1 = oracle.window_msa(x2.reshape(x.shape), p, heads, window, shift).reshape(-1, C)
    assert np.array_equal(y0[ti], y1[ti])                      # bitwise unchanged
    assert not np.array_equal(y0[tj], y1[tj])
    # same region, same window: must change
    k_slot = int(np.nonzero((lab[w] == lab[w][i_slot]) & (np.arange(g.N) != i_slot))[0][0])
    x3 = x.reshape(-1, C).copy()
    x3[int(m[w, k_slot])] += 10.0
    y3 = oracle.window_msa(x3.reshape(x.shape), p, heads, window, shift).reshape(-1, C)
    assert not np.array_equal(y0[ti], y3[ti])


def test_locality_outside_cell():
    B, size, C, heads, window, shift = 1, (6, 10, 10), 16, 2, (2, 5, 5), (1, 2, 2)
    p = _params(C, heads, window, seed=9)
    x = _tokens(B, *size, C, seed=10)
    y0 = oracle.block(x, p, heads, window, shift)[1]
    x2 = x.copy()
    x2[0, 5, 9, 9] += 5.0            # far corner: not in the cell of token (0,0,0)
    y1 = oracle.block(x2, p, heads, window, shift)[1]
    assert np.array_equal(y0[0, 0, 0, 0], y1[0, 0, 0, 0])


# ---------------------------------------------------------------- P-e library special cases
def test_layernorm_and_gelu_match_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((37, 96)) * 3 + 1
    g, b = rng.standard_normal(96), rng.standard_normal(96)
    ref = F.layer_norm(torch.from_numpy(x), (96,), torch.from_numpy(g), torch.from_numpy(b), 1e-5)
    assert np.max(np.abs(oracle.layer_norm(x, g, b) - ref.numpy())) < 1e-12
    ref = F.gelu(torch.from_numpy(x), approximate="none")
    assert np.max(np.abs(oracle.gelu(x) - ref.numpy())) < 1e-12


def test_global_window_is_sdpa_with_bias():
    # window >= grid and shift 0: one window per clip = global MHSA + bias
    B, size, C, heads, window = 2, (3, 4, 5), 32, 4, (8, 7, 7)
    p = _params(C, heads, window, seed=11)
    xn = _tokens(B, *size, C, seed=12)
    got = oracle.window_msa(xn, p, heads, window, (4, 3, 3))
    T, H, W = size
    N = T * H * W
    d = C // heads
    coords = [(t, h, w) for t in range(T) for h in range(H) for w in range(W)]
    bias = np.zeros((heads, N, N))
    for i, ci in enumerate(coords):
        for j, cj in enumerate(coords):
            r = ((ci[0] - cj[0] + 7) * 13 + (ci[1] - cj[1] + 6)) * 13 + (ci[2] - cj[2] + 6)
            bias[:, i, j] = p["rpb_table"][r]
    x = torch.from_numpy(xn.reshape(B, N, C))
    qkv = x @ torch.from_numpy(p["qkv_w"]).T + torch.from_numpy(p["qkv_b"])
    q, k, v = (qkv[..., i * C:(i + 1) * C].reshape(B, N, heads, d).transpose(1, 2) for i in range(3))
    o = F.scaled_dot_product_attention(q, k, v, attn_mask=torch.from_numpy(bias))
    o = o.transpose(1, 2).reshape(B, N, C) @ torch.from_numpy(p["proj_w"]).T + torch.from_numpy(p["proj_b"])
    assert np.max(np.abs(got.reshape(B, N, C) - o.numpy())) < 1e-12


def test_zero_table_is_plain_windowed_mha():
    B, size, C, heads, window = 1, (4, 14, 14), 32, 2, (2, 7, 7)
    p = _params(C, heads, window, seed=13)
    p["rpb_table"] = np.zeros_like(p["rpb_table"])
    xn = _tokens(B, *size, C, seed=14)
    got = oracle.window_msa(xn, p, heads, window, (0, 0, 0))
    mha = torch.nn.MultiheadAttention(C, heads, bias=True, batch_first=True).double()
    with torch.no_grad():
        mha.in_proj_weight.copy_(torch.from_numpy(p["qkv_w"]))
        mha.in_proj_bias.copy_(torch.from_numpy(p["qkv_b"]))
        mha.out_proj.weight.copy_(torch.from_numpy(p["proj_w"]))
        mha.out_proj.bias.copy_(torch.from_numpy(p["proj_b"]))
        # regular windows by plain reshaping (no roll, no pad)
        xw = torch.from_numpy(xn).reshape(1, 2, 2, 2, 7, 2, 7, C).permute(0, 1, 3, 5, 2, 4, 6, 7).reshape(-1, 98, C)
        o, _ = mha(xw, xw, xw, need_weights=False)
        o = o.reshape(1, 2, 2, 2, 2, 7, 7, C).permute(0, 1, 4, 2, 5, 3, 6, 7).reshape(xn.shape)
    assert np.max(np.abs(got - o.numpy())) < 1e-12


def test_patch_embed_is_conv3d():
    rng = np.random.default_rng(2)
    v = rng.standard_normal((2, 3, 6, 9, 13))          # non-divisible H, W: zero-padded
    w = rng.standard_normal((8, 3, 2, 4, 4))
    b = rng.standard_normal(8)
    got = oracle.patch_embed(v, w, b)
    vt = F.pad(torch.from_numpy(v), (0, 3, 0, 3, 0, 0))
    ref = F.conv3d(vt, torch.from_numpy(w), torch.from_numpy(b), stride=(2, 4, 4))
    assert np.max(np.abs(got - ref.permute(0, 2, 3, 4, 1).numpy())) < 1e-12


def test_merge_gather_layout():
    # tiny grid whose values encode (h, w): the 4C vector of output (0,0) is
    # the (0,0), (1,0), (0,1), (1,1) neighbours in that order
    x = np.zeros((1, 1, 2, 2, 1))
    for h in range(2):
        for w in range(2):
            x[0, 0, h, w, 0] = 10 * h + w
    g = ov.merge_gather(x)
    assert g.shape == (1, 1, 1, 1, 4)
    assert g[0, 0, 0, 0].tolist() == [0, 10, 1, 11]


# ---------------------------------------------------------------- P-f 2D reduction
def test_2d_partition_order():
    # T = P = 1: windows in (b, wh, ww) order, tokens (ph, pw) -- the 2D
    # window_partition of the Swin glossary page
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 1, 14, 21, 5))
    w = ov.partition(x, (1, 7, 7))
    k = 0
    for b in range(2):
        for i in range(2):
            for j in range(3):
                assert np.array_equal(w[k].reshape(7, 7, 5), x[b, 0, 7 * i:7 * i + 7, 7 * j:7 * j + 7])
                k += 1


# ---------------------------------------------------------------- P-g inflation, P-h coverage
def test_inflated_table_gives_frame_independent_bias():
    P, M = 8, 7
    rng = np.random.default_rng(4)
    t2 = rng.standard_normal(((2 * M - 1) ** 2, 3))
    t3 = np.tile(t2, (2 * P - 1, 1))            # repeated over the 2P-1 temporal offsets (§3.4)
    rel = ov.relative_index((P, M, M))
    bias = t3[rel]                              # (N, N, heads)
    N = P * M * M
    coords = np.array([(t, h, w) for t in range(P) for h in range(M) for w in range(M)])
    spatial = (coords[:, None, 1] - coords[None, :, 1] + M - 1) * (2 * M - 1) + \
              (coords[:, None, 2] - coords[None, :, 2] + M - 1)
    assert np.array_equal(bias, t2[spatial])


def test_relative_index_covers_every_row_once_per_offset():
    P, M = 8, 7
    rel = ov.relative_index((P, M, M))
    assert rel.shape == (392, 392)
    assert set(np.unique(rel).tolist()) == set(range((2 * P - 1) * (2 * M - 1) ** 2))
    assert rel.max() == 2534
    # diagonal (zero offset) is the centre row
    assert (np.diag(rel) == (P - 1) * 169 + (M - 1) * 13 + (M - 1)).all()


# ---------------------------------------------------------------- P-i mutation sensitivity
TOL_MAX = 3e-2
MUT_SHAPE = (1, (16, 14, 14), 96, 3, (8, 7, 7), (4, 3, 3))
MUT_PAD = (1, (16, 12, 13), 64, 2, (8, 7, 7), (4, 3, 3))


def _mut_run(shape, monkeypatch=None, **kw):
    B, size, C, heads, window, shift = shape
    p = _params(C, heads, window, seed=21, init="stress", dtype="bf16")
    rng = np.random.default_rng(22)
    x = synth.round_bf16(rng.standard_normal((B, *size, C)).astype(np.float32)).astype(np.float64)
    return oracle.block(x, p, heads, window, shift, **kw)[1], p, x


@pytest.fixture(scope="module")
def correct_out():
    return _mut_run(MUT_SHAPE)[0]


def test_mutant_no_bias(correct_out):
    B, size, C, heads, window, shift = MUT_SHAPE
    _, p, x = _mut_run(MUT_SHAPE)
    p = dict(p, rpb_table=np.zeros_like(p["rpb_table"]))
    y = oracle.block(x, p, heads, window, shift)[1]
    assert np.max(np.abs(y - correct_out)) > TOL_MAX


def test_mutant_flipped_offset_sign(correct_out, monkeypatch):
    real = ov.relative_index
    monkeypatch.setattr(ov, "relative_index", lambda *a, **k: real(*a, **k).T)
    y = _mut_run(MUT_SHAPE)[0]
    assert np.max(np.abs(y - correct_out)) > TOL_MAX


def test_mutant_no_mask(correct_out, monkeypatch):
    real = ov.region_labels
    monkeypatch.setattr(ov, "region_labels", lambda *a, **k: np.zeros_like(real(*a, **k)))
    y = _mut_run(MUT_SHAPE)[0]
    assert np.max(np.abs(y - correct_out)) > TOL_MAX


def test_mutant_roll_direction(correct_out, monkeypatch):
    real = ov.roll3
    monkeypatch.setattr(ov, "roll3", lambda u, s: real(u, [-v for v in s]))
    y = _mut_run(MUT_SHAPE)[0]
    assert np.max(np.abs(y - correct_out)) > TOL_MAX


def test_mutant_pads_visible():
    y0 = _mut_run(MUT_PAD)[0]
    y1 = _mut_run(MUT_PAD, pad_visible=True)[0]
    assert np.max(np.abs(y1 - y0)) > TOL_MAX


# ---------------------------------------------------------------- sampled evaluation
def test_block_sampled_matches_full():
    B, size, C, heads, window, shift = 2, (5, 9, 11), 16, 2, (2, 4, 3), (1, 2, 1)
    p = _params(C, heads, window, seed=30)
    x = _tokens(B, *size, C, seed=31)
    zh, y = oracle.block(x, p, heads, window, shift)
    toks = [0, 17, 200, 2 * 5 * 9 * 11 - 1]
    zs, ys = ov.block_sampled(x, p, heads, window, shift, toks)
    assert np.max(np.abs(zs - zh.reshape(-1, C)[toks])) < 1e-12
    assert np.max(np.abs(ys - y.reshape(-1, C)[toks])) < 1e-12


def test_clamp_reading():
    assert oracle.effective_window((16, 7, 7), (8, 7, 7), (4, 3, 3)) == ((8, 7, 7), (4, 0, 0))
    assert oracle.effective_window((16, 7, 7), (8, 7, 7), (4, 3, 3), clamp_strict=True) == ((8, 7, 7), (4, 3, 3))
    assert oracle.effective_window((4, 5, 9), (8, 7, 7), (4, 3, 3)) == ((4, 5, 7), (0, 0, 3))
