"""GPU parity: the HIP library (through the C ABI) against the fp64 oracle.

Permutations and the index map are compared bit for bit; floating-point
outputs within max-abs 3e-2 / mean-abs 3e-3 (bf16 I/O, fp32 accumulate) or
1e-4 (fp32 path).  Block stacks are compared per block, teacher-forced: the
oracle's block k consumes the GPU's input of block k.
"""
import numpy as np
import pytest
import torch

import synth
import oracle
from oracle import vswin as ov
import shifted_window_attention_amd as vs

from helpers import TOL_BF16_MAX, check, dev, dev_params, host64, say, tdt

pytestmark = pytest.mark.gpu

GEOMS = [
    # B, (T, H, W), C, heads, window, shift
    (1, (4, 14, 14), 32, 2, (2, 7, 7), (1, 3, 3)),
    (1, (16, 56, 56), 96, 3, (8, 7, 7), (4, 3, 3)),
    (2, (16, 60, 60), 128, 4, (8, 7, 7), (4, 3, 3)),
    (2, (16, 60, 60), 128, 4, (8, 7, 7), (0, 0, 0)),
    (2, (16, 7, 7), 768, 24, (8, 7, 7), (4, 3, 3)),
    (2, (5, 9, 11), 32, 2, (2, 4, 3), (1, 2, 1)),
    (1, (18, 15, 8), 32, 1, (8, 7, 7), (4, 3, 3)),
]


def _rng_tokens(shape, dtype, seed):
    x = np.random.default_rng(seed).standard_normal(shape).astype(np.float32)
    return synth.round_bf16(x) if dtype == "bf16" else x


@pytest.mark.parametrize("g", GEOMS)
@pytest.mark.parametrize("pad_visible", [False, True])
def test_index_map_bitexact(g, pad_visible):
    B, size, C, heads, window, shift = g
    say(f"index map {g} pad_visible={pad_visible}")
    flags = vs.F_PAD_VISIBLE if pad_visible else 0
    d = vs.make_desc(B, *size, C, heads, window, shift, dtype=torch.bfloat16, flags=flags)
    m, r = vs.vswin_index_map(d)
    o = ov.Geometry(B, size, window, shift, pad_visible=pad_visible)
    assert np.array_equal(m.cpu().numpy().astype(np.int64), o.index_map().ravel())
    lab = np.tile(o.win_labels, (B, 1)).ravel()
    lab = np.where(lab == ov.PAD_LABEL, 255, lab)
    assert np.array_equal(r.cpu().numpy().astype(np.int64), lab)


@pytest.mark.parametrize("g", GEOMS)
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_partition_and_reverse_bitexact(g, dtype):
    B, size, C, heads, window, shift = g
    say(f"partition/reverse {g} {dtype}")
    x = _rng_tokens((B, *size, C), dtype, 5)
    xt = dev(x, dtype)
    w = vs.vswin_partition_fwd(xt, window, shift)
    o = ov.Geometry(B, size, window, shift)
    ref = ov.partition(ov.roll3(ov.pad_end(x, o.padded), [-s for s in o.shift]), o.window)
    assert np.array_equal(w.float().cpu().numpy(), ref.astype(np.float32))
    back = vs.vswin_reverse_fwd(w, x.shape, window, shift)
    assert torch.equal(back, xt)
    r = _rng_tokens((B, *size, C), dtype, 6)
    both = vs.vswin_reverse_fwd(w, x.shape, window, shift, residual=dev(r, dtype))
    exp = (xt.float() + dev(r, dtype).float()).to(xt.dtype)
    assert torch.equal(both, exp)


@pytest.mark.parametrize("B,size,C,dtype", [
    (2, (16, 48, 47), 128, "bf16"),   # 76832 padded slots
    (2, (16, 48, 47), 128, "fp32"),
    (2, (16, 91, 91), 96, "bf16"),    # 264992 padded slots
])
def test_partition_reverse_layernorm_many_rows(B, size, C, dtype):
    """The gather, scatter + residual and LayerNorm kernels at large row counts
    (tens of thousands of workgroups) with padded windows: permutations
    bit-exact, LayerNorm against the oracle."""
    window, shift = (8, 7, 7), (4, 3, 3)
    say(f"many-row partition/reverse/LN {B} {size} C={C} {dtype}")
    x = _rng_tokens((B, *size, C), dtype, 25)
    xt = dev(x, dtype)
    w = vs.vswin_partition_fwd(xt, window, shift)
    o = ov.Geometry(B, size, window, shift)
    ref = ov.partition(ov.roll3(ov.pad_end(x, o.padded), [-s for s in o.shift]), o.window)
    assert np.array_equal(w.float().cpu().numpy(), ref.astype(np.float32))
    r = _rng_tokens((B, *size, C), dtype, 26)
    both = vs.vswin_reverse_fwd(w, x.shape, window, shift, residual=dev(r, dtype))
    assert torch.equal(both, (xt.float() + dev(r, dtype).float()).to(xt.dtype))
    rng = np.random.default_rng(C)
    g = synth.round_bf16((1 + 0.1 * rng.standard_normal(C)).astype(np.float32))
    b = synth.round_bf16((0.1 * rng.standard_normal(C)).astype(np.float32))
    rows = x.reshape(-1, C)
    y = vs.vswin_layernorm_fwd(dev(rows, dtype), dev(g, "bf16"), dev(b, "bf16"), out_dtype=tdt("bf16"))
    ref = oracle.layer_norm(rows.astype(np.float64), g, b)
    assert np.abs(host64(y) - ref).max() <= 2.0 ** -8 * np.abs(ref).max() + 1e-6


@pytest.mark.parametrize("C", [32, 96, 128, 192, 384, 768, 1536, 3072])
@pytest.mark.parametrize("io", [("fp32", "bf16"), ("bf16", "bf16"), ("fp32", "fp32")])
def test_layernorm(C, io):
    say(f"layernorm C={C} {io}")
    rows = 1000
    rng = np.random.default_rng(C)
    x = (rng.standard_normal((rows, C)) * 2 + 0.5).astype(np.float32)
    if io[0] == "bf16":
        x = synth.round_bf16(x)
    g = (1 + 0.1 * rng.standard_normal(C)).astype(np.float32)
    b = (0.1 * rng.standard_normal(C)).astype(np.float32)
    if io[1] == "bf16":
        g, b = synth.round_bf16(g), synth.round_bf16(b)
    y = vs.vswin_layernorm_fwd(dev(x, io[0]), dev(g, io[1]), dev(b, io[1]), out_dtype=tdt(io[1]))
    ref = oracle.layer_norm(x, g, b)
    if io[1] == "bf16":
        err = np.abs(host64(y) - ref)
        assert err.max() <= 2.0 ** -8 * np.abs(ref).max() + 1e-6
    else:
        check(host64(y), ref, "fp32", "layernorm")


# ----------------------------------------------------------------------------- window MSA branch
MSA_CASES = [
    # name, B, size, C, heads, window, shift, dtype, init, flags
    ("fp32 smoke regular", 1, (4, 14, 14), 32, 2, (2, 7, 7), (0, 0, 0), "fp32", "spec", 0),
    ("fp32 smoke shifted", 1, (4, 14, 14), 32, 2, (2, 7, 7), (1, 3, 3), "fp32", "stress", 0),
    # fp32 on the matrix cores: head_dim 32 and 64, padded grids, the -100 mask
    ("fp32 window 8 d=32 shifted", 1, (16, 14, 14), 64, 2, (8, 7, 7), (4, 3, 3), "fp32", "stress", 0),
    ("fp32 d=64 padded shifted", 2, (4, 12, 13), 128, 2, (2, 7, 7), (1, 3, 3), "fp32", "stress", 0),
    ("fp32 d=32 mask -100", 1, (4, 14, 14), 64, 2, (2, 7, 7), (1, 3, 3), "fp32", "stress", vs.F_MASK_M100),
    ("fp32 d=16 pads visible", 1, (5, 12, 13), 32, 2, (2, 7, 7), (1, 3, 3), "fp32", "stress", vs.F_PAD_VISIBLE),
    ("bf16 regular", 1, (16, 14, 14), 96, 3, (8, 7, 7), (0, 0, 0), "bf16", "stress", 0),
    ("bf16 shifted", 1, (16, 14, 14), 96, 3, (8, 7, 7), (4, 3, 3), "bf16", "stress", 0),
    ("bf16 shifted spec", 2, (16, 21, 14), 64, 2, (8, 7, 7), (4, 3, 3), "bf16", "spec", 0),
    ("bf16 padded shifted", 1, (16, 12, 13), 128, 4, (8, 7, 7), (4, 3, 3), "bf16", "stress", 0),
    ("bf16 padded regular", 1, (16, 12, 13), 128, 4, (8, 7, 7), (0, 0, 0), "bf16", "stress", 0),
    ("bf16 temporal pad", 1, (12, 14, 14), 64, 2, (8, 7, 7), (4, 3, 3), "bf16", "stress", 0),
    ("bf16 clamp (16,7,7)", 2, (16, 7, 7), 768, 24, (8, 7, 7), (4, 3, 3), "bf16", "stress", 0),
    ("bf16 generic P=2", 1, (4, 14, 14), 64, 2, (2, 7, 7), (1, 3, 3), "bf16", "stress", 0),
    ("bf16 generic d=16", 1, (8, 14, 14), 32, 2, (8, 7, 7), (4, 3, 3), "bf16", "stress", 0),
    ("bf16 pads visible", 1, (16, 12, 13), 64, 2, (8, 7, 7), (4, 3, 3), "bf16", "stress", vs.F_PAD_VISIBLE),
    ("bf16 mask -100", 1, (16, 14, 14), 64, 2, (8, 7, 7), (4, 3, 3), "bf16", "stress", vs.F_MASK_M100),
    ("bf16 clamp strict", 1, (16, 7, 7), 64, 2, (8, 7, 7), (4, 3, 3), "bf16", "stress", vs.F_CLAMP_STRICT),
    ("bf16 window 16", 1, (16, 7, 7), 64, 2, (16, 7, 7), (8, 3, 3), "bf16", "stress", vs.F_CLAMP_STRICT),
    ("bf16 window 4", 1, (16, 14, 14), 64, 2, (4, 7, 7), (2, 3, 3), "bf16", "stress", 0),
    # temporal window 16 (784 tokens): the MFMA kernel's scalar-table form
    ("bf16 window 16 regular", 1, (16, 14, 14), 96, 3, (16, 7, 7), (0, 0, 0), "bf16", "stress", 0),
    ("bf16 window 16 shifted", 1, (16, 14, 14), 96, 3, (16, 7, 7), (8, 3, 3), "bf16", "stress", 0),
    ("bf16 window 16 padded", 1, (16, 12, 13), 64, 2, (16, 7, 7), (8, 3, 3), "bf16", "stress", 0),
    ("bf16 window 16 spec", 1, (32, 14, 14), 64, 2, (16, 7, 7), (8, 3, 3), "bf16", "spec", 0),
    ("bf16 mask -100 padded", 1, (16, 12, 13), 64, 2, (8, 7, 7), (4, 3, 3), "bf16", "stress", vs.F_MASK_M100),
    # a temporal region boundary inside a group of 4 keys: labels compared key by key
    ("bf16 window 4 padded", 1, (14, 12, 13), 96, 3, (4, 7, 7), (2, 3, 3), "bf16", "stress", 0),
    ("bf16 window 4 pads visible", 1, (14, 12, 13), 64, 2, (4, 7, 7), (2, 3, 3), "bf16", "stress",
     vs.F_PAD_VISIBLE),
    ("bf16 window 12 shift 6", 1, (24, 14, 14), 64, 2, (12, 7, 7), (6, 3, 3), "bf16", "stress", 0),
    ("bf16 window 4 mask -100 (generic)", 1, (16, 14, 14), 64, 2, (4, 7, 7), (2, 3, 3), "bf16", "stress",
     vs.F_MASK_M100),
    ("bf16 spatial-only shift", 1, (16, 14, 14), 96, 3, (8, 7, 7), (0, 3, 3), "bf16", "stress", 0),
    ("bf16 window 16 mask -100", 1, (16, 14, 14), 64, 2, (16, 7, 7), (8, 3, 3), "bf16", "stress",
     vs.F_MASK_M100),
]


def _msa_params(C, heads, window, dtype, init, seed=11):
    rows = (2 * window[0] - 1) * (2 * window[1] - 1) * (2 * window[2] - 1)
    return synth.gen_block_params(C, heads, rows, 4, np.random.SeedSequence(seed), dtype, init)


@pytest.mark.parametrize("case", MSA_CASES, ids=[c[0] for c in MSA_CASES])
def test_window_msa(case):
    name, B, size, C, heads, window, shift, dtype, init, flags = case
    say(f"window_msa {name}")
    p = _msa_params(C, heads, window, dtype, init)
    x = _rng_tokens((B, *size, C), dtype, 3)
    y = vs.vswin_window_msa_fwd(dev(x, dtype), dev_params(p, dtype), heads, window, shift, flags=flags)
    ref = oracle.window_msa(x, p, heads, window, shift,
                            clamp_strict=bool(flags & vs.F_CLAMP_STRICT),
                            pad_visible=bool(flags & vs.F_PAD_VISIBLE),
                            mask_m100=bool(flags & vs.F_MASK_M100))
    check(host64(y), ref, dtype, name)


@pytest.mark.parametrize("window,shift", [((8, 7, 7), (0, 0, 0)), ((8, 7, 7), (4, 3, 3)), ((16, 7, 7), (8, 3, 3)),
                                          ((4, 7, 7), (2, 3, 3))])
def test_window_msa_forced_row_max_pass(window, shift, monkeypatch):
    """The exact row-max pass of the MFMA kernel at stress init."""
    say(f"window_msa forced max pass window {window} shift {shift}")
    monkeypatch.setenv("VSWIN_ATTN_MAXPASS", "1")
    C, heads = 96, 3
    p = _msa_params(C, heads, window, "bf16", "stress")
    x = _rng_tokens((1, 16, 14, 21, C), "bf16", 4)
    y = vs.vswin_window_msa_fwd(dev(x, "bf16"), dev_params(p, "bf16"), heads, window, shift)
    check(host64(y), oracle.window_msa(x, p, heads, window, shift), "bf16", "forced max pass")


def test_window_msa_logits_beyond_exp_range():
    """Logits of several hundred (exp2 would overflow without a max): tokens
    +-1, q = k = 8 x, v = x, so q.k is an exact integer on both sides and the
    kernel must take its row-max pass on its own."""
    say("window_msa logits beyond exp range")
    C, heads, window, shift = 64, 2, (8, 7, 7), (4, 3, 3)
    rng = np.random.default_rng(9)
    x = np.where(rng.random((1, 16, 14, 14, C)) < 0.5, -1.0, 1.0).astype(np.float32)
    eye = np.eye(C, dtype=np.float32)
    rows = 15 * 13 * 13
    p = {"qkv_w": np.concatenate([8 * eye, 8 * eye, eye]), "qkv_b": np.zeros(3 * C, np.float32),
         "proj_w": eye.copy(), "proj_b": np.zeros(C, np.float32),
         "rpb_table": synth.round_bf16(rng.standard_normal((rows, heads)).astype(np.float32))}
    y = vs.vswin_window_msa_fwd(dev(x, "bf16"), dev_params(p, "bf16"), heads, window, shift)
    ref = oracle.window_msa(x, p, heads, window, shift)
    assert np.abs(ref).max() > 0.5
    check(host64(y), ref, "bf16", "logits beyond exp range")


@pytest.mark.parametrize("window,shift", [((8, 7, 7), (4, 3, 3)), ((16, 7, 7), (8, 3, 3))])
def test_window_msa_m100_visible(window, shift):
    """The -100 mask where it changes the result: a few relative offsets carry
    a bias of +150, so a query whose only such keys lie in another region puts
    its weight on them (logit 50 against about 0) instead of excluding them;
    logits this large also take the kernel through its row-max pass.  The
    test first checks on the oracle that exclusion and -100 differ."""
    say(f"window_msa -100 visible, window {window}")
    C, heads = 64, 2
    rng = np.random.default_rng(17)
    rows = (2 * window[0] - 1) * 13 * 13
    table = np.zeros((rows, heads), np.float32)
    table[rng.random(rows) < 0.005] = 150.0
    p = _msa_params(C, heads, window, "bf16", "spec", seed=31)
    p["rpb_table"] = table
    # v = x and an identity projection, so the output is the weighted tokens
    eye = np.eye(C, dtype=np.float32)
    p["qkv_w"] = p["qkv_w"].copy()
    p["qkv_w"][2 * C:] = eye
    p["proj_w"] = eye.copy()
    x = synth.round_bf16(rng.standard_normal((1, 16, 14, 14, C)).astype(np.float32))
    ref = oracle.window_msa(x, p, heads, window, shift, mask_m100=True)
    excl = oracle.window_msa(x, p, heads, window, shift)
    assert np.abs(ref - excl).max() > 10 * TOL_BF16_MAX
    y = vs.vswin_window_msa_fwd(dev(x, "bf16"), dev_params(p, "bf16"), heads, window, shift, flags=vs.F_MASK_M100)
    check(host64(y), ref, "bf16", f"-100 visible {window}")


# ----------------------------------------------------------------------------- blocks
def _stack_check(x0, params, shape, dtype, flags=0, label=""):
    """Run the block stack on the GPU; check each block against the oracle fed
    the GPU's own input of that block."""
    s = shape
    xt = dev(x0, dtype)
    for k, p in enumerate(params):
        shift = (0, 0, 0) if k % 2 == 0 else s.shift
        yt = vs.vswin_block_fwd(xt, dev_params(p, dtype), s.heads, s.window, shift, flags=flags)
        xin = host64(xt)
        _, ref = oracle.block(xin, p, s.heads, s.window, shift,
                              pad_visible=bool(flags & vs.F_PAD_VISIBLE))
        check(host64(yt), ref, dtype, f"{label} block {k} shift {shift}")
        xt = yt
    return xt


# C = 96 bf16 blocks run qkv -> attention -> (projection + MLP in one kernel);
# these geometries take that path through pads, batches and the clamp
C96_CASES = [
    ("padded shifted", 1, (16, 12, 13), (4, 3, 3), 0),
    ("padded regular", 1, (16, 12, 13), (0, 0, 0), 0),
    ("temporal pad B=2", 2, (12, 14, 14), (4, 3, 3), 0),
    ("pads visible", 1, (16, 12, 13), (4, 3, 3), vs.F_PAD_VISIBLE),
    ("clamp (16,7,7)", 2, (16, 7, 7), (4, 3, 3), 0),
    ("B=2 non-square", 2, (16, 14, 21), (4, 3, 3), 0),
]


@pytest.mark.parametrize("case", C96_CASES, ids=[c[0] for c in C96_CASES])
def test_block_c96_fused_projection(case):
    name, B, size, shift, flags = case
    say(f"C=96 block {name}")
    C, heads, window = 96, 3, (8, 7, 7)
    p = _msa_params(C, heads, window, "bf16", "stress", seed=23)
    x = _rng_tokens((B, *size, C), "bf16", 5)
    y = vs.vswin_block_fwd(dev(x, "bf16"), dev_params(p, "bf16"), heads, window, shift, flags=flags)
    _, ref = oracle.block(x, p, heads, window, shift, pad_visible=bool(flags & vs.F_PAD_VISIBLE))
    check(host64(y), ref, "bf16", f"C=96 block {name}")


@pytest.mark.parametrize("case", C96_CASES[:3] + [("C=128 padded B=2", 2, (16, 12, 13), (4, 3, 3), 0)],
                         ids=[c[0] for c in C96_CASES[:3]] + ["C=128 padded B=2"])
def test_block_one_kernel_qkv_attention_path(case, monkeypatch):
    """VSWIN_FUSED=1 routes the block through the one-kernel LN1 + gather +
    qkv + attention (q, k, v on chip) instead of the separate launches; it
    must meet the same bar."""
    name, B, size, shift, flags = case
    C = 128 if "128" in name else 96
    heads, window = C // 32, (8, 7, 7)
    say(f"one-kernel qkv + attention path: {name}")
    monkeypatch.setenv("VSWIN_FUSED", "1")
    p = _msa_params(C, heads, window, "bf16", "stress", seed=23)
    x = _rng_tokens((B, *size, C), "bf16", 5)
    y = vs.vswin_block_fwd(dev(x, "bf16"), dev_params(p, "bf16"), heads, window, shift, flags=flags)
    _, ref = oracle.block(x, p, heads, window, shift, pad_visible=bool(flags & vs.F_PAD_VISIBLE))
    check(host64(y), ref, "bf16", f"one-kernel qkv + attention {name}")


@pytest.mark.parametrize("C,B,size", [(96, 1, (16, 56, 56)), (96, 2, (16, 56, 56)), (128, 2, (16, 12, 13)),
                                      (128, 1, (16, 60, 60))])
def test_block_fused_qkv_attention_equals_separate(C, B, size, monkeypatch):
    """The one-kernel LN1 + gather + qkv + attention rounds q, k and v to bf16
    exactly where the separate launches store them, and runs the same
    attention arithmetic: the block outputs agree bit for bit, on grids whose
    workgroup runs cross windows and heads."""
    heads, window = C // 32, (8, 7, 7)
    p = dev_params(_msa_params(C, heads, window, "bf16", "stress", seed=41), "bf16")
    x = dev(_rng_tokens((B, *size, C), "bf16", 9), "bf16")
    for shift in ((0, 0, 0), (4, 3, 3)):
        say(f"fused vs separate qkv + attention: C={C} B={B} {size} shift {shift}")
        monkeypatch.setenv("VSWIN_FUSED", "1")
        yf = vs.vswin_block_fwd(x, p, heads, window, shift)
        monkeypatch.setenv("VSWIN_FUSED", "0")
        ys = vs.vswin_block_fwd(x, p, heads, window, shift)
        torch.cuda.synchronize()
        assert torch.isfinite(yf.float()).all()
        assert torch.equal(yf, ys), f"max diff {(yf.float() - ys.float()).abs().max().item()}"


@pytest.mark.parametrize("window,shift", [((16, 7, 7), (0, 0, 0)), ((16, 7, 7), (8, 3, 3)), ((4, 7, 7), (2, 3, 3))])
def test_block_window_variants_stage1_grid(window, shift):
    """The other temporal windows on the Swin-T stage-1 token grid: 16 (784
    tokens per window; more than 4 query tiles per wave and window, the scalar
    bias tables written by the qkv launch) and 4 with temporal shift 2 (a
    region boundary inside a group of 4 keys)."""
    say(f"window {window} block, stage-1 grid, shift {shift}")
    C, heads = 96, 3
    plan = vs.vswin_plan_query(vs.make_desc(1, 16, 56, 56, C, heads, window, shift, dtype=1))
    assert plan["fast_attention"] and plan["tokens_per_window"] == window[0] * 49
    p = _msa_params(C, heads, window, "bf16", "stress", seed=29)
    x = _rng_tokens((1, 16, 56, 56, C), "bf16", 6)
    y = vs.vswin_block_fwd(dev(x, "bf16"), dev_params(p, "bf16"), heads, window, shift)
    _, ref = oracle.block(x, p, heads, window, shift)
    check(host64(y), ref, "bf16", f"window {window} block shift {shift}")


def test_block_swin_l_width():
    """Swin-L's stage-1 width (C = 192, 6 heads of 32): the generic GEMM path
    around the MFMA attention, regular and shifted."""
    C, heads, window = 192, 6, (8, 7, 7)
    p = _msa_params(C, heads, window, "bf16", "stress", seed=37)
    x = _rng_tokens((1, 16, 14, 14, C), "bf16", 12)
    for shift in ((0, 0, 0), (4, 3, 3)):
        say(f"Swin-L width block, shift {shift}")
        y = vs.vswin_block_fwd(dev(x, "bf16"), dev_params(p, "bf16"), heads, window, shift)
        _, ref = oracle.block(x, p, heads, window, shift)
        check(host64(y), ref, "bf16", f"C=192 block shift {shift}")


@pytest.mark.parametrize("C,heads,shape", [
    (64, 2, (1, 16, 28, 28)),    # K = 64: a single K stage; fc2 K = 256; 3- and 4-stage rings
    (320, 10, (1, 8, 28, 21)),   # K = 320: five stages; 4704 tokens (ragged last 128-row tile); 2-stage ring
])
def test_block_staged_k_gemm_shapes(C, heads, shape):
    """Widths outside the published models that route every linear layer
    through the staged-K GEMM: one and five K stages, a token count that is
    not a multiple of the 128-row tile, and tile counts that pick each ring
    depth; regular and shifted, stress init."""
    window = (8, 7, 7)
    p = _msa_params(C, heads, window, "bf16", "stress", seed=41)
    x = _rng_tokens(shape + (C,), "bf16", 14)
    for shift in ((0, 0, 0), (4, 3, 3)):
        say(f"staged-K widths: C={C} tokens {shape} shift {shift}")
        y = vs.vswin_block_fwd(dev(x, "bf16"), dev_params(p, "bf16"), heads, window, shift)
        _, ref = oracle.block(x, p, heads, window, shift)
        check(host64(y), ref, "bf16", f"C={C} block shift {shift}")


def test_workload1_fp32_pair():
    say("workload 1: fp32 block pair")
    x, params = synth.gen_workload(1)
    _stack_check(x, params, synth.WORKLOADS[1].shape, "fp32", label="wl1")


def test_workload1_fp32_pair_stress():
    say("workload 1: fp32 block pair, stress init")
    x, params = synth.gen_workload(1, init="stress")
    _stack_check(x, params, synth.WORKLOADS[1].shape, "fp32", label="wl1 stress")


def test_workload2_bf16_pair():
    say("workload 2: Swin-T stage-1 bf16 block pair (full size)")
    x, params = synth.gen_workload(2)
    _stack_check(x, params, synth.WORKLOADS[2].shape, "bf16", label="wl2")


def test_workload2_bf16_pair_stress():
    say("workload 2 shapes, stress init")
    x, params = synth.gen_workload(2, init="stress")
    _stack_check(x, params, synth.WORKLOADS[2].shape, "bf16", label="wl2 stress")


def test_workload3_bf16_six_blocks():
    say("workload 3: Swin-T stage-3 six blocks, B=4")
    x, params = synth.gen_workload(3)
    _stack_check(x, params, synth.WORKLOADS[3].shape, "bf16", label="wl3")


def _fresh_check(params, shape, dtype, label, seed):
    """Stress-init blocks, each on fresh N(0,1) tokens of the workload's shape
    (regular and shifted alternating): chained stress blocks grow the
    residual stream until one bf16 rounding of the output (half an ulp is
    0.031 at |y| >= 8) fills the absolute bar by itself."""
    s = shape
    for k, p in enumerate(params):
        shift = (0, 0, 0) if k % 2 == 0 else s.shift
        x = _rng_tokens((s.B, s.T, s.H, s.W, s.C), dtype, seed + k)
        y = vs.vswin_block_fwd(dev(x, dtype), dev_params(p, dtype), s.heads, s.window, shift)
        _, ref = oracle.block(x, p, s.heads, s.window, shift)
        check(host64(y), ref, dtype, f"{label} block {k} shift {shift}")


def test_workload3_bf16_six_blocks_stress():
    """Workload 3's shapes (C = 384: the generic GEMM + unfused MLP path) at
    stress init, where a missing bias, a flipped offset sign or a wrong mask
    moves the outputs far beyond the bar; all six blocks, every token."""
    say("workload 3 shapes, stress init")
    _, params = synth.gen_workload(3, init="stress")
    _fresh_check(params, synth.WORKLOADS[3].shape, "bf16", "wl3 stress", 300)


@pytest.mark.parametrize("init", ["spec", "stress"])
def test_workload4_bf16_pair_full(init):
    """Workload 4 (Swin-B stage 1, B=8, (16,60,60,128) padded to (16,63,63);
    the C = 128 fused MLP with its erf) on every output token of both blocks
    of the pair, at spec and at stress init."""
    say(f"workload 4: Swin-B stage-1 padded pair, B=8, every token, {init} init")
    x, params = synth.gen_workload(4, init=init)
    if init == "spec":
        _stack_check(x, params, synth.WORKLOADS[4].shape, "bf16", label="wl4 spec")
    else:
        _fresh_check(params, synth.WORKLOADS[4].shape, "bf16", "wl4 stress", 400)


def test_block_c128_padded_stress_full():
    """C = 128 (the fused MLP with its GELU table) on a small padded grid with
    B = 2, every output token, regular and shifted, stress init."""
    C, heads, window = 128, 4, (8, 7, 7)
    p = _msa_params(C, heads, window, "bf16", "stress", seed=41)
    x = _rng_tokens((2, 16, 12, 13, C), "bf16", 14)
    for shift in ((0, 0, 0), (4, 3, 3)):
        say(f"C=128 padded block B=2, stress, shift {shift}")
        y = vs.vswin_block_fwd(dev(x, "bf16"), dev_params(p, "bf16"), heads, window, shift)
        _, ref = oracle.block(x, p, heads, window, shift)
        check(host64(y), ref, "bf16", f"C=128 padded block shift {shift}")


def test_block_c96_more_pairs_than_waves_stress_full():
    """C = 96 with more 16-token tile pairs than the projection + MLP launch has
    waves (grid (8, 93, 93) padded to (8, 98, 98): 69192 tokens, 4325 tiles,
    the last one half full, 2163 pairs on 2048 waves), so some waves run the
    per-pair loop (inputs, projection and LN2 of a further pair after the
    pipelined chunk loop) and the last pair's second tile lies past the tokens;
    every output token, regular and shifted (the temporal window covers T, so
    only the spatial shift remains), stress init."""
    C, heads, window = 96, 3, (8, 7, 7)
    p = _msa_params(C, heads, window, "bf16", "stress", seed=43)
    x = _rng_tokens((1, 8, 93, 93, C), "bf16", 17)
    for shift in ((0, 0, 0), (4, 3, 3)):
        say(f"C=96 block (1,8,93,93), stress, shift {shift}")
        y = vs.vswin_block_fwd(dev(x, "bf16"), dev_params(p, "bf16"), heads, window, shift)
        _, ref = oracle.block(x, p, heads, window, shift)
        check(host64(y), ref, "bf16", f"C=96 multi-pair block shift {shift}")


def _backbone_dev(params):
    return {
        "embed_w": dev(params["embed_w"], "bf16"), "embed_b": dev(params["embed_b"], "bf16"),
        "stages": [[dev_params(p, "bf16") for p in st] for st in params["stages"]],
        "merges": [dev_params(m, "bf16") for m in params["merges"]],
        "norm_g": dev(params["norm_g"], "bf16"), "norm_b": dev(params["norm_b"], "bf16"),
    }


@pytest.mark.parametrize("dtype,shape,offset", [
    ("bf16", (1, 3, 5, 10, 12), False),   # T and H padded to the patch, 4-wide w groups
    ("fp32", (2, 3, 4, 8, 8), False),
    ("bf16", (1, 2, 6, 12, 16), False),   # 2 channels
    ("bf16", (1, 3, 4, 8, 10), False),    # W not a multiple of 4: element-wise gather
    ("bf16", (1, 3, 4, 8, 8), True),      # video not 16-byte aligned: refused before any launch
])
def test_patch_embed_grids(dtype, shape, offset):
    """Patch embedding (2x4x4 patches, C = 96) on grids that exercise the
    vector gather (4 consecutive w per thread), its zero fill past the video's
    end and the element-wise fallback; a misaligned video is an error."""
    say(f"patch embed {dtype} {shape} offset {offset}")
    rng = np.random.default_rng(53)
    video = rng.standard_normal(shape).astype(np.float32)
    w = (0.02 * rng.standard_normal((96, shape[1], 2, 4, 4))).astype(np.float32)
    b = (0.02 * rng.standard_normal(96)).astype(np.float32)
    if dtype == "bf16":   # values representable in bf16, so both sides see the same inputs
        video, w, b = (torch.from_numpy(a).to(torch.bfloat16).float().numpy() for a in (video, w, b))
    vt = dev(video, dtype)
    if offset:
        big = torch.empty(vt.numel() + 1, dtype=vt.dtype, device=vt.device)
        big[1:] = vt.reshape(-1)
        with pytest.raises(vs.VswinError, match="aligned"):
            vs.vswin_patch_embed_fwd(big[1:].view(vt.shape), dev(w, dtype), dev(b, dtype))
        return
    y = vs.vswin_patch_embed_fwd(vt, dev(w, dtype), dev(b, dtype))
    check(host64(y), oracle.patch_embed(video, w, b), dtype, f"patch embed {shape}")


@pytest.mark.parametrize("shape", [(1, 2, 2, 2, 192), (1, 3, 5, 7, 192), (2, 4, 16, 16, 384)])
def test_patch_merge_small_and_ragged(shape):
    """Patch merging through the staged-K GEMM (K = 4C = 768 or 1536) at token
    counts far below, just above and at a multiple of the 128-row tile,
    with odd H and W (zero-padded 2x2 groups); LN scale and shift spread
    around 1 and 0, weights sized for outputs of order 1."""
    say(f"patch merge {shape}")
    rng = np.random.default_rng(61)
    B, T, H, W, C = shape
    bf = lambda a: torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).float().numpy()
    x = bf(rng.standard_normal(shape))
    m = {"ln_g": bf(1.0 + 0.2 * rng.standard_normal(4 * C)), "ln_b": bf(0.2 * rng.standard_normal(4 * C)),
         "w": bf(0.025 * rng.standard_normal((2 * C, 4 * C)))}   # outputs of order 1 (the bar is absolute)
    y = vs.vswin_patch_merge_fwd(dev(x, "bf16"), dev(m["ln_g"], "bf16"), dev(m["ln_b"], "bf16"), dev(m["w"], "bf16"))
    check(host64(y), oracle.patch_merge(x, m), "bf16", f"merge {shape}")


def test_workload5_backbone():
    """Workload 5 (Swin-T backbone, B=2 clips of 3x32x224x224).  Gate: every
    block, merge, the embedding and the final LN teacher-forced (each compared
    with the oracle fed the GPU's own input).  Report: the composed
    vswin_backbone_fwd against oracle.backbone() on the same clip, end to end
    in fp64, per stage (the drift of bf16 storage between kernels, which no
    per-block bar covers)."""
    say("workload 5: Swin-T backbone B=2 (per-block teacher-forced, then end to end)")
    cfg = synth.WORKLOADS[5].backbone
    video = synth.gen_video(cfg["B"], cfg["in_chans"], cfg["frames"], cfg["height"], cfg["width"], 5, "bf16")
    params = synth.gen_backbone_params(cfg, 5, "bf16")
    dparams = _backbone_dev(params)
    vt = dev(video, "bf16")
    x = vs.vswin_patch_embed_fwd(vt, dparams["embed_w"], dparams["embed_b"])
    check(host64(x), oracle.patch_embed(video, params["embed_w"], params["embed_b"]), "bf16", "patch embed")
    half = tuple(w // 2 for w in cfg["window"])
    for i, depth in enumerate(cfg["depths"]):
        for j in range(depth):
            shift = (0, 0, 0) if j % 2 == 0 else half
            y = vs.vswin_block_fwd(x, dparams["stages"][i][j], cfg["heads"][i], cfg["window"], shift)
            _, ref = oracle.block(host64(x), params["stages"][i][j], cfg["heads"][i], cfg["window"], shift)
            check(host64(y), ref, "bf16", f"stage {i} block {j}")
            x = y
        if i < len(cfg["depths"]) - 1:
            m = dparams["merges"][i]
            y = vs.vswin_patch_merge_fwd(x, m["ln_g"], m["ln_b"], m["w"])
            check(host64(y), oracle.patch_merge(host64(x), params["merges"][i]), "bf16", f"merge {i}")
            x = y
    out = vs.vswin_layernorm_fwd(x, dparams["norm_g"], dparams["norm_b"])
    check(host64(out), oracle.layer_norm(host64(x), params["norm_g"], params["norm_b"]), "bf16", "final LN")
    # the composed forward: the same call sequence, so the same bits ...
    full, trace = vs.vswin_backbone_fwd(vt, dparams, cfg, collect=True)
    assert torch.equal(full, out)
    # ... and end to end against the oracle's own backbone (no teacher forcing)
    ref_out, ref_trace = oracle.backbone(video.astype(np.float64), params, cfg, collect=True)
    k = 0
    for i, depth in enumerate(cfg["depths"]):
        k += depth
        e = np.abs(host64(trace[k - 1][1]) - ref_trace[k - 1][1])
        say(f"  end-to-end drift after stage {i + 1}: max-abs {e.max():.3e} mean-abs {e.mean():.3e} "
            f"(output scale {np.abs(ref_trace[k - 1][1]).max():.2f})")
    e = np.abs(host64(full) - ref_out)
    say(f"  end-to-end drift of the final LN output: max-abs {e.max():.3e} mean-abs {e.mean():.3e}")
    # drift over 12 blocks and 3 merges of bf16 storage is reported, not gated
    # by the per-block bar; a composition mistake (stage order, shift
    # alternation, merge placement, the stage-4 clamp) moves the LN output by O(1)
    assert e.mean() <= 3e-2, f"end-to-end mean-abs drift {e.mean():.3e}"


def test_workload5_stage_blocks_stress():
    """One regular + shifted pair at each deeper Swin-T stage's shape (B=2;
    stage 2 (16,28,28,192), stage 3 (16,14,14,384), stage 4 (16,7,7,768) with
    its clamped shift (4,0,0)) at stress init, every output token."""
    cfg = synth.WORKLOADS[5].backbone
    params = synth.gen_backbone_params(cfg, 15, "bf16", init="stress")
    for i, (H, C) in enumerate([(28, 192), (14, 384), (7, 768)], start=1):
        for j in range(2):
            shift = (0, 0, 0) if j == 0 else (4, 3, 3)
            say(f"stage {i + 1} shapes, stress init, block {j}")
            x = _rng_tokens((2, 16, H, H, C), "bf16", 60 + 2 * i + j)
            p = params["stages"][i][j]
            y = vs.vswin_block_fwd(dev(x, "bf16"), dev_params(p, "bf16"), cfg["heads"][i], cfg["window"], shift)
            _, ref = oracle.block(x, p, cfg["heads"][i], cfg["window"], shift)
            check(host64(y), ref, "bf16", f"stage {i + 1} stress block {j}")


def test_block_is_deterministic():
    say("determinism: two runs bitwise equal")
    x, params = synth.gen_workload(2)
    s = synth.WORKLOADS[2].shape
    xt = dev(x, "bf16")
    p = dev_params(params[1], "bf16")
    a = vs.vswin_block_fwd(xt, p, s.heads, s.window, s.shift)
    b = vs.vswin_block_fwd(xt, p, s.heads, s.window, s.shift)
    assert torch.equal(a, b)


def test_block_pair_graph_replay_matches_eager():
    """The block pair captured in a HIP graph gives, on every replay, the
    bits of the eager calls (the library records only kernel launches)."""
    say("graph replay of the stage-1 block pair vs eager")
    x, params = synth.gen_workload(2)
    s = synth.WORKLOADS[2].shape
    xt = dev(x, "bf16")
    p = [dev_params(q, "bf16") for q in params]
    plan = vs.vswin_plan_query(vs.make_desc(s.B, s.T, s.H, s.W, s.C, s.heads, s.window, s.shift))
    ws = torch.empty(plan["workspace_bytes"], dtype=torch.uint8, device="cuda")
    y1, y2 = torch.empty_like(xt), torch.empty_like(xt)

    def pair(st):
        vs.vswin_block_fwd(xt, p[0], s.heads, s.window, (0, 0, 0), out=y1, workspace=ws, stream=st)
        vs.vswin_block_fwd(y1, p[1], s.heads, s.window, s.shift, out=y2, workspace=ws, stream=st)

    pair(None)
    torch.cuda.synchronize()
    ref1, ref2 = y1.clone(), y2.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pair(torch.cuda.current_stream())
    other = dev(np.random.default_rng(5).standard_normal(x.shape).astype(np.float32), "bf16")
    for r in range(3):
        y1.zero_()
        y2.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y1, ref1) and torch.equal(y2, ref2), f"replay {r} differs from the eager result"
        # eager work between replays, on the same workspace
        vs.vswin_block_fwd(other, p[1], s.heads, s.window, s.shift, workspace=ws)
        torch.cuda.synchronize()


def test_empty_batch_on_gpu():
    say("empty batch")
    x = torch.empty((0, 16, 14, 14, 96), dtype=torch.bfloat16, device="cuda")
    p = dev_params(synth.gen_block_params(96, 3, 2535, 4, np.random.SeedSequence(1), "bf16"), "bf16")
    y = vs.vswin_block_fwd(x, p, 3, (8, 7, 7), (4, 3, 3))
    assert y.shape == x.shape


def _slot_to_natural(N, P, Mh, Mw, fast):
    """Row order of the block's internal window buffers, as documented for
    vswin_attention_fwd: slot s = 4 m + i holds token (pt = 4 a + i, ph, pw)
    with m = (a * Mh + ph) * Mw + pw when the MFMA path serves the shape."""
    s = np.arange(N)
    if not fast:
        return s
    m, i = s // 4, s % 4
    a, r = m // (Mh * Mw), m % (Mh * Mw)
    return (4 * a + i) * (Mh * Mw) + r


@pytest.mark.parametrize("shift", [(0, 0, 0), (4, 3, 3)])
@pytest.mark.parametrize("size", [(16, 14, 14), (16, 12, 13)])
def test_attention_core_alone(shift, size):
    """vswin_attention_fwd on random projected windows against softmax(q k^T /
    sqrt(d) + B + mask) v in fp64, with the bias rows and region labels taken
    from the oracle's geometry."""
    say(f"attention core {size} shift {shift}")
    B, C, heads, window = 1, 96, 3, (8, 7, 7)
    d = C // heads
    desc = vs.make_desc(B, *size, C, heads, window, shift)
    plan = vs.vswin_plan_query(desc)
    nW, N = plan["num_windows"], plan["tokens_per_window"]
    perm = _slot_to_natural(N, *plan["eff_window"], plan["fast_attention"])
    rng = np.random.default_rng(17)
    q, k, v = (synth.round_bf16((1.5 * rng.standard_normal((nW, heads, N, d))).astype(np.float32))
               for _ in range(3))
    table = synth.round_bf16(rng.standard_normal((15 * 13 * 13, heads)).astype(np.float32))
    qs, ks, vs_ = q[:, :, perm], k[:, :, perm], v[:, :, perm]
    if plan["fast_attention"]:
        vs_ = np.ascontiguousarray(vs_.transpose(0, 1, 3, 2))
    o = host64(vs.vswin_attention_fwd(desc, dev(qs, "bf16"), dev(ks, "bf16"), dev(vs_, "bf16"),
                                      dev(table, "bf16")))
    o_nat = np.empty_like(o)
    o_nat[:, perm] = o
    g = ov.Geometry(B, size, window, shift)
    bias = table.astype(np.float64)[g.rel]
    ref = np.zeros((nW, N, C))
    for w in range(nW):
        lab = g.win_labels[w % g.nw_sample]
        allowed = lab[:, None] == lab[None, :]
        for h in range(heads):
            sc = q[w, h].astype(np.float64) @ k[w, h].astype(np.float64).T / np.sqrt(d) + bias[:, :, h]
            if g.use_mask:
                sc = np.where(allowed, sc, -np.inf)
            sc -= sc.max(1, keepdims=True)
            e = np.exp(sc)
            ref[w, :, h * d:(h + 1) * d] = (e / e.sum(1, keepdims=True)) @ v[w, h].astype(np.float64)
    # pad query rows are not outputs of the block; compare the real ones
    real = g.index_map() >= 0
    check(o_nat[real], ref[real], "bf16", "attention core")


@pytest.mark.parametrize("case", [(96, 1, (16, 56, 56), (4, 3, 3)), (96, 1, (16, 12, 13), (0, 0, 0)),
                                  (128, 2, (16, 12, 13), (4, 3, 3))],
                         ids=["stage-1 shifted", "C=96 padded regular", "C=128 padded shifted B=2"])
def test_qkv_attention_entry(case, monkeypatch):
    """vswin_qkv_attention_fwd against the oracle's branch with an identity
    output projection (so the branch output is the heads' concatenated
    attention output), token by token through the slot map; the one-kernel
    path and the separate launches agree bit for bit."""
    C, B, size, shift = case
    heads, window = C // 32, (8, 7, 7)
    say(f"qkv + attention entry C={C} B={B} {size} shift {shift}")
    p = _msa_params(C, heads, window, "bf16", "stress", seed=43)
    p["ln1_g"] = synth.round_bf16((1 + 0.2 * np.random.default_rng(1).standard_normal(C)).astype(np.float32))
    p["ln1_b"] = synth.round_bf16((0.2 * np.random.default_rng(2).standard_normal(C)).astype(np.float32))
    x = _rng_tokens((B, *size, C), "bf16", 13)
    dp, xt = dev_params(p, "bf16"), dev(x, "bf16")
    monkeypatch.setenv("VSWIN_FUSED", "1")
    o = vs.vswin_qkv_attention_fwd(xt, dp, heads, window, shift)
    monkeypatch.setenv("VSWIN_FUSED", "0")
    o2 = vs.vswin_qkv_attention_fwd(xt, dp, heads, window, shift)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    desc = vs.make_desc(B, *size, C, heads, window, shift, dtype=torch.bfloat16)
    plan = vs.vswin_plan_query(desc)
    nW, N = plan["num_windows"], plan["tokens_per_window"]
    perm = _slot_to_natural(N, *plan["eff_window"], plan["fast_attention"])
    o_nat = np.empty((nW, N, C))
    o_nat[:, perm] = host64(o).reshape(nW, N, C)
    tok = vs.vswin_index_map(desc)[0].cpu().numpy().astype(np.int64).reshape(nW, N)
    real = tok >= 0
    q = dict(p)
    q["proj_w"] = np.eye(C, dtype=np.float32)
    q["proj_b"] = np.zeros(C, dtype=np.float32)
    xn = ov.layer_norm(x.astype(np.float64), p["ln1_g"].astype(np.float64), p["ln1_b"].astype(np.float64))
    ref = ov.window_msa(xn, q, heads, window, shift).reshape(-1, C)
    check(o_nat[real], ref[tok[real]], "bf16", f"qkv + attention C={C} {size} {shift}")


def test_attention_prepared_tables_reuse():
    """The prepared bias tables live in the attention workspace: a call with
    F_TABLES_READY reuses them (same result, bit for bit), a call without it
    rebuilds them from the table it is given."""
    say("attention prepared-table reuse")
    B, C, heads, window, shift, size = 1, 96, 3, (8, 7, 7), (4, 3, 3), (16, 14, 14)
    d = C // heads
    desc = vs.make_desc(B, *size, C, heads, window, shift)
    ready = vs.make_desc(B, *size, C, heads, window, shift, flags=vs.F_TABLES_READY)
    plan = vs.vswin_plan_query(desc)
    assert plan["fast_attention"] == 1 and plan["attention_workspace_bytes"] > 0
    nW, N = plan["num_windows"], plan["tokens_per_window"]
    g = torch.Generator(device="cuda").manual_seed(5)
    q, k, vt = (torch.randn((nW, heads, *s), generator=g, device="cuda").to(torch.bfloat16)
                for s in ((N, d), (N, d), (d, N)))
    t1, t2 = (torch.randn((15 * 13 * 13, heads), generator=g, device="cuda").to(torch.bfloat16) for _ in range(2))
    ws = torch.empty(plan["attention_workspace_bytes"], dtype=torch.uint8, device="cuda")
    o1 = vs.vswin_attention_fwd(desc, q, k, vt, t1, workspace=ws).clone()
    o1r = vs.vswin_attention_fwd(ready, q, k, vt, t1, workspace=ws).clone()
    o2 = vs.vswin_attention_fwd(desc, q, k, vt, t2, workspace=ws).clone()
    ws2 = torch.empty_like(ws)
    o2f = vs.vswin_attention_fwd(desc, q, k, vt, t2, workspace=ws2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o1r)
    assert torch.equal(o2, o2f)
    assert not torch.equal(o1, o2)


def test_mfma_rate_probe_runs():
    """The MFMA throughput helper launches and leaves finite values; the FLOP
    count it reports is blocks x 8 waves x 8 MFMAs x iters x 16384."""
    say("mfma rate probe")
    out = torch.full((4 * 512,), float("nan"), dtype=torch.float32, device="cuda")
    flops = vs.vswin_mfma_rate_probe(out, 4, 16)
    torch.cuda.synchronize()
    assert flops == 4 * 8 * 8 * 16 * 16384
    assert torch.isfinite(out).all()
