"""Host-side checks of the C ABI (no GPU): the library loads and exports every
entry point include/vswin.h declares, the host plan matches the oracle's
geometry exactly, and every argument error is reported before any launch."""
import ctypes
import os
import re

import numpy as np
import pytest

import synth
from oracle import vswin as ov
import shifted_window_attention_amd as vs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vswin.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(vswin_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = vs.lib()
    names = _declared()
    assert "vswin_block_fwd" in names and "vswin_window_msa_fwd" in names
    for n in names:
        assert hasattr(L, n), n
    assert L.vswin_abi_version() == 1


def test_status_strings():
    L = vs.lib()
    for s, txt in [(0, b"ok"), (-1, b"invalid argument"), (-2, b"unsupported"),
                   (-3, b"workspace too small"), (-4, b"HIP error")]:
        assert L.vswin_status_string(s) == txt


GEOMS = [
    (1, (4, 14, 14), 32, 2, (2, 7, 7), (1, 3, 3), "fp32"),
    (1, (16, 56, 56), 96, 3, (8, 7, 7), (0, 0, 0), "bf16"),
    (1, (16, 56, 56), 96, 3, (8, 7, 7), (4, 3, 3), "bf16"),
    (4, (16, 14, 14), 384, 12, (8, 7, 7), (4, 3, 3), "bf16"),
    (8, (16, 60, 60), 128, 4, (8, 7, 7), (0, 0, 0), "bf16"),
    (8, (16, 60, 60), 128, 4, (8, 7, 7), (4, 3, 3), "bf16"),
    (2, (16, 7, 7), 768, 24, (8, 7, 7), (4, 3, 3), "bf16"),       # backbone stage 4: clamp
    (2, (5, 9, 11), 32, 2, (2, 4, 3), (1, 2, 1), "bf16"),
    (1, (3, 5, 5), 64, 2, (8, 7, 7), (4, 3, 3), "fp32"),
]


@pytest.mark.parametrize("g", GEOMS)
@pytest.mark.parametrize("strict", [False, True])
def test_plan_matches_oracle_geometry(g, strict):
    B, size, C, heads, window, shift, dt = g
    d = vs.make_desc(B, *size, C, heads, window, shift, dtype=0 if dt == "fp32" else 1,
                     flags=vs.F_CLAMP_STRICT if strict else 0)
    p = vs.vswin_plan_query(d)
    o = ov.Geometry(B, size, window, shift, clamp_strict=strict)
    assert p["eff_window"] == o.window
    assert p["eff_shift"] == o.shift
    assert p["padded"] == o.padded
    assert p["tokens_per_window"] == o.N
    assert p["num_windows"] == o.nW
    assert p["tokens"] == B * int(np.prod(size))
    assert p["masked"] == o.use_mask
    assert p["workspace_bytes"] >= p["msa_workspace_bytes"] > 0


def test_fast_path_selection():
    for wid in (2, 3, 4):
        s = synth.WORKLOADS[wid].shape
        for shift in ((0, 0, 0), s.shift):
            d = vs.make_desc(s.B, s.T, s.H, s.W, s.C, s.heads, s.window, shift, dtype=1)
            assert vs.vswin_plan_query(d)["fast_attention"], (wid, shift)
    # fp32 and windows whose temporal extent is not a multiple of 4 use the generic kernel
    assert not vs.vswin_plan_query(vs.make_desc(1, 4, 14, 14, 32, 2, (2, 7, 7), (1, 3, 3), dtype=0))["fast_attention"]
    assert not vs.vswin_plan_query(vs.make_desc(1, 6, 14, 14, 64, 2, (6, 7, 7), (3, 3, 3), dtype=1))["fast_attention"]
    # temporal window 16 (784 tokens) runs on the MFMA kernel's scalar-table form;
    # longer windows, or N > 512 with another spatial window, do not
    assert vs.vswin_plan_query(vs.make_desc(1, 16, 56, 56, 96, 3, (16, 7, 7), (8, 3, 3), dtype=1))["fast_attention"]
    assert not vs.vswin_plan_query(vs.make_desc(1, 24, 14, 14, 64, 2, (24, 7, 7), (12, 3, 3),
                                                dtype=1))["fast_attention"]
    assert not vs.vswin_plan_query(vs.make_desc(1, 16, 12, 12, 64, 2, (16, 6, 6), (8, 3, 3),
                                                dtype=1))["fast_attention"]
    # window 4 with temporal shift 2 (labels compared key by key) runs on the MFMA
    # kernel, except with the -100 mask
    assert vs.vswin_plan_query(vs.make_desc(1, 16, 56, 56, 96, 3, (4, 7, 7), (2, 3, 3), dtype=1))["fast_attention"]
    assert not vs.vswin_plan_query(vs.make_desc(1, 16, 56, 56, 96, 3, (4, 7, 7), (2, 3, 3), dtype=1,
                                                flags=vs.F_MASK_M100))["fast_attention"]
    # the code-compat -100 mask runs on the MFMA kernel too
    assert vs.vswin_plan_query(vs.make_desc(1, 16, 14, 14, 64, 2, (8, 7, 7), (4, 3, 3), dtype=1,
                                            flags=vs.F_MASK_M100))["fast_attention"]


BAD = [
    dict(C=96, heads=5),                       # C % heads
    dict(shift=(8, 3, 3)),                     # shift >= window
    dict(shift=(-1, 0, 0)),
    dict(window=(0, 7, 7)),
    dict(T=0),
    dict(eps=0.0),
    dict(flags=64),
]


@pytest.mark.parametrize("bad", BAD)
def test_plan_rejects_bad_descriptors(bad):
    kw = dict(B=1, T=16, H=14, W=14, C=96, heads=3, window=(8, 7, 7), shift=(4, 3, 3), eps=1e-5, flags=0)
    kw.update(bad)
    d = vs.make_desc(kw["B"], kw["T"], kw["H"], kw["W"], kw["C"], kw["heads"], kw["window"], kw["shift"],
                     dtype=1, eps=kw["eps"], flags=kw["flags"])
    with pytest.raises(vs.VswinError) as e:
        vs.vswin_plan_query(d)
    assert e.value.status == -1


def test_unsupported_head_dim():
    d = vs.make_desc(1, 16, 14, 14, 256, 2, (8, 7, 7), (0, 0, 0), dtype=1)   # head_dim 128
    with pytest.raises(vs.VswinError) as e:
        vs.vswin_plan_query(d)
    assert e.value.status == -2


def _fake_weights(base=0x10000):
    w = vs.BlockWeights()
    for i, (n, _) in enumerate(vs.BlockWeights._fields_):
        setattr(w, n, base + 256 * i)
    return w


def _call_block(d, x, w, y, ws, nbytes, fn="vswin_block_fwd"):
    return getattr(vs.lib(), fn)(ctypes.byref(d), x, ctypes.byref(w) if w is not None else None, y, ws,
                                 nbytes, None)


def test_block_argument_errors_before_launch():
    d = vs.make_desc(1, 16, 14, 14, 96, 3, (8, 7, 7), (4, 3, 3), dtype=1)
    need = vs.vswin_plan_query(d)["workspace_bytes"]
    w = _fake_weights()
    X, Y, WS = 0x100000, 0x200000, 0x300000
    L = vs.lib()
    assert _call_block(d, None, w, Y, WS, need) == -1                 # null x
    assert _call_block(d, X + 8, w, Y, WS, need) == -1                # misaligned x
    assert _call_block(d, X, w, X, WS, need) == -1                    # aliasing
    assert _call_block(d, X, None, Y, WS, need) == -1                 # null weights
    w2 = _fake_weights(); w2.rpb_table = None
    assert _call_block(d, X, w2, Y, WS, need) == -1
    assert b"rpb_table" in L.vswin_last_error()
    assert _call_block(d, X, w, Y, WS, need - 1) == -3                # workspace too small
    assert _call_block(d, X, w, Y, WS + 16, need) == -3               # workspace misaligned
    need_msa = vs.vswin_plan_query(d)["msa_workspace_bytes"]
    assert _call_block(d, X, w, Y, WS, need_msa - 1, "vswin_window_msa_fwd") == -3


def test_qkv_attention_argument_errors_before_launch():
    """vswin_qkv_attention_fwd: argument, support and workspace errors come
    back before anything is enqueued."""
    d = vs.make_desc(1, 16, 14, 14, 96, 3, (8, 7, 7), (4, 3, 3), dtype=1)
    need = vs.vswin_plan_query(d)["msa_workspace_bytes"]
    w = _fake_weights()
    X, O, WS = 0x100000, 0x200000, 0x300000
    fn = "vswin_qkv_attention_fwd"
    L = vs.lib()
    assert _call_block(d, None, w, O, WS, need, fn) == -1             # null x
    assert _call_block(d, X, w, X, WS, need, fn) == -1                # aliasing
    w2 = _fake_weights(); w2.ln1_g = None
    assert _call_block(d, X, w2, O, WS, need, fn) == -1
    assert b"ln1_g" in L.vswin_last_error()
    assert _call_block(d, X, w, O, WS, need - 1, fn) == -3            # workspace too small
    assert _call_block(d, X, w, O, WS + 16, need, fn) == -3           # workspace misaligned
    # fp32, and a width whose qkv projection cannot gather its own rows
    for dd in (vs.make_desc(1, 4, 14, 14, 32, 2, (2, 7, 7), (1, 3, 3), dtype=0),
               vs.make_desc(1, 16, 14, 14, 192, 6, (8, 7, 7), (4, 3, 3), dtype=1)):
        n = vs.vswin_plan_query(dd)["msa_workspace_bytes"]
        assert _call_block(dd, X, w, O, WS, n, fn) == -2
    # nothing to do for an empty batch
    d0 = vs.make_desc(0, 16, 14, 14, 96, 3, (8, 7, 7), (4, 3, 3), dtype=1)
    assert _call_block(d0, X, w, O, None, 0, fn) == 0


def test_fault_hook_reports_hip_error(monkeypatch):
    monkeypatch.setenv("VSWIN_FAULT", "launch")
    d = vs.make_desc(1, 16, 14, 14, 96, 3, (8, 7, 7), (4, 3, 3), dtype=1)
    need = vs.vswin_plan_query(d)["workspace_bytes"]
    assert _call_block(d, 0x100000, _fake_weights(), 0x200000, 0x300000, need) == -4
    assert b"injected" in vs.lib().vswin_last_error()


def test_empty_batch_is_a_no_op():
    d = vs.make_desc(0, 16, 14, 14, 96, 3, (8, 7, 7), (4, 3, 3), dtype=1)
    p = vs.vswin_plan_query(d)
    assert p["num_windows"] == 0 and p["tokens"] == 0
    # nothing is enqueued, so this runs without a GPU
    assert _call_block(d, 0x100000, _fake_weights(), 0x200000, None, 0) == 0


def test_mfma_rate_probe_rejects_bad_arguments():
    """The measurement helper validates its arguments on the host (no launch)."""
    L = vs.lib()
    for blocks, iters in [(0, 10), (1, 0), (-3, 5)]:
        assert L.vswin_mfma_rate_probe(None, blocks, iters, None) == -1
    assert L.vswin_mfma_rate_probe(None, 1, 1, None) == -1   # NULL out


def test_bwd_workspace_query_refuses_unsupported_shapes():
    """The backward serves the bf16 MFMA-attention shapes (the -100 mask,
    key-by-key labels and windows of up to 1024 tokens included); -100 with a
    boundary inside a key group, windows over 1024 tokens and fp32 are refused
    on the host."""
    ok = vs.vswin_bwd_workspace_query(vs.make_desc(1, 16, 56, 56, 96, 3, (8, 7, 7), (4, 3, 3), dtype=1))
    assert ok["block"] > ok["msa"] > 0
    for d in (vs.make_desc(1, 16, 14, 14, 64, 2, (8, 7, 7), (4, 3, 3), dtype=1, flags=vs.F_MASK_M100),
              vs.make_desc(1, 16, 14, 14, 64, 2, (4, 7, 7), (2, 3, 3), dtype=1),
              vs.make_desc(1, 16, 14, 14, 64, 2, (16, 7, 7), (8, 3, 3), dtype=1)):
        assert vs.vswin_bwd_workspace_query(d)["block"] > 0
    for d in (vs.make_desc(1, 16, 14, 14, 64, 2, (4, 7, 7), (2, 3, 3), dtype=1, flags=vs.F_MASK_M100),
              vs.make_desc(1, 24, 14, 14, 64, 2, (24, 7, 7), (12, 3, 3), dtype=1),
              vs.make_desc(1, 4, 14, 14, 32, 2, (2, 7, 7), (1, 3, 3), dtype=0)):
        with pytest.raises(vs.VswinError) as e:
            vs.vswin_bwd_workspace_query(d)
        assert e.value.status == -2


def test_head_views_inflation_reject_bad_arguments():
    """Argument checks of the inference entry points return before any device
    work (no GPU needed)."""
    L = vs.lib()
    # head: C not a multiple of 4; negative K; bad dtype
    assert L.vswin_head_fwd(1, 10, 6, 4, 0, None, None, None, None, None, 0, None) == -1
    assert L.vswin_head_fwd(1, 10, 8, -1, 0, None, None, None, None, None, 0, None) == -1
    assert L.vswin_head_fwd(1, 10, 8, 4, 7, None, None, None, None, None, 0, None) == -1
    # empty batch or no classes: nothing to do
    assert L.vswin_head_fwd(0, 10, 8, 4, 0, None, None, None, None, None, 0, None) == 0
    assert L.vswin_head_fwd(1, 10, 8, 0, 0, None, None, None, None, None, 0, None) == 0
    # views: too many views, no views
    assert L.vswin_multiview_average(1, 4097, 10, None, None, None) == -1
    assert L.vswin_multiview_average(1, 0, 10, None, None, None) == -1
    assert L.vswin_multiview_average(0, 2, 10, None, None, None) == 0
    # inflation: bad sizes
    assert L.vswin_inflate_patch_embed(96, 3, 0, 4, 4, 0, None, None, None) == -1
    assert L.vswin_inflate_bias_table(169, 3, 0, 0, None, None, None) == -1
    assert L.vswin_head_workspace(2, 392, 768) >= 2 * 768 * 4 * 2


def test_issue_probe_rejects_bad_arguments():
    L = vs.lib()
    assert L.vswin_issue_probe(None, 1, 1, 4, None) == -1
    assert L.vswin_issue_probe(None, 0, 1, 0, None) == -1
    assert L.vswin_issue_probe(None, 1, 1, 0, None) == -1   # NULL out


def _host_block(C=32, heads=2, window=(2, 7, 7), dtype="fp32"):
    import torch
    p = synth.gen_block_params(C, heads, (2 * window[0] - 1) * (2 * window[1] - 1) * (2 * window[2] - 1), 4,
                               np.random.SeedSequence(3), dtype)
    td = torch.float32 if dtype == "fp32" else torch.bfloat16
    w = {k: torch.from_numpy(v).to(td) for k, v in p.items()}
    x = torch.zeros((1, 4, 14, 14, C), dtype=td)
    return x, w


@pytest.mark.parametrize("mutate", [
    "table for another window", "qkv_w transposed", "weight dtype", "proj_w missing", "fc2_w width",
    "heads not dividing C",
])
def test_binding_rejects_mismatched_weights(mutate):
    """The binding checks every weight's shape, dtype and device against x
    before any library call, so a mismatch is a ValueError, not a kernel
    reading past an allocation."""
    import torch
    x, w = _host_block()
    heads = 2
    if mutate == "table for another window":
        w["rpb_table"] = torch.zeros((15 * 13 * 13, 2))
    elif mutate == "qkv_w transposed":
        w["qkv_w"] = w["qkv_w"].t().contiguous()
    elif mutate == "weight dtype":
        w["fc1_w"] = w["fc1_w"].to(torch.bfloat16)
    elif mutate == "proj_w missing":
        del w["proj_w"]
    elif mutate == "fc2_w width":
        w["fc2_w"] = torch.zeros((32, 100))
    elif mutate == "heads not dividing C":
        heads = 3
    for fn in (vs.vswin_block_fwd, vs.vswin_window_msa_fwd):
        if fn is vs.vswin_window_msa_fwd and mutate in ("weight dtype", "fc2_w width"):
            continue          # the MSA branch does not read the MLP weights
        with pytest.raises(ValueError):
            fn(x, w, heads, (2, 7, 7), (1, 3, 3))
    with pytest.raises(ValueError):
        vs.vswin_block_bwd(x, w, torch.zeros_like(x), heads, (2, 7, 7), (1, 3, 3))


def test_binding_rejects_mismatched_outputs_and_grads():
    import torch
    x, w = _host_block()
    args = (w, 2, (2, 7, 7), (1, 3, 3))
    with pytest.raises(ValueError):
        vs.vswin_block_fwd(x, *args, out=torch.zeros((1, 4, 14, 14, 32), dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        vs.vswin_window_msa_fwd(x, *args, out=torch.zeros((1, 4, 14, 13, 32)))
    with pytest.raises(ValueError):
        vs.vswin_block_bwd(x, w, torch.zeros((1, 4, 14, 14, 16)), 2, (2, 7, 7), (1, 3, 3))
    with pytest.raises(ValueError):
        vs.vswin_block_bwd(x, w, torch.zeros_like(x), 2, (2, 7, 7), (1, 3, 3), dx=torch.zeros((5,)))
    with pytest.raises(ValueError):        # gradients are fp32 and shaped like their weight
        vs.vswin_block_bwd(x, w, torch.zeros_like(x), 2, (2, 7, 7), (1, 3, 3),
                           grads={"qkv_w": torch.zeros((96, 32), dtype=torch.bfloat16)})
    with pytest.raises(ValueError):
        vs.vswin_block_bwd(x, w, torch.zeros_like(x), 2, (2, 7, 7), (1, 3, 3),
                           grads={"proj_w": torch.zeros((32, 33))})
    with pytest.raises(ValueError):        # the MSA backward writes no MLP gradient
        vs.vswin_window_msa_bwd(x, w, torch.zeros_like(x), 2, (2, 7, 7), (1, 3, 3),
                                grads={"fc1_w": torch.zeros((128, 32))})


def test_binding_attention_core_checks_buffer_sizes():
    import torch
    d = vs.make_desc(1, 16, 14, 14, 96, 3, (8, 7, 7), (4, 3, 3))
    plan = vs.vswin_plan_query(d)
    nW, N = plan["num_windows"], plan["tokens_per_window"]
    q = torch.zeros((nW, 3, N, 32), dtype=torch.bfloat16)
    tab = torch.zeros((15 * 13 * 13, 3), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        vs.vswin_attention_fwd(d, q, q, q[:, :, :-1], tab)
    with pytest.raises(ValueError):
        vs.vswin_attention_fwd(d, q, q, q, tab[:-1])
    with pytest.raises(ValueError):
        vs.vswin_attention_fwd(d, q, q, q, tab, out=torch.zeros((nW, N, 95), dtype=torch.bfloat16))
