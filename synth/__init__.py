"""Seeded synthetic inputs for the Video Swin window-attention block.

This module is shared by the oracle tests and by the GPU path's tests and
benchmark.  It holds only workload shapes and random-number recipes: no step
of the method (no LayerNorm, roll, partition, attention, clamp or padding
rule) lives here, so that the oracle and the HIP path stay independent.

Workloads follow the shapes of the Video Swin pages: a 32x224x224 RGB clip
cut into 2x4x4 patches gives 16x56x56 tokens (Video Swin Transformer, §3.1),
windows of 8x7x7 tokens (§3.3), Swin-T / Swin-B widths and head counts
(§3.3 and the paper-vs-code notes on heads per stage).

Recipe (identical bytes on both sides of every comparison):
  * RNG: numpy Generator(PCG64) seeded from SeedSequence(seed).spawn(k);
    one child stream per tensor, in the fixed order of ``_BLOCK_TENSORS``.
  * tokens / video: N(0, 1).
  * "spec" init: Linear weights truncated normal std 0.02 (resampled
    outside +-2 sigma), relative-position table truncated normal std 0.02
    (plain N(0, 0.02) for the fp32 smoke workload), biases 0, LN gamma 1,
    LN beta 0.
  * "stress" init (parity only, never timed): Linear weights N(0, 1/fan_in),
    table N(0, 1), biases N(0, 0.1), gamma 1 + N(0, 0.1), beta N(0, 0.1).
    It makes bias, mask and roll mistakes visible above the tolerances.
  * bf16 workloads round every tensor to bf16 (round to nearest even) once,
    so both sides consume the same stored values.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Tuple

import numpy as np

__all__ = [
    "BlockShape", "Workload", "WORKLOADS", "round_bf16", "gen_tokens",
    "gen_block_params", "gen_stack_params", "gen_backbone_params",
    "gen_video", "BLOCK_TENSORS",
]


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even).

    Returns float32 whose low 16 mantissa bits are zero.  NaN stays NaN.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16) << 16
    out = rounded.astype(np.uint32).view(np.float32)
    nan = np.isnan(a)
    if nan.any():
        out = out.copy()
        out[nan] = np.nan
    return out.reshape(a.shape)


@dataclasses.dataclass(frozen=True)
class BlockShape:
    """Shape of one Video Swin block's input and its hyper-parameters."""
    B: int
    T: int
    H: int
    W: int
    C: int
    heads: int
    window: Tuple[int, int, int]
    shift: Tuple[int, int, int]
    mlp_ratio: int = 4

    @property
    def tokens(self) -> int:
        return self.B * self.T * self.H * self.W

    @property
    def table_rows(self) -> int:
        P, Mh, Mw = self.window
        return (2 * P - 1) * (2 * Mh - 1) * (2 * Mw - 1)


@dataclasses.dataclass(frozen=True)
class Workload:
    """A named synthetic workload.

    ``blocks`` lists the block stack (regular / shifted alternate: even index
    uses shift 0, odd index uses ``shape.shift``).  The backbone workload sets
    ``backbone`` instead.
    """
    wid: int
    name: str
    dtype: str                      # "fp32" or "bf16"
    shape: Optional[BlockShape]
    depth: int                      # number of blocks in the stack
    table_truncated: bool = True
    backbone: Optional[dict] = None


WORKLOADS: Dict[int, Workload] = {
    1: Workload(1, "smoke fp32 block pair (4,14,14,32)", "fp32",
                BlockShape(1, 4, 14, 14, 32, 2, (2, 7, 7), (1, 3, 3)), 2,
                table_truncated=False),
    2: Workload(2, "Swin-T stage-1 block pair (16,56,56,96)", "bf16",
                BlockShape(1, 16, 56, 56, 96, 3, (8, 7, 7), (4, 3, 3)), 2),
    3: Workload(3, "Swin-T stage-3 six blocks B=4 (16,14,14,384)", "bf16",
                BlockShape(4, 16, 14, 14, 384, 12, (8, 7, 7), (4, 3, 3)), 6),
    4: Workload(4, "Swin-B stage-1 block pair B=8 (16,60,60,128) padded", "bf16",
                BlockShape(8, 16, 60, 60, 128, 4, (8, 7, 7), (4, 3, 3)), 2),
    5: Workload(5, "Swin-T backbone B=2 video (3,32,224,224)", "bf16", None, 12,
                backbone=dict(B=2, in_chans=3, frames=32, height=224, width=224,
                              patch=(2, 4, 4), embed_dim=96,
                              depths=(2, 2, 6, 2), heads=(3, 6, 12, 24),
                              window=(8, 7, 7), shift=(4, 3, 3), mlp_ratio=4)),
}

# Order in which each block's tensors draw their child seed streams.
BLOCK_TENSORS: List[str] = [
    "ln1_g", "ln1_b", "qkv_w", "qkv_b", "proj_w", "proj_b", "rpb_table",
    "ln2_g", "ln2_b", "fc1_w", "fc1_b", "fc2_w", "fc2_b",
]


def _trunc_normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    """N(0, std^2) truncated to +-2 std by resampling (float32)."""
    out = rng.standard_normal(size=shape, dtype=np.float32)
    bad = np.abs(out) > 2.0
    while bad.any():
        out[bad] = rng.standard_normal(size=int(bad.sum()), dtype=np.float32)
        bad = np.abs(out) > 2.0
    return out * np.float32(std)


def _finish(a: np.ndarray, dtype: str) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    return round_bf16(a) if dtype == "bf16" else a


def gen_tokens(shape: BlockShape, seed: int, dtype: str) -> np.ndarray:
    """Tokens (B, T, H, W, C), N(0, 1), as float32 holding `dtype` values."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    x = rng.standard_normal(size=(shape.B, shape.T, shape.H, shape.W, shape.C),
                            dtype=np.float32)
    return _finish(x, dtype)


def gen_block_params(C: int, heads: int, table_rows: int, mlp_ratio: int,
                     seed_seq: np.random.SeedSequence, dtype: str,
                     init: str = "spec", table_truncated: bool = True
                     ) -> Dict[str, np.ndarray]:
    """One block's parameters in PyTorch layouts (Linear weight = (out, in)).

    rpb_table is ((2P-1)(2Mh-1)(2Mw-1), heads).
    """
    hid = mlp_ratio * C
    shapes = {
        "ln1_g": (C,), "ln1_b": (C,),
        "qkv_w": (3 * C, C), "qkv_b": (3 * C,),
        "proj_w": (C, C), "proj_b": (C,),
        "rpb_table": (table_rows, heads),
        "ln2_g": (C,), "ln2_b": (C,),
        "fc1_w": (hid, C), "fc1_b": (hid,),
        "fc2_w": (C, hid), "fc2_b": (C,),
    }
    children = seed_seq.spawn(len(BLOCK_TENSORS))
    out: Dict[str, np.ndarray] = {}
    for name, child in zip(BLOCK_TENSORS, children):
        rng = np.random.Generator(np.random.PCG64(child))
        shp = shapes[name]
        if init == "spec":
            if name.endswith("_w"):
                a = _trunc_normal(rng, shp, 0.02)
            elif name == "rpb_table":
                a = (_trunc_normal(rng, shp, 0.02) if table_truncated else
                     rng.standard_normal(size=shp, dtype=np.float32) * np.float32(0.02))
            elif name.endswith("_g"):
                a = np.ones(shp, np.float32)
            else:
                a = np.zeros(shp, np.float32)
        elif init == "stress":
            if name.endswith("_w"):
                a = rng.standard_normal(size=shp, dtype=np.float32) / np.float32(np.sqrt(shp[1]))
            elif name == "rpb_table":
                a = rng.standard_normal(size=shp, dtype=np.float32)
            elif name.endswith("_g"):
                a = 1.0 + 0.1 * rng.standard_normal(size=shp, dtype=np.float32)
            else:
                a = 0.1 * rng.standard_normal(size=shp, dtype=np.float32)
        else:
            raise ValueError(f"unknown init {init!r}")
        out[name] = _finish(a, dtype)
    return out


def gen_stack_params(wl: Workload, seed: int, init: str = "spec") -> List[Dict[str, np.ndarray]]:
    """Parameters of every block of a block-stack workload."""
    s = wl.shape
    assert s is not None
    ss = np.random.SeedSequence(seed).spawn(wl.depth + 1)[1:]
    return [gen_block_params(s.C, s.heads, s.table_rows, s.mlp_ratio, ss[i],
                             wl.dtype, init, wl.table_truncated)
            for i in range(wl.depth)]


def gen_workload(wid: int, init: str = "spec", seed: Optional[int] = None):
    """(tokens, [block params]) for a block-stack workload; seed = workload id."""
    wl = WORKLOADS[wid]
    seed = wid if seed is None else seed
    ss_tok = np.random.SeedSequence(seed).spawn(1)[0]
    x = gen_tokens(wl.shape, ss_tok.generate_state(1)[0], wl.dtype)
    return x, gen_stack_params(wl, seed, init)


def gen_video(B: int, chans: int, frames: int, height: int, width: int,
              seed: int, dtype: str) -> np.ndarray:
    """Video clip (B, chans, frames, height, width), N(0, 1)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    v = rng.standard_normal(size=(B, chans, frames, height, width), dtype=np.float32)
    return _finish(v, dtype)


def gen_backbone_params(cfg: dict, seed: int, dtype: str, init: str = "spec") -> dict:
    """Parameters of a Video Swin backbone (patch embed, stages, merges, final LN).

    Layout:
      embed_w (C, in_chans, pt, ph, pw) -- Conv3d weight layout; embed_b (C,)
      stages[i] = list of block param dicts (width C_i = C * 2**i)
      merges[i] (i < n_stages-1) = dict(ln_g (4C_i,), ln_b (4C_i,), w (2C_i, 4C_i))
      norm_g, norm_b (C_last,)
    """
    C0 = cfg["embed_dim"]
    pt, ph, pw = cfg["patch"]
    P, Mh, Mw = cfg["window"]
    rows = (2 * P - 1) * (2 * Mh - 1) * (2 * Mw - 1)
    depths, heads = cfg["depths"], cfg["heads"]
    n_st = len(depths)
    ss = np.random.SeedSequence(seed).spawn(4 + n_st * 2)
    rng = lambda i: np.random.Generator(np.random.PCG64(ss[i]))
    kin = cfg["in_chans"] * pt * ph * pw
    p: dict = {}
    if init == "spec":
        p["embed_w"] = _finish(_trunc_normal(rng(1), (C0, cfg["in_chans"], pt, ph, pw), 0.02), dtype)
        p["embed_b"] = np.zeros((C0,), np.float32)
    else:
        p["embed_w"] = _finish(rng(1).standard_normal(size=(C0, cfg["in_chans"], pt, ph, pw),
                                                       dtype=np.float32) / np.float32(np.sqrt(kin)), dtype)
        p["embed_b"] = _finish(0.1 * rng(2).standard_normal(size=(C0,), dtype=np.float32), dtype)
    p["stages"], p["merges"] = [], []
    for i in range(n_st):
        Ci = C0 * 2 ** i
        bss = ss[4 + 2 * i].spawn(depths[i])
        p["stages"].append([gen_block_params(Ci, heads[i], rows, cfg["mlp_ratio"], bss[j],
                                             dtype, init) for j in range(depths[i])])
        if i < n_st - 1:
            r = np.random.Generator(np.random.PCG64(ss[5 + 2 * i]))
            if init == "spec":
                m = dict(ln_g=np.ones((4 * Ci,), np.float32), ln_b=np.zeros((4 * Ci,), np.float32),
                         w=_trunc_normal(r, (2 * Ci, 4 * Ci), 0.02))
            else:
                m = dict(ln_g=1.0 + 0.1 * r.standard_normal(size=(4 * Ci,), dtype=np.float32),
                         ln_b=0.1 * r.standard_normal(size=(4 * Ci,), dtype=np.float32),
                         w=r.standard_normal(size=(2 * Ci, 4 * Ci), dtype=np.float32) / np.float32(np.sqrt(4 * Ci)))
            p["merges"].append({k: _finish(v, dtype) for k, v in m.items()})
    Cl = C0 * 2 ** (n_st - 1)
    if init == "spec":
        p["norm_g"], p["norm_b"] = np.ones((Cl,), np.float32), np.zeros((Cl,), np.float32)
    else:
        r = rng(3)
        p["norm_g"] = _finish(1.0 + 0.1 * r.standard_normal(size=(Cl,), dtype=np.float32), dtype)
        p["norm_b"] = _finish(0.1 * r.standard_normal(size=(Cl,), dtype=np.float32), dtype)
    return p
