"""CPU fp64 oracle of the Video Swin 3D (shifted-)window attention block.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke entry point and the
benchmark's CPU-baseline leg may import this module.  The product path (the
HIP library and its Python binding) never calls it, and it shares no code,
tables or helpers with that path.

Everything here is the plain definition, step by step, in float64:
explicit zero padding, an explicit ``np.roll``, a per-window Python loop, a
region-label mask and a max-subtracted softmax.  Inputs are the exact stored
values (bf16 or fp32) upcast to float64.

Sources (Video Swin Transformer pages):
  * block pair and pre-norm residual structure: §3.1 and eq. 1 (page
    "Video Swin Transformer", Method steps 3 and 5);
  * window partition, half-window shift by cyclic roll, region mask, relative
    position bias and scaled softmax: §3.2 and eq. 2;
  * window (8,7,7), head width 32: §3.3;
  * padding to window multiples and the window/shift clamp: the
    paper-vs-code notes ("Mask value and padding") and Pitfalls;
  * op order LN -> pad -> roll -> partition, qkv = Linear(C, 3C), q scaled by
    head_dim**-0.5: the mmaction2 walk-through (CSDN page, section 1.2);
  * patch embedding and patch merging: §3.1 steps 1-2 and the CSDN page's
    PatchEmbed3D / PatchMerging description.

Readings of points the pages leave open (each listed in the design notes):
  D1 roll by -shift before, +shift after (torch/numpy roll semantics);
  D2 pad first, then roll the padded grid; un-roll, then crop;
  D3 shift = window // 2 per axis;
  D4 an axis whose size is <= its window takes window = size, shift 0
     (``clamp_strict`` gives the literal "smaller than");
  D5 zeros appended at the end of each axis, after LN1;
  D6 pad tokens form their own region (``pad_visible`` gives the code's
     behaviour of leaving them visible);
  D7 region = slice label [0, n-w) / [n-w, n-s) / [n-s, n) per shifted axis
     on the rolled padded grid;
  D8 masked pairs are excluded (weight exactly 0); ``mask_m100`` adds -100;
  D9 relative offset = query - key, table row = (dt+P-1)(2Mh-1)(2Mw-1) +
     (dh+Mh-1)(2Mw-1) + (dw+Mw-1), temporal offset outermost;
  D11 qkv output = [q | k | v], channel = head * d + e;
  D12 LayerNorm with biased variance, eps 1e-5;  D13 exact erf GELU;
  D15 dropout / drop-path are identity (inference);
  D16 windows ordered (b, wt, wh, ww), tokens (pt, ph, pw), row-major;
  D17 patch vector order (c, kt, kh, kw), no patch norm;
  D18 merge concat order (h,w) offsets (0,0),(1,0),(0,1),(1,1), LN(4C), Linear;
  D23 classification head = mean of the final tokens over (T', H', W'), then
      Linear(C -> classes) (the 2D Swin page's global average pooling and
      linear classifier, applied to the 3D token grid);
  D24 several views of one video (temporal clips x spatial crops, Table 1)
      combine as the mean over views of each view's softmax probabilities;
  D25 inflation (§3.4): the 2D patch kernel is repeated over the pt temporal
      slots and divided by pt (0.5 for pt = 2); the 2D bias table is repeated
      over the 2P - 1 temporal offsets, temporal offset outermost (D9).

Parity unpinned (no page value separates the alternatives; shared written
conventions): D9 offset sign and h/w order, D12 eps, D13 erf vs tanh, D17/D18
flatten and concat orders, D4 equality case, D24 probabilities vs logits.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
from scipy.special import erf as _erf

PAD_LABEL = -1

Int3 = Tuple[int, int, int]


# --------------------------------------------------------------------------
# geometry: clamp, padding, window counts
# --------------------------------------------------------------------------
def effective_window(size: Sequence[int], window: Sequence[int], shift: Sequence[int],
                     clamp_strict: bool = False) -> Tuple[Int3, Int3]:
    """Window/shift clamp (paper-vs-code notes: window = size, shift 0 when the
    input is not larger than the window; reading D4)."""
    win, sh = [], []
    for n, w, s in zip(size, window, shift):
        small = (n < w) if clamp_strict else (n <= w)
        if small:
            win.append(int(n)); sh.append(0)
        else:
            win.append(int(w)); sh.append(int(s))
    return tuple(win), tuple(sh)


def padded_size(size: Sequence[int], window: Sequence[int]) -> Int3:
    """Each axis rounded up to a multiple of its window (Pitfalls: padding)."""
    return tuple(int(math.ceil(n / w) * w) for n, w in zip(size, window))


def num_windows(B: int, size: Sequence[int], window: Sequence[int]) -> int:
    """B * prod(ceil(n / w)); the same for regular and shifted blocks (§3.2)."""
    return int(B * np.prod([math.ceil(n / w) for n, w in zip(size, window)]))


# --------------------------------------------------------------------------
# elementwise pieces
# --------------------------------------------------------------------------
def layer_norm(x: np.ndarray, g: np.ndarray, b: np.ndarray, eps: float = 1e-5) -> np.ndarray:
    """LayerNorm over the last axis, biased variance (reading D12)."""
    x = np.asarray(x, np.float64)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * np.asarray(g, np.float64) + np.asarray(b, np.float64)


def gelu(x: np.ndarray) -> np.ndarray:
    """Exact GELU x * Phi(x) (reading D13)."""
    x = np.asarray(x, np.float64)
    return 0.5 * x * (1.0 + _erf(x / math.sqrt(2.0)))


def linear(x: np.ndarray, w: np.ndarray, b: Optional[np.ndarray]) -> np.ndarray:
    """y = x W^T + b with W in PyTorch (out, in) layout."""
    y = np.asarray(x, np.float64) @ np.asarray(w, np.float64).T
    if b is not None:
        y = y + np.asarray(b, np.float64)
    return y


# --------------------------------------------------------------------------
# pad / roll / partition and their inverses (§3.2, fig. 3; CSDN 1.2)
# --------------------------------------------------------------------------
def pad_end(u: np.ndarray, padded: Sequence[int], value: float = 0.0) -> np.ndarray:
    """Append `value` at the end of axes 1..3 of (B, T, H, W, C) (reading D5)."""
    B, T, H, W = u.shape[:4]
    pads = [(0, 0), (0, padded[0] - T), (0, padded[1] - H), (0, padded[2] - W)]
    pads += [(0, 0)] * (u.ndim - 4)
    return np.pad(u, pads, mode="constant", constant_values=value)


def roll3(u: np.ndarray, shift: Sequence[int]) -> np.ndarray:
    """Cyclic roll of axes 1..3: out[i] = in[(i - shift) mod n] (numpy/torch)."""
    return np.roll(u, shift=tuple(int(s) for s in shift), axis=(1, 2, 3))


def partition(u: np.ndarray, window: Sequence[int]) -> np.ndarray:
    """(B, Tp, Hp, Wp, ...) -> (B*nW, N, ...): windows (b, wt, wh, ww) row-major,
    tokens (pt, ph, pw) row-major (reading D16)."""
    B, Tp, Hp, Wp = u.shape[:4]
    P, Mh, Mw = window
    rest = u.shape[4:]
    v = u.reshape((B, Tp // P, P, Hp // Mh, Mh, Wp // Mw, Mw) + rest)
    order = (0, 1, 3, 5, 2, 4, 6) + tuple(range(7, 7 + len(rest)))
    v = v.transpose(order)
    return v.reshape((-1, P * Mh * Mw) + rest)


def reverse(windows: np.ndarray, B: int, padded: Sequence[int], window: Sequence[int]) -> np.ndarray:
    """Inverse of `partition`: (B*nW, N, ...) -> (B, Tp, Hp, Wp, ...)."""
    Tp, Hp, Wp = padded
    P, Mh, Mw = window
    rest = windows.shape[2:]
    v = windows.reshape((B, Tp // P, Hp // Mh, Wp // Mw, P, Mh, Mw) + rest)
    order = (0, 1, 4, 2, 5, 3, 6) + tuple(range(7, 7 + len(rest)))
    return v.transpose(order).reshape((B, Tp, Hp, Wp) + rest)


def crop(u: np.ndarray, size: Sequence[int]) -> np.ndarray:
    return u[:, :size[0], :size[1], :size[2]]


# --------------------------------------------------------------------------
# region labels and relative position index
# --------------------------------------------------------------------------
def axis_labels(n_pad: int, w: int, s: int) -> np.ndarray:
    """Per rolled position r of one axis: 0 for r < n-w, 1 for r < n-s, else 2
    (reading D7); all 0 when the axis is not shifted."""
    r = np.arange(n_pad)
    if s == 0:
        return np.zeros(n_pad, np.int64)
    return np.where(r < n_pad - w, 0, np.where(r < n_pad - s, 1, 2)).astype(np.int64)


def region_labels(size: Sequence[int], padded: Sequence[int], window: Sequence[int],
                  shift: Sequence[int], pad_visible: bool = False) -> np.ndarray:
    """Label of every rolled padded grid position (Tp, Hp, Wp).

    Real tokens: 9*lt + 3*lh + lw.  Pad tokens: PAD_LABEL (reading D6) unless
    `pad_visible`.  A rolled position r holds original padded coordinate
    (r + s) mod n, which is a pad when it is >= the real size.
    """
    lt, lh, lw = (axis_labels(p, w, s) for p, w, s in zip(padded, window, shift))
    lab = 9 * lt[:, None, None] + 3 * lh[None, :, None] + lw[None, None, :]
    if not pad_visible:
        pads = [((np.arange(p) + s) % p) >= n for p, s, n in zip(padded, shift, size)]
        is_pad = pads[0][:, None, None] | pads[1][None, :, None] | pads[2][None, None, :]
        lab = np.where(is_pad, PAD_LABEL, lab)
    return lab


def relative_index(window: Sequence[int], table_window: Optional[Sequence[int]] = None) -> np.ndarray:
    """(N, N) table rows for query i, key j of a window (eq. 2; reading D9).

    Offset = coord(i) - coord(j); the temporal offset is the outermost index so
    that a 2D table tiled over the 2P-1 temporal rows (§3.4 inflation) gives a
    bias independent of the temporal offset.  `table_window` is the configured
    window that sized the table (equal to `window` unless clamped).
    """
    P, Mh, Mw = window
    tP, tMh, tMw = table_window if table_window is not None else window
    t, h, w = np.meshgrid(np.arange(P), np.arange(Mh), np.arange(Mw), indexing="ij")
    coords = np.stack([t.ravel(), h.ravel(), w.ravel()], axis=1)          # (N, 3)
    d = coords[:, None, :] - coords[None, :, :]                             # (N, N, 3)
    return ((d[..., 0] + tP - 1) * (2 * tMh - 1) * (2 * tMw - 1)
            + (d[..., 1] + tMh - 1) * (2 * tMw - 1)
            + (d[..., 2] + tMw - 1))


def table_rows(window: Sequence[int]) -> int:
    P, Mh, Mw = window
    return (2 * P - 1) * (2 * Mh - 1) * (2 * Mw - 1)


# --------------------------------------------------------------------------
# attention of one window (eq. 2; CSDN 1.2 WindowAttention3D)
# --------------------------------------------------------------------------
def attend_window(X: np.ndarray, labels: np.ndarray, bias: np.ndarray, p: Dict[str, np.ndarray],
                  heads: int, use_mask: bool, mask_m100: bool = False) -> np.ndarray:
    """One window: X (N, C), labels (N,), bias (N, N, heads) -> proj output (N, C)."""
    N, C = X.shape
    d = C // heads
    qkv = linear(X, p["qkv_w"], p.get("qkv_b"))
    q, k, v = qkv[:, :C], qkv[:, C:2 * C], qkv[:, 2 * C:]
    allowed = labels[:, None] == labels[None, :]
    out = np.empty((N, C), np.float64)
    for h in range(heads):
        sl = slice(h * d, (h + 1) * d)
        s = (q[:, sl] * d ** -0.5) @ k[:, sl].T + bias[:, :, h]
        if use_mask:
            if mask_m100:
                s = s + np.where(allowed, 0.0, -100.0)
            else:
                s = np.where(allowed, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        e = np.exp(s)
        prob = e / e.sum(axis=1, keepdims=True)
        out[:, sl] = prob @ v[:, sl]
    return linear(out, p["proj_w"], p.get("proj_b"))


# --------------------------------------------------------------------------
# the window multi-head self-attention branch and the block
# --------------------------------------------------------------------------
class Geometry:
    """Everything the per-window loop needs for one block of a given input."""

    def __init__(self, B: int, size: Sequence[int], window: Sequence[int], shift: Sequence[int],
                 clamp_strict: bool = False, pad_visible: bool = False):
        self.B = B
        self.size = tuple(int(v) for v in size)
        self.table_window = tuple(int(v) for v in window)
        self.window, self.shift = effective_window(size, window, shift, clamp_strict)
        self.padded = padded_size(self.size, self.window)
        self.N = int(np.prod(self.window))
        self.nw_sample = num_windows(1, self.size, self.window)
        self.nW = B * self.nw_sample
        self.shifted = any(s > 0 for s in self.shift)
        self.has_pad = self.padded != self.size
        self.pad_visible = pad_visible
        lab = region_labels(self.size, self.padded, self.window, self.shift, pad_visible)
        self.win_labels = partition(lab[None, ..., None], self.window)[..., 0]   # (nw_sample, N)
        # mask is needed when shifted, or when pad tokens must be hidden
        self.use_mask = self.shifted or (self.has_pad and not pad_visible)
        self.rel = relative_index(self.window, self.table_window)

    def index_map(self) -> np.ndarray:
        """(nW, N) source token (flat b,t,h,w index) of every window slot, -1 for
        pads: the oracle's own pad/roll/partition applied to an iota."""
        T, H, W = self.size
        iota = np.arange(self.B * T * H * W, dtype=np.int64).reshape(self.B, T, H, W, 1)
        u = pad_end(iota, self.padded, value=-1)
        u = roll3(u, [-s for s in self.shift])
        return partition(u, self.window)[..., 0]


def window_msa(xn: np.ndarray, p: Dict[str, np.ndarray], heads: int, window: Sequence[int],
               shift: Sequence[int], *, clamp_strict: bool = False, pad_visible: bool = False,
               mask_m100: bool = False, windows: Optional[Sequence[int]] = None):
    """3D (S)W-MSA branch of the pages' ``window_msa`` (without LN or residual).

    xn: (B, T, H, W, C), the LayerNorm output.  Returns (B, T, H, W, C) float64.
    With `windows` given, only those window indices are computed and the
    function returns {window index: (N, C) output in window token order}.
    """
    xn = np.asarray(xn, np.float64)
    B, T, H, W, C = xn.shape
    g = Geometry(B, (T, H, W), window, shift, clamp_strict, pad_visible)
    u = pad_end(xn, g.padded)
    u = roll3(u, [-s for s in g.shift])
    xw = partition(u, g.window)                                   # (nW, N, C)
    bias = np.asarray(p["rpb_table"], np.float64)[g.rel]         # (N, N, heads)
    todo = range(g.nW) if windows is None else windows
    res = {}
    for w in todo:
        res[w] = attend_window(xw[w], g.win_labels[w % g.nw_sample], bias, p, heads,
                               g.use_mask, mask_m100)
    if windows is not None:
        return res
    yw = np.stack([res[w] for w in range(g.nW)])
    y = reverse(yw, B, g.padded, g.window)
    y = roll3(y, g.shift)
    return crop(y, g.size)


def mlp(v: np.ndarray, p: Dict[str, np.ndarray]) -> np.ndarray:
    """Linear(C, 4C) -> GELU -> Linear(4C, C) (reading D14)."""
    return linear(gelu(linear(v, p["fc1_w"], p["fc1_b"])), p["fc2_w"], p["fc2_b"])


def block(x: np.ndarray, p: Dict[str, np.ndarray], heads: int, window: Sequence[int],
          shift: Sequence[int], *, eps: float = 1e-5, clamp_strict: bool = False,
          pad_visible: bool = False, mask_m100: bool = False):
    """One pre-norm Video Swin block (eq. 1): returns (z_hat, y) in float64.

    z_hat = x + MSA(LN1(x));  y = z_hat + MLP(LN2(z_hat)).
    """
    x = np.asarray(x, np.float64)
    u = layer_norm(x, p["ln1_g"], p["ln1_b"], eps)
    zh = x + window_msa(u, p, heads, window, shift, clamp_strict=clamp_strict,
                        pad_visible=pad_visible, mask_m100=mask_m100)
    y = zh + mlp(layer_norm(zh, p["ln2_g"], p["ln2_b"], eps), p)
    return zh, y


def block_sampled(x: np.ndarray, p: Dict[str, np.ndarray], heads: int, window: Sequence[int],
                  shift: Sequence[int], tokens: Sequence[int], *, eps: float = 1e-5,
                  clamp_strict: bool = False, pad_visible: bool = False,
                  mask_m100: bool = False):
    """The block evaluated only at the given flat token indices (b,t,h,w order).

    Computes just the windows that contain those tokens, so it scales to the
    largest workloads.  Returns (z_hat rows, y rows), each (len(tokens), C).
    """
    x = np.asarray(x, np.float64)
    B, T, H, W, C = x.shape
    g = Geometry(B, (T, H, W), window, shift, clamp_strict, pad_visible)
    imap = g.index_map()
    where = {}
    flat = imap.ravel()
    pos = np.full(B * T * H * W, -1, np.int64)
    valid = flat >= 0
    pos[flat[valid]] = np.nonzero(valid)[0]
    need = sorted({int(pos[t]) // g.N for t in tokens})
    xf = x.reshape(-1, C)
    res = {}
    for w in need:
        src = imap[w]
        rows = np.zeros((g.N, C), np.float64)
        rows[src >= 0] = layer_norm(xf[src[src >= 0]], p["ln1_g"], p["ln1_b"], eps)
        bias = np.asarray(p["rpb_table"], np.float64)[g.rel]
        res[w] = attend_window(rows, g.win_labels[w % g.nw_sample], bias, p, heads,
                               g.use_mask, mask_m100)
    zh = np.stack([xf[t] + res[int(pos[t]) // g.N][int(pos[t]) % g.N] for t in tokens])
    y = zh + mlp(layer_norm(zh, p["ln2_g"], p["ln2_b"], eps), p)
    return zh, y


# --------------------------------------------------------------------------
# backbone pieces (§3.1 steps 1-2; CSDN PatchEmbed3D / PatchMerging)
# --------------------------------------------------------------------------
def patch_embed(video: np.ndarray, w: np.ndarray, b: Optional[np.ndarray]) -> np.ndarray:
    """(B, Cin, T, H, W) -> (B, T/pt, H/ph, W/pw, C): each patch's values in
    (c, kt, kh, kw) order times the projection (reading D17).  Non-divisible
    axes are zero-padded at the end."""
    v = np.asarray(video, np.float64)
    C, Cin, pt, ph, pw = w.shape
    B, _, T, H, W = v.shape
    Tp, Hp, Wp = (int(math.ceil(n / k) * k) for n, k in zip((T, H, W), (pt, ph, pw)))
    v = np.pad(v, [(0, 0), (0, 0), (0, Tp - T), (0, Hp - H), (0, Wp - W)])
    v = v.reshape(B, Cin, Tp // pt, pt, Hp // ph, ph, Wp // pw, pw)
    v = v.transpose(0, 2, 4, 6, 1, 3, 5, 7).reshape(B, Tp // pt, Hp // ph, Wp // pw, Cin * pt * ph * pw)
    return linear(v, np.asarray(w, np.float64).reshape(C, -1), b)


def merge_gather(x: np.ndarray) -> np.ndarray:
    """(B, T, H, W, C) -> (B, T, H/2, W/2, 4C): concat of the 2x2 spatial group
    in (h, w) offset order (0,0), (1,0), (0,1), (1,1) (reading D18); odd H or W
    is zero-padded at the end."""
    x = np.asarray(x, np.float64)
    B, T, H, W, C = x.shape
    x = np.pad(x, [(0, 0), (0, 0), (0, H % 2), (0, W % 2), (0, 0)])
    parts = [x[:, :, a::2, b::2] for (a, b) in ((0, 0), (1, 0), (0, 1), (1, 1))]
    return np.concatenate(parts, axis=-1)


def patch_merge(x: np.ndarray, m: Dict[str, np.ndarray], eps: float = 1e-5) -> np.ndarray:
    """Patch merging: gather 2x2 -> LN(4C) -> Linear(4C -> 2C)."""
    return linear(layer_norm(merge_gather(x), m["ln_g"], m["ln_b"], eps), m["w"], m.get("b"))


def backbone(video: np.ndarray, params: dict, cfg: dict, *, eps: float = 1e-5,
             collect: bool = False):
    """Full Video Swin backbone forward: embed -> stages (blocks alternate
    shift 0 / half window) with merging between stages -> final LN.

    With `collect`, also returns the list of every block's input and output
    (for per-block teacher-forced comparisons).
    """
    x = patch_embed(video, params["embed_w"], params["embed_b"])
    window = tuple(cfg["window"])
    half = tuple(w // 2 for w in window)
    trace: List[Tuple[np.ndarray, np.ndarray]] = []
    n_st = len(cfg["depths"])
    for i in range(n_st):
        for j, p in enumerate(params["stages"][i]):
            shift = (0, 0, 0) if j % 2 == 0 else half
            _, y = block(x, p, cfg["heads"][i], window, shift, eps=eps)
            if collect:
                trace.append((x, y))
            x = y
        if i < n_st - 1:
            x = patch_merge(x, params["merges"][i], eps)
    out = layer_norm(x, params["norm_g"], params["norm_b"], eps)
    return (out, trace) if collect else out


# --------------------------------------------------------------------------
# closed-form counters (tab. 4, tab. 5)
# --------------------------------------------------------------------------
def block_macs(B: int, size: Sequence[int], C: int, heads: int, window: Sequence[int],
               shift: Sequence[int], mlp_ratio: int = 4) -> Dict[str, int]:
    """Multiply-accumulates of one block, counted op by op on dense padded
    windows: QKV and proj on padded tokens, QK^T and AV per window, MLP on
    real tokens."""
    g = Geometry(B, size, window, shift)
    L = B * int(np.prod(size))
    Lp = g.nW * g.N
    d = C // heads
    macs = {
        "qkv": Lp * C * 3 * C,
        "qk": g.nW * heads * g.N * g.N * d,
        "av": g.nW * heads * g.N * g.N * d,
        "proj": Lp * C * C,
        "fc1": L * C * mlp_ratio * C,
        "fc2": L * mlp_ratio * C * C,
    }
    macs["total"] = sum(macs.values())
    return macs


def backbone_macs(cfg: dict) -> Dict[str, int]:
    """Multiply-accumulates of one clip through the backbone (patch embed,
    blocks, merges); LayerNorm, softmax and GELU are not counted."""
    pt, ph, pw = cfg["patch"]
    T, H, W = (int(math.ceil(n / k)) for n, k in zip(
        (cfg["frames"], cfg["height"], cfg["width"]), (pt, ph, pw)))
    C = cfg["embed_dim"]
    kin = cfg["in_chans"] * pt * ph * pw
    window = tuple(cfg["window"])
    half = tuple(w // 2 for w in window)
    out = {"embed": T * H * W * kin * C, "blocks": 0, "merges": 0}
    for i, depth in enumerate(cfg["depths"]):
        for j in range(depth):
            shift = (0, 0, 0) if j % 2 == 0 else half
            out["blocks"] += block_macs(1, (T, H, W), C, cfg["heads"][i], window, shift,
                                        cfg["mlp_ratio"])["total"]
        if i < len(cfg["depths"]) - 1:
            H, W = (H + 1) // 2, (W + 1) // 2
            out["merges"] += T * H * W * 4 * C * 2 * C
            C *= 2
    out["total"] = out["embed"] + out["blocks"] + out["merges"]
    return out


# --------------------------------------------------------------------------
# around the backbone: 2D -> 3D inflation (§3.4), classification head and
# multi-view scores (readings D23-D25)
# --------------------------------------------------------------------------
def inflate_patch_embed(w2d: np.ndarray, pt: int) -> np.ndarray:
    """2D patch kernel (C, Cin, ph, pw) -> 3D (C, Cin, pt, ph, pw): the same
    kernel in each of the pt temporal slots, divided by pt (§3.4 "Initialisation
    from an image model": 0.5 for the two slots), so a video whose pt frames
    are equal embeds as its single frame did in 2D."""
    w = np.asarray(w2d, np.float64)
    return np.repeat(w[:, :, None, :, :], pt, axis=2) / pt


def inflate_bias_table(t2d: np.ndarray, P: int) -> np.ndarray:
    """2D relative-bias table ((2M-1)^2, heads) -> 3D ((2P-1)(2M-1)^2, heads):
    one copy per temporal offset (§3.4), temporal offset outermost as in the
    3D table's row order (reading D9), so every frame pair sees the 2D bias."""
    t = np.asarray(t2d, np.float64)
    return np.concatenate([t] * (2 * P - 1), axis=0)


def head(x: np.ndarray, w: np.ndarray, b: Optional[np.ndarray]) -> np.ndarray:
    """Final tokens (B, T', H', W', C) -> class logits (B, classes): the mean
    over all tokens of a clip, then Linear(C -> classes) (reading D23)."""
    v = np.asarray(x, np.float64)
    pooled = v.reshape(v.shape[0], -1, v.shape[-1]).mean(axis=1)
    return linear(pooled, w, b)


def multiview_average(logits: np.ndarray) -> np.ndarray:
    """Logits of V views of each video (B, V, classes) -> (B, classes): the
    mean over the views of each view's softmax (reading D24)."""
    z = np.asarray(logits, np.float64)
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return (e / e.sum(axis=-1, keepdims=True)).mean(axis=1)


def backbone_params(cfg: dict, num_classes: int = 0, qkv_bias: bool = True) -> int:
    """Learnable parameters of the backbone (+ a linear head when
    num_classes > 0).  The relative position index is not a parameter."""
    pt, ph, pw = cfg["patch"]
    C = cfg["embed_dim"]
    kin = cfg["in_chans"] * pt * ph * pw
    rows = table_rows(cfg["window"])
    n = kin * C + C
    for i, depth in enumerate(cfg["depths"]):
        per = (2 * C + 3 * C * C + (3 * C if qkv_bias else 0) + rows * cfg["heads"][i]
               + C * C + C + 2 * C + cfg["mlp_ratio"] * C * C + cfg["mlp_ratio"] * C
               + cfg["mlp_ratio"] * C * C + C)
        n += depth * per
        if i < len(cfg["depths"]) - 1:
            n += 2 * 4 * C + 4 * C * 2 * C
            C *= 2
    n += 2 * C
    if num_classes:
        n += C * num_classes + num_classes
    return n
