"""CPU fp64 oracle of the Video Swin block's backward pass (training).

TEST INFRASTRUCTURE ONLY.  Only the test-suite and the benchmark's
CPU-baseline leg may import this module; the HIP library never calls it and
shares nothing with it.

The block is the one of ``oracle.vswin.block`` (page "Video Swin
Transformer", §3.1 / eq. 1 and §3.2 / eq. 2):

    u  = LN1(x);  windows of u (pad, roll by -shift, partition)
    per window and head: S = q k^T / sqrt(d) + B[idx],  masked pairs excluded
    (or -100 added), P = softmax(S), O = P v
    z^ = x + crop(roll(reverse(O W_proj^T + b_proj), +shift))
    y  = z^ + fc2(GELU(fc1(LN2(z^))))

Given dy = dL/dy this module returns dL/dx and dL/d(every weight) by the
chain rule written out step by step in the forward's order, reversed.  Each
backward step is the derivative of the forward step it undoes:

  * linear y = x W^T + b:      dx = dy W,  dW = dy^T x,  db = sum_rows dy;
  * GELU y = x Phi(x):         dx = dy (Phi(x) + x phi(x));
  * LayerNorm y = g x^ + b, x^ = (x - mu) / sigma (biased variance):
        dx = (1/sigma) (dx^ - mean(dx^) - x^ mean(dx^ x^)), dx^ = dy g,
        dg = sum_rows dy x^,  db = sum_rows dy;
  * softmax P = softmax(S) per row:  dS = P (dP - rowsum(dP P));
  * the relative position bias: dB[row, h] = sum of dS over the pairs whose
    offset maps to that table row (scatter-add through the index);
  * pad / roll / partition are permutations (and zero fills): their
    backward is the inverse permutation, pads receiving nothing.

Pinned by central finite differences of <dy, block(x, p)> in fp64 (the
tests), independently of any GPU code.
"""
from __future__ import annotations

import math
from typing import Dict, Sequence, Tuple

import numpy as np
from scipy.special import erf as _erf

from . import vswin as fw


def layer_norm_bwd(x: np.ndarray, g: np.ndarray, dy: np.ndarray, eps: float = 1e-5):
    """LayerNorm over the last axis (biased variance): (dx, dg, db)."""
    x = np.asarray(x, np.float64)
    C = x.shape[-1]
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    xh = (x - mu) * rstd
    dxh = dy * np.asarray(g, np.float64)
    dx = rstd * (dxh - dxh.mean(axis=-1, keepdims=True) - xh * (dxh * xh).mean(axis=-1, keepdims=True))
    rows = dy.reshape(-1, C)
    return dx, (rows * xh.reshape(-1, C)).sum(axis=0), rows.sum(axis=0)


def gelu_bwd(x: np.ndarray, dy: np.ndarray) -> np.ndarray:
    """d/dx of x Phi(x) = Phi(x) + x phi(x), times dy."""
    x = np.asarray(x, np.float64)
    Phi = 0.5 * (1.0 + _erf(x / math.sqrt(2.0)))
    phi = np.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)
    return dy * (Phi + x * phi)


def linear_bwd(x: np.ndarray, w: np.ndarray, dy: np.ndarray):
    """y = x W^T + b: (dx, dW, db) over rows of x (any leading shape)."""
    x2 = np.asarray(x, np.float64).reshape(-1, x.shape[-1])
    d2 = np.asarray(dy, np.float64).reshape(-1, dy.shape[-1])
    dx = (d2 @ np.asarray(w, np.float64)).reshape(x.shape[:-1] + (w.shape[1],))
    return dx, d2.T @ x2, d2.sum(axis=0)


def attend_window_bwd(X: np.ndarray, labels: np.ndarray, rel: np.ndarray, p: Dict[str, np.ndarray],
                      heads: int, use_mask: bool, dOut: np.ndarray, mask_m100: bool = False):
    """Backward of ``oracle.vswin.attend_window`` for one window.

    X (N, C) window rows of LN1(x); dOut (N, C) the gradient of the
    projection output.  Returns dX (N, C) and the window's contributions to
    the qkv / proj weights and biases and to the bias table.
    """
    N, C = X.shape
    d = C // heads
    table = np.asarray(p["rpb_table"], np.float64)
    bias = table[rel]                                            # (N, N, heads)
    qkv = fw.linear(X, p["qkv_w"], p.get("qkv_b"))
    q, k, v = qkv[:, :C], qkv[:, C:2 * C], qkv[:, 2 * C:]
    allowed = labels[:, None] == labels[None, :]
    # forward again, keeping P and the head outputs
    O = np.empty((N, C), np.float64)
    probs = []
    for h in range(heads):
        sl = slice(h * d, (h + 1) * d)
        s = (q[:, sl] * d ** -0.5) @ k[:, sl].T + bias[:, :, h]
        if use_mask:
            s = s + np.where(allowed, 0.0, -100.0) if mask_m100 else np.where(allowed, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        e = np.exp(s)
        P = e / e.sum(axis=1, keepdims=True)
        probs.append(P)
        O[:, sl] = P @ v[:, sl]
    # projection
    dO, dWp, dbp = linear_bwd(O, p["proj_w"], dOut)
    # attention per head
    dq = np.zeros((N, C)); dk = np.zeros((N, C)); dv = np.zeros((N, C))
    dtable = np.zeros_like(table)
    for h in range(heads):
        sl = slice(h * d, (h + 1) * d)
        P = probs[h]
        dv[:, sl] = P.T @ dO[:, sl]
        dP = dO[:, sl] @ v[:, sl].T
        dS = P * (dP - (dP * P).sum(axis=1, keepdims=True))
        dq[:, sl] = dS @ k[:, sl] * d ** -0.5
        dk[:, sl] = dS.T @ q[:, sl] * d ** -0.5
        np.add.at(dtable[:, h], rel.ravel(), dS.ravel())
    dqkv = np.concatenate([dq, dk, dv], axis=1)
    dX, dWqkv, dbqkv = linear_bwd(X, p["qkv_w"], dqkv)
    return dX, {"qkv_w": dWqkv, "qkv_b": dbqkv, "proj_w": dWp, "proj_b": dbp, "rpb_table": dtable}


def window_msa_bwd(xn: np.ndarray, p: Dict[str, np.ndarray], heads: int, window: Sequence[int],
                   shift: Sequence[int], dy: np.ndarray, *, clamp_strict: bool = False,
                   pad_visible: bool = False, mask_m100: bool = False):
    """Backward of ``oracle.vswin.window_msa``: (d xn, weight grads)."""
    xn = np.asarray(xn, np.float64)
    B, T, H, W, C = xn.shape
    g = fw.Geometry(B, (T, H, W), window, shift, clamp_strict, pad_visible)
    xw = fw.partition(fw.roll3(fw.pad_end(xn, g.padded), [-s for s in g.shift]), g.window)
    # y = crop(roll(reverse(yw), +s)): its backward is the forward gather of dy
    dyw = fw.partition(fw.roll3(fw.pad_end(np.asarray(dy, np.float64), g.padded),
                                [-s for s in g.shift]), g.window)
    dxw = np.zeros_like(xw)
    grads = None
    for w in range(g.nW):
        dX, gw = attend_window_bwd(xw[w], g.win_labels[w % g.nw_sample], g.rel, p, heads, g.use_mask,
                                   dyw[w], mask_m100)
        dxw[w] = dX
        grads = gw if grads is None else {k: grads[k] + gw[k] for k in grads}
    # xw = partition(roll(pad(xn), -s)): scatter back, pads dropped
    dxn = fw.crop(fw.roll3(fw.reverse(dxw, B, g.padded, g.window), g.shift), g.size)
    return dxn, grads


def block_bwd(x: np.ndarray, p: Dict[str, np.ndarray], heads: int, window: Sequence[int],
              shift: Sequence[int], dy: np.ndarray, *, eps: float = 1e-5, clamp_strict: bool = False,
              pad_visible: bool = False, mask_m100: bool = False) -> Tuple[np.ndarray, Dict[str, np.ndarray]]:
    """Backward of ``oracle.vswin.block``: (dx, grads of all 13 weights)."""
    x = np.asarray(x, np.float64)
    dy = np.asarray(dy, np.float64)
    u = fw.layer_norm(x, p["ln1_g"], p["ln1_b"], eps)
    zh = x + fw.window_msa(u, p, heads, window, shift, clamp_strict=clamp_strict,
                           pad_visible=pad_visible, mask_m100=mask_m100)
    n2 = fw.layer_norm(zh, p["ln2_g"], p["ln2_b"], eps)
    a1 = fw.linear(n2, p["fc1_w"], p["fc1_b"])
    h = fw.gelu(a1)
    # y = z^ + fc2(GELU(fc1(LN2(z^))))
    dh, dW2, db2 = linear_bwd(h, p["fc2_w"], dy)
    da1 = gelu_bwd(a1, dh)
    dn2, dW1, db1 = linear_bwd(n2, p["fc1_w"], da1)
    dzh, dg2, dbe2 = layer_norm_bwd(zh, p["ln2_g"], dn2, eps)
    dzh = dzh + dy
    # z^ = x + MSA(LN1(x))
    du, gm = window_msa_bwd(u, p, heads, window, shift, dzh, clamp_strict=clamp_strict,
                            pad_visible=pad_visible, mask_m100=mask_m100)
    dx, dg1, dbe1 = layer_norm_bwd(x, p["ln1_g"], du, eps)
    dx = dx + dzh
    grads = {"ln1_g": dg1, "ln1_b": dbe1, "ln2_g": dg2, "ln2_b": dbe2,
             "fc1_w": dW1, "fc1_b": db1, "fc2_w": dW2, "fc2_b": db2}
    grads.update(gm)
    return dx, grads
