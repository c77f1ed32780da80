"""Python binding of libvswin.so -- the MI355X (gfx950) Video Swin 3D
(shifted-)window attention block.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/vswin.h.  PyTorch provides device
memory and the current HIP stream.  There is no CPU fallback: if the library
is missing or fails to load, every call raises.

The functions carry the C entry points' names (``vswin_block_fwd`` ...).
Tensors must be contiguous, on the current HIP device, float32 or bfloat16
(all of one dtype per call), and 16-byte aligned (fresh torch allocations are).
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence

import torch

__all__ = [
    "VswinError", "lib", "Desc", "BlockWeights", "PlanInfo", "make_desc",
    "vswin_plan_query", "vswin_block_fwd", "vswin_block_fwd_noalloc", "vswin_window_msa_fwd", "vswin_attention_fwd",
    "vswin_qkv_attention_fwd", "vswin_index_map",
    "vswin_partition_fwd", "vswin_reverse_fwd", "vswin_layernorm_fwd",
    "vswin_patch_embed_fwd", "vswin_patch_merge_fwd", "vswin_backbone_fwd", "vswin_mfma_rate_probe",
    "vswin_issue_probe",
    "BlockGrads", "vswin_bwd_workspace_query", "vswin_block_bwd", "vswin_window_msa_bwd",
    "vswin_head_fwd", "vswin_multiview_average", "vswin_inflate_patch_embed", "vswin_inflate_bias_table",
    "F_PAD_VISIBLE", "F_CLAMP_STRICT", "F_MASK_M100", "F_TABLES_READY", "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libvswin.so")

F_PAD_VISIBLE = 1
F_CLAMP_STRICT = 2
F_MASK_M100 = 4
F_TABLES_READY = 8

_STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported", -3: "workspace too small", -4: "HIP error"}


class VswinError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"vswin status {status} ({_STATUS.get(status, '?')}): {msg}")
        self.status = status


class Desc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
                ("W", ctypes.c_int32), ("C", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("window", ctypes.c_int32 * 3), ("shift", ctypes.c_int32 * 3),
                ("mlp_hidden", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("ln_eps", ctypes.c_float), ("flags", ctypes.c_uint32)]


class BlockWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "ln1_g", "ln1_b", "qkv_w", "qkv_b", "proj_w", "proj_b", "rpb_table",
        "ln2_g", "ln2_b", "fc1_w", "fc1_b", "fc2_w", "fc2_b")]


class BlockGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "ln1_g", "ln1_b", "qkv_w", "qkv_b", "proj_w", "proj_b", "rpb_table",
        "ln2_g", "ln2_b", "fc1_w", "fc1_b", "fc2_w", "fc2_b")]


class PlanInfo(ctypes.Structure):
    _fields_ = [("eff_window", ctypes.c_int32 * 3), ("eff_shift", ctypes.c_int32 * 3),
                ("padded", ctypes.c_int32 * 3), ("tokens_per_window", ctypes.c_int32),
                ("num_windows", ctypes.c_int64), ("tokens", ctypes.c_int64),
                ("masked", ctypes.c_int32), ("fast_attention", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_size_t), ("msa_workspace_bytes", ctypes.c_size_t),
                ("attention_workspace_bytes", ctypes.c_size_t)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libvswin.so (built in-tree by shifted_window_attention_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m shifted_window_attention_amd.build` (no CPU fallback exists)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    pdesc = ctypes.POINTER(Desc)
    pw = ctypes.POINTER(BlockWeights)
    i3 = ctypes.POINTER(ctypes.c_int32)
    sig = {
        "vswin_plan_query": (i32, [pdesc, ctypes.POINTER(PlanInfo)]),
        "vswin_block_fwd": (i32, [pdesc, vp, pw, vp, vp, sz, vp]),
        "vswin_block_fwd_noalloc": (i32, [pdesc, vp, pw, vp, vp]),
        "vswin_window_msa_fwd": (i32, [pdesc, vp, pw, vp, vp, sz, vp]),
        "vswin_attention_fwd": (i32, [pdesc, vp, vp, vp, vp, vp, vp, sz, vp]),
        "vswin_qkv_attention_fwd": (i32, [pdesc, vp, pw, vp, vp, sz, vp]),
        "vswin_index_map": (i32, [pdesc, vp, vp, vp]),
        "vswin_partition_fwd": (i32, [pdesc, vp, vp, vp]),
        "vswin_reverse_fwd": (i32, [pdesc, vp, vp, vp, vp]),
        "vswin_layernorm_fwd": (i32, [i64, i32, i32, i32, vp, vp, vp, f32, vp, vp]),
        "vswin_patch_embed_workspace": (sz, [i32, i32, i32, i32, i32, i3, i32]),
        "vswin_patch_embed_fwd": (i32, [i32, i32, i32, i32, i32, i3, i32, i32, vp, vp, vp, vp, vp, sz, vp]),
        "vswin_patch_merge_workspace": (sz, [i32, i32, i32, i32, i32, i32]),
        "vswin_patch_merge_fwd": (i32, [i32, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, f32, vp,
                                        vp, sz, vp]),
        "vswin_head_workspace": (sz, [i32, i64, i32]),
        "vswin_head_fwd": (i32, [i32, i64, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]),
        "vswin_multiview_average": (i32, [i32, i32, i32, vp, vp, vp]),
        "vswin_inflate_patch_embed": (i32, [i32, i32, i32, i32, i32, i32, vp, vp, vp]),
        "vswin_inflate_bias_table": (i32, [i32, i32, i32, i32, vp, vp, vp]),
        "vswin_status_string": (ctypes.c_char_p, [i32]),
        "vswin_last_error": (ctypes.c_char_p, []),
        "vswin_abi_version": (i32, []),
        "vswin_mfma_rate_probe": (i32, [vp, i32, i32, vp]),
        "vswin_issue_probe": (i32, [vp, i32, i32, i32, vp]),
        "vswin_bwd_workspace_query": (i32, [pdesc, ctypes.POINTER(sz), ctypes.POINTER(sz)]),
        "vswin_block_bwd": (i32, [pdesc, vp, pw, vp, vp, ctypes.POINTER(BlockGrads), vp, sz, vp]),
        "vswin_window_msa_bwd": (i32, [pdesc, vp, pw, vp, vp, ctypes.POINTER(BlockGrads), vp, sz, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype, fn.argtypes = res, args
    _lib = L
    return L


def _check(status: int) -> None:
    if status != 0:
        raise VswinError(status, lib().vswin_last_error().decode())


def _dt(t: torch.dtype) -> int:
    if t == torch.float32:
        return 0
    if t == torch.bfloat16:
        return 1
    raise TypeError(f"unsupported dtype {t}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    if t.device.type != "cuda":
        raise ValueError("tensors must be on the HIP device")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def make_desc(B: int, T: int, H: int, W: int, C: int, heads: int, window: Sequence[int],
              shift: Sequence[int], *, mlp_hidden: Optional[int] = None, dtype=torch.bfloat16,
              eps: float = 1e-5, flags: int = 0) -> Desc:
    d = Desc()
    d.B, d.T, d.H, d.W, d.C, d.heads = B, T, H, W, C, heads
    for i in range(3):
        d.window[i], d.shift[i] = int(window[i]), int(shift[i])
    d.mlp_hidden = 4 * C if mlp_hidden is None else mlp_hidden
    d.dtype = _dt(dtype) if isinstance(dtype, torch.dtype) else int(dtype)
    d.ln_eps, d.flags = eps, flags
    return d


def vswin_plan_query(desc: Desc, geometry_only: bool = False) -> dict:
    """Host-only planning: clamped window/shift, padded grid, counts, workspace.

    With geometry_only, a descriptor the compute entry points cannot serve
    (status unsupported) still returns its geometry."""
    p = PlanInfo()
    st = lib().vswin_plan_query(ctypes.byref(desc), ctypes.byref(p))
    if not (geometry_only and st == -2):
        _check(st)
    return dict(eff_window=tuple(p.eff_window), eff_shift=tuple(p.eff_shift), padded=tuple(p.padded),
                tokens_per_window=p.tokens_per_window, num_windows=p.num_windows, tokens=p.tokens,
                masked=bool(p.masked), fast_attention=bool(p.fast_attention),
                workspace_bytes=p.workspace_bytes, msa_workspace_bytes=p.msa_workspace_bytes,
                attention_workspace_bytes=p.attention_workspace_bytes)


def _desc_for(x: torch.Tensor, heads, window, shift, eps, flags, mlp_hidden) -> Desc:
    B, T, H, W, C = x.shape
    return make_desc(B, T, H, W, C, heads, window, shift, mlp_hidden=mlp_hidden, dtype=x.dtype,
                     eps=eps, flags=flags)


# weights the C ABI accepts as NULL (their term is then zero)
_OPTIONAL = ("qkv_b", "proj_b", "fc1_b", "fc2_b")


def _weight_shapes(C: int, heads: int, window: Sequence[int], hid: int) -> Dict[str, tuple]:
    """PyTorch layouts of one block's tensors; the table is sized by the
    requested (unclamped) window."""
    P, Mh, Mw = (int(v) for v in window)
    return {"ln1_g": (C,), "ln1_b": (C,), "qkv_w": (3 * C, C), "qkv_b": (3 * C,),
            "proj_w": (C, C), "proj_b": (C,), "rpb_table": ((2 * P - 1) * (2 * Mh - 1) * (2 * Mw - 1), heads),
            "ln2_g": (C,), "ln2_b": (C,), "fc1_w": (hid, C), "fc1_b": (hid,),
            "fc2_w": (C, hid), "fc2_b": (C,)}


def _like(t: torch.Tensor, ref: torch.Tensor, what: str) -> None:
    if tuple(t.shape) != tuple(ref.shape) or t.dtype != ref.dtype or t.device != ref.device:
        raise ValueError(f"{what} must match x: shape {tuple(ref.shape)}, {ref.dtype}, {ref.device} "
                         f"(got {tuple(t.shape)}, {t.dtype}, {t.device})")


def _check_weights(x: torch.Tensor, w: Dict[str, torch.Tensor], heads: int, window: Sequence[int],
                   names: Sequence[str]) -> int:
    """Every weight the call reads must have x's dtype and device and its
    block layout, so that no kernel reads past an allocation.  Returns the
    MLP width (fc1_w rows, or 4C when the call does not read fc1_w)."""
    C = x.shape[-1]
    if x.dim() != 5:
        raise ValueError(f"x must be (B, T, H, W, C), got shape {tuple(x.shape)}")
    if heads <= 0 or C % heads:
        raise ValueError(f"C={C} is not a multiple of heads={heads}")
    fc1 = w.get("fc1_w")
    hid = int(fc1.shape[0]) if ("fc1_w" in names and fc1 is not None and fc1.dim() == 2) else 4 * C
    shapes = _weight_shapes(C, heads, window, hid)
    for n in names:
        t = w.get(n)
        if t is None:
            if n in _OPTIONAL:
                continue
            raise ValueError(f"weight {n} is missing")
        if tuple(t.shape) != shapes[n]:
            raise ValueError(f"weight {n} must have shape {shapes[n]}, got {tuple(t.shape)}")
        if t.dtype != x.dtype:
            raise ValueError(f"weight {n} must be {x.dtype} like x, got {t.dtype}")
        if t.device != x.device:
            raise ValueError(f"weight {n} is on {t.device}, x on {x.device}")
    return hid


def _weights(w: Dict[str, torch.Tensor]) -> BlockWeights:
    bw = BlockWeights()
    for name, _ in BlockWeights._fields_:
        t = w.get(name)
        setattr(bw, name, _ptr(t) if t is not None else None)
    return bw


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]) -> torch.Tensor:
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError(f"workspace too small: need {nbytes} bytes")
        return workspace
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def vswin_block_fwd(x: torch.Tensor, w: Dict[str, torch.Tensor], heads: int, window: Sequence[int],
                    shift: Sequence[int], *, eps: float = 1e-5, flags: int = 0,
                    out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """One Video Swin block (eq. 1) on x (B, T, H, W, C); returns y of x's shape."""
    hid = _check_weights(x, w, heads, window, GRAD_NAMES)
    d = _desc_for(x, heads, window, shift, eps, flags, hid)
    plan = vswin_plan_query(d)
    y = torch.empty_like(x) if out is None else out
    _like(y, x, "out")
    ws = _workspace(plan["workspace_bytes"], x.device, workspace)
    bw = _weights(w)
    _check(lib().vswin_block_fwd(ctypes.byref(d), _ptr(x), ctypes.byref(bw), _ptr(y), _ptr(ws),
                                 ws.numel() * ws.element_size(), _stream(stream)))
    return y


def vswin_block_fwd_noalloc(x: torch.Tensor, w: Dict[str, torch.Tensor], heads: int, window: Sequence[int],
                            shift: Sequence[int], *, eps: float = 1e-5, flags: int = 0,
                            out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """vswin_block_fwd on the library's static scratch array (the C entry
    point allocates nothing; calls overlapping on one GPU race)."""
    hid = _check_weights(x, w, heads, window, GRAD_NAMES)
    d = _desc_for(x, heads, window, shift, eps, flags, hid)
    y = torch.empty_like(x) if out is None else out
    _like(y, x, "out")
    bw = _weights(w)
    _check(lib().vswin_block_fwd_noalloc(ctypes.byref(d), _ptr(x), ctypes.byref(bw), _ptr(y), _stream(stream)))
    return y


def vswin_window_msa_fwd(x_norm: torch.Tensor, w: Dict[str, torch.Tensor], heads: int,
                         window: Sequence[int], shift: Sequence[int], *, eps: float = 1e-5,
                         flags: int = 0, out: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """The (S)W-MSA branch (§3.2) on the LayerNorm output; no residual."""
    _check_weights(x_norm, w, heads, window, MSA_GRAD_NAMES)
    d = _desc_for(x_norm, heads, window, shift, eps, flags, 4 * x_norm.shape[-1])
    plan = vswin_plan_query(d)
    y = torch.empty_like(x_norm) if out is None else out
    _like(y, x_norm, "out")
    ws = _workspace(plan["msa_workspace_bytes"], x_norm.device, workspace)
    bw = _weights(w)
    _check(lib().vswin_window_msa_fwd(ctypes.byref(d), _ptr(x_norm), ctypes.byref(bw), _ptr(y),
                                      _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return y


def vswin_attention_fwd(desc: Desc, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                        table: torch.Tensor, out: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Attention core on projected windows in the block's internal layout (see
    vswin_attention_fwd in include/vswin.h): o (nW, N, C), heads concatenated."""
    plan = vswin_plan_query(desc)
    nW, N, C, h = plan["num_windows"], plan["tokens_per_window"], desc.C, desc.heads
    n_qkv = nW * h * N * (C // h)
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.numel() != n_qkv or t.dtype != q.dtype or t.device != q.device:
            raise ValueError(f"{name} must hold num_windows*heads*N*d = {n_qkv} elements of {q.dtype} "
                             f"(got {t.numel()} of {t.dtype} on {t.device})")
    P, Mh, Mw = (int(v_) for v_ in desc.window)
    rows = (2 * P - 1) * (2 * Mh - 1) * (2 * Mw - 1)
    if tuple(table.shape) != (rows, h) or table.dtype != q.dtype or table.device != q.device:
        raise ValueError(f"table must be ({rows}, {h}) {q.dtype}, got {tuple(table.shape)} {table.dtype}")
    o = out if out is not None else torch.empty((nW, N, C), dtype=q.dtype, device=q.device)
    if o.numel() != nW * N * C or o.dtype != q.dtype or o.device != q.device:
        raise ValueError(f"out must hold num_windows*N*C = {nW * N * C} elements of {q.dtype}")
    ws = _workspace(plan["attention_workspace_bytes"], q.device, workspace)
    _check(lib().vswin_attention_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(table), _ptr(o),
                                     _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return o


QKV_ATTN_NAMES = ("ln1_g", "ln1_b", "qkv_w", "qkv_b", "rpb_table")


def vswin_qkv_attention_fwd(x: torch.Tensor, w: Dict[str, torch.Tensor], heads: int, window: Sequence[int],
                            shift: Sequence[int], *, eps: float = 1e-5, flags: int = 0,
                            out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                            stream=None) -> torch.Tensor:
    """LN1 + window partition + qkv + attention of one block on its input x
    (B, T, H, W, C): the heads' outputs in window rows (num_windows * N, C),
    slot order as vswin_attention_fwd's o (see include/vswin.h)."""
    _check_weights(x, w, heads, window, QKV_ATTN_NAMES)
    d = _desc_for(x, heads, window, shift, eps, flags, 4 * x.shape[-1])
    plan = vswin_plan_query(d)
    rows = plan["num_windows"] * plan["tokens_per_window"]
    o = torch.empty((rows, x.shape[-1]), dtype=x.dtype, device=x.device) if out is None else out
    if o.numel() != rows * x.shape[-1] or o.dtype != x.dtype or o.device != x.device:
        raise ValueError(f"out must hold num_windows*N*C = {rows * x.shape[-1]} elements of {x.dtype} on {x.device}")
    ws = _workspace(plan["msa_workspace_bytes"], x.device, workspace)
    bw = _weights(w)
    _check(lib().vswin_qkv_attention_fwd(ctypes.byref(d), _ptr(x), ctypes.byref(bw), _ptr(o), _ptr(ws),
                                         ws.numel() * ws.element_size(), _stream(stream)))
    return o


def vswin_index_map(desc: Desc, device="cuda", stream=None):
    """(map int32 (nW*N,), region uint8 (nW*N,)) of the pad+roll+partition permutation."""
    plan = vswin_plan_query(desc, geometry_only=True)
    n = plan["num_windows"] * plan["tokens_per_window"]
    m = torch.empty(max(n, 1), dtype=torch.int32, device=device)
    r = torch.empty(max(n, 1), dtype=torch.uint8, device=device)
    _check(lib().vswin_index_map(ctypes.byref(desc), _ptr(m), _ptr(r), _stream(stream)))
    return m[:n], r[:n]


def vswin_partition_fwd(x: torch.Tensor, window, shift, *, flags: int = 0, stream=None) -> torch.Tensor:
    B, T, H, W, C = x.shape
    d = make_desc(B, T, H, W, C, 1, window, shift, dtype=x.dtype, flags=flags)
    plan = vswin_plan_query(d, geometry_only=True)
    out = torch.empty((plan["num_windows"], plan["tokens_per_window"], C), dtype=x.dtype, device=x.device)
    _check(lib().vswin_partition_fwd(ctypes.byref(d), _ptr(x), _ptr(out), _stream(stream)))
    return out


def vswin_reverse_fwd(windows: torch.Tensor, shape, window, shift, *, residual=None, flags: int = 0,
                      stream=None) -> torch.Tensor:
    B, T, H, W, C = shape
    d = make_desc(B, T, H, W, C, 1, window, shift, dtype=windows.dtype, flags=flags)
    y = torch.empty(tuple(shape), dtype=windows.dtype, device=windows.device)
    _check(lib().vswin_reverse_fwd(ctypes.byref(d), _ptr(windows), _ptr(residual), _ptr(y),
                                   _stream(stream)))
    return y


GRAD_NAMES = ("ln1_g", "ln1_b", "qkv_w", "qkv_b", "proj_w", "proj_b", "rpb_table",
              "ln2_g", "ln2_b", "fc1_w", "fc1_b", "fc2_w", "fc2_b")
MSA_GRAD_NAMES = ("qkv_w", "qkv_b", "proj_w", "proj_b", "rpb_table")


def vswin_bwd_workspace_query(desc: Desc) -> Dict[str, int]:
    """Workspace bytes of vswin_block_bwd ("block") and vswin_window_msa_bwd ("msa")."""
    b, m = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(lib().vswin_bwd_workspace_query(ctypes.byref(desc), ctypes.byref(b), ctypes.byref(m)))
    return {"block": b.value, "msa": m.value}


def _grads(w: Dict[str, torch.Tensor], names, grads: Optional[Dict[str, torch.Tensor]]):
    """fp32 gradient buffers shaped like the weights (allocated unless given)."""
    out = {} if grads is None else dict(grads)
    for n, t in out.items():
        if n not in names:
            raise ValueError(f"no gradient {n} is written by this call (it writes {', '.join(names)})")
        ref = w.get(n)
        if ref is None:
            raise ValueError(f"gradient {n} given for an absent weight")
        if t.dtype != torch.float32 or tuple(t.shape) != tuple(ref.shape) or t.device != ref.device:
            raise ValueError(f"gradient {n} must be float32 with shape {tuple(ref.shape)} on {ref.device} "
                             f"(got {t.dtype}, {tuple(t.shape)}, {t.device})")
    for n in names:
        if n not in out and w.get(n) is not None:
            out[n] = torch.empty(w[n].shape, dtype=torch.float32, device=w[n].device)
    bg = BlockGrads()
    for n in GRAD_NAMES:
        setattr(bg, n, _ptr(out[n]) if n in out else None)
    return out, bg


def vswin_block_bwd(x: torch.Tensor, w: Dict[str, torch.Tensor], dy: torch.Tensor, heads: int,
                    window: Sequence[int], shift: Sequence[int], *, eps: float = 1e-5, flags: int = 0,
                    dx: Optional[torch.Tensor] = None, grads: Optional[Dict[str, torch.Tensor]] = None,
                    workspace: Optional[torch.Tensor] = None, stream=None):
    """Backward of vswin_block_fwd: (dx, {weight name: fp32 gradient})."""
    hid = _check_weights(x, w, heads, window, GRAD_NAMES)
    _like(dy, x, "dy")
    dxo = torch.empty_like(x) if dx is None else dx
    _like(dxo, x, "dx")
    g, bg = _grads(w, GRAD_NAMES, grads)
    d = _desc_for(x, heads, window, shift, eps, flags, hid)
    nbytes = vswin_bwd_workspace_query(d)["block"]
    ws = _workspace(nbytes, x.device, workspace)
    bw = _weights(w)
    _check(lib().vswin_block_bwd(ctypes.byref(d), _ptr(x), ctypes.byref(bw), _ptr(dy), _ptr(dxo),
                                 ctypes.byref(bg), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return dxo, g


def vswin_window_msa_bwd(x_norm: torch.Tensor, w: Dict[str, torch.Tensor], dy: torch.Tensor, heads: int,
                         window: Sequence[int], shift: Sequence[int], *, eps: float = 1e-5, flags: int = 0,
                         dx: Optional[torch.Tensor] = None, grads: Optional[Dict[str, torch.Tensor]] = None,
                         workspace: Optional[torch.Tensor] = None, stream=None):
    """Backward of vswin_window_msa_fwd: (dx_norm, {qkv/proj/table name: fp32 gradient})."""
    _check_weights(x_norm, w, heads, window, MSA_GRAD_NAMES)
    _like(dy, x_norm, "dy")
    dxo = torch.empty_like(x_norm) if dx is None else dx
    _like(dxo, x_norm, "dx")
    g, bg = _grads(w, MSA_GRAD_NAMES, grads)
    d = _desc_for(x_norm, heads, window, shift, eps, flags, 4 * x_norm.shape[-1])
    nbytes = vswin_bwd_workspace_query(d)["msa"]
    ws = _workspace(nbytes, x_norm.device, workspace)
    bw = _weights(w)
    _check(lib().vswin_window_msa_bwd(ctypes.byref(d), _ptr(x_norm), ctypes.byref(bw), _ptr(dy), _ptr(dxo),
                                      ctypes.byref(bg), _ptr(ws), ws.numel() * ws.element_size(),
                                      _stream(stream)))
    return dxo, g


def vswin_mfma_rate_probe(out: torch.Tensor, blocks: int, iters: int, stream=None) -> int:
    """Launch the MFMA throughput kernel (measurement helper; see include/vswin.h).
    out: float32 device tensor of >= blocks * 512 elements.  Returns the FLOPs
    one launch performs."""
    if out.dtype != torch.float32 or out.numel() < blocks * 512:
        raise ValueError("out must be float32 with at least blocks * 512 elements")
    _check(lib().vswin_mfma_rate_probe(_ptr(out), blocks, iters, _stream(stream)))
    return blocks * 8 * 8 * iters * 16384


def vswin_issue_probe(out: torch.Tensor, blocks: int, iters: int, mode: int, stream=None) -> None:
    """Launch the MFMA / VALU overlap probe (measurement helper; see
    include/vswin.h).  out: float32 device tensor of >= blocks * 512 elements."""
    if out.dtype != torch.float32 or out.numel() < blocks * 512:
        raise ValueError("out must be float32 with at least blocks * 512 elements")
    _check(lib().vswin_issue_probe(_ptr(out), blocks, iters, mode, _stream(stream)))


def vswin_layernorm_fwd(x: torch.Tensor, g: torch.Tensor, b: torch.Tensor, eps: float = 1e-5,
                        out_dtype=None, stream=None) -> torch.Tensor:
    C = x.shape[-1]
    out_dtype = g.dtype if out_dtype is None else out_dtype
    y = torch.empty(x.shape, dtype=out_dtype, device=x.device)
    _check(lib().vswin_layernorm_fwd(x.numel() // C, C, _dt(x.dtype), _dt(out_dtype), _ptr(x), _ptr(g),
                                     _ptr(b), eps, _ptr(y), _stream(stream)))
    return y


def vswin_patch_embed_fwd(video: torch.Tensor, w: torch.Tensor, b: Optional[torch.Tensor],
                          stream=None) -> torch.Tensor:
    """video (B, Cin, T, H, W), w (C, Cin, pt, ph, pw) -> tokens (B, T', H', W', C)."""
    B, Cin, T, H, W = video.shape
    C, _, pt, ph, pw = w.shape
    patch = (ctypes.c_int32 * 3)(pt, ph, pw)
    dt = _dt(video.dtype)
    nbytes = lib().vswin_patch_embed_workspace(B, Cin, T, H, W, patch, dt)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=video.device)
    y = torch.empty((B, -(-T // pt), -(-H // ph), -(-W // pw), C), dtype=video.dtype, device=video.device)
    _check(lib().vswin_patch_embed_fwd(B, Cin, T, H, W, patch, C, dt, _ptr(video), _ptr(w), _ptr(b),
                                       _ptr(y), _ptr(ws), ws.numel(), _stream(stream)))
    return y


def vswin_patch_merge_fwd(x: torch.Tensor, ln_g, ln_b, w, b=None, eps: float = 1e-5,
                          stream=None) -> torch.Tensor:
    """x (B, T, H, W, C) -> (B, T, ceil(H/2), ceil(W/2), Cout)."""
    B, T, H, W, C = x.shape
    Cout = w.shape[0]
    dt = _dt(x.dtype)
    nbytes = lib().vswin_patch_merge_workspace(B, T, H, W, C, dt)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=x.device)
    y = torch.empty((B, T, -(-H // 2), -(-W // 2), Cout), dtype=x.dtype, device=x.device)
    _check(lib().vswin_patch_merge_fwd(B, T, H, W, C, Cout, dt, _ptr(x), _ptr(ln_g), _ptr(ln_b), _ptr(w),
                                       _ptr(b), eps, _ptr(y), _ptr(ws), ws.numel(), _stream(stream)))
    return y


def vswin_head_fwd(x: torch.Tensor, w: torch.Tensor, b: Optional[torch.Tensor] = None, *, out=None,
                   workspace=None, stream=None) -> torch.Tensor:
    """Final tokens x (B, T', H', W', C) (or (B, L, C)), w (K, C), b (K) ->
    logits (B, K) fp32: the mean over the tokens, then the linear classifier."""
    B, C = x.shape[0], x.shape[-1]
    L = 1
    for n in x.shape[1:-1]:
        L *= n
    K = w.shape[0]
    nbytes = lib().vswin_head_workspace(B, L, C)
    ws = workspace if workspace is not None else torch.empty(max(nbytes, 256), dtype=torch.uint8,
                                                             device=x.device)
    y = out if out is not None else torch.empty((B, K), dtype=torch.float32, device=x.device)
    _check(lib().vswin_head_fwd(B, L, C, K, _dt(x.dtype), _ptr(x), _ptr(w), _ptr(b), _ptr(y), _ptr(ws),
                                ws.numel(), _stream(stream)))
    return y


def vswin_multiview_average(logits: torch.Tensor, *, out=None, stream=None) -> torch.Tensor:
    """logits (B, V, K) fp32 of V views per video -> (B, K): the mean of the
    views' softmax probabilities."""
    B, V, K = logits.shape
    y = out if out is not None else torch.empty((B, K), dtype=torch.float32, device=logits.device)
    _check(lib().vswin_multiview_average(B, V, K, _ptr(logits), _ptr(y), _stream(stream)))
    return y


def vswin_inflate_patch_embed(w2: torch.Tensor, pt: int, *, stream=None) -> torch.Tensor:
    """2D patch kernel (C, Cin, ph, pw) -> 3D (C, Cin, pt, ph, pw), divided by pt."""
    C, Cin, ph, pw = w2.shape
    w3 = torch.empty((C, Cin, pt, ph, pw), dtype=w2.dtype, device=w2.device)
    _check(lib().vswin_inflate_patch_embed(C, Cin, pt, ph, pw, _dt(w2.dtype), _ptr(w2), _ptr(w3),
                                           _stream(stream)))
    return w3


def vswin_inflate_bias_table(t2: torch.Tensor, P: int, *, stream=None) -> torch.Tensor:
    """2D relative-bias table (rows2d, heads) -> ((2P-1) rows2d, heads)."""
    rows2d, heads = t2.shape
    t3 = torch.empty(((2 * P - 1) * rows2d, heads), dtype=t2.dtype, device=t2.device)
    _check(lib().vswin_inflate_bias_table(rows2d, heads, P, _dt(t2.dtype), _ptr(t2), _ptr(t3), _stream(stream)))
    return t3


def vswin_backbone_fwd(video: torch.Tensor, params: dict, cfg: dict, *, eps: float = 1e-5,
                       collect: bool = False, stream=None):
    """Video Swin backbone forward as a sequence of library calls: patch
    embedding -> stages of blocks (shift 0 / half window alternating) with
    patch merging between stages -> final LayerNorm (§3.1)."""
    x = vswin_patch_embed_fwd(video, params["embed_w"], params.get("embed_b"), stream=stream)
    window = tuple(cfg["window"])
    half = tuple(v // 2 for v in window)
    trace = []
    n_st = len(cfg["depths"])
    for i in range(n_st):
        for j, p in enumerate(params["stages"][i]):
            shift = (0, 0, 0) if j % 2 == 0 else half
            y = vswin_block_fwd(x, p, cfg["heads"][i], window, shift, eps=eps, stream=stream)
            if collect:
                trace.append((x, y))
            x = y
        if i < n_st - 1:
            m = params["merges"][i]
            x = vswin_patch_merge_fwd(x, m["ln_g"], m["ln_b"], m["w"], m.get("b"), eps=eps, stream=stream)
    out = vswin_layernorm_fwd(x, params["norm_g"], params["norm_b"], eps=eps, stream=stream)
    return (out, trace) if collect else out
