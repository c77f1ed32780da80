"""Build libvswin.so (gfx950) in-tree with hipcc.

Usage: python -m shifted_window_attention_amd.build [--verbose]
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libvswin.so")
SOURCES = ["vswin_api.hip", "k_layout.hip", "k_gemm.hip", "k_winproj.hip", "k_attention.hip", "k_attn_mfma.hip",
           "k_mlp.hip", "k_patch.hip", "k_probe.hip", "k_backward.hip", "k_head.hip", "k_attn_fused.hip",
           "k_attn_f32.hip"]
ARCH = os.environ.get("VSWIN_ARCH", "gfx950")

# -packed-fp32-ops: keep the compiler from forming v_pk_{add,mul,fma}_f32.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-ffp-contract=fast",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-result", "-munsafe-fp-atomics"]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.sep not in c or os.path.exists(c)):
            return c
    raise RuntimeError("hipcc not found")


# per-file extras: the attention kernel keeps MFMA operands/results in VGPRs
# (no accumulation-register round trips between score tiles and VALU work)
# MFMA accumulators in ordinary VGPRs (no AGPR copies) for the MFMA kernels
_VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
EXTRA = {"k_attn_mfma.hip": _VGPR_FORM, "k_attn_fused.hip": _VGPR_FORM, "k_mlp.hip": _VGPR_FORM, "k_winproj.hip": _VGPR_FORM,
         "k_probe.hip": _VGPR_FORM}


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    noise = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if verbose and noise:
        print("\n".join(noise), flush=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
