"""Static check of the kernels' argument-block prefetch (kernarg_warm in
vswin_common.h): every kernel that issues it loads only lines inside its own
argument segment and covers all of its explicit arguments (and the first
hidden ones where the kernel has any).  Compiles the sources to gfx950
assembly with the library's flags and reads the code object metadata; no
GPU is needed."""
import concurrent.futures as cf
import os
import re
import subprocess

import pytest
import yaml

from shifted_window_attention_amd import build as b


def _asm(src, out_dir):
    out = os.path.join(out_dir, src.replace(".hip", ".s"))
    cmd = [b._hipcc(), *b.FLAGS, *b.EXTRA.get(src, []), "--cuda-device-only", "-S",
           os.path.join(b.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out


def _warm_blocks(path):
    txt = open(path).read()
    meta = txt[txt.index(".amdgpu_metadata") + 16:txt.index(".end_amdgpu_metadata")].replace("\t", "    ")
    for k in yaml.safe_load(meta)["amdhsa.kernels"]:
        name = k[".symbol"][:-3] if k[".symbol"].endswith(".kd") else k[".symbol"]
        hidden = [a[".offset"] for a in k[".args"] if a[".value_kind"].startswith("hidden")]
        size = k[".kernarg_segment_size"]
        i = txt.find("\n" + name + ":")
        j = txt.find(".Lfunc_end", i)
        m = re.search(r";;#ASMSTART\n((?:\s*s_load_dword s\d+, s\[\d+:\d+\], 0x[0-9a-f]+\n)+)"
                      r"\s*s_waitcnt lgkmcnt\(0\)", txt[i:j])
        if m:
            offs = [int(x, 16) for x in re.findall(r"0x([0-9a-f]+)", m.group(1))]
            yield name, offs, hidden, size


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc"), reason="needs hipcc")
def test_kernarg_warm_stays_in_segment(tmp_path):
    srcs = [s for s in b.SOURCES if "warm_args" in open(os.path.join(b.CSRC, s)).read()]
    assert srcs
    with cf.ThreadPoolExecutor(min(8, len(srcs))) as ex:
        outs = list(ex.map(lambda s: _asm(s, str(tmp_path)), srcs))
    n = 0
    for path in outs:
        for name, offs, hidden, size in _warm_blocks(path):
            n += 1
            explicit_end = min(hidden) if hidden else size
            assert max(offs) + 4 <= size, f"{name}: line {max(offs)} beyond the {size}-byte segment"
            assert offs == list(range(0, max(offs) + 1, 64)), f"{name}: lines {offs}"
            assert max(offs) >= (explicit_end - 1) // 64 * 64, f"{name}: explicit arguments not covered"
            if hidden:
                assert max(offs) >= min(hidden) // 64 * 64, f"{name}: first hidden line not covered"
    assert n >= 20
