"""Writes the two text summaries in this folder from rocprofv3 output.

    python profiles/make_summaries.py <stats_dir> <pmc_dir>

<stats_dir> holds bench_kernel_stats.csv from
    rocprofv3 --kernel-trace --stats --output-format csv -d <stats_dir> -o bench -- \
        python bench.py --steps 10 --warmup 2 --no-cpu-baseline
<pmc_dir> holds FETCH_SIZE/ and WRITE_SIZE/ from
    rocprofv3 --pmc FETCH_SIZE --output-format csv -d <pmc_dir>/FETCH_SIZE -o FETCH_SIZE -- python bench.py --counter-pass
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d <pmc_dir>/WRITE_SIZE -o WRITE_SIZE -- python bench.py --counter-pass
"""
import csv
import hashlib
import os
import re
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ATTN_SRC = os.path.join(ROOT, "shifted_window_attention_amd", "csrc", "k_attn_mfma.hip")


def short(name: str) -> str:
    name = name.replace("void ", "").replace("(anonymous namespace)::", "")
    name = re.sub(r"\(.*", "", name)
    return name[:80]


def stats(stats_dir: str) -> str:
    rows = list(csv.DictReader(open(os.path.join(stats_dir, "bench_kernel_stats.csv"))))
    out = ["# Kernel times, Swin-T stage-1 block pair (bf16 tokens (1,16,56,56,96), 3 heads x 32, window (8,7,7))", "",
           "Command (one MI355X):", "",
           "    cd /tmp && export TMPDIR=/tmp && cd -",
           "    rocprofv3 --kernel-trace --stats --output-format csv -d out -o bench -- \\",
           "        python bench.py --steps 10 --warmup 2 --no-cpu-baseline", "",
           "The run covers 12 block pairs (10 timed + 2 warm-up), 70 individually timed pairs (50 warm, then 20 with",
           "a 512 MiB fill, the torch FillFunctor kernel, between them), 2 x (5 + 50) standalone attention launches",
           "for the roofline leg, and 23 launches each of the gather (`ln_rows_v8_kernel` with the slot map), the",
           "scatter + residual (`reverse_v8_kernel`) and LayerNorm (`ln_rows_v8_kernel`) on the Swin-T stage-1 grid",
           "(<4, 3> instances, C = 96) and the Swin-B stage-1 B=8 grid (<16, 1> instances, C = 128), then the",
           "window variants on the stage-1 grid (window 4 with shift (2,3,3): the per-key-label form `Cfg<8, 4,",
           "false, false, true>`; window 16: the scalar-table form `Cfg<8, 8, true, false, false>`; window 8 with the",
           "-100 mask: `Cfg<8, 4, false, true, false>`), each 23 block pairs and 21 standalone attention launches;",
           "the main workload's attention is `Cfg<8, 4, false, false, false>`; then 11 backward block pairs",
           "(`vswin_block_bwd`: the forward recomputed, then the `attn_bwd_*`, `wgrad_kernel`, `ln_bwd_kernel`, GELU",
           "and GEMM kernels of the backward); then the inference pieces, 23 launches each (the head's",
           "`head_pool_kernel` / `head_reduce_kernel` / `head_fc_kernel` on 24 clips of (16,7,7,768) tokens,",
           "`view_avg_kernel`, `inflate_patch_kernel`, `inflate_table_kernel`), and the MFMA / VALU overlap probe",
           "(`issue_probe_kernel`, 4 modes x 4 launches) next to the MFMA rate probe (`mfma_rate_kernel`). Other",
           "torch kernels are input generation.", "",
           "| kernel | calls | avg us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| `{short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    return "\n".join(out) + "\n"


def traffic(pmc_dir: str) -> str:
    def vals(c, pat):
        rows = list(csv.DictReader(open(os.path.join(pmc_dir, c, f"{c}_counter_collection.csv"))))
        return [float(r["Counter_Value"]) for r in rows if pat in r["Kernel_Name"]]
    fc, wc = vals("FETCH_SIZE", "copyBuffer"), vals("WRITE_SIZE", "copyBuffer")
    fa, wa = vals("FETCH_SIZE", "attn_mfma"), vals("WRITE_SIZE", "attn_mfma")
    copy_kib = 256 * 1024
    ff, fw = copy_kib / statistics.mean(fc), copy_kib / statistics.mean(wc)
    fb, wb = statistics.mean(fa) * 1024 * ff, statistics.mean(wa) * 1024 * fw
    alg_r, alg_w = 3 * 128 * 3 * 392 * 32 * 2, 128 * 392 * 96 * 2
    src = hashlib.sha256(open(ATTN_SRC, "rb").read()).hexdigest()
    kib = lambda v: ", ".join(str(round(x)) for x in v)
    return f"""# HBM traffic of the fused window attention, Swin-T stage 1 (q, k, V^T of 128 windows x 3 heads x 392 x 32)

Commands (one counter per run, one MI355X):

    cd /tmp && export TMPDIR=/tmp && cd -
    rocprofv3 --pmc FETCH_SIZE --output-format csv -d out/FETCH_SIZE -o FETCH_SIZE -- python bench.py --counter-pass
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d out/WRITE_SIZE -o WRITE_SIZE -- python bench.py --counter-pass

`bench.py --counter-pass` copies 256 MiB three times with a plain device copy (`__amd_rocclr_copyBuffer`), then launches
the attention kernel three times with shift (0,0,0) and three times with shift (4,3,3), then the gather, scatter and
LayerNorm kernels once each (section at the end).

Per-dispatch counter values (KiB):

| kernel | FETCH_SIZE | WRITE_SIZE |
|---|---|---|
| copyBuffer, 256 MiB | {kib(fc)} | {kib(wc)} |
| attn_mfma_kernel (3 regular, 3 shifted) | {kib(fa)} | {kib(wa)} |

Calibration against the copy of known size (262144 KiB read and written): FETCH_SIZE x {ff:.4f}, WRITE_SIZE x {fw:.4f}.

- fetch bytes per launch: {int(round(fb))}
- write bytes per launch: {int(round(wb))}
- hbm bytes per launch: {int(round(fb + wb))}
- algorithmic bytes per launch: {alg_r + alg_w} (q, k, V^T read once: {alg_r}; o written once: {alg_w})
- kernel source sha256: `{src}`

The kernel fetches {fb / alg_r:.2f}x the algorithmic q/k/V^T bytes (a window shared by two workgroups' runs is read
by both; each workgroup also copies its head's prepared bias table, built once per call, from L2) and writes the output exactly once.
""" + memory_traffic(pmc_dir, ff, fw)


def memory_traffic(pmc_dir: str, ff: float, fw: float) -> str:
    """The gather, scatter + residual and LayerNorm dispatches of the counter
    pass (in that order), Swin-B stage-1 grid B=8, C=128, bf16."""
    def rows(c):
        rs = list(csv.DictReader(open(os.path.join(pmc_dir, c, f"{c}_counter_collection.csv"))))
        rs = [r for r in rs if "ln_rows" in r["Kernel_Name"] or "reverse" in r["Kernel_Name"]]
        key = "Dispatch_Id" if rs and "Dispatch_Id" in rs[0] else None
        if key:
            rs.sort(key=lambda r: int(r[key]))
        return [float(r["Counter_Value"]) for r in rs]
    f, w = rows("FETCH_SIZE"), rows("WRITE_SIZE")
    if len(f) < 3 or len(w) < 3:
        return ""
    L, Lp, C = 8 * 16 * 60 * 60, 8 * 16 * 63 * 63, 128
    alg = [((L + Lp) * C * 2, "read x once, write the padded windows once"),
           (3 * L * C * 2, "read the windows' real slots and the residual, write y"),
           (2 * L * C * 2, "read x, write y")]
    names = ["gather (pad + roll + partition)", "scatter + residual (reverse + un-roll + crop)", "LayerNorm"]
    out = ["", "## Memory-bound kernels, Swin-B stage-1 grid (B=8, 16x60x60x128 -> 16x63x63), bf16", "",
           "One dispatch each at the end of the same counter pass, scaled by the same copy calibration.", "",
           "| kernel | FETCH bytes | WRITE bytes | HBM bytes | algorithmic bytes | ratio |", "|---|---|---|---|---|---|"]
    for i in range(3):
        fb, wb = f[i] * 1024 * ff, w[i] * 1024 * fw
        out.append(f"| {names[i]} | {int(round(fb))} | {int(round(wb))} | {int(round(fb + wb))} | "
                   f"{alg[i][0]} ({alg[i][1]}) | {(fb + wb) / alg[i][0]:.2f} |")
    return "\n".join(out) + "\n"


if __name__ == "__main__":
    sdir, pdir = sys.argv[1], sys.argv[2]
    open(os.path.join(HERE, "block_pair_swin_t_stage1_kernel_stats.md"), "w").write(stats(sdir))
    open(os.path.join(HERE, "attn_mfma_swin_t_stage1_traffic.md"), "w").write(traffic(pdir))
    print("written")
