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
           "The run covers 12 block pairs (10 timed + 2 warm-up) and 2 x (5 + 50) standalone attention launches",
           "for the roofline leg; torch kernels are input generation.", "",
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
the attention kernel three times with shift (0,0,0) and three times with shift (4,3,3).

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
"""


if __name__ == "__main__":
    sdir, pdir = sys.argv[1], sys.argv[2]
    open(os.path.join(HERE, "block_pair_swin_t_stage1_kernel_stats.md"), "w").write(stats(sdir))
    open(os.path.join(HERE, "attn_mfma_swin_t_stage1_traffic.md"), "w").write(traffic(pdir))
    print("written")
