#!/usr/bin/env python
"""Throughput of the Video Swin window-attention block on one MI355X.

A step is one regular + shifted block pair (eq. 1) of the Swin-T stage-1
workload: bf16 tokens (B=1, T'=16, H'=56, W'=56, C=96) from a 32x224x224
clip with 2x4x4 patches, 3 heads of 32, window (8,7,7), shift (4,3,3), MLP
ratio 4, seeded synthetic inputs and weights (no dataset).  Inputs, weights,
outputs and workspace are resident in HBM before the timed region.

The K timed steps are captured into one HIP graph and replayed once between
two events, right behind at least W untimed steps replayed from the same
graph (every kernel of every pair runs; the graph only removes the Python
binding's per-call host work, reported separately as the eager rate).  Prints one JSON line: tokens/s through a block (tokens x blocks per
second), TFLOP/s and the fraction of the bf16 MFMA peak, the roofline of the
dominant kernel (the window attention, launched alone and timed with HIP
events on its stream), the one-kernel LN1 + gather + qkv + attention
variant, and the fp64 CPU oracle's rate on the same workload.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "window-attention block tokens/s + TFLOP/s (% of MFMA peak) at Swin-T stage 1"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
CSRC = os.path.join(ROOT, "shifted_window_attention_amd", "csrc")
# the sources whose sha256 a counter summary records (the kernel's own file
# and the attention core it includes)
ATTN_SOURCES = [os.path.join(CSRC, "k_attn_mfma.hip"), os.path.join(CSRC, "attn_core.h")]
FUSED_SOURCES = [os.path.join(CSRC, "k_attn_fused.hip"), os.path.join(CSRC, "attn_core.h")]
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "attn_mfma_swin_t_stage1_traffic.md")
FUSED_TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "wattn_fused_swin_t_stage1_traffic.md")


def sources_sha256(paths) -> str:
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        h.update(open(p, "rb").read())
    return h.hexdigest()


def counter_traffic(path: str, sources) -> int:
    """HBM bytes per launch from a committed FETCH_SIZE / WRITE_SIZE summary,
    or None when the summary is missing or was taken on another version of
    the kernel's sources (their sha256 is recorded in the summary)."""
    if not path or not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and line.lstrip().startswith("- "):
            k, v = line.lstrip()[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel source sha256") != sources_sha256(sources) or "hbm bytes per launch" not in fields:
        return None
    return int(fields["hbm bytes per launch"])


def block_flops(plan: dict, C: int, hid: int) -> dict:
    """Closed-form FLOPs (2 per multiply-accumulate) of one block on dense
    padded windows: qkv and proj on padded tokens, QK^T and AV per window,
    MLP on real tokens."""
    Lp = plan["num_windows"] * plan["tokens_per_window"]
    L = plan["tokens"]
    N = plan["tokens_per_window"]
    f = {"qkv": 2 * Lp * C * 3 * C, "attn": 2 * 2 * Lp * N * C, "proj": 2 * Lp * C * C,
         "fc1": 2 * L * C * hid, "fc2": 2 * L * hid * C}
    f["total"] = sum(f.values())
    return f


def cpu_baseline(x, params, shape, min_seconds=12.0, max_reps=20):
    """The fp64 oracle, untouched, on the same workload: full block pairs
    repeated until about `min_seconds` of CPU work."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        cores = os.cpu_count() or 1
    x64 = x.astype(np.float64)
    reps, t0 = 0, time.perf_counter()
    while True:
        _, y = oracle.block(x64, params[0], shape.heads, shape.window, (0, 0, 0))
        oracle.block(y, params[1], shape.heads, shape.window, shape.shift)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or reps >= max_reps:
            break
    info = host_info()
    return {"value": 2 * shape.tokens * reps / el, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{reps} full block pair(s) of the same workload in fp64 numpy "
                      f"({el:.1f} s, BLAS threads={cores})",
            "cpu_model": info["cpu_model"], "nproc": info["nproc"], "usable_cpus": info["usable_cpus"]}


def host_info() -> dict:
    """The host the CPU baseline runs on: CPU model, logical CPUs, the CPUs
    this process may use, and the BLAS pool size."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        blas = None
    return {"cpu_model": model, "nproc": os.cpu_count(), "usable_cpus": usable, "blas_threads": blas}


def oracle_per_config(max_seconds: float = 8.0) -> dict:
    """The fp64 oracle, untouched, on a bounded sample of each other workload:
    whole windows of one shifted block (every real token of the sampled
    windows through attention and MLP, oracle.block_sampled), the fp32 smoke
    pair whole, and the backbone on one clip; real tokens per second through
    a block (backbone: clips per second)."""
    import numpy as np
    import oracle
    from oracle import vswin as ov
    import synth
    out = {}
    x1, p1 = synth.gen_workload(1)
    s1 = synth.WORKLOADS[1].shape
    t0 = time.perf_counter()
    _, y = oracle.block(x1.astype(np.float64), p1[0], s1.heads, s1.window, (0, 0, 0))
    oracle.block(y, p1[1], s1.heads, s1.window, s1.shift)
    el = time.perf_counter() - t0
    out["workload1"] = {"value": round(2 * s1.tokens / el, 1), "unit": "tokens/s", "sample": "the whole fp32 pair"}
    for wid, nwin in ((3, 4), (4, 6)):
        x, params = synth.gen_workload(wid)
        s = synth.WORKLOADS[wid].shape
        g = ov.Geometry(s.B, (s.T, s.H, s.W), s.window, s.shift)
        imap = g.index_map()
        toks, done, t0 = [], 0, time.perf_counter()
        for w in np.linspace(0, g.nW - 1, nwin).astype(int):
            tk = imap[w][imap[w] >= 0].tolist()
            oracle.vswin.block_sampled(x.astype(np.float64), params[1], s.heads, s.window, s.shift, tk)
            done += len(tk)
            if time.perf_counter() - t0 > max_seconds:
                break
        el = time.perf_counter() - t0
        out[f"workload{wid}"] = {"value": round(done / el, 1), "unit": "tokens/s",
                                 "sample": f"{done} real tokens (whole windows) of one shifted block"}
    cfg = dict(synth.WORKLOADS[5].backbone)
    video = synth.gen_video(1, cfg["in_chans"], cfg["frames"], cfg["height"], cfg["width"], 5, "bf16")
    params = synth.gen_backbone_params(cfg, 5, "bf16")
    t0 = time.perf_counter()
    oracle.vswin.backbone(video.astype(np.float64), params, cfg)
    el = time.perf_counter() - t0
    out["workload5"] = {"value": round(1 / el, 4), "unit": "clips/s", "sample": "the whole backbone on one clip"}
    return out


def other_workloads(vs, torch, np, stream, reps: int = 5) -> dict:
    """GPU throughput of the other workloads (eager library calls, HIP events
    on the calls' stream, inputs and weights resident): Swin-T stage-3 six
    blocks at B=4 (C=384), the Swin-B stage-1 padded pair at B=8 (C=128), the
    Swin-T backbone on two clips, and the fp32 smoke pair.  TFLOP/s from the
    closed form (2 per multiply-accumulate; padded windows for qkv, attention
    and proj, real tokens for the MLP; backbone: embed and merges added)."""
    import synth
    dev = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dt).cuda()
    out = {}

    def timeit(fn, n):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    for wid, n in ((1, 20), (3, reps), (4, reps)):
        wl = synth.WORKLOADS[wid]
        s = wl.shape
        td = torch.float32 if wl.dtype == "fp32" else torch.bfloat16
        x_np, params = synth.gen_workload(wid)
        x = dev(x_np, td)
        w = [{k: dev(v, td) for k, v in p.items()} for p in params]
        hid = s.mlp_ratio * s.C
        shifts = [(0, 0, 0) if k % 2 == 0 else s.shift for k in range(len(params))]
        plans = [vs.vswin_plan_query(vs.make_desc(s.B, s.T, s.H, s.W, s.C, s.heads, s.window, sh, mlp_hidden=hid,
                                                  dtype=td)) for sh in shifts]
        ws = torch.empty(max(p["workspace_bytes"] for p in plans), dtype=torch.uint8, device="cuda")
        ys = [torch.empty_like(x), torch.empty_like(x)]

        def stack():
            cur = x
            for k, p in enumerate(w):
                vs.vswin_block_fwd(cur, p, s.heads, s.window, shifts[k], out=ys[k % 2], workspace=ws, stream=stream)
                cur = ys[k % 2]

        ms = timeit(stack, n)
        flops = sum(block_flops(p, s.C, hid)["total"] for p in plans)
        out[f"workload{wid}"] = {"workload": wl.name, "dtype": wl.dtype, "blocks": len(params),
                                 "ms_per_stack": round(ms, 4),
                                 "tokens_per_s": round(s.tokens * len(params) / (ms * 1e-3), 1),
                                 "tflops": round(flops / (ms * 1e-3) / 1e12, 2), "gflop": round(flops / 1e9, 3)}
    cfg = synth.WORKLOADS[5].backbone
    video = dev(synth.gen_video(cfg["B"], cfg["in_chans"], cfg["frames"], cfg["height"], cfg["width"], 5, "bf16"),
                torch.bfloat16)
    bp = synth.gen_backbone_params(cfg, 5, "bf16")
    dp = {"embed_w": dev(bp["embed_w"], torch.bfloat16), "embed_b": dev(bp["embed_b"], torch.bfloat16),
          "stages": [[{k: dev(v, torch.bfloat16) for k, v in p.items()} for p in st] for st in bp["stages"]],
          "merges": [{k: dev(v, torch.bfloat16) for k, v in m.items()} for m in bp["merges"]],
          "norm_g": dev(bp["norm_g"], torch.bfloat16), "norm_b": dev(bp["norm_b"], torch.bfloat16)}
    ms = timeit(lambda: vs.vswin_backbone_fwd(video, dp, cfg, stream=stream), reps)
    # closed form of the backbone: embed, blocks, merges
    B, C = cfg["B"], cfg["embed_dim"]
    T, H, W = cfg["frames"] // 2, cfg["height"] // 4, cfg["width"] // 4
    flops = 2 * B * T * H * W * (cfg["in_chans"] * 2 * 4 * 4) * C
    for i, depth in enumerate(cfg["depths"]):
        for j in range(depth):
            sh = (0, 0, 0) if j % 2 == 0 else tuple(v // 2 for v in cfg["window"])
            p = vs.vswin_plan_query(vs.make_desc(B, T, H, W, C, cfg["heads"][i], cfg["window"], sh))
            flops += block_flops(p, C, 4 * C)["total"]
        if i < len(cfg["depths"]) - 1:
            H, W = (H + 1) // 2, (W + 1) // 2
            flops += 2 * B * T * H * W * 4 * C * 2 * C
            C *= 2
    out["workload5"] = {"workload": synth.WORKLOADS[5].name, "dtype": "bf16", "ms_per_forward": round(ms, 4),
                        "clips_per_s": round(B / (ms * 1e-3), 2), "stage1_tokens_per_s":
                        round(B * (cfg["frames"] // 2) * (cfg["height"] // 4) * (cfg["width"] // 4) / (ms * 1e-3), 1),
                        "tflops": round(flops / (ms * 1e-3) / 1e12, 2), "gflop": round(flops / 1e9, 3)}
    return out


def memory_kernels(vs, torch, stream, launches: int = 20, cold_launches: int = 10) -> dict:
    """HBM rates of the standalone permutation / normalisation kernels (the
    block path fuses them into its GEMMs): the pad + roll + partition gather,
    the reverse + un-roll scatter with the residual, and LayerNorm, on the
    Swin-T stage-1 token grid and on the Swin-B stage-1 grid (B=8,
    16x60x60x128, padded to 16x63x63).  Bytes are algorithmic: each tensor once
    at its stored width.  Two timings per kernel:
      warm  `launches` launches back to back on the same buffers (a kernel's
            working set of up to ~250 MB can stay in the 256 MB last-level
            cache between launches);
      cold  each launch alone between HIP events after a 512 MiB fill of a
            scrub buffer (larger than that cache), median of `cold_launches`:
            the inputs come from HBM; this is the figure the HBM fractions
            rest on."""
    import statistics
    out = {}
    shapes = {"swin_t_s1": ((1, 16, 56, 56, 96), (4, 3, 3)), "swin_b_s1_b8": ((8, 16, 60, 60, 128), (4, 3, 3))}
    g = torch.Generator(device="cuda").manual_seed(4)
    scrub = torch.empty(512 * 1024 * 1024 // 4, device="cuda")
    for name, (shape, shift) in shapes.items():
        B, T, H, W, C = shape
        x = torch.randn(shape, generator=g, device="cuda").to(torch.bfloat16)
        gam = torch.ones(C, dtype=torch.bfloat16, device="cuda")
        bet = torch.zeros(C, dtype=torch.bfloat16, device="cuda")
        win = vs.vswin_partition_fwd(x, (8, 7, 7), shift, stream=stream)
        L, Lp = x.numel() // C, win.numel() // C
        runs = {
            "gather": (lambda: vs.vswin_partition_fwd(x, (8, 7, 7), shift, stream=stream), (L + Lp) * C * 2),
            "scatter_residual": (lambda: vs.vswin_reverse_fwd(win, shape, (8, 7, 7), shift, residual=x,
                                                              stream=stream), 3 * L * C * 2),
            "layernorm": (lambda: vs.vswin_layernorm_fwd(x, gam, bet, stream=stream), 2 * L * C * 2),
        }
        res = {}
        for k, (fn, nbytes) in runs.items():
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(launches):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            warm_us = e0.elapsed_time(e1) * 1e3 / launches
            cold = []
            for _ in range(cold_launches):
                scrub.fill_(1.0)
                torch.cuda.synchronize()
                e0.record(stream)
                fn()
                e1.record(stream)
                torch.cuda.synchronize()
                cold.append(e0.elapsed_time(e1) * 1e3)
            cold_us = statistics.median(cold)
            rate = lambda us: nbytes / (us * 1e-6) / 1e9
            res[k] = {"bytes": nbytes,
                      "cold_us": round(cold_us, 2), "cold_GB/s": round(rate(cold_us), 1),
                      "cold_frac": round(rate(cold_us) / PEAK_HBM_GBS, 3),
                      "warm_us": round(warm_us, 2), "warm_GB/s": round(rate(warm_us), 1),
                      "warm_frac": round(rate(warm_us) / PEAK_HBM_GBS, 3)}
        out[name] = res
    del scrub
    return out


def inference_head(vs, torch, stream, launches: int = 20) -> dict:
    """The pieces around the backbone at the Swin-T K400 test protocol: the
    classification head on 2 videos x 12 views (4 clips x 3 crops) of final
    tokens (16, 7, 7, 768) in bf16 with 400 classes, then the average of the
    views' softmax probabilities; plus the inflation of a Swin-T 2D patch
    kernel and (13*13, 3) bias table.  us per launch (HIP events) and the
    head's algorithmic bytes (tokens and weights once) over its time."""
    g = torch.Generator(device="cuda").manual_seed(6)
    B, V, K, C = 2, 12, 400, 768
    x = torch.randn((B * V, 16, 7, 7, C), generator=g, device="cuda").to(torch.bfloat16)
    w = (0.02 * torch.randn((K, C), generator=g, device="cuda")).to(torch.bfloat16)
    b = torch.zeros(K, dtype=torch.bfloat16, device="cuda")
    logits = torch.empty((B * V, K), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(vs.lib().vswin_head_workspace(B * V, 16 * 49, C), 256), dtype=torch.uint8, device="cuda")
    w2 = (0.02 * torch.randn((96, 3, 4, 4), generator=g, device="cuda")).to(torch.bfloat16)
    t2 = (0.02 * torch.randn((169, 3), generator=g, device="cuda")).to(torch.bfloat16)
    runs = {
        "head": (lambda: vs.vswin_head_fwd(x, w, b, out=logits, workspace=ws, stream=stream),
                 x.numel() * 2 + w.numel() * 2 + B * V * K * 4),
        "multiview_average": (lambda: vs.vswin_multiview_average(logits.view(B, V, K), stream=stream), None),
        "inflate_patch_embed": (lambda: vs.vswin_inflate_patch_embed(w2, 2, stream=stream), None),
        "inflate_bias_table": (lambda: vs.vswin_inflate_bias_table(t2, 8, stream=stream), None),
    }
    out = {"workload": "2 videos x 12 views, tokens (16,7,7,768) bf16, 400 classes"}
    for k, (fn, nbytes) in runs.items():
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(launches):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / launches
        r = {"us": round(us, 2)}
        if nbytes:
            gbs = nbytes / (us * 1e-6) / 1e9
            r.update({"bytes": nbytes, "GB/s": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 3)})
        out[k] = r
    return out


def window_variants(vs, torch, np, stream, steps: int = 20) -> dict:
    """The block pair on the Swin-T stage-1 token grid (1,16,56,56,96) with
    the other temporal windows of the window-size ablation, 4 and 16 (196 and
    784 tokens per window; shift half the window), and with the -100 form of
    the region mask at window 8: ms per pair (eager, HIP events) and the
    attention kernel alone (prepared tables reused) in us and TFLOP/s."""
    import synth
    C, heads, hid = 96, 3, 384
    shape = (1, 16, 56, 56, C)
    g = np.random.default_rng(5)
    xd = torch.from_numpy(g.standard_normal(shape).astype(np.float32)).to(torch.bfloat16).cuda()
    cases = {"window_4": ((4, 7, 7), (2, 3, 3), 0), "window_16": ((16, 7, 7), (8, 3, 3), 0),
             "window_8_mask_m100": ((8, 7, 7), (4, 3, 3), vs.F_MASK_M100)}
    out = {}
    for name, (window, shift, flags) in cases.items():
        rows = (2 * window[0] - 1) * 13 * 13
        ps = [synth.gen_block_params(C, heads, rows, 4, np.random.SeedSequence(40 + k), "bf16", "spec")
              for k in range(2)]
        w = [{k: torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.bfloat16).cuda()
              for k, v in p.items()} for p in ps]
        shifts = [(0, 0, 0), shift]
        descs = [vs.make_desc(*shape, heads, window, sh, mlp_hidden=hid, dtype=torch.bfloat16, flags=flags)
                 for sh in shifts]
        plans = [vs.vswin_plan_query(d) for d in descs]
        ws = torch.empty(max(p["workspace_bytes"] for p in plans), dtype=torch.uint8, device="cuda")
        y1, y2 = torch.empty_like(xd), torch.empty_like(xd)

        def pair():
            vs.vswin_block_fwd(xd, w[0], heads, window, shifts[0], out=y1, workspace=ws, flags=flags, stream=stream)
            vs.vswin_block_fwd(y1, w[1], heads, window, shifts[1], out=y2, workspace=ws, flags=flags, stream=stream)

        for _ in range(3):
            pair()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            pair()
        e1.record(stream)
        torch.cuda.synchronize()
        pair_ms = e0.elapsed_time(e1) / steps
        # the attention kernel alone, shifted block
        nW, N = plans[1]["num_windows"], plans[1]["tokens_per_window"]
        gq = torch.Generator(device="cuda").manual_seed(6)
        qkv = [torch.randn((nW, heads, N, C // heads), generator=gq, device="cuda").to(torch.bfloat16)
               for _ in range(3)]
        o = torch.empty((nW, N, C), dtype=torch.bfloat16, device="cuda")
        aws = torch.empty(max(256, plans[1]["attention_workspace_bytes"]), dtype=torch.uint8, device="cuda")
        vs.vswin_attention_fwd(descs[1], *qkv, w[1]["rpb_table"], out=o, workspace=aws, stream=stream)
        ready = vs.make_desc(*shape, heads, window, shift, mlp_hidden=hid, dtype=torch.bfloat16,
                             flags=flags | vs.F_TABLES_READY)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            vs.vswin_attention_fwd(ready, *qkv, w[1]["rpb_table"], out=o, workspace=aws, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        attn_us = e0.elapsed_time(e1) * 1e3 / steps
        fl = block_flops(plans[1], C, hid)
        pair_flops = sum(block_flops(p, C, hid)["total"] for p in plans)
        out[name] = {"window": list(window), "shift": list(shift), "tokens_per_window": N,
                     "fast_attention": bool(plans[1]["fast_attention"]),
                     "pair_ms": round(pair_ms, 4), "pair_tflops": round(pair_flops / (pair_ms * 1e-3) / 1e12, 2),
                     "tokens_per_s": round(2 * 50176 / (pair_ms * 1e-3), 1),
                     "attn_us_shifted": round(attn_us, 3),
                     "attn_tflops": round(fl["attn"] / (attn_us * 1e-6) / 1e12, 2)}
    return out


def backward_pair(vs, torch, np, x, w, s, shifts, stream, steps: int = 10) -> dict:
    """Training backward of the same block pair (vswin_block_bwd, forward
    recomputed inside each call): ms per pair (HIP events) and the backward
    FLOPs of the closed form: the forward again plus, per linear layer, 2x
    its forward FLOPs (dX and dW), and 5 attention products per (query, key)
    (S and dP in the key-owned kernel, S^T, dP^T and dQ in the query-owned one
    recompute S and dP, so 7 products are issued; 4 of them are necessary:
    dP, dV, dK, dQ, plus S)."""
    hid = s.mlp_ratio * s.C
    dy = torch.randn(x.shape, device="cuda", generator=torch.Generator(device="cuda").manual_seed(7)).to(x.dtype)
    descs = [vs.make_desc(s.B, s.T, s.H, s.W, s.C, s.heads, s.window, sh, mlp_hidden=hid, dtype=torch.bfloat16)
             for sh in shifts]
    nbytes = max(vs.vswin_bwd_workspace_query(d)["block"] for d in descs)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dx = torch.empty_like(x)
    grads = [{k: torch.empty(v.shape, dtype=torch.float32, device="cuda") for k, v in wi.items()} for wi in w]

    def pair():
        for i, sh in enumerate(shifts):
            vs.vswin_block_bwd(x, w[i], dy, s.heads, s.window, sh, dx=dx, grads=grads[i], workspace=ws,
                               stream=stream)

    pair()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        pair()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    plans = [vs.vswin_plan_query(d) for d in descs]
    fwd = [block_flops(p, s.C, hid) for p in plans]
    lin = sum(f["qkv"] + f["proj"] + f["fc1"] + f["fc2"] for f in fwd)
    attn = sum(f["attn"] for f in fwd)           # 2 products (S, PV) per (query, key)
    flops = sum(f["total"] for f in fwd) + 2 * lin + 2.5 * attn
    return {"ms_per_pair": round(ms, 4), "tokens_per_s": round(2 * s.tokens / (ms * 1e-3), 1),
            "gflop_per_pair": round(flops / 1e9, 3), "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
            "note": "forward recomputed inside the call; FLOPs = forward + 2x linear + 5 attention products"}


def mfma_measured_peak(vs, torch, stream, iters: int = 4000) -> float:
    """TFLOP/s of the library's v_mfma_f32_16x16x32_bf16 throughput kernel with
    two workgroups of 8 waves per CU (four waves per SIMD)."""
    blocks = 2 * torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(blocks * 512, dtype=torch.float32, device="cuda")
    flops = vs.vswin_mfma_rate_probe(out, blocks, iters, stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(5):
        vs.vswin_mfma_rate_probe(out, blocks, iters, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    return flops / (e0.elapsed_time(e1) * 1e-3 / 5) / 1e12


def issue_overlap(vs, torch, stream, iters: int = 2000) -> dict:
    """us per launch of the library's MFMA / VALU overlap probe (4 waves per
    SIMD): MFMA part only, VALU part only, the two split over the waves, both
    in every wave.  serial_fraction = t_both / (t_mfma + t_valu): 1 when the
    SIMD runs the two kinds of work back to back, max / sum when it overlaps
    them fully."""
    blocks = 2 * torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(blocks * 512, dtype=torch.float32, device="cuda")
    t = {}
    for mode, name in enumerate(["mfma_us", "valu_us", "split_us", "both_us"]):
        vs.vswin_issue_probe(out, blocks, iters, mode, stream=stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(3):
            vs.vswin_issue_probe(out, blocks, iters, mode, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        t[name] = round(e0.elapsed_time(e1) * 1e3 / 3, 1)
    t["serial_fraction"] = round(t["both_us"] / (t["mfma_us"] + t["valu_us"]), 3)
    t["full_overlap_would_be"] = round(max(t["mfma_us"], t["valu_us"]) / (t["mfma_us"] + t["valu_us"]), 3)
    return t


def step_percentiles(step, torch, stream, n: int, scrub=None) -> dict:
    """Per-step times (ms) from HIP events around each step; with `scrub` (a
    callable run between steps, outside the events) the caches start cold."""
    ts = []
    for _ in range(n):
        if scrub is not None:
            scrub()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step(stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ts.sort()
    q = lambda f: ts[min(len(ts) - 1, int(f * (len(ts) - 1) + 0.5))]
    return {"p10": round(q(0.1), 4), "p50": round(q(0.5), 4), "p90": round(q(0.9), 4), "n": n}


def counter_pass():
    """A plain copy of known size (the scale of FETCH_SIZE / WRITE_SIZE), then
    the attention kernel alone on seeded q, k, V^T of the Swin-T stage-1 shape,
    the one-kernel qkv + attention and one block pair on the stage-1 tokens,
    and the standalone memory-bound kernels."""
    import torch
    import synth
    import shifted_window_attention_amd as vs
    n = 256 * 1024 * 1024
    src = torch.ones(n // 4, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    s = synth.WORKLOADS[2].shape
    g = torch.Generator(device="cuda").manual_seed(2)
    for sh in [(0, 0, 0), s.shift]:
        d = vs.make_desc(s.B, s.T, s.H, s.W, s.C, s.heads, s.window, sh)
        p = vs.vswin_plan_query(d)
        nW, N = p["num_windows"], p["tokens_per_window"]
        q, k, v = (torch.randn((nW, s.heads, N, s.C // s.heads), generator=g, device="cuda").to(torch.bfloat16)
                   for _ in range(3))
        tab = (0.02 * torch.randn((15 * 13 * 13, s.heads), generator=g, device="cuda")).to(torch.bfloat16)
        o = torch.empty((nW, N, s.C), dtype=torch.bfloat16, device="cuda")
        for _ in range(3):
            vs.vswin_attention_fwd(d, q, k, v, tab, out=o)
    torch.cuda.synchronize()
    # LN1 + gather + qkv + attention in one kernel on the stage-1 tokens, 3
    # launches per shift
    x_np, params = synth.gen_workload(2)
    x = torch.from_numpy(x_np).to(torch.bfloat16).cuda()
    ws = [{k_: torch.from_numpy(v_).to(torch.bfloat16).cuda() for k_, v_ in p_.items()} for p_ in params]
    os.environ["VSWIN_FUSED"] = "1"
    for i, sh in enumerate([(0, 0, 0), s.shift]):
        for _ in range(3):
            vs.vswin_qkv_attention_fwd(x, ws[i], s.heads, s.window, sh)
    os.environ.pop("VSWIN_FUSED")
    # one block pair (qkv, attention, projection + MLP kernels, twice)
    y1 = vs.vswin_block_fwd(x, ws[0], s.heads, s.window, (0, 0, 0))
    vs.vswin_block_fwd(y1, ws[1], s.heads, s.window, s.shift)
    torch.cuda.synchronize()
    # the standalone gather, scatter + residual and LayerNorm, once each, in this
    # order, on the Swin-B stage-1 grid (B=8, 16x60x60x128 padded to 16x63x63)
    shape, C = (8, 16, 60, 60, 128), 128
    x = torch.randn(shape, generator=g, device="cuda").to(torch.bfloat16)
    gam = torch.ones(C, dtype=torch.bfloat16, device="cuda")
    bet = torch.zeros(C, dtype=torch.bfloat16, device="cuda")
    win = vs.vswin_partition_fwd(x, (8, 7, 7), (4, 3, 3))
    vs.vswin_reverse_fwd(win, shape, (8, 7, 7), (4, 3, 3), residual=x)
    vs.vswin_layernorm_fwd(x, gam, bet)
    torch.cuda.synchronize()
    print("counter pass done", flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=200,
                    help="untimed steps before the timed ones (the first 10 eager, all of them as graph replays)")
    ap.add_argument("--kernel-launches", type=int, default=50,
                    help="attention-kernel launches timed for the roofline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--counter-pass", action="store_true",
                    help="no timing: one 256 MiB device copy (counter calibration), 3 attention launches per "
                         "shift of the stage-1 shape, 3 one-kernel qkv + attention launches per shift and one "
                         "block pair on the stage-1 tokens, then one gather, scatter and LayerNorm of the Swin-B "
                         "stage-1 B=8 grid; for rocprofv3 --pmc runs")
    ap.add_argument("--no-traffic", action="store_true",
                    help="leave roofline.traffic null (ignore the committed counter summaries)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the block shards by clip with no exchange, so run one process per GPU.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import shifted_window_attention_amd as vs

    torch.cuda.set_device(0)
    if args.counter_pass:
        counter_pass()
        return
    wl = synth.WORKLOADS[2]
    s = wl.shape
    x_np, params = synth.gen_workload(2)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).cuda()
    x = dev(x_np)
    w = [{k: dev(v) for k, v in p.items()} for p in params]
    hid = s.mlp_ratio * s.C
    shifts = [(0, 0, 0), s.shift]
    descs = [vs.make_desc(s.B, s.T, s.H, s.W, s.C, s.heads, s.window, sh, mlp_hidden=hid,
                          dtype=torch.bfloat16) for sh in shifts]
    plans = [vs.vswin_plan_query(d) for d in descs]
    ws = torch.empty(max(p["workspace_bytes"] for p in plans), dtype=torch.uint8, device="cuda")
    y1 = torch.empty_like(x)
    y2 = torch.empty_like(x)
    stream = torch.cuda.current_stream()

    def step(st):
        vs.vswin_block_fwd(x, w[0], s.heads, s.window, shifts[0], out=y1, workspace=ws, stream=st)
        vs.vswin_block_fwd(y1, w[1], s.heads, s.window, shifts[1], out=y2, workspace=ws, stream=st)

    def timed(run, st):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(st)
        for _ in range(args.steps):
            run()
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps, (time.perf_counter() - t0) * 1e3 / args.steps

    for _ in range(min(args.warmup, 10)):
        step(stream)
    torch.cuda.synchronize()
    ref_y = y2.clone()
    # The K timed steps are captured into one HIP graph and replayed once: the
    # same kernels on the same buffers, K times over, without the Python
    # binding's per-call argument checks on the host (which take about as long
    # as the GPU work).  The eager rate through the binding is reported too.
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(args.steps):
            step(torch.cuda.current_stream())
    graph.replay()
    torch.cuda.synchronize()
    if not torch.equal(y2, ref_y):
        raise RuntimeError("the graph replay differs from the eager pair")
    # warm-up: at least W steps as untimed replays of the same graph, queued
    # right before the timed one (no host synchronisation in between), so that
    # the timed replay starts on a GPU already in its steady state under load
    # (the first replays after a pause run up to 10 % slower)
    warm_replays = max(1, -(-args.warmup // args.steps))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(warm_replays):
        graph.replay()
    e0.record(stream)
    graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    # host clock over the warm-up and timed replays together
    wall = (time.perf_counter() - t0) * 1e3 / ((warm_replays + 1) * args.steps)
    del graph
    eager_ms, eager_wall = timed(lambda: step(stream), stream)
    # per-step distribution (one pair per graph replay, events around each),
    # warm, then with a 512 MiB scrub between steps (larger than the 256 MB
    # last-level cache) so that each step starts from HBM
    g1 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g1):
        step(torch.cuda.current_stream())
    replay = lambda st: g1.replay()
    warm = step_percentiles(replay, torch, stream, 50)
    scrub_buf = torch.empty(512 * 1024 * 1024 // 4, device="cuda")
    cold = step_percentiles(replay, torch, stream, 20, scrub=lambda: scrub_buf.fill_(1.0))
    del scrub_buf, g1
    flops = [block_flops(p, s.C, hid) for p in plans]
    step_flops = sum(f["total"] for f in flops)
    tokens_per_step = s.tokens * len(shifts)
    tflops = step_flops / (ms * 1e-3) / 1e12

    def time_launches(fn, n):
        """Average time of one launch of fn(stream): n launches captured into
        one graph, replayed once between two events right behind at least W
        untimed launches (replays of the same graph), like the timed pairs."""
        fn(stream)
        torch.cuda.synchronize()
        gl = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gl):
            for _ in range(n):
                fn(torch.cuda.current_stream())
        gl.replay()
        torch.cuda.synchronize()
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(max(1, -(-args.warmup // n))):
            gl.replay()
        a0.record(stream)
        gl.replay()
        a1.record(stream)
        torch.cuda.synchronize()
        return a0.elapsed_time(a1) * 1e3 / n

    # the same pair with LN1 + gather + qkv + attention as one kernel
    # (VSWIN_FUSED=1), and that kernel alone, for comparison
    os.environ["VSWIN_FUSED"] = "1"
    g10 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g10):
        for _ in range(10):
            step(torch.cuda.current_stream())
    g10.replay()
    torch.cuda.synchronize()
    f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(max(1, -(-args.warmup // 10))):   # the same warm-up as the timed pairs
        g10.replay()
    f0.record(stream)
    g10.replay()
    f1.record(stream)
    torch.cuda.synchronize()
    one_kernel_pair_ms = f0.elapsed_time(f1) / 10
    del g10
    Lp = plans[0]["num_windows"] * plans[0]["tokens_per_window"]
    o_rows = torch.empty((Lp, s.C), dtype=torch.bfloat16, device="cuda")
    msa_ws = torch.empty(max(p["msa_workspace_bytes"] for p in plans), dtype=torch.uint8, device="cuda")
    fused_us = [time_launches(lambda st: vs.vswin_qkv_attention_fwd(x, w[i], s.heads, s.window, shifts[i],
                                                                     out=o_rows, workspace=msa_ws, stream=st),
                              args.kernel_launches) for i in range(len(shifts))]
    os.environ.pop("VSWIN_FUSED")
    fused_flops = flops[0]["qkv"] + flops[0]["attn"]
    f_us = sum(fused_us) / len(fused_us)
    one_kernel = {"kernel": "wattn_fused_kernel<96> (LN1 + gather + qkv + window attention, VSWIN_FUSED=1)",
                  "pair_ms": round(one_kernel_pair_ms, 4), "avg_us": round(f_us, 3),
                  "tflops": round(fused_flops / (f_us * 1e-6) / 1e12, 2),
                  "frac": round(fused_flops / (f_us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4),
                  "flops_per_launch": fused_flops,
                  "traffic": None if args.no_traffic else counter_traffic(FUSED_TRAFFIC_SUMMARY, FUSED_SOURCES)}

    # ---- the attention core alone (the kernel of the separate-launch path) on
    # prepared q, k, V^T; the first calls prepare the bias tables in attn_ws,
    # the timed ones reuse them (F_TABLES_READY)
    d = s.C // s.heads
    g = torch.Generator(device="cuda").manual_seed(2)
    qkv = [torch.randn((plans[0]["num_windows"], s.heads, plans[0]["tokens_per_window"], d),
                       generator=g, device="cuda").to(torch.bfloat16) for _ in range(3)]
    o = torch.empty((plans[0]["num_windows"], plans[0]["tokens_per_window"], s.C), dtype=torch.bfloat16,
                    device="cuda")
    attn_ws = torch.empty(max(256, max(p["attention_workspace_bytes"] for p in plans)), dtype=torch.uint8,
                          device="cuda")
    ready = [vs.make_desc(s.B, s.T, s.H, s.W, s.C, s.heads, s.window, sh, mlp_hidden=hid,
                          dtype=torch.bfloat16, flags=vs.F_TABLES_READY) for sh in shifts]
    kern_us = []
    for i, dsc in enumerate(descs):
        vs.vswin_attention_fwd(dsc, *qkv, w[i]["rpb_table"], out=o, workspace=attn_ws, stream=stream)
        kern_us.append(time_launches(lambda st: vs.vswin_attention_fwd(ready[i], *qkv, w[i]["rpb_table"], out=o,
                                                                       workspace=attn_ws, stream=st),
                                     args.kernel_launches))
    attn_flops = flops[0]["attn"]
    attn_us = sum(kern_us) / len(kern_us)
    achieved = attn_flops / (attn_us * 1e-6) / 1e12
    measured_peak = mfma_measured_peak(vs, torch, stream)
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": None if args.no_traffic else counter_traffic(TRAFFIC_SUMMARY, ATTN_SOURCES),
                "kernel": "attn_mfma_kernel", "avg_us": round(attn_us, 3),
                "avg_us_regular": round(kern_us[0], 3), "avg_us_shifted": round(kern_us[1], 3),
                "flops_per_launch": attn_flops, "measured_mfma_peak": round(measured_peak, 1),
                "frac_of_measured_peak": round(achieved / measured_peak, 4),
                "mfma_valu_issue": issue_overlap(vs, torch, stream)}

    out = {
        "metric": METRIC, "value": round(tokens_per_step / (ms * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "Swin-T stage-1 regular+shifted block pair: bf16 tokens (1,16,56,56,96), "
                               "3 heads x 32, window (8,7,7), shift (4,3,3), MLP ratio 4, seeded synthetic",
                   "global_batch": s.B, "tokens_per_block": s.tokens, "blocks_per_step": len(shifts),
                   "parallelism": "single GPU"},
        "tflops": round(tflops, 2), "mfma_peak_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        "mfma_measured_peak_frac": round(tflops / measured_peak, 4),
        "step_gflop": round(step_flops / 1e9, 3), "wall_ms_per_step": round(wall, 4),
        "timing": "the K steps captured in one HIP graph, replayed once (eager binding calls: eager_ms_per_step)",
        "eager_ms_per_step": round(eager_ms, 4), "eager_wall_ms_per_step": round(eager_wall, 4),
        "roofline": roofline, "one_kernel_qkv_attention": one_kernel,
        "step_ms_warm": warm, "step_ms_cold": cold,
        "memory_kernels": memory_kernels(vs, torch, stream),
        "window_variants": window_variants(vs, torch, np, stream),
        "backward": backward_pair(vs, torch, np, x, w, s, shifts, stream),
        "inference_head": inference_head(vs, torch, stream),
        "other_workloads": other_workloads(vs, torch, np, stream),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(x_np, params, s)
        out["cpu_baseline_per_workload"] = oracle_per_config()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
