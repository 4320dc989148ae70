#!/usr/bin/env python3
"""Benchmark of the MoE expert-decode path on one MI355X.

A step is one decode step of M tokens (M = 1 for the headline stacks, M = 4
or 16 for the 120B-shape small-M workload) through every layer: per layer the
router (a route kernel, or partial sums from the previous down kernel), the
grouped gate_up dequant-GEMV with SwiGLU over the chosen experts, and the
grouped down dequant-GEMV with the weighted combine and residual - replayed
from one captured HIP graph per step.  Every token gets a fresh N(0,1) bf16
hidden state; all inputs and weights are resident in HBM before the timed
region.  W untimed warmup steps, then K timed steps bracketed by stream
events and device synchronisation.

Prints one JSON line: the expert-path HBM rate (algorithmic packed-weight
bytes of every (layer, expert) matrix the step uses, once, plus the router
weights, over GPU time), the per-kernel roofline figure of the dominant
kernel (gate_up), the measured streaming-read rate, and the CPU oracle timed
on a bounded sample.  After the timed run the same steps run again twice,
untimed for the headline: with an event pair around each step (the per-step
median / mean / spread) and with a host sync after each step (sync mode, the
wall time when the host picks every next token).

Other workloads (``--workload``): the five expert-path configurations, dense
packed GEMVs on non-expert shapes, the large-M (prefill) path on the
MX-scaled matrix cores, and the decode attention of a gpt-oss-shape stack
(``gptoss20b_attn_8k``: KV-cache bytes read per token over GPU time).
"""

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0     # MI355X HBM3E, published peak
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense FP8 matrix-core peak (no sparsity)
METRIC = "expert-path HBM GB/s (% of peak) + us/token, gpt-oss-20B-shape MoE at M=1"
SHARE_NOTE = ("duration_us = the dispatch's own time (start/stop events of the directly launched "
              "per-kernel pass) plus gap_share_us, an equal share of the replayed step's launch gaps "
              "(replayed step time minus the step's dispatch times, over its launches): the duration a "
              "kernel trace of graph replays gives each launch; achieved_kernel_only divides by the "
              "dispatch time alone")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def expert_bytes(cfg):
    """Packed bytes (codes + scales + zeros) of one expert's gate_up and down."""
    def mat(n, k):
        codes = n * k // 2
        if cfg.fmt == "mxfp4":
            return codes + n * (k // 32)
        groups = k // cfg.group
        return codes + n * groups * 2 + n * ((groups + 1) // 2)
    return mat(2 * cfg.inter, cfg.hidden), mat(cfg.hidden, cfg.inter)


def router_bytes(cfg):
    return cfg.n_experts * cfg.hidden * 4 + (cfg.n_experts * 4 if cfg.hot_experts else 0)


def step_bytes(cfg, unique_experts_per_layer):
    gu, dn = expert_bytes(cfg)
    return sum(router_bytes(cfg) + u * (gu + dn) for u in unique_experts_per_layer)


KERNEL_SOURCES = tuple("bit_dequant_gemv_amd/csrc/" + f for f in (
    "moe.hip", "moe_down.hip", "moe_layer.hip", "moe_mfma.hip", "gemv.hip",
    "bdg_gemv.hpp", "bdg_device.hpp", "bdg_topk.hpp", "bdg_moe.hpp", "bdg_moe_down.hpp", "bdg_moe_layer.hpp",
    "bdg_moe_mfma.hpp"))


def kernel_sources_sha(sources=KERNEL_SOURCES):
    """Hash of the kernel sources' code (comments and blank lines dropped), so a
    counter summary stays valid across comment-only edits and no longer."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in sources:
        text = open(os.path.join(ROOT, f)).read()
        lines = [re.sub(r"//.*", "", ln).rstrip() for ln in text.splitlines()]
        h.update("\n".join(ln for ln in lines if ln).encode())
    return h.hexdigest()[:16]


ATTN_SOURCES = ("bit_dequant_gemv_amd/csrc/attn.hip", "bit_dequant_gemv_amd/csrc/bdg_device.hpp")
MX_SOURCES = ("bit_dequant_gemv_amd/csrc/mxgemm.hip", "bit_dequant_gemv_amd/csrc/router.hip",
              "bit_dequant_gemv_amd/csrc/bdg_device.hpp")
SOURCE_SETS = {"moe": KERNEL_SOURCES, "attn": ATTN_SOURCES, "mx": MX_SOURCES}


def measured_traffic(workload, kernel, sources=KERNEL_SOURCES):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, copy-calibrated), or None when there is
    none or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if kernel_sources_sha(sources) != rec.get("kernel_sources_sha"):
        return None
    t = rec["per_launch"].get(kernel)
    return None if t is None else t["fetch_bytes"] + t["write_bytes"]


# ---------------------------------------------------------------- rocprofv3 summaries
#
# `python bench.py summarize ...` turns rocprofv3 CSV output (kernel-trace
# statistics, FETCH_SIZE / WRITE_SIZE passes, SQ counter passes) into the
# text summaries kept under profiles/.  Host-only; reads the CSV files given.

KERNEL_KIND_PATTERNS = (          # kernel name fragment -> kind (per-launch traffic keys)
    ("moe_layer_kernel", "layer"), ("moe_gateup_kernel", "gate_up"), ("moe_gu_group_kernel", "gate_up"),
    ("moe_down_kernel", "down"), ("moe_dn_group_kernel", "down"), ("moe_route", "route"),
    ("moe_combine_kernel", "combine"), ("moe_gu_mfma_kernel", "gate_up"), ("moe_dn_mfma_kernel", "down"),
    ("qgemv_kernel", "qgemv"),
    # the split kernel's one-block form (every cached key in one block, merged in place)
    ("attn_split_kernel<unsigned short, true>", "attn_fused"), ("attn_split_kernel<float, true>", "attn_fused"),
    ("attn_split_kernel", "attn_split"),
    ("attn_merge_kernel", "attn_merge"), ("mx_gemm_kernel", "mx_gemm"), ("mxfp8_quant_kernel", "mx_quant"),
    ("mx_stage_scales_kernel", "mx_stage"),
    ("stream_copy_kernel", "copy"),
)


def kernel_kind(name):
    for frag, kind in KERNEL_KIND_PATTERNS:
        if frag in name:
            return kind
    return None


def short_kernel(name):
    name = name.split("(")[0]
    return name.replace("void ", "").replace("bdg::", "")


def _find(src, suffix):
    import glob
    hits = sorted(glob.glob(os.path.join(src, "**", "*" + suffix), recursive=True))
    if not hits:
        raise SystemExit(f"no *{suffix} under {src}")
    return hits[0]


def _counter_rows(src):
    import csv
    return list(csv.DictReader(open(_find(src, "counter_collection.csv"))))


def _per_kernel_counter(src, counter):
    """{kernel name: [value per dispatch]} for one counter of a pass."""
    out = {}
    for r in _counter_rows(src):
        if r["Counter_Name"] == counter:
            out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def summarize(argv):
    import csv
    import statistics as st
    ap = argparse.ArgumentParser(prog="bench.py summarize")
    ap.add_argument("what", choices=["trace", "traffic", "sq"])
    ap.add_argument("--workload", required=True)
    ap.add_argument("--src", action="append", default=[],
                    help="rocprofv3 output directory (the trace; for sq, one per counter pass, merged)")
    ap.add_argument("--fetch", help="FETCH_SIZE pass of the workload")
    ap.add_argument("--write", help="WRITE_SIZE pass of the workload")
    ap.add_argument("--cal-fetch", help="FETCH_SIZE pass of bench.py --copy-calibration BYTES")
    ap.add_argument("--cal-write", help="WRITE_SIZE pass of the same")
    ap.add_argument("--cal-bytes", type=int, default=268435456)
    ap.add_argument("--command", action="append", default=[], help="the rocprofv3 command(s), for the record")
    ap.add_argument("--note", default="", help="a paragraph of reading under the table")
    ap.add_argument("--name", default=None, help="output file stem (default: kind_workload)")
    ap.add_argument("--sources", default="moe", choices=sorted(SOURCE_SETS))
    ap.add_argument("--out-dir", default=os.path.join(ROOT, "profiles"), help="where the summary goes")
    a = ap.parse_args(argv)
    sha = kernel_sources_sha(SOURCE_SETS[a.sources])
    cmds = "\n".join(f"    {c}" for c in a.command)
    if a.what == "trace":
        rows = list(csv.DictReader(open(_find(a.src[0], "kernel_stats.csv"))))
        total = sum(float(r["TotalDurationNs"]) for r in rows)
        # per dispatch: back to back (its start is the previous dispatch's end on
        # the queue: a graph replay) or not (a direct launch the host issued late)
        disp = sorted(csv.DictReader(open(_find(a.src[0], "kernel_trace.csv"))),
                      key=lambda r: (r["Queue_Id"], int(r["Start_Timestamp"])))
        split = {}
        prev_q, prev_end = None, None
        for r in disp:
            t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
            b2b = prev_q == r["Queue_Id"] and prev_end is not None and t0 <= prev_end
            d = split.setdefault(r["Kernel_Name"], {True: [], False: []})
            d[b2b].append((t1 - t0) / 1e3)
            prev_q, prev_end = r["Queue_Id"], t1
        lines = [f"# Kernel trace: {a.workload}", "", "Command (from the repository root, on one MI355X):", "",
                 cmds, "",
                 "rocprofv3 kernel statistics.  In a run of back-to-back launches (graph replays) a",
                 "kernel's recorded start is the previous kernel's end, so each duration covers the",
                 "kernel and the launch gap before it, and the durations tile the replayed steps.  The",
                 "last two columns split the dispatches by that test: back to back (start = the previous",
                 "dispatch's end on the queue) and the rest (launched directly, e.g. the per-kernel pass).", "",
                 "| kernel | calls | avg us | min us | max us | share | avg us back to back (n) | avg us other (n) |",
                 "|---|---|---|---|---|---|---|---|"]

        def avg(v):
            return f"{st.mean(v):.2f} ({len(v)})" if v else "-"
        for r in rows:
            sp = split.get(r["Name"], {True: [], False: []})
            lines.append(f"| `{short_kernel(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                         f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                         f"{100.0 * float(r['TotalDurationNs']) / total:.1f}% | {avg(sp[True])} | {avg(sp[False])} |")
        stem = a.name or f"kernel_trace_{a.workload}"
    elif a.what == "traffic":
        calf = _per_kernel_counter(a.cal_fetch, "FETCH_SIZE")
        calw = _per_kernel_counter(a.cal_write, "WRITE_SIZE")
        kib = a.cal_bytes / 1024.0
        cf = st.mean(next(v for k, v in calf.items() if "bdg_stream_copy" in k or "copy_kernel" in k))
        cw = st.mean(next(v for k, v in calw.items() if "bdg_stream_copy" in k or "copy_kernel" in k))
        fs, ws = kib / cf, kib / cw
        fetch = _per_kernel_counter(a.fetch, "FETCH_SIZE")
        write = _per_kernel_counter(a.write, "WRITE_SIZE")
        per, table = {}, []
        for name, vals in sorted(fetch.items()):
            kind = kernel_kind(name)
            if kind is None or kind == "copy":
                continue
            f = st.mean(vals)
            w = st.mean(write.get(name, [0.0]))
            fb, wb = int(round(f * fs * 1024)), int(round(w * ws * 1024))
            prev = per.get(kind)
            n = len(vals)
            if prev:      # several template instances of one kind: launch-weighted mean
                tot = prev["launches"] + n
                fb = int(round((prev["fetch_bytes"] * prev["launches"] + fb * n) / tot))
                wb = int(round((prev["write_bytes"] * prev["launches"] + wb * n) / tot))
                n = tot
            per[kind] = {"fetch_bytes": fb, "write_bytes": wb, "launches": n}
            table.append(f"| `{short_kernel(name)}` | {len(vals)} | {f:.1f} | {w:.1f} | {int(round(f * fs * 1024)):,} "
                         f"| {int(round(w * ws * 1024)):,} |")
        lines = [f"# HBM traffic per launch: {a.workload}", "",
                 "Commands (one counter pass each; FETCH_SIZE and WRITE_SIZE cannot share a pass):", "",
                 cmds, "",
                 f"Calibration: the 16-byte copy kernel over {a.cal_bytes} B reads and writes {kib:.0f} KiB;",
                 f"the counters read FETCH_SIZE {cf:.1f} KiB (scale x{fs:.3f}) and WRITE_SIZE {cw:.1f} KiB "
                 f"(scale x{ws:.3f}) per launch.", "",
                 "| kernel | launches | FETCH_SIZE KiB | WRITE_SIZE KiB | fetched bytes (scaled) | written bytes (scaled) |",
                 "|---|---|---|---|---|---|"] + table
        rec = {"workload": a.workload, "kernel_sources_sha": sha, "fetch_scale": fs, "write_scale": ws,
               "per_launch": {k: {"fetch_bytes": v["fetch_bytes"], "write_bytes": v["write_bytes"]}
                              for k, v in per.items()}}
        stem = a.name or f"hbm_traffic_{a.workload}"
        json.dump(rec, open(os.path.join(a.out_dir, stem + ".json"), "w"), indent=1)
    else:
        ctr = {}
        for src in a.src:
            for r in _counter_rows(src):
                ctr.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], []).append(
                    float(r["Counter_Value"]))
        have = set(k for c in ctr.values() for k in c)
        cols = [("dispatches", None), ("waves / dispatch", None)]
        if "SQ_INSTS_VALU" in have:
            cols += [("VALU instr / wave", lambda m, wv, wc: f"{m.get('SQ_INSTS_VALU', 0) / wv:.0f}")]
        if "SQ_INSTS_MFMA" in have:
            cols += [("MFMA instr / wave", lambda m, wv, wc: f"{m.get('SQ_INSTS_MFMA', 0) / wv:.0f}")]
        if "SQ_INSTS_VMEM_RD" in have:
            cols += [("VMEM read instr / wave", lambda m, wv, wc: f"{m.get('SQ_INSTS_VMEM_RD', 0) / wv:.1f}")]
        if "SQ_WAVE_CYCLES" in have:
            cols += [("VALU active / wave-cycles", lambda m, wv, wc: f"{m.get('SQ_ACTIVE_INST_VALU', 0) / wc:.2f}"),
                     ("waiting (any) / wave-cycles", lambda m, wv, wc: f"{m.get('SQ_WAIT_ANY', 0) / wc:.2f}"),
                     ("waiting for issue / wave-cycles",
                      lambda m, wv, wc: f"{m.get('SQ_WAIT_INST_ANY', 0) / wc:.2f}")]
        if "SQ_VALU_MFMA_BUSY_CYCLES" in have:
            cols += [("MFMA busy, M SIMD-cycles / dispatch",
                      lambda m, wv, wc: f"{m.get('SQ_VALU_MFMA_BUSY_CYCLES', 0) / 1e6:.2f}")]
        if "TA_BUSY_avr" in have and "GRBM_GUI_ACTIVE" in have:
            cols += [("TA busy / GUI-active cycles (mean TA)",
                      lambda m, wv, wc: f"{m.get('TA_BUSY_avr', 0) / max(m['GRBM_GUI_ACTIVE'], 1):.2f}")]
        if "SQ_LDS_BANK_CONFLICT" in have and "SQ_ACTIVE_INST_LDS" in have:
            cols += [("LDS bank-conflict cycles / LDS instr",
                      lambda m, wv, wc: f"{m.get('SQ_LDS_BANK_CONFLICT', 0) / max(m['SQ_ACTIVE_INST_LDS'], 1):.2f}")]
        if "SQ_WAIT_INST_LDS" in have and "SQ_WAVE_CYCLES" in have:
            cols += [("waiting for LDS / wave-cycles", lambda m, wv, wc: f"{m.get('SQ_WAIT_INST_LDS', 0) / wc:.3f}")]
        if "GRBM_GUI_ACTIVE" in have:
            cols += [("GUI-active cycles / dispatch", lambda m, wv, wc: f"{m.get('GRBM_GUI_ACTIVE', 0):.0f}")]
        lines = [f"# SQ counters: {a.workload}", "",
                 "Commands (from the repository root, on one MI355X; counter passes of their own, no trace "
                 "options, merged per kernel):", "", cmds, "",
                 "Counters averaged over the dispatches of the run (a counter pass serialises dispatches, so no",
                 "timing is taken from it).  The wave-cycle ratios divide counters that share a unit (summed over",
                 "all waves): SQ_ACTIVE_INST_VALU, SQ_WAIT_ANY and SQ_WAIT_INST_ANY over SQ_WAVE_CYCLES.  MFMA busy",
                 "is SQ_VALU_MFMA_BUSY_CYCLES summed over the SIMDs; divided by a launch's traced duration times",
                 "2.4 GHz times the 1024 SIMDs it gives the matrix cores' share of the launch (a counter pass",
                 "stretches the launches, so GRBM_GUI_ACTIVE is no clock for it).  TA busy is the mean",
                 "texture-address unit's busy cycles (TA_BUSY_avr) over GRBM_GUI_ACTIVE.", "",
                 "| kernel | " + " | ".join(c for c, _ in cols) + " |",
                 "|---|" + "---:|" * len(cols)]
        for name, c in sorted(ctr.items()):
            if kernel_kind(name) is None or "SQ_WAVES" not in c:
                continue
            m = {k: st.mean(v) for k, v in c.items()}
            wv = max(m["SQ_WAVES"], 1.0)
            wc = max(m.get("SQ_WAVE_CYCLES", 0.0), 1.0)
            vals = [str(len(c["SQ_WAVES"])), f"{wv:.0f}"] + [f(m, wv, wc) for _, f in cols[2:]]
            lines.append(f"| `{short_kernel(name)}` | " + " | ".join(vals) + " |")
        stem = a.name or f"sq_counters_{a.workload}"
    if a.note:
        lines += ["", a.note]
    lines += ["", f"Kernel sources sha256[:16]: `{sha}`", ""]
    path = os.path.join(a.out_dir, stem + ".md")
    open(path, "w").write("\n".join(lines))
    print(path)


def blas_threads():
    """Threads the oracle's NumPy BLAS uses (its matrix products run on them)."""
    from threadpoolctl import threadpool_info
    return int(max([p.get("num_threads", 1) for p in threadpool_info()] or [1]))


def cpu_baseline(cfg, sample_layers, m):
    """The oracle as it stands on `sample_layers` layers of one step (M tokens).

    Packed weights of the sampled layers are generated first (untimed), the
    oracle then dequantizes the chosen experts on demand and runs its float64
    layer; the per-layer time is scaled to a whole step of every layer.
    """
    import numpy as np

    import synth
    from oracle import formats, moe as omoe

    log(f"cpu baseline: generating {sample_layers} layers of packed weights (untimed)")
    gen = []
    for l in range(sample_layers):
        w_r, b_r, _ = synth.router(cfg, l)
        experts = [synth.expert_weights(cfg, l, e) for e in range(cfg.n_experts)]
        gen.append((w_r, b_r, experts))
    log("cpu baseline: timing the oracle")
    uniq = []
    passes = 0
    t0 = time.perf_counter()
    # whole passes over the sampled layers, each on fresh tokens, until at
    # least 10 s of CPU work
    while passes < 1 or time.perf_counter() - t0 < 10.0:
        x = synth.hidden_batch(cfg, range(passes * m, (passes + 1) * m))[0].astype(np.float64)
        for l in range(sample_layers):
            w_r, b_r, experts = gen[l]

            def get(e, experts=experts):
                w = experts[e]
                if cfg.fmt == "mxfp4":
                    return formats.mxfp4_dequant(*w["gu"]), formats.mxfp4_dequant(*w["dn"])
                return (formats.int4g_dequant(*w["gu"], cfg.group),
                        formats.int4g_dequant(*w["dn"], cfg.group))
            res = omoe.moe_layer(x, w_r, get, cfg.top_k, bias=b_r, norm=cfg.norm, residual=cfg.norm)
            uniq.append(len(np.unique(res["idx"])))
            x = res["y"]
        passes += 1
    dt = time.perf_counter() - t0
    per_step_s = dt / (passes * sample_layers) * cfg.n_layers
    n_threads = blas_threads()
    nbytes = step_bytes(cfg, [float(np.mean(uniq))] * cfg.n_layers)
    return {
        "value": round(nbytes / per_step_s / 1e9, 4),
        "unit": "GB/s",
        "cores": n_threads,
        "kind": "oracle",
        "us_per_token": round(per_step_s / m * 1e6, 1),
        "sample": f"{sample_layers} of {cfg.n_layers} layers of a step of M={m} tokens, {passes} pass{'es' if passes != 1 else ''} "
                  f"on fresh tokens, {dt:.1f} s of CPU time, scaled to a whole step; float64 NumPy, "
                  f"elementwise dequant on one thread, BLAS matvecs on {n_threads}",
    }


def stream_read_rate(torch, bdg, dev, phase_bytes, gbytes=4.0, reps=5):
    """Streaming-read rate over 4 GiB, and back-to-back reads of phase-sized
    slices (distinct data) - the floor of a kernel that only reads that much."""
    n = int(gbytes * (1 << 30)) // 16 * 16
    buf = torch.empty(n, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    rates = []
    for _ in range(reps + 1):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        bdg.stream_read(buf)
        b.record()
        b.synchronize()
        rates.append(n / (a.elapsed_time(b) * 1e-3) / 1e9)
    phases = {}
    sink = torch.empty(1024, dtype=torch.float32, device=dev)
    for name, nb in phase_bytes.items():
        nb = nb // 256 * 256
        cnt = min(64, n // nb)
        views = [buf[i * nb:(i + 1) * nb] for i in range(cnt)]
        # back-to-back reads of distinct slices replayed from a graph, so the
        # figure is the GPU's and not the host's launch rate
        graph = torch.cuda.CUDAGraph()
        stream = torch.cuda.Stream()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            with torch.cuda.graph(graph, stream=stream):
                for v in views:
                    bdg.stream_read(v, n_blocks=1024, sink=sink)
        torch.cuda.current_stream().wait_stream(stream)
        graph.replay()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        graph.replay()
        b.record()
        b.synchronize()
        us = a.elapsed_time(b) * 1e3 / cnt
        del graph
        phases[name] = {"bytes": nb, "us": round(us, 2), "GBps": round(nb / (us * 1e-6) / 1e9, 1)}
    del buf
    return max(rates[1:]), statistics.median(rates[1:]), phases


def base_record(cfg, value, K, W, ms_per_step, config):
    return {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": config,
        "pct_of_peak": round(100.0 * value / PEAK_HBM_GBPS, 2),
    }


def bench_gemv(torch, bdg, synth, sdev, dev, cfg, args):
    """Single MXFP4 GEMV, 2880 x 2880: R distinct matrices (more than L2 + the
    Infinity Cache) called in rotation so every call reads from HBM (cold), and
    the same matrix called R times (hot, a cache figure).  The calls of one
    pass are replayed from a captured graph, so the time per call is the GPU's
    (kernel plus the gap between graph nodes)."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    from oracle import formats, gemv as ogemv

    R = 256
    K = args.steps if args.steps is not None else 16
    W = args.warmup if args.warmup is not None else 2
    t0 = time.time()
    with ThreadPoolExecutor(16) as ex:
        mats = list(ex.map(lambda i: synth.gemv_matrix(cfg, i), range(R)))
    qws = [sdev.qweight_from_arrays(cfg.fmt, m, cfg.group, dev) for m in mats]
    log(f"uploaded {R} matrices ({time.time() - t0:.1f} s)")
    x = torch.from_numpy(synth.hidden(cfg, 0)[0]).to(dev)
    y = torch.empty(cfg.hidden, dtype=torch.float32, device=dev)
    nbytes = cfg.hidden * cfg.hidden // 2 + cfg.hidden * (cfg.hidden // 32)

    def timed(order):
        g = torch.cuda.CUDAGraph()
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            with torch.cuda.graph(g, stream=st):
                for i in order:
                    bdg.qgemv(qws[i], x, out=y)
        torch.cuda.current_stream().wait_stream(st)
        for _ in range(W):
            g.replay()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(K):
            g.replay()
        b.record()
        b.synchronize()
        us = a.elapsed_time(b) * 1e3 / (K * len(order))
        del g
        return us

    cold_us = timed(list(range(R)))
    hot_us = timed([0] * R)
    value = nbytes / (cold_us * 1e-6) / 1e9
    log(f"cold {cold_us:.2f} us/call ({value:.1f} GB/s), hot {hot_us:.2f} us/call "
        f"({nbytes / (hot_us * 1e-6) / 1e9:.1f} GB/s)")
    cpu = None
    if not args.no_cpu_baseline:
        w = formats.mxfp4_dequant(*mats[0])
        xv = synth.hidden(cfg, 0)[0]
        t1 = time.perf_counter()
        n = 0
        while time.perf_counter() - t1 < 10.0 or n < 2:
            ogemv.gemv(formats.mxfp4_dequant(*mats[n % R]), xv)
            n += 1
        dt = (time.perf_counter() - t1) / n
        cpu = {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "kind": "oracle",
               "cores": blas_threads(),
               "sample": f"{n} calls, dequant (NumPy, one thread) + float64 matvec each"}
        del w
    out = base_record(cfg, value, K * R, W * R, cold_us * 1e-3, {
        "workload": cfg.name, "fmt": cfg.fmt, "n": cfg.hidden, "k": cfg.hidden,
        "matrices_rotated": R, "bytes_per_call": nbytes,
        "timing": "graph of 256 calls replayed; per call = kernel + node gap"})
    out.update({"us_per_call_cold": round(cold_us, 3), "us_per_call_hot": round(hot_us, 3),
                "hot_GBps_cache": round(nbytes / (hot_us * 1e-6) / 1e9, 1), "cpu_baseline": cpu,
                "roofline": {"kernel": "qgemv_kernel", "bound": "hbm", "achieved": round(value, 1),
                             "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(value / PEAK_HBM_GBPS, 4),
                             "traffic": None, "traffic_algorithmic_bytes": nbytes}})
    print(json.dumps(out), flush=True)


def dense_bytes(cfg):
    """Packed bytes of one dense matrix: codes + scales (+ int4 zero points)."""
    if cfg.fmt == "mxfp4":
        return cfg.n * cfg.k // 2 + cfg.n * (cfg.k // 32)
    groups = cfg.k // cfg.group
    return cfg.n * cfg.k // 2 + cfg.n * groups * 2 + cfg.n * ((groups + 1) // 2)


def bench_dense(torch, bdg, synth, sdev, dev, cfg, args):
    """One dense packed GEMV on a non-expert shape at M=1 (bf16 x): cfg.rotate
    distinct matrices, together larger than L2 and the Infinity Cache, called
    in turn from a captured graph, so every call reads its matrix from HBM.
    The time per call (events around the replays) is the kernel plus the gap
    between graph nodes, so the roofline figure from it is a lower bound."""
    import numpy as np

    R = cfg.rotate
    nbytes = dense_bytes(cfg)
    calls = max(R, (64 // R) * R)                      # calls per graph replay
    K = args.steps if args.steps is not None else 8
    W = args.warmup if args.warmup is not None else 2
    t0 = time.time()
    qws = []
    for i in range(R):
        arrs = synth.dense_matrix(cfg, i)
        qws.append(sdev.qweight_from_arrays(cfg.fmt, arrs, cfg.group, dev))
        del arrs
    log(f"uploaded {R} matrices of {nbytes / 1e6:.1f} MB ({time.time() - t0:.1f} s)")
    _, xbits = synth.hidden(cfg, 0)
    x = torch.from_numpy(xbits.view(np.int16)).to(dev).view(torch.bfloat16)
    y = torch.empty(cfg.n, dtype=torch.float32, device=dev)

    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            for c in range(calls):
                bdg.qgemv(qws[c % R], x, out=y)
    torch.cuda.current_stream().wait_stream(st)
    for _ in range(W):
        g.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(K):
        g.replay()
    b.record()
    b.synchronize()
    call_us = a.elapsed_time(b) * 1e3 / (K * calls)
    value = nbytes / (call_us * 1e-6) / 1e9
    if not torch.isfinite(y).all():
        raise SystemExit("non-finite output")
    log(f"{cfg.name}: {call_us:.2f} us/call in the graph ({value:.1f} GB/s)")

    cpu = None
    if not args.no_cpu_baseline:
        # the oracle on a bounded row sample (dequantize + float64 matvec), scaled by bytes
        from oracle import formats, gemv as ogemv
        arrs = synth.dense_matrix(cfg, 0)
        xv = synth.hidden(cfg, 0)[0]
        rows = min(cfg.n, 16384)
        sample = tuple(a_[:rows] for a_ in arrs)
        sbytes = nbytes * rows / cfg.n
        t1 = time.perf_counter()
        n = 0
        while time.perf_counter() - t1 < 10.0 or n < 2:
            if cfg.fmt == "mxfp4":
                w = formats.mxfp4_dequant(*sample)
            else:
                w = formats.int4g_dequant(*sample, cfg.group)
            ogemv.gemv(w, xv)
            n += 1
        dt = (time.perf_counter() - t1) / n
        cpu = {"value": round(sbytes / dt / 1e9, 4), "unit": "GB/s", "kind": "oracle",
               "cores": blas_threads(),
               "sample": f"{rows} of {cfg.n} rows, {n} passes of dequant (NumPy) + float64 matvec"}
    out = base_record(cfg, value, K * calls, W * calls, call_us * 1e-3, {
        "workload": cfg.name, "fmt": cfg.fmt, "n": cfg.n, "k": cfg.k, "m": 1,
        "matrices_rotated": R, "bytes_per_call": nbytes,
        "timing": f"graph of {calls} calls replayed; per call = kernel + node gap"})
    out.update({"us_per_call": round(call_us, 3), "cpu_baseline": cpu,
                "roofline": {"kernel": "qgemv_kernel", "bound": "hbm", "achieved": round(value, 1),
                             "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(value / PEAK_HBM_GBPS, 4),
                             "traffic": measured_traffic(cfg.name, "qgemv"),
                             "traffic_algorithmic_bytes": nbytes}})
    print(json.dumps(out), flush=True)


def bench_mx(torch, bdg, synth, sdev, dev, cfg, args):
    """Large-M product on the MX-scaled matrix cores: cfg.m tokens (bf16) are
    quantized to MXFP8, then multiplied by one MXFP4 matrix [n][k].  Both
    kernels are timed from captured graphs of 16 calls each (events around
    the replays); the product is priced against the dense FP8 MFMA peak (the
    FP4 x FP8 instruction issues at the FP8 rate)."""
    import numpy as np

    m = args.m if args.m else cfg.m
    K = args.steps if args.steps is not None else 8
    W = args.warmup if args.warmup is not None else 2
    calls = 16
    arrs = synth.dense_matrix(cfg, 0)
    qw = sdev.qweight_from_arrays(cfg.fmt, arrs, cfg.group, dev)
    if not args.mx_scales_per_call:
        qw.stage_mx_scales()          # weight layout, once per matrix (untimed, like the upload)
    _, xbits = synth.hidden_batch(cfg, range(m))
    x = torch.from_numpy(xbits.view(np.int16)).to(dev).view(torch.bfloat16)
    codes = torch.empty((m, cfg.k), dtype=torch.uint8, device=dev)
    scales = torch.empty((m, cfg.k // 32), dtype=torch.uint8, device=dev)
    y = torch.empty((m, cfg.n), dtype=torch.float32, device=dev)
    ws = torch.empty(bdg.mx_gemm_workspace_bytes(cfg.n, cfg.k, m), dtype=torch.uint8, device=dev)

    def graph_time(fn):
        g = torch.cuda.CUDAGraph()
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            with torch.cuda.graph(g, stream=st):
                for _ in range(calls):
                    fn()
        torch.cuda.current_stream().wait_stream(st)
        for _ in range(W):
            g.replay()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(K):
            g.replay()
        b.record()
        b.synchronize()
        return a.elapsed_time(b) * 1e3 / (K * calls)

    q_us = graph_time(lambda: bdg.mxfp8_quantize(x, codes, scales))
    g_us = graph_time(lambda: bdg.mx_gemm(qw, codes, scales, out=y, workspace=ws))
    if not torch.isfinite(y).all():
        raise SystemExit("non-finite output")
    flops = 2.0 * cfg.n * m * cfg.k
    tflops = flops / (g_us * 1e-6) / 1e12
    q_bytes = m * cfg.k * 2 + m * cfg.k + m * (cfg.k // 32)
    log(f"{cfg.name} m={m}: quantize {q_us:.2f} us ({q_bytes / (q_us * 1e-6) / 1e9:.1f} GB/s), "
        f"gemm {g_us:.2f} us ({tflops:.1f} TFLOP/s)")
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import mxq
        xv = synth.hidden_batch(cfg, range(8))[0]
        t1 = time.perf_counter()
        n = 0
        while time.perf_counter() - t1 < 10.0 or n < 2:
            oc, os_ = mxq.mxfp8_quantize(xv)
            mxq.mx_gemm(*arrs, oc, os_)
            n += 1
        dt = (time.perf_counter() - t1) / n
        cpu = {"value": round(2.0 * cfg.n * 8 * cfg.k / dt / 1e12, 6), "unit": "TFLOP/s", "kind": "oracle",
               "cores": blas_threads(),
               "sample": f"8 of {m} tokens, {n} passes of quantize + dequantize + float64 product"}
    out = {
        "metric": "mx_gemm TFLOP/s (MXFP4 weights x MXFP8 activations)",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": K * calls, "warmup": W * calls,
        "ms_per_step": round(g_us * 1e-3, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp4 x mxfp8 -> f32", "data": "synthetic",
        "config": {"workload": cfg.name, "n": cfg.n, "k": cfg.k, "m": m,
                   "weight_scale_words": "per call" if args.mx_scales_per_call else "staged once",
                   "timing": f"graphs of {calls} calls replayed; per call = kernel + node gap"},
        "quantize_us": round(q_us, 3), "quantize_GBps": round(q_bytes / (q_us * 1e-6) / 1e9, 1),
        "gemm_us": round(g_us, 3),
        "roofline": {"kernel": "mx_gemm_kernel", "bound": "mfma", "achieved": round(tflops, 1),
                     "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s", "frac": round(tflops / PEAK_FP8_TFLOPS, 4),
                     "traffic": measured_traffic(cfg.name, "mx_gemm", MX_SOURCES) if m == cfg.m else None},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def bench_prefill(torch, bdg, synth, sdev, dev, cfg, args):
    """One bare MoE layer over cfg.m tokens at once (prefill): router + top-k,
    MXFP8 quantization, grouped gate_up GEMM with SwiGLU and requantization,
    grouped down GEMM, combine - replayed from a captured graph (the entry
    point takes a preallocated workspace and allocates nothing)."""
    m = args.m if args.m else cfg.m
    K = args.steps if args.steps is not None else 8
    W = args.warmup if args.warmup is not None else 2
    layer = sdev.upload_layer(cfg, 0, dev, threads=16)
    if not args.mx_scales_per_call:   # weight layout, once per matrix (untimed, like the upload)
        layer["gate_up"].stage_mx_scales()
        layer["down"].stage_mx_scales()
    x, _ = sdev.hidden_device(cfg, range(m), dev)
    ws = torch.empty(bdg.prefill_workspace_bytes(m, cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k),
                     dtype=torch.uint8, device=dev)
    y = torch.empty((m, cfg.hidden), dtype=torch.float32, device=dev)
    bdg.moe_prefill_mx(layer, cfg.n_experts, cfg.top_k, x, y=y, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            bdg.moe_prefill_mx(layer, cfg.n_experts, cfg.top_k, x, y=y, workspace=ws)
    torch.cuda.current_stream().wait_stream(st)
    for _ in range(W):
        g.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(K):
        g.replay()
    b.record()
    b.synchronize()
    us = a.elapsed_time(b) * 1e3 / K
    if not torch.isfinite(y).all():
        raise SystemExit("non-finite output")
    flops = 2.0 * m * cfg.top_k * (2 * cfg.inter * cfg.hidden + cfg.hidden * cfg.inter)
    tflops = flops / (us * 1e-6) / 1e12
    log(f"{cfg.name} m={m}: {us:.1f} us per layer, {m / (us * 1e-6):.0f} tokens/s, {tflops:.1f} TFLOP/s")
    out = {
        "metric": "prefill MoE layer tokens/s (grouped MX GEMM)", "value": round(m / (us * 1e-6), 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": round(us * 1e-3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "mxfp4 x mxfp8 -> f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "m": m, "hidden": cfg.hidden, "inter": cfg.inter,
                   "experts": cfg.n_experts, "top_k": cfg.top_k,
                   "weight_scale_words": "per call" if args.mx_scales_per_call else "staged once",
                   "timing": "graph of one layer replayed; events around the replays"},
        "layer_TFLOPs": round(tflops, 1),
        "roofline": {"kernel": "whole layer", "bound": "mfma", "achieved": round(tflops, 1),
                     "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s", "frac": round(tflops / PEAK_FP8_TFLOPS, 4),
                     "traffic": measured_traffic(cfg.name, "mx_gemm", MX_SOURCES) if m == cfg.m else None},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def bench_layer_rotation(torch, bdg, synth, sdev, dev, cfg, args):
    """One bare MoE layer (no norm, no residual) at M=1, rotating over 8
    independently seeded layers (3.4 GB, beyond every cache) with a fresh
    hidden state per token.  A token here is two kernels, too little GPU
    work to hide the host's launch of a graph per token, so the whole
    sequence of tokens is captured into one graph; each token's layer reads
    its hidden state where it lies in HBM (the plans launch directly, so no
    per-call graph is keyed on the input's address)."""
    NL = 8
    K = args.steps if args.steps is not None else 64
    W = args.warmup if args.warmup is not None else 8
    t0 = time.time()
    plans, keep = [], []
    for l in range(NL):
        lay = sdev.upload_layer(cfg, l, dev, threads=16)
        plan, _ = sdev.build_plan(cfg, dev, max_m=1, layers=[lay], use_graph=False)
        plans.append(plan)
        keep.append(lay)
    log(f"uploaded {NL} layers ({time.time() - t0:.1f} s)")
    x_all, _ = sdev.hidden_device(cfg, range(W + K), dev)
    y_buf = torch.empty((1, cfg.hidden), dtype=torch.float32, device=dev)
    def seq(tokens):
        g = torch.cuda.CUDAGraph()
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            with torch.cuda.graph(g, stream=st):
                for t in tokens:
                    bdg.moe_expert_decode(plans[t % NL], x_all[t:t + 1], y=y_buf)
        torch.cuda.current_stream().wait_stream(st)
        return g

    warm = seq(range(W))
    timed_g = seq(range(W, W + K))
    warm.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    timed_g.replay()
    b.record()
    b.synchronize()
    gpu_ms = a.elapsed_time(b)
    if not torch.isfinite(y_buf).all():
        raise SystemExit("non-finite output")
    nbytes = step_bytes(cfg, [cfg.top_k])
    value = nbytes * K / (gpu_ms * 1e-3) / 1e9
    log(f"timed {K} tokens: {gpu_ms / K * 1e3:.2f} us/token, {value:.1f} GB/s")
    if args.graph_only:
        print(json.dumps({"workload": cfg.name, "steps": K, "us_per_token": round(gpu_ms / K * 1e3, 2)}),
              flush=True)
        for pl in plans:
            pl.close()
        return
    acc = None
    for t in range(W, W + K):
        acc = bdg.moe_expert_decode_profiled(plans[t % NL], x_all[t:t + 1], y_buf, acc)
    gu_bytes, dn_bytes = expert_bytes(cfg)
    # a self-routing gate_up launch also reads the layer's router weights
    per_step = {k: acc.count[i] / K for i, k in enumerate(bdg.KERNEL_KINDS)}
    sr = self_routed_launches(cfg, False, per_step["gate_up"], per_step["route"])
    gu_launch = int(round(cfg.top_k * gu_bytes + (sr / per_step["gate_up"]) * router_bytes(cfg)))
    kernels, gap_us, _ = kernel_figures(bdg, acc, {"gate_up": gu_launch, "down": cfg.top_k * dn_bytes,
                                                   "route": router_bytes(cfg)}, gpu_ms / K * 1e3, K)
    achieved = kernels["gate_up"]["GBps"]
    log(f"per-kernel: {kernels}")
    cpu = None if args.no_cpu_baseline else cpu_baseline(cfg, 1, 1)
    out = base_record(cfg, value, K, W, gpu_ms / K, {
        "workload": cfg.name, "fmt": cfg.fmt, "layers_rotated": NL, "hidden": cfg.hidden,
        "inter": cfg.inter, "experts": cfg.n_experts, "top_k": cfg.top_k, "m": 1, "bytes_per_step": nbytes,
        "timing": "all timed tokens in one captured graph, stream-ordered"})
    out.update({"us_per_token": round(gpu_ms / K * 1e3, 2), "kernels": kernels, "cpu_baseline": cpu,
                "roofline": {"kernel": "moe_gateup_kernel", "bound": "hbm", "achieved": round(achieved, 1),
                             "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                             "traffic": measured_traffic(cfg.name, "gate_up"), "traffic_algorithmic_bytes": gu_launch,
                             "duration_us": kernels["gate_up"]["share_us"], "gap_share_us": round(gap_us, 3),
                             "duration": SHARE_NOTE,
                             "achieved_kernel_only": kernels["gate_up"]["GBps_kernel_only"]}})
    print(json.dumps(out), flush=True)
    for pl in plans:
        pl.close()


def attn_layer_keys(cfg, layer):
    return min(cfg.window, cfg.ctx) if cfg.sliding(layer) else cfg.ctx


def attn_layer_bytes(cfg, layer):
    """KV-cache bytes one decode token reads in a layer: n_kv_heads x keys x
    head_dim x 2 (keys and values) x element size."""
    es = 2 if cfg.cache_dtype == "bf16" else 4
    return cfg.n_kv_heads * attn_layer_keys(cfg, layer) * cfg.head_dim * 2 * es


def attn_traffic(workload):
    """HBM bytes of one full-attention call (split + merge kernels) from the
    committed counter summary, or None."""
    parts = [measured_traffic(workload, k, ATTN_SOURCES) for k in ("attn_split", "attn_merge")]
    return None if None in parts else sum(parts)


def bench_attn(torch, bdg, synth, dev, cfg, args):
    """Decode attention of a gpt-oss-shape stack: per layer one attn_decode
    launch (rotation, cache append, sink + window attention, split merge) at a
    context of cfg.ctx keys (even layers: the 128-key window).  One captured
    graph per token replays all layers; the rate is KV-cache bytes read per
    token over GPU time.  The roofline figure times the full-attention
    launches alone in a graph (per launch = kernel + node gap)."""
    import numpy as np

    K = args.steps if args.steps is not None else 64
    W = args.warmup if args.warmup is not None else 8
    L, m = cfg.n_layers, cfg.m
    pos0, cap = cfg.ctx - m, cfg.ctx
    t0 = time.time()
    caches, sinks = [], []
    for l in range(L):
        kv, vv, kb, vb = synth.attn_cache(cfg, l, pos0, cap)
        if cfg.cache_dtype == "bf16":
            kc = torch.from_numpy(kb.view(np.int16)).to(dev).view(torch.bfloat16)
            vc = torch.from_numpy(vb.view(np.int16)).to(dev).view(torch.bfloat16)
        else:
            kc, vc = torch.from_numpy(kv).to(dev), torch.from_numpy(vv).to(dev)
        caches.append((kc, vc))
        sinks.append(torch.from_numpy(synth.attn_sinks(cfg, l)).to(dev))
    table, _, _ = bdg.attn_rope_table(cfg.rope, cfg.head_dim, cap, device=dev)
    ws = bdg.attn_workspace(cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, m, cfg.ctx, dev)
    n_sets = 8                                   # distinct token inputs, used in turn
    inputs = [[tuple(torch.from_numpy(a).to(dev) for a in synth.attn_token(cfg, l, s)) for l in range(L)]
              for s in range(n_sets)]
    outs = [torch.empty((m, cfg.n_heads, cfg.head_dim), dtype=torch.float32, device=dev) for _ in range(L)]
    log(f"uploaded {L} layers of KV cache ({time.time() - t0:.1f} s)")

    def layer_call(s, l):
        q, k, v = inputs[s][l]
        window = cfg.window if cfg.sliding(l) else 0
        bdg.attn_decode(q, k, v, caches[l][0], caches[l][1], pos0, table, cfg.sm_scale, sinks[l], window,
                        o=outs[l], workspace=ws)

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            with torch.cuda.graph(g, stream=st):
                fn()
        torch.cuda.current_stream().wait_stream(st)
        return g

    graphs = [capture(lambda s=s: [layer_call(s, l) for l in range(L)]) for s in range(n_sets)]
    for i in range(W):
        graphs[i % n_sets].replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(K):
        graphs[i % n_sets].replay()
    b.record()
    b.synchronize()
    us_tok = a.elapsed_time(b) * 1e3 / K
    nbytes = sum(attn_layer_bytes(cfg, l) for l in range(L))
    value = nbytes / (us_tok * 1e-6) / 1e9
    for o in outs:
        if not torch.isfinite(o).all():
            raise SystemExit("non-finite attention output")
    log(f"{cfg.name}: {us_tok:.2f} us/token, {value:.1f} GB/s of KV cache")

    # dominant kernel: the full-attention launches, alone in a graph
    full = [l for l in range(L) if not cfg.sliding(l)]
    reps = 4
    gf = capture(lambda: [layer_call(0, l) for _ in range(reps) for l in full])
    gf.replay()
    torch.cuda.synchronize()
    a.record()
    for _ in range(4):
        gf.replay()
    b.record()
    b.synchronize()
    launch_us = a.elapsed_time(b) * 1e3 / (4 * reps * len(full))
    fbytes = attn_layer_bytes(cfg, full[0])
    achieved = fbytes / (launch_us * 1e-6) / 1e9
    slide = [l for l in range(L) if cfg.sliding(l)]
    gs = capture(lambda: [layer_call(0, l) for _ in range(reps) for l in slide])
    gs.replay()
    torch.cuda.synchronize()
    a.record()
    for _ in range(4):
        gs.replay()
    b.record()
    b.synchronize()
    slide_us = a.elapsed_time(b) * 1e3 / (4 * reps * max(1, len(slide)))
    log(f"full-attention launch {launch_us:.2f} us ({achieved:.1f} GB/s), sliding launch {slide_us:.2f} us")

    cpu = None
    if not args.no_cpu_baseline:
        # the oracle on one full-attention layer of one token, repeated for >= 10 s
        from oracle import attn as oattn
        l = full[0]
        kv, vv, _, _ = synth.attn_cache(cfg, l, pos0, cap)
        kv64, vv64 = np.nan_to_num(kv.astype(np.float64)), np.nan_to_num(vv.astype(np.float64))
        inv32, a32 = oattn.rope_constants(cfg.head_dim, **{k_: cfg.rope[k_] for k_ in (
            "theta", "factor", "orig_ctx", "beta_fast", "beta_slow", "truncate")})
        sk = synth.attn_sinks(cfg, l)
        t1 = time.perf_counter()
        n = 0
        while time.perf_counter() - t1 < 10.0 or n < 2:
            q, k, v = synth.attn_token(cfg, l, n)
            oattn.decode_step(q, k, v, kv64, vv64, cfg.cache_dtype, pos0, inv32, a32, 0, cfg.sm_scale, sk)
            n += 1
        dt = (time.perf_counter() - t1) / n
        cpu = {"value": round(fbytes / dt / 1e9, 4), "unit": "GB/s", "kind": "oracle",
               "cores": blas_threads(),
               "us_per_token": round(dt * 1e6 * nbytes / fbytes, 1),
               "sample": f"one full-attention layer (ctx {cfg.ctx}) of one token, {n} passes of the float64 "
                         f"oracle step (rotation, cache store, 64 heads of attention), per-byte rate"}
    out = base_record(cfg, value, K, W, us_tok * 1e-3, {
        "workload": cfg.name, "layers": L, "heads": cfg.n_heads, "kv_heads": cfg.n_kv_heads,
        "head_dim": cfg.head_dim, "ctx": cfg.ctx, "window": cfg.window, "m": m,
        "cache_dtype": cfg.cache_dtype, "kv_bytes_per_token": nbytes,
        "timing": "one graph per token (all layers), replayed back to back"})
    out.update({"metric": "decode-attention KV-cache HBM GB/s + us/token, gpt-oss-20B shape",
                "us_per_token": round(us_tok, 2),
                "sliding_launch_us": round(slide_us, 3),
                "cpu_baseline": cpu,
                "roofline": {"kernel": "attn_decode on a full-attention layer: attn_split_kernel + "
                                       "attn_merge_kernel", "bound": "hbm",
                             "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                             "frac": round(achieved / PEAK_HBM_GBPS, 4),
                             "launch_us": round(launch_us, 3),
                             "traffic": attn_traffic(cfg.name),
                             "traffic_algorithmic_bytes": fbytes}})
    print(json.dumps(out), flush=True)


def bench_timeline(bdg, plan, cfg, x_all, x_buf, y_buf, W, K):
    """Where a fused layer kernel's time goes: per-block 100 MHz clock stamps
    at its phase boundaries (moe_expert_decode_timeline, direct launches).
    Per phase, the median and the latest block's time after the kernel's
    first block started, over the timed tokens and layers 1..L-1, and the
    gap from a layer's last block to the next layer's first."""
    import numpy as np
    names = bdg.api.LAYER_STAMPS
    rows, gaps = [], []
    for s in range(W, W + K):
        x_buf.copy_(x_all[s])
        st = bdg.moe_expert_decode_timeline(plan, x_buf, y_buf).astype(np.int64)   # [L][blocks][16]
        for l in range(1, st.shape[0]):
            blk = st[l][:, :len(names)]
            t0 = blk[:, 0][blk[:, 0] > 0].min()
            rec = {}
            for i, nm in enumerate(names):
                v = blk[:, i][blk[:, i] > 0]
                if v.size:
                    rec[nm] = ((np.median(v) - t0) * 0.01, (v.max() - t0) * 0.01)
            rows.append(rec)
            if l + 1 < st.shape[0]:
                nxt = st[l + 1][:, 0]
                end = blk[:, names.index("end")]
                gaps.append((nxt[nxt > 0].min() - max(end.max(), blk[:, names.index("barrier")].max())) * 0.01)
    out = {}
    for nm in names:
        vals = [r[nm] for r in rows if nm in r]
        if vals:
            out[nm] = {"median_block_us": round(float(np.mean([v[0] for v in vals])), 2),
                       "last_block_us": round(float(np.mean([v[1] for v in vals])), 2)}
    res = {"workload": cfg.name, "kernel": "moe_layer_kernel", "tokens": K, "layers_averaged": cfg.n_layers - 1,
           "clock": "s_memrealtime, 100 MHz", "phases_after_first_block_start": out,
           "gap_to_next_layer_us": round(float(np.mean(gaps)), 2) if gaps else None}
    log(f"timeline: {res}")
    print(json.dumps(res), flush=True)
    plan.close()


def routing_stats(bdg, np, synth, plan, cfg, m, x_all, x_buf, y_buf, W, K):
    """Unique (layer, expert) matrices per step of the K steps after W: M=1
    reads k experts per layer; for M > 1 the steps are replayed untimed with
    routing traces.  Returns (uniq [K][L], routing summary or None)."""
    routing = None
    if m == 1:
        return [[cfg.top_k] * cfg.n_layers for _ in range(K)], None
    uniq, hot_frac, tpe = [], [], []
    hot_sets = [synth.router(cfg, l)[2] for l in range(cfg.n_layers)]
    for s in range(W, W + K):
        x_buf.copy_(x_all[s])
        _, tr = bdg.moe_expert_decode(plan, x_buf, y=y_buf, traces=True)
        topk = tr["topk"].cpu().numpy()                       # [L][m][k]
        uniq.append([len(set(topk[l].ravel().tolist())) for l in range(cfg.n_layers)])
        if hot_sets[0] is not None:
            hot_frac.append([float(np.isin(topk[l], hot_sets[l]).mean()) for l in range(cfg.n_layers)])
        for l in range(cfg.n_layers):
            tpe.extend(np.bincount(topk[l].ravel(), minlength=cfg.n_experts)[
                np.unique(topk[l].ravel())].tolist())
    hist = np.bincount(np.array(tpe), minlength=m + 1)[1:].tolist()
    routing = {
        "unique_experts_per_layer_mean": round(float(np.mean(uniq)), 3),
        "picks_per_layer": m * cfg.top_k,
        "tokens_per_active_expert_hist": {str(i + 1): c for i, c in enumerate(hist) if c},
    }
    if hot_frac:
        routing["hot_pick_fraction_per_layer"] = [round(v, 3) for v in np.mean(hot_frac, axis=0)]
        routing["hot_pick_fraction_mean"] = round(float(np.mean(hot_frac)), 3)
    return uniq, routing


def kernel_figures(bdg, acc, launch_bytes, replay_us_per_step, steps):
    """Per-kind figures of a KernelTimes over `steps` steps: avg_us (the
    dispatch's own start-to-end time), share_us = avg_us plus an equal share
    of the replayed step's launch gaps ((replayed step time - the step's
    dispatch times) / launches per step: in a graph replay each launch
    waits one gap behind the previous kernel, and a kernel trace of the
    replay starts each launch at the previous kernel's end), launches, and
    for kinds with algorithmic bytes per launch GBps = bytes / share_us (the
    roofline figure) and GBps_kernel_only = bytes / avg_us."""
    kinds = range(len(bdg.KERNEL_KINDS))
    launches = sum(acc.count[i] for i in kinds) / steps
    dispatch_us = sum(acc.ms[i] for i in kinds) / steps * 1e3
    gap_us = max(0.0, (replay_us_per_step - dispatch_us) / launches) if launches else 0.0
    kernels = {}
    for i, name in enumerate(bdg.KERNEL_KINDS):
        if acc.count[i]:
            avg = acc.ms[i] / acc.count[i] * 1e3
            k = {"avg_us": round(avg, 3), "share_us": round(avg + gap_us, 3), "launches": int(acc.count[i])}
            if name in launch_bytes:
                k["GBps"] = round(launch_bytes[name] / ((avg + gap_us) * 1e-6) / 1e9, 1)
                k["GBps_kernel_only"] = round(launch_bytes[name] / (avg * 1e-6) / 1e9, 1)
            kernels[name] = k
    return kernels, gap_us, dispatch_us


def self_routed_launches(cfg, route_every_layer, gate_up_per_step, route_per_step):
    """gate_up launches per step that compute their layer's router inside the
    launch (and read its router weights): the layers that need a router of
    their own - the first, and every later one unless a down kernel hands it
    router sums (a stack of <= 64 experts) - less the route kernels launched."""
    down_routes = cfg.norm and cfg.n_layers > 1 and cfg.n_experts <= 64 and not route_every_layer
    own = min(1.0, gate_up_per_step) if down_routes else gate_up_per_step
    return max(0.0, own - route_per_step)


def kernel_pass(bdg, plan, cfg, x_all, x_buf, y_buf, W, K, mean_uniq, replay_us_per_step, route_every_layer=False):
    """Per-kernel figures over the K steps after W: the same kernels and
    grids launched directly, each dispatch with start/stop events (see
    kernel_figures; replay_us_per_step is the graph replay's step time, or
    None for no gap share).  Returns (per-kind figures, dominant kernel
    name, its algorithmic bytes per launch, its GB/s, gap share us,
    dispatch us per step, fused-layer flag)."""
    gu_bytes, dn_bytes = expert_bytes(cfg)
    acc = None
    for s in range(W, W + K):
        x_buf.copy_(x_all[s])
        acc = bdg.moe_expert_decode_profiled(plan, x_buf, y_buf, acc)
    # a self-routing gate_up launch also reads its layer's router weights
    per_step = {k: acc.count[i] / K for i, k in enumerate(bdg.KERNEL_KINDS)}
    sr = self_routed_launches(cfg, route_every_layer, per_step["gate_up"], per_step["route"])
    sr_share = sr / per_step["gate_up"] if per_step["gate_up"] else 0.0
    gu_launch_bytes = int(round(mean_uniq * gu_bytes + sr_share * router_bytes(cfg)))
    layer_launch_bytes = int(round(mean_uniq * (gu_bytes + dn_bytes)))
    dispatch_only = sum(acc.ms[i] for i in range(len(bdg.KERNEL_KINDS))) / K * 1e3
    kernels, gap_us, dispatch_us = kernel_figures(
        bdg, acc, {"gate_up": gu_launch_bytes, "down": int(round(mean_uniq * dn_bytes)),
                   "route": router_bytes(cfg), "layer": layer_launch_bytes},
        replay_us_per_step if replay_us_per_step else dispatch_only, K)
    fused = "layer" in kernels
    if fused:
        # the fused per-layer kernel: the chosen experts' gate_up and down bytes per launch
        dom_kernel, dom_kind, dom_bytes = "moe_layer_kernel", "layer", layer_launch_bytes
    else:
        dom_kernel, dom_kind, dom_bytes = "moe_gateup_kernel", "gate_up", gu_launch_bytes
    achieved = kernels[dom_kind]["GBps"]
    return kernels, dom_kernel, dom_bytes, achieved, gap_us, dispatch_us, fused


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default 64 at M=1, 16 at M>1)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps (default 8 at M=1, 4 at M>1)")
    ap.add_argument("--workload", default="gptoss20b_stack")
    ap.add_argument("--m", type=int, default=0, help="tokens per step (default: the workload's own)")
    ap.add_argument("--mx-scales-per-call", action="store_true",
                    help="MX workloads: let each call stage the weights' scale words (default: staged once)")
    ap.add_argument("--cpu-sample-layers", type=int, default=1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stream-read", action="store_true")
    ap.add_argument("--mfma", action="store_true",
                    help="steps of M > 1: the grouped expert products on the matrix cores (BDG_MOE_MFMA) "
                         "instead of the VALU kernels (A/B)")
    ap.add_argument("--fused-layer", action="store_true",
                    help="one-token steps run each layer as the fused per-layer kernel instead of two "
                         "kernels (gate_up, down): the A/B of the fused design")
    ap.add_argument("--route-every-layer", action="store_true",
                    help="stacks: a route kernel before every layer instead of the router partial sums "
                         "from the previous down kernel (BDG_MOE_ROUTE_EVERY_LAYER): the A/B of fused routing")
    ap.add_argument("--route-kernel", action="store_true",
                    help="layers after the first that need their own router launch the route kernel "
                         "instead of routing inside their gate_up launch (BDG_MOE_ROUTE_KERNEL): the "
                         "A/B of self-routing")
    ap.add_argument("--timeline", action="store_true",
                    help="one-token stacks: phase timeline of the fused per-layer kernel (per-block clock "
                         "stamps of moe_expert_decode_timeline), summarized per phase, then exit")
    ap.add_argument("--graph-only", action="store_true",
                    help="only the warmup and the timed graph replays (no per-step events, sync mode, "
                         "per-kernel event pass, stream read or CPU baseline): the run a kernel trace "
                         "of graph replays alone is taken from")
    ap.add_argument("--kernel-pass-only", action="store_true",
                    help="only the per-kernel pass: every step launched directly (no graph), each kernel "
                         "timed by its dispatch's start/stop events; prints the per-kernel figures.  A "
                         "kernel trace of this command holds exactly the dispatches the events time")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run the 16-byte copy kernel 4 times over BYTES (for scaling "
                         "HBM counters against a kernel of known traffic), then exit")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the expert decode runs on one MI355X; see the sharding notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import bit_dequant_gemv_amd as bdg
    import synth
    from synth import device as sdev

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        nb = args.copy_calibration // 256 * 256
        src = torch.ones(nb, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(4):
            bdg.stream_copy(src, dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": nb, "launches": 4}), flush=True)
        return
    if args.workload in synth.ATTN:
        return bench_attn(torch, bdg, synth, dev, synth.ATTN[args.workload], args)
    if args.workload in synth.PREFILL:
        return bench_prefill(torch, bdg, synth, sdev, dev, synth.PREFILL[args.workload], args)
    if args.workload in synth.DENSE and synth.DENSE[args.workload].m > 1:
        return bench_mx(torch, bdg, synth, sdev, dev, synth.DENSE[args.workload], args)
    if args.workload in synth.DENSE:
        return bench_dense(torch, bdg, synth, sdev, dev, synth.DENSE[args.workload], args)
    cfg = synth.CONFIGS[args.workload]
    if cfg.name == "gemv_2880":
        return bench_gemv(torch, bdg, synth, sdev, dev, cfg, args)
    if cfg.name == "gptoss20b_layer":
        return bench_layer_rotation(torch, bdg, synth, sdev, dev, cfg, args)
    m = args.m if args.m else cfg.m
    if not 1 <= m <= 16:
        raise SystemExit("--m must be in 1..16")
    K = args.steps if args.steps is not None else (64 if m == 1 else 16)
    W = args.warmup if args.warmup is not None else (8 if m == 1 else 4)

    t0 = time.time()
    layers = []
    for l in range(cfg.n_layers):
        layers.append(sdev.upload_layer(cfg, l, dev, threads=16))
        if l % 6 == 5 or l == cfg.n_layers - 1:
            log(f"uploaded {l + 1}/{cfg.n_layers} layers ({time.time() - t0:.1f} s)")
    plan, _ = sdev.build_plan(cfg, dev, max_m=m, layers=layers, fused_layer=args.fused_layer or args.timeline,
                              mfma=args.mfma, route_every_layer=args.route_every_layer,
                              route_kernel=args.route_kernel, use_graph=not args.kernel_pass_only)
    x_all, _ = sdev.hidden_device(cfg, range((W + K) * m), dev)
    x_all = x_all.reshape(W + K, m, cfg.hidden)
    x_buf = torch.empty_like(x_all[0])
    y_buf = torch.empty((m, cfg.hidden), dtype=torch.float32, device=dev)

    for s in range(W):
        x_buf.copy_(x_all[s])
        bdg.moe_expert_decode(plan, x_buf, y=y_buf)
    torch.cuda.synchronize()
    log(f"warmup done ({W} steps of M={m})")
    if args.timeline:
        return bench_timeline(bdg, plan, cfg, x_all, x_buf, y_buf, W, K)
    if args.kernel_pass_only:
        uniq, _ = routing_stats(bdg, np, synth, plan, cfg, m, x_all, x_buf, y_buf, W, K)
        kernels, dom_kernel, dom_bytes, achieved, _, dispatch_us, _ = kernel_pass(
            bdg, plan, cfg, x_all, x_buf, y_buf, W, K, float(np.mean(uniq)), None, args.route_every_layer)
        if not torch.isfinite(y_buf).all() or not plan.check():
            raise SystemExit("non-finite output or a failed in-kernel wait")
        log(f"kernel pass ({K} steps of M={m}, direct launches): {kernels}")
        print(json.dumps({"workload": cfg.name, "m": m, "steps": K, "kernels": kernels,
                          "roofline_kernel": dom_kernel, "algorithmic_bytes_per_launch": dom_bytes,
                          "achieved_GBps": achieved, "dispatch_us_per_step": round(dispatch_us, 2)}), flush=True)
        plan.close()
        return

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for s in range(W, W + K):
        x_buf.copy_(x_all[s])                  # the next step's hidden states land in the input buffer
        bdg.moe_expert_decode(plan, x_buf, y=y_buf)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    gpu_ms = start.elapsed_time(end)
    if not torch.isfinite(y_buf).all() or not plan.check():
        raise SystemExit("non-finite output or a failed in-kernel wait")
    if args.graph_only:
        log(f"graph-only run: {K} steps of M={m}, {gpu_ms / K * 1e3:.1f} us/step")
        print(json.dumps({"workload": cfg.name, "m": m, "steps": K, "us_per_step": round(gpu_ms / K * 1e3, 2),
                          "fused_layer": bool(args.fused_layer), "route_kernel": bool(args.route_kernel)}),
              flush=True)
        plan.close()
        return

    gu_bytes, dn_bytes = expert_bytes(cfg)
    uniq, routing = routing_stats(bdg, np, synth, plan, cfg, m, x_all, x_buf, y_buf, W, K)
    nbytes = sum(step_bytes(cfg, u) for u in uniq)
    value = nbytes / (gpu_ms * 1e-3) / 1e9
    mean_uniq = float(np.mean(uniq))
    log(f"timed {K} steps of M={m}: {gpu_ms / K * 1e3:.1f} us/step GPU, {gpu_ms / K / m * 1e3:.1f} us/token, "
        f"{wall / K * 1e6:.1f} us/step wall, {value:.1f} GB/s (unique experts/layer {mean_uniq:.2f})")

    # per-step distribution: an event pair around each replay (stream mode), and
    # sync mode: a host sync after every step, as when the host picks the next
    # token; both on the same steps, after the timed run
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for i, s in enumerate(range(W, W + K)):
        x_buf.copy_(x_all[s])
        ev[i][0].record()
        bdg.moe_expert_decode(plan, x_buf, y=y_buf)
        ev[i][1].record()
    torch.cuda.synchronize()
    step_us = [a.elapsed_time(b) * 1e3 for a, b in ev]
    sync_us = []
    for s in range(W, W + K):
        t1 = time.perf_counter()
        x_buf.copy_(x_all[s])
        bdg.moe_expert_decode(plan, x_buf, y=y_buf)
        torch.cuda.synchronize()
        sync_us.append((time.perf_counter() - t1) * 1e6)
    per_step = {"median_us": round(statistics.median(step_us), 2), "mean_us": round(statistics.mean(step_us), 2),
                "min_us": round(min(step_us), 2), "max_us": round(max(step_us), 2)}
    sync_mode = {"median_us": round(statistics.median(sync_us), 2), "mean_us": round(statistics.mean(sync_us), 2)}
    log(f"per step (events around each replay): {per_step}; sync mode wall per step: {sync_mode}")

    kernels, dom_kernel, dom_bytes, achieved, gap_us, dispatch_us, fused = kernel_pass(
        bdg, plan, cfg, x_all, x_buf, y_buf, W, K, mean_uniq, gpu_ms / K * 1e3, args.route_every_layer)
    gu_launch_bytes = int(round(mean_uniq * gu_bytes))
    layer_launch_bytes = int(round(mean_uniq * (gu_bytes + dn_bytes)))
    log(f"per-kernel: {kernels}; dispatch time {dispatch_us:.1f} us/step of {gpu_ms / K * 1e3:.1f} replayed "
        f"(gap share {gap_us:.2f} us per launch)")

    stream = None
    if not args.no_stream_read:
        best, med, phases = stream_read_rate(
            torch, bdg, dev, {"gate_up": gu_launch_bytes, "down": int(round(mean_uniq * dn_bytes)),
                              "layer": layer_launch_bytes, "router": router_bytes(cfg)})
        stream = {"best_GBps": round(best, 1), "median_GBps": round(med, 1), "bytes": "4 GiB",
                  "phase_sized_reads": phases}
        log(f"stream read: best {best:.1f} GB/s, median {med:.1f} GB/s; phase-sized: {phases}")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, args.cpu_sample_layers, m)
        log(f"cpu baseline: {cpu}")

    config = {
        "workload": cfg.name,
        "fmt": cfg.fmt, "layers": cfg.n_layers, "hidden": cfg.hidden, "inter": cfg.inter,
        "experts": cfg.n_experts, "top_k": cfg.top_k, "m": m,
        "bytes_per_step": int(round(nbytes / K)),
        "timing": "HIP graph per step (M tokens), stream-ordered",
        "layer_kernels": ("fused per-layer kernel" if fused else
                          "grouped gate_up and down on the matrix cores" if (m > 1 and args.mfma) else
                          "two kernels per layer (gate_up, down)"),
    }
    if routing:
        config["routing"] = routing
    if args.route_every_layer:
        config["router"] = "route kernel before every layer"
    if args.route_kernel:
        config["router"] = "route kernel before every layer that needs its own router"
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(gpu_ms / K, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": config,
        "pct_of_peak": round(100.0 * value / PEAK_HBM_GBPS, 2),
        "us_per_token": round(gpu_ms / K / m * 1e3, 2),
        "wall_us_per_token": round(wall / K / m * 1e6, 2),
        "per_step_gpu": per_step,
        "sync_mode_wall_per_step": sync_mode,
        "pct_of_stream_read": round(100.0 * value / stream["best_GBps"], 2) if stream else None,
        "roofline": {
            "kernel": dom_kernel,
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4),
            "traffic": (measured_traffic(cfg.name + ("_mfma" if args.mfma and m > 1 else ""),
                                         "layer" if fused else "gate_up") if m == cfg.m else None),
            "traffic_algorithmic_bytes": dom_bytes,
            "duration_us": kernels["layer" if fused else "gate_up"]["share_us"],
            "gap_share_us": round(gap_us, 3),
            "duration": SHARE_NOTE,
            "achieved_kernel_only": kernels["layer" if fused else "gate_up"]["GBps_kernel_only"],
        },
        "kernels": kernels,
        "kernel_us_per_step": round(dispatch_us, 2),
        "stream_read": stream,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    plan.close()


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "summarize":
        summarize(sys.argv[2:])
    else:
        main()
