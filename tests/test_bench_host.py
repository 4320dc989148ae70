"""Host logic of bench.py's measurement figures (no GPU): the per-kernel
duration with its share of the replayed step's launch gaps, and the
rocprofv3 summarizers (kernel trace, copy-calibrated HBM traffic, merged SQ
counter passes) on small synthetic CSV files."""

import csv
import json
import os
import types

import pytest

import bench


def _fake_bdg():
    return types.SimpleNamespace(KERNEL_KINDS=("route", "gate_up", "down", "combine", "layer"))


def _acc(ms, count):
    return types.SimpleNamespace(ms=list(ms), count=list(count))


def test_kernel_figures_gap_share():
    bdg = _fake_bdg()
    # 2 steps; per step one route (4 us) and 24 gate_up (11 us) + 24 down (8 us) dispatches
    steps = 2
    acc = _acc([steps * 4e-3, steps * 24 * 11e-3, steps * 24 * 8e-3, 0.0, 0.0],
               [steps, steps * 24, steps * 24, 0, 0])
    dispatch = 4.0 + 24 * 11.0 + 24 * 8.0
    replay = dispatch + 49 * 1.5            # a 1.5 us gap in front of each of the 49 launches
    kernels, gap, disp = bench.kernel_figures(bdg, acc, {"gate_up": 35_251_200}, replay, steps)
    assert disp == pytest.approx(dispatch)
    assert gap == pytest.approx(1.5)
    g = kernels["gate_up"]
    assert g["avg_us"] == pytest.approx(11.0)
    assert g["share_us"] == pytest.approx(12.5)
    assert g["launches"] == steps * 24
    assert g["GBps"] == pytest.approx(35_251_200 / 12.5e-6 / 1e9, rel=1e-3)
    assert g["GBps_kernel_only"] == pytest.approx(35_251_200 / 11.0e-6 / 1e9, rel=1e-3)
    assert "GBps" not in kernels["down"]          # no bytes given for it
    assert "combine" not in kernels               # never launched


def test_kernel_figures_no_negative_gap():
    """Directly launched dispatches can sum above the replayed step: no gap
    is shared then (never a negative one)."""
    bdg = _fake_bdg()
    acc = _acc([0.0, 10e-3, 0.0, 0.0, 0.0], [0, 1, 0, 0, 0])
    kernels, gap, _ = bench.kernel_figures(bdg, acc, {"gate_up": 1_000_000}, 8.0, 1)
    assert gap == 0.0
    assert kernels["gate_up"]["share_us"] == pytest.approx(10.0)


def _write_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0].keys()))
        w.writeheader()
        w.writerows(rows)


def test_summarize_trace_splits_back_to_back(tmp_path):
    src = tmp_path / "trace"
    gu = "void bdg::moe_gateup_kernel<0, 3, 6, 1>(bdg::GateUpParams)"
    dn = "void bdg::moe_down_kernel<0, 32, 3, 3, 6, 8>(bdg::DownParams)"
    # a replay: gu 0-12, dn 12-20, gu 20-32 (back to back); then direct launches with gaps
    disp = [(gu, 0, 12_000), (dn, 12_000, 20_000), (gu, 20_000, 32_000),
            (gu, 40_000, 51_000), (dn, 60_000, 67_000)]
    _write_csv(str(src / "c_kernel_trace.csv"),
               [{"Queue_Id": "1", "Kernel_Name": k, "Start_Timestamp": a, "End_Timestamp": b} for k, a, b in disp])
    stats = []
    for name in (gu, dn):
        d = [b - a for k, a, b in disp if k == name]
        stats.append({"Name": name, "Calls": len(d), "TotalDurationNs": sum(d), "AverageNs": sum(d) / len(d),
                      "MinNs": min(d), "MaxNs": max(d)})
    _write_csv(str(src / "c_kernel_stats.csv"), stats)
    bench.summarize(["trace", "--workload", "t", "--src", str(src), "--command", "cmd", "--out-dir", str(tmp_path)])
    text = (tmp_path / "kernel_trace_t.md").read_text()
    gu_line = next(l for l in text.splitlines() if "moe_gateup_kernel" in l)
    cells = [c.strip() for c in gu_line.strip("|").split("|")]
    assert cells[1] == "3"
    assert cells[6] == "12.00 (1)"            # the first gate_up starts the queue: not back to back
    assert cells[7] == "11.50 (2)"            # 0-12 and 40-51 (after a gap)
    dn_line = next(l for l in text.splitlines() if "moe_down_kernel" in l)
    dcells = [c.strip() for c in dn_line.strip("|").split("|")]
    assert dcells[6] == "8.00 (1)" and dcells[7] == "7.00 (1)"


def _counter_dir(path, rows):
    _write_csv(str(path / "c_counter_collection.csv"),
               [{"Kernel_Name": k, "Counter_Name": c, "Counter_Value": v} for k, c, v in rows])


def test_summarize_traffic_calibration(tmp_path):
    copy = "bdg::stream_copy_kernel(uint4 const*, uint4*, long)"
    gu = "void bdg::moe_gateup_kernel<0, 3, 6, 1>(bdg::GateUpParams)"
    cal_bytes = 1 << 20                                   # 1024 KiB read and written
    _counter_dir(tmp_path / "calf", [(copy, "FETCH_SIZE", 512.0)] * 2)    # reads half: scale x2
    _counter_dir(tmp_path / "calw", [(copy, "WRITE_SIZE", 1024.0)] * 2)   # scale x1
    _counter_dir(tmp_path / "f", [(gu, "FETCH_SIZE", 100.0), (gu, "FETCH_SIZE", 102.0)])
    _counter_dir(tmp_path / "w", [(gu, "WRITE_SIZE", 4.0), (gu, "WRITE_SIZE", 4.0)])
    bench.summarize(["traffic", "--workload", "t", "--fetch", str(tmp_path / "f"), "--write", str(tmp_path / "w"),
                     "--cal-fetch", str(tmp_path / "calf"), "--cal-write", str(tmp_path / "calw"),
                     "--cal-bytes", str(cal_bytes), "--out-dir", str(tmp_path)])
    rec = json.load(open(tmp_path / "hbm_traffic_t.json"))
    assert rec["fetch_scale"] == pytest.approx(2.0)
    assert rec["write_scale"] == pytest.approx(1.0)
    assert rec["per_launch"]["gate_up"]["fetch_bytes"] == round(101.0 * 2.0 * 1024)
    assert rec["per_launch"]["gate_up"]["write_bytes"] == round(4.0 * 1024)
    assert rec["kernel_sources_sha"] == bench.kernel_sources_sha()


def test_summarize_sq_merges_passes(tmp_path):
    gu = "void bdg::moe_gu_mfma_kernel<2>(bdg::MfmaParams)"
    _counter_dir(tmp_path / "a", [(gu, "SQ_WAVES", 100.0), (gu, "SQ_WAVE_CYCLES", 1000.0),
                                  (gu, "SQ_ACTIVE_INST_VALU", 250.0), (gu, "SQ_WAIT_ANY", 300.0),
                                  (gu, "SQ_WAIT_INST_ANY", 100.0), (gu, "SQ_INSTS_VALU", 5000.0),
                                  (gu, "SQ_INSTS_VMEM_RD", 400.0), (gu, "GRBM_GUI_ACTIVE", 2000.0)])
    _counter_dir(tmp_path / "b", [(gu, "SQ_WAVES", 100.0), (gu, "SQ_INSTS_MFMA", 800.0),
                                  (gu, "SQ_VALU_MFMA_BUSY_CYCLES", 3.0e6), (gu, "TA_BUSY_avr", 500.0),
                                  (gu, "GRBM_GUI_ACTIVE", 2000.0)])
    bench.summarize(["sq", "--workload", "t", "--src", str(tmp_path / "a"), "--src", str(tmp_path / "b"),
                     "--out-dir", str(tmp_path)])
    text = (tmp_path / "sq_counters_t.md").read_text()
    header = next(l for l in text.splitlines() if l.startswith("| kernel"))
    row = next(l for l in text.splitlines() if "moe_gu_mfma_kernel" in l)
    cols = [c.strip() for c in header.strip("|").split("|")]
    vals = dict(zip(cols, [c.strip() for c in row.strip("|").split("|")]))
    assert vals["waves / dispatch"] == "100"
    assert vals["VALU instr / wave"] == "50"
    assert vals["MFMA instr / wave"] == "8"
    assert vals["VALU active / wave-cycles"] == "0.25"
    assert vals["waiting (any) / wave-cycles"] == "0.30"
    assert vals["MFMA busy, M SIMD-cycles / dispatch"] == "3.00"
    assert vals["TA busy / GUI-active cycles (mean TA)"] == "0.25"


def test_kernel_kinds_of_rocprof_names():
    """Trace and counter names map to the per-launch traffic keys the bench
    reads: the attention split kernel's one-block form (merging in place) is
    a kind of its own, and both gate_up instances (self-routing or not) are
    gate_up."""
    kk = bench.kernel_kind
    assert kk("void bdg::attn_split_kernel<unsigned short, false>(bdg::AttnArgs)") == "attn_split"
    assert kk("void bdg::attn_split_kernel<unsigned short, true>(bdg::AttnArgs)") == "attn_fused"
    assert kk("void bdg::attn_split_kernel<float, true>(bdg::AttnArgs)") == "attn_fused"
    assert kk("void bdg::attn_merge_kernel<float>(bdg::AttnArgs)") == "attn_merge"
    assert kk("void bdg::moe_gateup_kernel<1, 2, 6, 2, true>(bdg::GateUpParams)") == "gate_up"
    assert kk("void bdg::moe_gateup_kernel<0, 3, 6, 1, false>(bdg::GateUpParams)") == "gate_up"
    assert kk("void bdg::moe_route_direct_kernel<8>(bdg::RouteParams)") == "route"
    assert kk("void bdg::stream_copy_kernel(uint4 const*, uint4*, long)") == "copy"
    assert kk("__amd_rocclr_copyBuffer") is None


def test_self_routed_launches():
    """gate_up launches per step that read their layer's router weights: the
    layers needing a router of their own (the first; every later one unless
    the down kernels hand on router sums, a stack of <= 64 experts) less the
    route kernels launched."""
    cfg = types.SimpleNamespace(norm=True, n_layers=48, n_experts=128)
    assert bench.self_routed_launches(cfg, False, 48.0, 0.0) == 48.0
    assert bench.self_routed_launches(cfg, False, 48.0, 48.0) == 0.0       # route kernel flag
    cfg = types.SimpleNamespace(norm=True, n_layers=24, n_experts=32)
    assert bench.self_routed_launches(cfg, False, 24.0, 0.0) == 1.0        # the first layer; sums from down after
    assert bench.self_routed_launches(cfg, False, 24.0, 1.0) == 0.0
    assert bench.self_routed_launches(cfg, True, 24.0, 0.0) == 24.0        # every layer routed on its own
    assert bench.self_routed_launches(cfg, False, 0.0, 24.0) == 0.0        # fused per-layer kernel
    cfg = types.SimpleNamespace(norm=False, n_layers=1, n_experts=32)
    assert bench.self_routed_launches(cfg, False, 1.0, 0.0) == 1.0
    assert bench.self_routed_launches(cfg, False, 1.0, 1.0) == 0.0
