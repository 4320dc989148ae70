"""GPU parity of the MoE expert-decode path (moe_expert_decode, moe_experts_routed).

Layers are compared with the oracle element by element; stacks are checked
layer by layer with teacher forcing (the oracle runs layer l on the GPU's own
input residual of layer l, taken from resid_trace), and routing is checked
against the float64 logits with the near-tie band.
"""

import functools

import numpy as np
import pytest
import torch

import bit_dequant_gemv_amd as bdg
import synth
from oracle import formats, moe as omoe
from synth import device as sdev

from helpers import assert_close, banner, to_np

pytestmark = pytest.mark.gpu

W_TOL = 1e-5    # router weights inside the stack vs the oracle's float64 softmax


def oracle_expert_getter(cfg, layer):
    @functools.lru_cache(maxsize=None)
    def get(e):
        w = synth.expert_weights(cfg, layer, e)
        if cfg.fmt == synth.FMT_MXFP4:
            return formats.mxfp4_dequant(*w["gu"]), formats.mxfp4_dequant(*w["dn"])
        return (formats.int4g_dequant(*w["gu"], cfg.group),
                formats.int4g_dequant(*w["dn"], cfg.group))
    return get


def check_layer(cfg, layer, x_in, y_gpu, topk_gpu, wts_gpu, stack, what):
    """Teacher-forced check of one layer: oracle on the GPU's input."""
    w_r, b_r, _ = synth.router(cfg, layer)
    res = omoe.moe_layer(x_in, w_r, oracle_expert_getter(cfg, layer), cfg.top_k, bias=b_r,
                         norm=stack, residual=stack, forced_idx=topk_gpu)
    rel, cos = assert_close(y_gpu, res["y"], res["den"], what)
    assert np.array_equal(res["idx"], topk_gpu)
    assert np.max(np.abs(res["w"] - wts_gpu)) <= W_TOL, f"{what}: router weights"
    return rel, cos, res["ties"]


def small_cfg(fmt, base, E=8, k=2, H=320, I=96, L=1, stack=False, m=3, group=64):
    if fmt == "mxfp4" or H % group or I % group:
        group = 32
    return synth.MoEConfig(name=f"small{base}", base=base, fmt=fmt, n_layers=L, hidden=H,
                           inter=I, n_experts=E, top_k=k, group=group, norm=stack, m=m)


def run_and_check(cfg, dev, m, use_graph=True, tokens=None, **plan_opts):
    plan, layers = sdev.build_plan(cfg, dev, max_m=m, use_graph=use_graph, **plan_opts)
    tokens = list(range(m)) if tokens is None else tokens
    x, xv = sdev.hidden_device(cfg, tokens, dev)
    banner(f"moe_expert_decode {cfg.name} fmt={cfg.fmt} L={cfg.n_layers} E={cfg.n_experts} "
           f"k={cfg.top_k} H={cfg.hidden} I={cfg.inter} m={m} graph={use_graph}")
    y, tr = bdg.moe_expert_decode(plan, x, traces=True)
    torch.cuda.synchronize()
    y, topk, wts, resid = to_np(y), to_np(tr["topk"]), to_np(tr["wts"]), to_np(tr["resid"])
    # layer 0 input is x itself, exactly
    assert np.array_equal(resid[0], xv)
    for l in range(cfg.n_layers):
        out = resid[l + 1] if l + 1 < cfg.n_layers else y
        check_layer(cfg, l, resid[l], out, topk[l], wts[l], cfg.norm, f"{cfg.name} layer {l}")
    return plan, layers, x, y, tr


@pytest.mark.parametrize("fmt", ["mxfp4", "int4g"])
@pytest.mark.parametrize("m", [1, 3])
def test_layer_small(dev, fmt, m):
    cfg = small_cfg(fmt, 1000 + m, m=m)
    run_and_check(cfg, dev, m)


def route_launches(plan, x):
    """Route-kernel launches of one decode step (per-kernel event pass)."""
    y = torch.empty((x.shape[0], plan.hidden), dtype=torch.float32, device=x.device)
    cnt = bdg.moe_expert_decode_profiled(plan, x, y).count
    torch.cuda.synchronize()
    return int(cnt[bdg.KERNEL_KINDS.index("route")])


@pytest.mark.parametrize("fmt", ["mxfp4", "int4g"])
@pytest.mark.parametrize("fuse", ["1", "0", "kernel"])
@pytest.mark.parametrize("E", [16, 96])
@pytest.mark.parametrize("m", [1, 2])
def test_stack_small_end_to_end(dev, fmt, fuse, E, m):
    """The per-token path of a 3-layer stack.  fuse=1: for E <= 64, layers
    after the first route from the partial router sums of the previous down
    kernel; E = 96 (more router rows than the down epilogue covers) and
    fuse=0: every layer routes inside its gate_up launch (so does the first
    layer in every case); fuse=kernel (BDG_MOE_ROUTE_KERNEL with every layer
    routed on its own): every layer runs the route kernel."""
    cfg = small_cfg(fmt, 1100 + E, E=E, k=4, H=512, I=256, L=3, stack=True, m=m)
    plan, layers, x, y, tr = run_and_check(cfg, dev, m, route_every_layer=fuse != "1", per_token=True,
                                           route_kernel=fuse == "kernel")
    assert route_launches(plan, x) == (cfg.n_layers if fuse == "kernel" else 0)
    # end to end without teacher forcing on the residual (routing forced only in band)
    layers_o = [(synth.router(cfg, l)[0], None, oracle_expert_getter(cfg, l)) for l in range(3)]
    xv = synth.hidden_batch(cfg, list(range(m)))[0]
    results, out = omoe.moe_stack(xv, layers_o, cfg.top_k, forced_idx=to_np(tr["topk"]))
    assert_close(y, out, results[-1]["den"], "stack end to end")


def test_graph_and_direct_launch_identical(dev):
    cfg = small_cfg("mxfp4", 1200, E=16, k=4, H=512, I=256, L=3, stack=True, m=2)
    plan_g, layers = sdev.build_plan(cfg, dev, max_m=2, use_graph=True)
    plan_d, _ = sdev.build_plan(cfg, dev, max_m=2, use_graph=False, layers=layers)
    x, _ = sdev.hidden_device(cfg, [0, 1], dev)
    y_g = bdg.moe_expert_decode(plan_g, x)
    y_d = bdg.moe_expert_decode(plan_d, x)
    # replay the graph into a NaN-filled output, several times, with eager work between
    for rep in range(3):
        y_r = torch.full_like(y_g, float("nan"))
        bdg.moe_expert_decode(plan_g, x, y=y_r)
        torch.cuda.synchronize()
        assert torch.equal(y_r, y_g), f"replay {rep}"
        _ = bdg.moe_expert_decode(plan_d, x)
    assert torch.equal(y_g, y_d)


def test_graph_cache_many_keys(dev):
    cfg = small_cfg("int4g", 1300, E=8, k=2, H=256, I=128, L=2, stack=True, m=1)
    plan, layers = sdev.build_plan(cfg, dev, max_m=1)
    xs = [sdev.hidden_device(cfg, [t], dev)[0] for t in range(12)]    # > cache size of 8
    first = [bdg.moe_expert_decode(plan, x).clone() for x in xs]
    again = [bdg.moe_expert_decode(plan, x) for x in xs]
    torch.cuda.synchronize()
    for a, b in zip(first, again):
        assert torch.equal(a, b)


# ---------------------------------------------------------------- fixed routing

def oracle_routed(cfg, layer, x, idx, wts):
    get = oracle_expert_getter(cfg, layer)
    y = np.zeros((x.shape[0], cfg.hidden))
    den = np.zeros_like(y)
    for t in range(x.shape[0]):
        for j in range(idx.shape[1]):
            d, _, dd = omoe.expert_ffn(*get(int(idx[t, j])), x[t])
            y[t] += wts[t, j] * d
            den[t] += abs(wts[t, j]) * dd
    return y, den


@pytest.mark.parametrize("case", ["duplicates", "one_expert", "k_equals_e", "skew"])
def test_experts_routed(dev, case):
    if case == "k_equals_e":
        cfg = small_cfg("mxfp4", 1400, E=4, k=4, H=256, I=160, m=4)
    else:
        cfg = small_cfg("int4g" if case == "skew" else "mxfp4", 1401, E=8, k=3, H=384, I=128, m=5)
    m = cfg.m
    plan, layers = sdev.build_plan(cfg, dev, max_m=m)
    x, xv = sdev.hidden_device(cfg, range(m), dev)
    rng = np.random.default_rng(5)
    if case == "duplicates":
        idx = np.array([[1, 2, 3], [3, 2, 1], [1, 1, 1], [0, 7, 0], [5, 5, 6]], dtype=np.int32)
    elif case == "one_expert":
        idx = np.full((m, 3), 4, dtype=np.int32)
    elif case == "k_equals_e":
        idx = np.stack([rng.permutation(4) for _ in range(m)]).astype(np.int32)
    else:
        idx = rng.choice([0, 0, 0, 1, 2, 7], size=(m, 3)).astype(np.int32)
    wts = rng.uniform(0.1, 1.0, (m, idx.shape[1])).astype(np.float32)
    banner(f"moe_experts_routed case={case}")
    y = to_np(bdg.moe_experts_routed(plan, 0, x, torch.from_numpy(idx).to(dev),
                                     torch.from_numpy(wts).to(dev)))
    y_ref, den = oracle_routed(cfg, 0, xv, idx, wts)
    assert_close(y, y_ref, den, f"routed {case}")


# ---------------------------------------------------------------- full-size configs

def test_gptoss20b_layer_full(dev):
    cfg = synth.CONFIGS["gptoss20b_layer"]
    run_and_check(cfg, dev, 2)


@pytest.mark.parametrize("name,check_layers", [("gptoss20b_stack", (0, 11, 23)),
                                               ("q4_30b_stack", (0, 23, 47))])
def test_stack_full(dev, name, check_layers):
    """Full 24-layer MXFP4 / 48-layer int4 stacks at M=1 in the benchmark's launch
    configuration: routing validated on every layer, outputs on sampled layers."""
    cfg = synth.CONFIGS[name]
    plan, layers = sdev.build_plan(cfg, dev, max_m=1)
    for tok in (0, 1):
        x, xv = sdev.hidden_device(cfg, [tok], dev)
        banner(f"moe_expert_decode {name} full token {tok}")
        y, tr = bdg.moe_expert_decode(plan, x, traces=True)
        torch.cuda.synchronize()
        y, topk, wts, resid = to_np(y), to_np(tr["topk"]), to_np(tr["wts"]), to_np(tr["resid"])
        assert np.array_equal(resid[0], xv)
        assert np.all(np.isfinite(y))
        for l in range(cfg.n_layers):
            xin = omoe.rmsnorm(resid[l])
            w_r, b_r, _ = synth.router(cfg, l)
            lg, sc = omoe.router_logits(w_r, xin, b_r)
            ok, _, msg = omoe.check_routing(lg[0], sc[0], topk[l, 0], cfg.top_k)
            assert ok, f"layer {l}: {msg}"
        for l in check_layers:
            out = resid[l + 1] if l + 1 < cfg.n_layers else y
            check_layer(cfg, l, resid[l], out, topk[l], wts[l], True, f"{name} layer {l} token {tok}")


@pytest.mark.parametrize("E,k", [(32, 4), (128, 8), (256, 8), (300, 16)])
@pytest.mark.parametrize("L", [1, 2])
@pytest.mark.parametrize("group", ["0", "1"])
def test_layer_routing_ties(dev, E, k, L, group):
    """The expert selection inside the fused path on tie-heavy logits: zero
    router rows, so each logit is its bias, drawn from a small value set with
    -inf entries.  The selection must match the oracle's order exactly (ties
    to the lower index), and the layer output the oracle's for those picks.
    L=2 checks the second layer of a residual stack, which on the per-token
    path (group=0; for E <= 64) routes from the partial sums written by the
    first layer's down kernel; group=1 runs the grouped kernels."""
    cfg = small_cfg("mxfp4", 1500 + E, E=E, k=k, H=128, I=64, m=2, L=L, stack=L > 1)
    rng = np.random.default_rng(E)
    b = rng.choice(np.array([1.0, 0.5, 0.5, 0.0, -np.inf], dtype=np.float32), size=E)
    b[rng.choice(E, size=k + 1, replace=False)] = 0.25
    w_r = np.zeros((E, cfg.hidden), dtype=np.float32)
    layers = [sdev.upload_layer(cfg, l, dev) for l in range(L)]
    layers[-1]["w_router"] = torch.from_numpy(w_r).to(dev)
    layers[-1]["b_router"] = torch.from_numpy(b).to(dev)
    plan, _ = sdev.build_plan(cfg, dev, max_m=2, layers=layers, per_token=group == "0")
    x, xv = sdev.hidden_device(cfg, [0, 1], dev)
    banner(f"moe_expert_decode routing ties E={E} k={k} L={L}")
    y, tr = bdg.moe_expert_decode(plan, x, traces=True)
    torch.cuda.synchronize()
    y, topk, wts = to_np(y), to_np(tr["topk"])[L - 1], to_np(tr["wts"])[L - 1]
    o_idx, o_w = omoe.topk_softmax(np.tile(b.astype(np.float64), (2, 1)), k)
    assert np.array_equal(topk, o_idx)
    assert np.max(np.abs(wts - o_w)) <= W_TOL
    xin = to_np(tr["resid"])[L - 1] if L > 1 else xv
    res = omoe.moe_layer(xin, w_r, oracle_expert_getter(cfg, L - 1), k, bias=b, norm=L > 1,
                         residual=L > 1, forced_idx=topk)
    assert_close(y, res["y"], res["den"], f"ties E={E} L={L}")


def _decode_with(cfg, dev, m, group):
    # the grouped path routes every layer with the route kernel; so must the
    # per-token path here (no partial sums from the previous down kernel)
    plan, _ = sdev.build_plan(cfg, dev, max_m=m, per_token=group == "0", route_every_layer=True)
    x, _ = sdev.hidden_device(cfg, range(m), dev)
    y, tr = bdg.moe_expert_decode(plan, x, traces=True)
    torch.cuda.synchronize()
    out = to_np(y), to_np(tr["topk"]), to_np(tr["wts"]), to_np(tr["resid"])
    plan.close()
    return out


@pytest.mark.parametrize("fmt", ["mxfp4", "int4g"])
@pytest.mark.parametrize("m", [3, 16])
def test_grouped_equals_per_token(dev, fmt, m):
    """Steps of M > 1 tokens read each chosen expert once (grouped kernels);
    every output row is the same arithmetic as on the per-token path (same
    row dot products, the combine in slot order), so the two agree bit for
    bit.  The per-token side routes every layer with the route kernel, as the
    grouped path does."""
    cfg = small_cfg(fmt, 1700 + m, E=80, k=4, H=384, I=192, L=3, stack=True, m=m)
    banner(f"grouped vs per-token fmt={fmt} m={m}")
    g = _decode_with(cfg, dev, m, "1")
    t = _decode_with(cfg, dev, m, "0")
    for a, b, what in zip(g, t, ("y", "topk", "wts", "resid")):
        assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                              b.view(np.uint32) if b.dtype == np.float32 else b), what


def test_small_m_120b_stack_full(dev):
    """The 36-layer 120B-shape stack (128 experts, top-4, biased hot set) at
    M = 4 and M = 16 through the grouped path, in the launch configuration
    the benchmark times (one plan of max_m 16, graph replay): routing of
    every token checked on every layer, outputs teacher-forced on sampled
    layers (first, two inner, last) for every token."""
    cfg = synth.CONFIGS["gptoss120b_smallm"]
    plan, layers = sdev.build_plan(cfg, dev, max_m=16)
    for m in (4, 16):
        x, xv = sdev.hidden_device(cfg, range(m), dev)
        banner(f"moe_expert_decode gptoss120b_smallm M={m}")
        y, tr = bdg.moe_expert_decode(plan, x, traces=True)
        torch.cuda.synchronize()
        y, topk, wts, resid = to_np(y), to_np(tr["topk"]), to_np(tr["wts"]), to_np(tr["resid"])
        assert np.array_equal(resid[0], xv)
        assert np.all(np.isfinite(y))
        for l in range(cfg.n_layers):
            w_r, b_r, _ = synth.router(cfg, l)
            lg, sc = omoe.router_logits(w_r, omoe.rmsnorm(resid[l]), b_r)
            for t in range(m):
                ok, _, msg = omoe.check_routing(lg[t], sc[t], topk[l, t], cfg.top_k)
                assert ok, f"M={m} layer {l} token {t}: {msg}"
        for l in (0, 11, 23, cfg.n_layers - 1):
            out = resid[l + 1] if l + 1 < cfg.n_layers else y
            check_layer(cfg, l, resid[l], out, topk[l], wts[l], True, f"120B M={m} layer {l}")
    plan.close()
    del layers
    torch.cuda.empty_cache()


@pytest.mark.parametrize("E,k,m", [(4, 2, 16), (2, 2, 16), (8, 8, 16), (6, 1, 9)])
def test_grouped_heavy_sharing(dev, E, k, m):
    """Few experts shared by every token (up to 16 picks of one expert, so an
    expert spans several chunks; k = E; k = 1): the grouped path against the
    per-token path bit for bit, and the first layer against the oracle."""
    cfg = small_cfg("mxfp4", 1800 + 10 * E + k, E=E, k=k, H=256, I=128, L=2, stack=True, m=m)
    banner(f"grouped heavy sharing E={E} k={k} m={m}")
    g = _decode_with(cfg, dev, m, "1")
    t = _decode_with(cfg, dev, m, "0")
    for a, b, what in zip(g, t, ("y", "topk", "wts", "resid")):
        assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                              b.view(np.uint32) if b.dtype == np.float32 else b), what
    y, topk, wts, resid = g
    check_layer(cfg, 0, resid[0], resid[1], topk[0], wts[0], True, f"sharing E={E} layer 0")
