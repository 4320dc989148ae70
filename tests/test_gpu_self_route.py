"""GPU parity of self-routing gate_up launches: layers after the first that
need their own router (more than 64 experts, or every layer routed on its
own) compute it inside the gate_up launch by default, and launch the router
kernel only with BDG_MOE_ROUTE_KERNEL.  The launch's first blocks take one
router row per wave and publish the sums tagged with the token's sequence
number; every block waits for the token's tags (a bounded wait).

The router arithmetic is the router kernel's, so a self-routing plan agrees
bit for bit with the same plan launching the router kernel (the flag): outputs,
routing, weights and residuals, over several tokens in a row (a stale sum
from an earlier token would change the routing), from graph replays with
eager work between them, and for steps of two tokens.  The first token is
also checked against the oracle layer by layer (teacher forcing on the
GPU's own residual inputs and near-tie routing).  The wait's failure path is
driven from the host (a plan whose waits give up at once)."""

import numpy as np
import pytest
import torch

import bit_dequant_gemv_amd as bdg
import synth
from synth import device as sdev

from helpers import banner, to_np
from test_gpu_moe import check_layer

pytestmark = pytest.mark.gpu

SHAPES = {
    # name: (fmt, H, I, E, k, layers, stack, route_every_layer)
    "q4_30b_3layers": ("int4g", 2048, 768, 128, 8, 3, True, False),        # 128 router rows, H = 8 float4 / lane
    "gptoss120b_3layers": ("mxfp4", 2880, 2880, 128, 4, 3, True, False),   # H = 2880: a ragged last float4
    "gptoss20b_every_layer": ("mxfp4", 2880, 2880, 32, 4, 3, True, True),  # 32 experts, one logit per lane
    "int4_e256_3layers": ("int4g", 1024, 512, 256, 8, 3, True, False),     # four logits per lane
    "gptoss120b_bare": ("mxfp4", 2880, 2880, 128, 4, 2, False, False),     # bare layers (no residual)
}


def shape_cfg(name, base, m=1):
    fmt, H, I, E, k, L, stack, _ = SHAPES[name]
    return synth.MoEConfig(name=name, base=base, fmt=fmt, n_layers=L, hidden=H, inter=I, n_experts=E, top_k=k,
                           group=64 if fmt == "int4g" else 32, norm=stack, m=m)


def kernel_counts(plan, x):
    y = torch.empty((x.shape[0], plan.hidden), dtype=torch.float32, device=x.device)
    cnt = bdg.moe_expert_decode_profiled(plan, x, y).count
    torch.cuda.synchronize()
    return {k: int(cnt[i]) for i, k in enumerate(bdg.KERNEL_KINDS)}


def decode(plan, x):
    y, tr = bdg.moe_expert_decode(plan, x, traces=True)
    torch.cuda.synchronize()
    return to_np(y), to_np(tr["topk"]), to_np(tr["wts"]), to_np(tr["resid"])


def same_bits(a, b):
    if a.dtype == np.float32:
        return np.array_equal(a.view(np.uint32), b.view(np.uint32))
    return np.array_equal(a, b)


@pytest.mark.parametrize("name", sorted(SHAPES))
def test_self_route_equals_router_kernel_and_oracle(dev, name):
    every = SHAPES[name][7]
    cfg = shape_cfg(name, 3500 + len(name))
    plan_s, layers = sdev.build_plan(cfg, dev, max_m=1, route_every_layer=every)
    plan_r, _ = sdev.build_plan(cfg, dev, max_m=1, layers=layers, route_every_layer=every, route_kernel=True)
    x0, _ = sdev.hidden_device(cfg, [0], dev)
    cnt_s, cnt_r = kernel_counts(plan_s, x0), kernel_counts(plan_r, x0)
    assert cnt_s["route"] == 0 and cnt_s["gate_up"] == cfg.n_layers, f"self-routing not taken: {cnt_s}"
    assert cnt_r["route"] == cfg.n_layers, cnt_r
    for tok in range(4):
        x, xv = sdev.hidden_device(cfg, [tok], dev)
        banner(f"self-routing gate_up {name} token {tok}")
        s = decode(plan_s, x)
        r = decode(plan_r, x)
        for a, b, what in zip(s, r, ("y", "topk", "wts", "resid")):
            assert same_bits(a, b), f"token {tok}: {what}"
        y, topk, wts, resid = s
        assert np.array_equal(resid[0], xv)
        if tok == 0:
            for l in range(cfg.n_layers):
                out = resid[l + 1] if l + 1 < cfg.n_layers else y
                check_layer(cfg, l, resid[l], out, topk[l], wts[l], cfg.norm, f"{name} layer {l}")
    assert plan_s.check() and plan_r.check()
    plan_s.close()
    plan_r.close()
    del layers
    torch.cuda.empty_cache()


def test_self_route_two_token_steps(dev):
    """Steps of two tokens on the per-token kernels: each token's router rows
    come from its own blocks (grid row t) and carry the step's tag."""
    cfg = shape_cfg("q4_30b_3layers", 3600, m=2)
    plan_s, layers = sdev.build_plan(cfg, dev, max_m=2, per_token=True)
    plan_r, _ = sdev.build_plan(cfg, dev, max_m=2, per_token=True, layers=layers, route_kernel=True)
    for step in range(3):
        x, _ = sdev.hidden_device(cfg, [2 * step, 2 * step + 1], dev)
        banner(f"self-routing gate_up, two-token step {step}")
        s = decode(plan_s, x)
        r = decode(plan_r, x)
        for a, b, what in zip(s, r, ("y", "topk", "wts", "resid")):
            assert same_bits(a, b), f"step {step}: {what}"
    assert kernel_counts(plan_s, x)["route"] == 0
    assert plan_s.check()
    plan_s.close()
    plan_r.close()
    del layers
    torch.cuda.empty_cache()


def test_self_route_graph_replays_match_direct_launches(dev):
    """The tags carry over from launch to launch: many graph replays of
    alternating tokens (with eager work between them) equal direct
    launches of a plan that runs the router kernel, bit for bit."""
    cfg = shape_cfg("q4_30b_3layers", 3700)
    plan_g, layers = sdev.build_plan(cfg, dev, max_m=1)
    plan_d, _ = sdev.build_plan(cfg, dev, max_m=1, layers=layers, use_graph=False, route_kernel=True)
    xs = [sdev.hidden_device(cfg, [t], dev)[0] for t in range(3)]
    want = [bdg.moe_expert_decode(plan_d, x).clone() for x in xs]
    banner("self-routing gate_up: 30 graph replays")
    for rep in range(10):
        for i, x in enumerate(xs):
            y = torch.full((1, cfg.hidden), float("nan"), device=dev)
            bdg.moe_expert_decode(plan_g, x, y=y)
            torch.cuda.synchronize()
            assert torch.equal(y, want[i]), f"replay {rep} token {i}"
        _ = bdg.moe_expert_decode(plan_d, xs[rep % 3])
    assert plan_g.check() and plan_d.check()
    plan_g.close()
    plan_d.close()
    del layers
    torch.cuda.empty_cache()


def test_self_route_wait_failure_is_reported(dev):
    """A plan whose in-kernel waits give up at once (negative wait_polls, set
    from the host): every kernel still exits, the blocks that gave up write
    NaN h (so y is NaN), and moe_plan_check reports it once.  The same
    weights on a normal plan then decode cleanly."""
    cfg = shape_cfg("q4_30b_3layers", 3800)
    plan_bad, layers = sdev.build_plan(cfg, dev, max_m=1, wait_polls=-1)
    x, _ = sdev.hidden_device(cfg, [0], dev)
    banner("self-routing gate_up: waits that give up at once")
    y = bdg.moe_expert_decode(plan_bad, x)
    torch.cuda.synchronize()
    assert torch.isnan(y).all(), "a self-routing wait did not give up"
    assert plan_bad.check() is False
    assert plan_bad.check() is True            # the fault word was cleared
    plan_bad.close()
    plan_ok, _ = sdev.build_plan(cfg, dev, max_m=1, layers=layers)
    y = bdg.moe_expert_decode(plan_ok, x)
    torch.cuda.synchronize()
    assert torch.isfinite(y).all() and plan_ok.check()
    plan_ok.close()


# (fmt, H, I, E, k): the self-routing edges.  65 experts leave 63 idle lanes
# in the second logit half; H = 32 is one float4 of a router row on half a
# wave; H = 3072 is the largest hidden size a router row covers.
# (I is wide enough for the gate_up grid to hold a wave per router row.)
EDGE_SHAPES = [("int4g", 128, 128, 65, 4), ("mxfp4", 32, 320, 100, 2), ("mxfp4", 3072, 128, 72, 4)]


@pytest.mark.parametrize("fmt,H,I,E,k", EDGE_SHAPES)
def test_self_route_edges(dev, fmt, H, I, E, k):
    cfg = synth.MoEConfig(name=f"sr_edge_{fmt}_{H}_{E}", base=3900 + E, fmt=fmt, n_layers=3, hidden=H, inter=I,
                          n_experts=E, top_k=k, group=64 if fmt == "int4g" else 32, norm=True, m=1)
    plan_s, layers = sdev.build_plan(cfg, dev, max_m=1)
    plan_r, _ = sdev.build_plan(cfg, dev, max_m=1, layers=layers, route_kernel=True)
    x0, _ = sdev.hidden_device(cfg, [0], dev)
    assert kernel_counts(plan_s, x0)["route"] == 0
    for tok in range(3):
        x, _ = sdev.hidden_device(cfg, [tok], dev)
        banner(f"self-routing gate_up edge {cfg.name} token {tok}")
        s = decode(plan_s, x)
        r = decode(plan_r, x)
        for a, b, what in zip(s, r, ("y", "topk", "wts", "resid")):
            assert same_bits(a, b), f"token {tok}: {what}"
        if tok == 0:
            y, topk, wts, resid = s
            for l in range(cfg.n_layers):
                out = resid[l + 1] if l + 1 < cfg.n_layers else y
                check_layer(cfg, l, resid[l], out, topk[l], wts[l], cfg.norm, f"{cfg.name} layer {l}")
    assert plan_s.check()
    plan_s.close()
    plan_r.close()


def test_self_route_falls_back_when_the_grid_is_too_small(dev):
    """A gate_up grid with fewer waves than router rows (200 experts, k * I =
    64 pairs: 3 blocks of 4 waves) keeps the route kernel before every layer."""
    cfg = synth.MoEConfig(name="sr_fallback", base=3990, fmt="mxfp4", n_layers=3, hidden=256, inter=64,
                          n_experts=200, top_k=1, group=32, norm=True, m=1)
    plan, layers = sdev.build_plan(cfg, dev, max_m=1)
    x, _ = sdev.hidden_device(cfg, [0], dev)
    assert kernel_counts(plan, x)["route"] == cfg.n_layers
    y, topk, wts, resid = decode(plan, x)
    for l in range(cfg.n_layers):
        out = resid[l + 1] if l + 1 < cfg.n_layers else y
        check_layer(cfg, l, resid[l], out, topk[l], wts[l], cfg.norm, f"fallback layer {l}")
    assert plan.check()
    plan.close()


@pytest.mark.parametrize("x_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("E,L,stack", [(32, 3, True), (128, 2, True), (32, 1, False)])
def test_self_route_first_layer(dev, x_dtype, E, L, stack):
    """The first layer routes inside its gate_up launch on the caller's input
    (bf16 bits or fp32, widened exactly as the route kernel's copy) and writes
    that copy for the down kernel's residual; its down kernel advances the
    token number, so a single bare layer (no later layer) still tags every
    token apart.  32 experts: later layers take router sums from the down
    kernel; 128: every layer routes itself.  Bit for bit the route-kernel plan
    over several tokens, within the oracle tolerance."""
    cfg = synth.MoEConfig(name=f"sr_first_{E}_{L}_{x_dtype}", base=4100 + E + L, fmt="mxfp4", n_layers=L,
                          hidden=2880, inter=2880, n_experts=E, top_k=4, group=32, norm=stack, m=1,
                          x_dtype=x_dtype)
    plan_s, layers = sdev.build_plan(cfg, dev, max_m=1)
    plan_r, _ = sdev.build_plan(cfg, dev, max_m=1, layers=layers, route_kernel=True)
    x0, _ = sdev.hidden_device(cfg, [0], dev)
    assert kernel_counts(plan_s, x0)["route"] == 0
    for tok in range(4):
        x, xv = sdev.hidden_device(cfg, [tok], dev)
        banner(f"self-routing first layer {cfg.name} token {tok}")
        s = decode(plan_s, x)
        r = decode(plan_r, x)
        for a, b, what in zip(s, r, ("y", "topk", "wts", "resid")):
            assert same_bits(a, b), f"token {tok}: {what}"
        y, topk, wts, resid = s
        assert np.array_equal(resid[0], xv)
        if tok == 0:
            for l in range(cfg.n_layers):
                out = resid[l + 1] if l + 1 < cfg.n_layers else y
                check_layer(cfg, l, resid[l], out, topk[l], wts[l], cfg.norm, f"{cfg.name} layer {l}")
    assert plan_s.check() and plan_r.check()
    plan_s.close()
    plan_r.close()
    del layers
    torch.cuda.empty_cache()
