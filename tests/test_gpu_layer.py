"""GPU parity of the fused per-layer decode kernel (moe_layer.hip): one-token
steps run each layer as one kernel that streams the down weights into LDS
during gate_up and exchanges h through a grid barrier.

It is opt-in (BDG_MOE_FUSED_LAYER) and computes every row with the same
arithmetic as the default two-kernel path, so the two agree bit for bit; the fused path is also
checked against the oracle layer by layer (teacher forcing on the GPU's own
residual inputs and near-tie routing), replayed from graphs many times, and
driven into its bounded wait's failure path from the host."""

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
    # name: (fmt, H, I, E, k, layers, stack)
    "gptoss20b_3layers": ("mxfp4", 2880, 2880, 32, 4, 3, True),
    "gptoss20b_bare": ("mxfp4", 2880, 2880, 32, 4, 1, False),
    "gptoss120b_3layers": ("mxfp4", 2880, 2880, 128, 4, 3, True),
    "q4_30b_e16_3layers": ("int4g", 2048, 768, 16, 8, 3, True),
    "q4_30b_2layers": ("int4g", 2048, 768, 128, 8, 2, True),
}


def shape_cfg(name, base):
    fmt, H, I, E, k, L, stack = SHAPES[name]
    return synth.MoEConfig(name=name, base=base, fmt=fmt, n_layers=L, hidden=H, inter=I, n_experts=E, top_k=k,
                           group=64 if fmt == "int4g" else 32, norm=stack, m=1)


def kernel_counts(plan, x):
    y = torch.empty((1, plan.hidden), dtype=torch.float32, device=x.device)
    cnt = bdg.moe_expert_decode_profiled(plan, x, y).count
    torch.cuda.synchronize()
    return {k: int(cnt[i]) for i, k in enumerate(bdg.KERNEL_KINDS)}


def decode(plan, x):
    y, tr = bdg.moe_expert_decode(plan, x, traces=True)
    torch.cuda.synchronize()
    return to_np(y), to_np(tr["topk"]), to_np(tr["wts"]), to_np(tr["resid"])


@pytest.mark.parametrize("name", sorted(SHAPES))
def test_fused_equals_two_kernel_and_oracle(dev, name):
    cfg = shape_cfg(name, 3100 + len(name))
    plan_f, layers = sdev.build_plan(cfg, dev, max_m=1, fused_layer=True)
    plan_t, _ = sdev.build_plan(cfg, dev, max_m=1, layers=layers)
    x0, _ = sdev.hidden_device(cfg, [0], dev)
    cnt_f, cnt_t = kernel_counts(plan_f, x0), kernel_counts(plan_t, x0)
    assert cnt_f["layer"] == cfg.n_layers and cnt_f["gate_up"] == 0, f"fused path not taken: {cnt_f}"
    assert cnt_t["layer"] == 0 and cnt_t["gate_up"] == cfg.n_layers
    for tok in range(3):
        x, xv = sdev.hidden_device(cfg, [tok], dev)
        banner(f"fused layer kernel {name} token {tok}")
        f = decode(plan_f, x)
        t = decode(plan_t, x)
        for a, b, what in zip(f, t, ("y", "topk", "wts", "resid")):
            assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                                  b.view(np.uint32) if b.dtype == np.float32 else b), f"token {tok}: {what}"
        y, topk, wts, resid = f
        assert np.array_equal(resid[0], xv)
        if tok == 0:
            for l in range(cfg.n_layers):
                out = resid[l + 1] if l + 1 < cfg.n_layers else y
                check_layer(cfg, l, resid[l], out, topk[l], wts[l], cfg.norm, f"{name} layer {l}")
    assert plan_f.check() and plan_t.check()
    plan_f.close()
    plan_t.close()
    del layers
    torch.cuda.empty_cache()


def test_fused_graph_replays_match_direct_launches(dev):
    """The barrier's words carry over from launch to launch: many graph
    replays (with eager work between them) equal direct launches bit for bit."""
    cfg = shape_cfg("gptoss20b_3layers", 3200)
    plan_g, layers = sdev.build_plan(cfg, dev, max_m=1, fused_layer=True)
    plan_d, _ = sdev.build_plan(cfg, dev, max_m=1, layers=layers, use_graph=False, fused_layer=True)
    xs = [sdev.hidden_device(cfg, [t], dev)[0] for t in range(3)]
    want = [bdg.moe_expert_decode(plan_d, x).clone() for x in xs]
    banner("fused layer kernel: 30 graph replays")
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


def test_fused_wait_failure_is_reported(dev):
    """A plan whose in-kernel waits give up at once (negative wait_polls, set
    from the host): every kernel still exits, the blocks that gave up write
    NaN, and moe_plan_check reports it once.  The same weights on a normal
    plan then decode cleanly."""
    cfg = shape_cfg("q4_30b_e16_3layers", 3300)
    plan_bad, layers = sdev.build_plan(cfg, dev, max_m=1, wait_polls=-1, fused_layer=True)
    x, _ = sdev.hidden_device(cfg, [0], dev)
    banner("fused layer kernel: waits that give up at once")
    y = bdg.moe_expert_decode(plan_bad, x)
    torch.cuda.synchronize()
    assert torch.isnan(y).any(), "no block gave up"
    assert plan_bad.check() is False
    assert plan_bad.check() is True            # the fault word was cleared
    plan_bad.close()
    plan_ok, _ = sdev.build_plan(cfg, dev, max_m=1, layers=layers, fused_layer=True)
    y = bdg.moe_expert_decode(plan_ok, x)
    torch.cuda.synchronize()
    assert torch.isfinite(y).all() and plan_ok.check()
    plan_ok.close()
