"""GPU parity of the grouped expert products on the matrix cores
(BDG_MOE_MFMA, moe_mfma.hip): steps of M > 1 tokens with up to 8 of a
distinct expert's picks per chunk (an expert with more spans several
chunks), K split over a block's 4 waves (a wave may get no K group at all
when the rows are short), weights decoded to bf16 with their block scale
(the conversion pinned by the exhaustive bf16 dequant test), activations as
bf16 hi + lo parts, fp32 accumulation.  Held to the same oracle tolerance as
the VALU path: max |y - y_ref| / (|W| . |x|) <= 1e-4, cosine >= 0.99999, per
layer with teacher forcing, routing validated on every layer."""

import numpy as np
import pytest
import torch

import bit_dequant_gemv_amd as bdg
import synth
from oracle import moe as omoe
from synth import device as sdev

from helpers import assert_close, banner, to_np
from test_gpu_moe import check_layer, oracle_routed, small_cfg

pytestmark = pytest.mark.gpu


def kernel_counts(plan, x):
    y = torch.empty((x.shape[0], plan.hidden), dtype=torch.float32, device=x.device)
    cnt = bdg.moe_expert_decode_profiled(plan, x, y).count
    torch.cuda.synchronize()
    return {k: int(cnt[i]) for i, k in enumerate(bdg.KERNEL_KINDS)}


@pytest.mark.parametrize("m", [2, 5, 16])
def test_mfma_stack_small(dev, m):
    """A 3-layer MXFP4 stack (80 experts, top-4): every layer against the
    oracle on the GPU's own inputs, routing checked on every layer."""
    cfg = small_cfg("mxfp4", 4000 + m, E=80, k=4, H=384, I=192, L=3, stack=True, m=m)
    plan, layers = sdev.build_plan(cfg, dev, max_m=m, mfma=True)
    x, xv = sdev.hidden_device(cfg, range(m), dev)
    banner(f"mfma stack small m={m}")
    y, tr = bdg.moe_expert_decode(plan, x, traces=True)
    torch.cuda.synchronize()
    y, topk, wts, resid = to_np(y), to_np(tr["topk"]), to_np(tr["wts"]), to_np(tr["resid"])
    assert np.array_equal(resid[0], xv)
    for l in range(cfg.n_layers):
        out = resid[l + 1] if l + 1 < cfg.n_layers else y
        check_layer(cfg, l, resid[l], out, topk[l], wts[l], True, f"mfma m={m} layer {l}")
    cnt = kernel_counts(plan, x)
    assert cnt["gate_up"] == cfg.n_layers and cnt["down"] == cfg.n_layers


@pytest.mark.parametrize("case", ["all_on_two", "spread", "k_equals_e"])
def test_mfma_routed(dev, case):
    """Fixed routing through the matrix-core pair: 16 tokens on the same two
    experts (16 picks per expert: two chunks of 8), picks spread over many
    experts (one pick per chunk; H = 320 gives 10 MX blocks, so one wave of
    the block gets no K group and the last group is half empty), and k = E
    (every token on every expert)."""
    if case == "k_equals_e":
        cfg = small_cfg("mxfp4", 4100, E=4, k=4, H=256, I=128, m=7)
    else:
        cfg = small_cfg("mxfp4", 4101, E=40, k=2, H=320, I=256, m=16)
    m = cfg.m
    plan, _ = sdev.build_plan(cfg, dev, max_m=m, mfma=True)
    x, xv = sdev.hidden_device(cfg, range(m), dev)
    rng = np.random.default_rng(9)
    if case == "all_on_two":
        idx = np.tile(np.array([[3, 17]], dtype=np.int32), (m, 1))
    elif case == "spread":
        idx = np.stack([rng.choice(cfg.n_experts, 2, replace=False) for _ in range(m)]).astype(np.int32)
    else:
        idx = np.stack([rng.permutation(4) for _ in range(m)]).astype(np.int32)
    wts = rng.uniform(0.1, 1.0, idx.shape).astype(np.float32)
    banner(f"mfma routed case={case}")
    y = to_np(bdg.moe_experts_routed(plan, 0, x, torch.from_numpy(idx).to(dev), torch.from_numpy(wts).to(dev)))
    y_ref, den = oracle_routed(cfg, 0, xv, idx, wts)
    assert_close(y, y_ref, den, f"mfma routed {case}")


def test_mfma_close_to_valu_grouped(dev):
    """The matrix-core and VALU grouped paths on the same layer input: the
    same routing, both within the oracle tolerance, and within the sum of
    the two tolerances of each other (different summation, not bit for bit)."""
    cfg = small_cfg("mxfp4", 4200, E=64, k=4, H=512, I=256, L=1, stack=True, m=16)
    plan_m, layers = sdev.build_plan(cfg, dev, max_m=16, mfma=True)
    plan_v, _ = sdev.build_plan(cfg, dev, max_m=16, layers=layers)
    x, _ = sdev.hidden_device(cfg, range(16), dev)
    banner("mfma vs VALU grouped m=16")
    ym, trm = bdg.moe_expert_decode(plan_m, x, traces=True)
    yv, trv = bdg.moe_expert_decode(plan_v, x, traces=True)
    torch.cuda.synchronize()
    topk = to_np(trm["topk"])[0]
    assert np.array_equal(topk, to_np(trv["topk"])[0])
    resid = to_np(trm["resid"])[0]
    wts = to_np(trm["wts"])[0]
    _, _, _ = check_layer(cfg, 0, resid, to_np(ym), topk, wts, True, "mfma layer")
    _, _, _ = check_layer(cfg, 0, resid, to_np(yv), topk, wts, True, "VALU layer")
    w_r, b_r, _ = synth.router(cfg, 0)
    from test_gpu_moe import oracle_expert_getter
    res = omoe.moe_layer(resid, w_r, oracle_expert_getter(cfg, 0), cfg.top_k, bias=b_r, norm=True,
                         residual=True, forced_idx=topk)
    assert omoe.max_rel_err(to_np(ym), to_np(yv), res["den"]) <= 2e-4


def test_mfma_120b_stack_full(dev):
    """The 36-layer 120B-shape stack (128 experts, top-4, biased hot set) at
    M = 4 and M = 16 on the matrix cores, in the launch configuration the
    benchmark's --mfma run times: routing of every token checked on every
    layer, outputs teacher-forced on sampled layers for every token."""
    cfg = synth.CONFIGS["gptoss120b_smallm"]
    plan, layers = sdev.build_plan(cfg, dev, max_m=16, mfma=True)
    for m in (4, 16):
        x, xv = sdev.hidden_device(cfg, range(m), dev)
        banner(f"mfma gptoss120b_smallm M={m}")
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
        for l in (0, 17, cfg.n_layers - 1):
            out = resid[l + 1] if l + 1 < cfg.n_layers else y
            check_layer(cfg, l, resid[l], out, topk[l], wts[l], True, f"mfma 120B M={m} layer {l}")
    plan.close()
    del layers
    torch.cuda.empty_cache()
