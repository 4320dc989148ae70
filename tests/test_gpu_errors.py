"""Failure handling on the GPU path: NaN scales propagate as NaN exactly
where the oracle's arithmetic puts them, and the decode entry points reject
bad arguments on the host (checked through the C ABI, past the Python
binding's own checks).  Every kernel here runs on valid, in-bounds inputs."""

import ctypes

import numpy as np
import pytest
import torch

import bit_dequant_gemv_amd as bdg
import synth
from bit_dequant_gemv_amd import _lib
from oracle import formats, gemv as ogemv, moe as omoe
from synth import device as sdev

from helpers import assert_close, banner, to_np

pytestmark = pytest.mark.gpu


def dev_t(a, dev):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(dev)


def check_nan_and_values(y, y_ref, den, what):
    """NaN exactly where the oracle has NaN; elsewhere within the tolerance."""
    gn, wn = np.isnan(y), np.isnan(y_ref)
    assert np.array_equal(gn, wn), f"{what}: NaN positions differ ({gn.sum()} vs {wn.sum()})"
    assert wn.any(), f"{what}: the case plants no NaN"
    keep = ~wn
    assert_close(y[keep], y_ref[keep], den[keep], what)


@pytest.mark.parametrize("fmt", ["mxfp4", "int4g"])
def test_qgemv_nan_scale_poisons_its_row_only(dev, fmt):
    """E8M0 255 (MXFP4) or an fp16 NaN scale (int4) makes the block's weights
    NaN, so exactly the rows holding such a block are NaN."""
    rng = np.random.default_rng(31)
    n, k = 70, 2880
    codes = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    x = rng.standard_normal((2, k)).astype(np.float32)
    bad_rows = [0, 17, 69]
    banner(f"qgemv NaN scales {fmt}")
    if fmt == "mxfp4":
        scales = rng.integers(118, 129, (n, k // 32), dtype=np.uint8)
        for i, r in enumerate(bad_rows):
            scales[r, [0, 44, 89][i]] = 255              # first, middle and last block
        w = formats.mxfp4_dequant(codes, scales)
        qw = bdg.QWeight("mxfp4", dev_t(codes, dev), dev_t(scales, dev))
    else:
        group = 64
        g = k // group
        scales = synth.fp16_bits_of(rng.uniform(0.005, 0.02, (n, g)))
        zeros = rng.integers(0, 256, (n, (g + 1) // 2), dtype=np.uint8)
        for i, r in enumerate(bad_rows):
            scales[r, [0, 22, 44][i]] = 0x7E00           # fp16 quiet NaN
        w = formats.int4g_dequant(codes, scales, zeros, group)
        qw = bdg.QWeight("int4g", dev_t(codes, dev), dev_t(scales, dev), dev_t(zeros, dev), group)
    y = to_np(bdg.qgemv(qw, dev_t(x, dev)))
    y_ref, den = ogemv.gemv(w, x)
    check_nan_and_values(y, y_ref, den, f"qgemv NaN {fmt}")
    assert set(np.nonzero(np.isnan(y[0]))[0]) == set(bad_rows)


@pytest.mark.parametrize("per_token", [True, False])
def test_expert_nan_scales_through_the_layer(dev, per_token):
    """A NaN block in an expert's gate_up makes one element of h NaN, and
    every output row of that expert reads it: the token's whole output is
    NaN.  A NaN block in a down row poisons that output row only.  Tokens
    routed around both stay finite and match the oracle."""
    cfg = synth.MoEConfig(name="nan", base=2600, fmt="mxfp4", n_layers=1, hidden=320, inter=96,
                          n_experts=6, top_k=2, norm=False, m=3)
    layer = sdev.upload_layer(cfg, 0, dev)
    gu_sc = layer["gate_up"].scales
    dn_sc = layer["down"].scales
    gu_sc[1, 50, 3] = 255          # expert 1, gate row 50, block 3
    dn_sc[4, 200, 1] = 255         # expert 4, down row 200, block 1
    plan, _ = sdev.build_plan(cfg, dev, max_m=3, layers=[layer], per_token=per_token)
    x, xv = sdev.hidden_device(cfg, range(3), dev)
    idx = np.array([[1, 0], [4, 2], [3, 5]], dtype=np.int32)
    wts = np.array([[0.6, 0.4], [0.7, 0.3], [0.5, 0.5]], dtype=np.float32)
    banner(f"moe_experts_routed NaN scales per_token={per_token}")
    y = to_np(bdg.moe_experts_routed(plan, 0, x, dev_t(idx, dev), dev_t(wts, dev)))
    torch.cuda.synchronize()

    def get(e):
        # the seeded host weights with the same blocks poisoned
        w = synth.expert_weights(cfg, 0, e)
        gu_codes, gu_scales = w["gu"][0], w["gu"][1].copy()
        dn_codes, dn_scales = w["dn"][0], w["dn"][1].copy()
        if e == 1:
            gu_scales[50, 3] = 255
        if e == 4:
            dn_scales[200, 1] = 255
        return formats.mxfp4_dequant(gu_codes, gu_scales), formats.mxfp4_dequant(dn_codes, dn_scales)
    y_ref = np.zeros((3, cfg.hidden))
    den = np.zeros((3, cfg.hidden))
    for t in range(3):
        for j in range(2):
            w_gu, w_d = get(int(idx[t, j]))
            d, _, den_d = omoe.expert_ffn(w_gu, w_d, xv[t])
            y_ref[t] += float(wts[t, j]) * d
            den[t] += float(wts[t, j]) * den_d
    check_nan_and_values(y, y_ref, den, "NaN scales through the layer")
    assert np.all(np.isnan(y[0]))
    assert set(np.nonzero(np.isnan(y[1]))[0]) == {200}
    assert np.all(np.isfinite(y[2]))
    plan.close()


def test_decode_rejects_bad_arguments_on_the_host(dev):
    """Arguments the plan cannot take fail before anything is enqueued."""
    cfg = synth.MoEConfig(name="rej", base=2700, fmt="mxfp4", n_layers=2, hidden=256, inter=64,
                          n_experts=4, top_k=2, norm=True, m=2)
    plan, _ = sdev.build_plan(cfg, dev, max_m=2)
    lib = _lib.load()
    x = torch.zeros((4, cfg.hidden + 4), dtype=torch.float32, device=dev)
    y = torch.full((4, cfg.hidden), 7.0, dtype=torch.float32, device=dev)
    xp, yp = ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(y.data_ptr())
    h = plan.handle
    banner("moe_expert_decode host-side rejections")
    assert lib.moe_expert_decode(h, xp, _lib.BDG_F32, 3, yp, None, None, None, None) == _lib.BDG_E_INVALID
    assert lib.moe_expert_decode(h, xp, _lib.BDG_F32, 0, yp, None, None, None, None) == _lib.BDG_E_INVALID
    assert lib.moe_expert_decode(h, xp, 5, 1, yp, None, None, None, None) == _lib.BDG_E_INVALID
    misaligned = ctypes.c_void_p(x.data_ptr() + 4)
    assert lib.moe_expert_decode(h, misaligned, _lib.BDG_F32, 1, yp, None, None, None, None) == _lib.BDG_E_ALIGN
    idx = torch.zeros((2, 2), dtype=torch.int32, device=dev)
    ip = ctypes.c_void_p(idx.data_ptr())
    assert lib.moe_experts_routed(h, 2, xp, _lib.BDG_F32, 1, ip, yp, yp, None) == _lib.BDG_E_INVALID
    assert lib.moe_experts_routed(h, -1, xp, _lib.BDG_F32, 1, ip, yp, yp, None) == _lib.BDG_E_INVALID
    assert lib.moe_experts_routed(h, 0, xp, _lib.BDG_F32, 3, ip, yp, yp, None) == _lib.BDG_E_INVALID
    torch.cuda.synchronize()
    assert torch.all(y == 7.0), "a rejected call wrote its output"
    # the binding refuses wrong shapes before the C call
    with pytest.raises(ValueError):
        bdg.moe_expert_decode(plan, torch.zeros((1, cfg.hidden + 32), device=dev))
    with pytest.raises(ValueError):
        bdg.moe_expert_decode(plan, torch.zeros((3, cfg.hidden), device=dev))
    with pytest.raises(ValueError):
        bdg.moe_expert_decode(plan, torch.zeros((1, cfg.hidden), device=dev),
                              y=torch.zeros((1, cfg.hidden - 32), device=dev))
    with pytest.raises(ValueError):
        bdg.moe_experts_routed(plan, 0, torch.zeros((1, cfg.hidden), device=dev),
                               torch.zeros((1, 3), dtype=torch.int32, device=dev),
                               torch.zeros((1, 2), device=dev))
    plan.close()
