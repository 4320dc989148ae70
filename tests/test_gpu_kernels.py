"""GPU parity: dequantisation (bit-exact), qgemv and the router vs the oracle.

All calls go through the C ABI of libbdg (via the ctypes binding).
"""

import numpy as np
import pytest
import torch

import bit_dequant_gemv_amd as bdg
import synth
from oracle import formats, gemv as ogemv, moe as omoe

from helpers import (ROUTER_REL, WEIGHT_ABS, assert_bit_exact, assert_close, banner, f32_bits,
                     to_np)
from test_oracle_formats import int4_exhaustive_inputs, mxfp4_exhaustive_inputs

pytestmark = pytest.mark.gpu


def dev_t(a, dev):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(dev)


# ---------------------------------------------------------------- dequant

def test_mxfp4_dequant_exhaustive(dev):
    codes, scales = mxfp4_exhaustive_inputs()
    banner("mxfp4_dequant exhaustive 16 codes x 256 E8M0")
    got = to_np(bdg.mxfp4_dequant(dev_t(codes, dev), dev_t(scales, dev)))
    torch.cuda.synchronize()
    assert_bit_exact(got, formats.mxfp4_dequant(codes, scales))


def test_mxfp4_dequant_bf16_output(dev):
    """bf16 output over all 16 codes x 256 E8M0: produced by the scaled FP4 ->
    bf16 conversion the matrix-core decode path uses, so this pins that
    instruction to the exact values (subnormals, -0, overflow to inf)."""
    codes, scales = mxfp4_exhaustive_inputs()
    got = bdg.mxfp4_dequant(dev_t(codes, dev), dev_t(scales, dev), out_dtype=torch.bfloat16)
    got_bits = to_np(got.view(torch.int16)).view(np.uint16)
    ref = formats.mxfp4_dequant(codes, scales)
    finite = ~np.isnan(ref)
    want_bits = synth.bf16_bits_of(ref)
    assert np.array_equal(got_bits[finite], want_bits[finite])
    assert np.all(np.isnan(synth.bf16_to_f32(got_bits[~finite])))


@pytest.mark.parametrize("index", [0, 1])
def test_mxfp4_dequant_full_gemv_matrix(dev, index):
    cfg = synth.CONFIGS["gemv_2880"]
    codes, scales = synth.gemv_matrix(cfg, index)
    banner(f"mxfp4_dequant 2880x2880 matrix {index}")
    got = to_np(bdg.mxfp4_dequant(dev_t(codes, dev), dev_t(scales, dev)))
    assert_bit_exact(got, formats.mxfp4_dequant(codes, scales))


@pytest.mark.parametrize("part", range(4))
def test_int4_dequant_exhaustive(dev, part):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)[part * 16384:(part + 1) * 16384]
    codes, scales, zeros = int4_exhaustive_inputs(bits)
    banner(f"int4g_dequant exhaustive slice {part}")
    got = to_np(bdg.int4g_dequant(dev_t(codes, dev), dev_t(scales, dev), dev_t(zeros, dev), 32))
    assert_bit_exact(got, formats.int4g_dequant(codes, scales, zeros, 32))


def test_int4_dequant_full_expert(dev):
    cfg = synth.CONFIGS["q4_30b_stack"]
    w = synth.expert_weights(cfg, 3, 17)
    for name in ("gu", "dn"):
        codes, scales, zeros = w[name]
        banner(f"int4g_dequant 30B expert {name} {codes.shape}")
        got = to_np(bdg.int4g_dequant(dev_t(codes, dev), dev_t(scales, dev), dev_t(zeros, dev), 64))
        assert_bit_exact(got, formats.int4g_dequant(codes, scales, zeros, 64))


def test_dequant_odd_group_count(dev):
    # k = 96, group 32 -> 3 groups (zero row of 2 bytes, last high nibble unused)
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 256, (5, 48), dtype=np.uint8)
    zeros = rng.integers(0, 256, (5, 2), dtype=np.uint8)
    scales = synth.fp16_bits_of(rng.uniform(-2, 2, (5, 3)))
    got = to_np(bdg.int4g_dequant(dev_t(codes, dev), dev_t(scales, dev), dev_t(zeros, dev), 32))
    assert_bit_exact(got, formats.int4g_dequant(codes, scales, zeros, 32))


# ---------------------------------------------------------------- qgemv

def mx_weight(codes, scales, dev):
    return bdg.QWeight("mxfp4", dev_t(codes, dev), dev_t(scales, dev))


def i4_weight(codes, scales, zeros, group, dev):
    return bdg.QWeight("int4g", dev_t(codes, dev), dev_t(scales, dev), dev_t(zeros, dev), group)


@pytest.mark.parametrize("index", range(4))
def test_qgemv_gemv_2880(dev, index):
    cfg = synth.CONFIGS["gemv_2880"]
    codes, scales = synth.gemv_matrix(cfg, index)
    x = synth.hidden(cfg, index)[0]
    banner(f"qgemv 2880x2880 MXFP4 matrix {index}")
    y = to_np(bdg.qgemv(mx_weight(codes, scales, dev), dev_t(x, dev)))
    y_ref, den = ogemv.gemv(formats.mxfp4_dequant(codes, scales), x)
    assert_close(y, y_ref, den, "qgemv")


@pytest.mark.parametrize("name", sorted(n for n, c in synth.DENSE.items() if c.m == 1))
@pytest.mark.parametrize("m", [1, 4])
def test_qgemv_dense_workloads(dev, name, m):
    """The dense non-expert shapes (201,088-row MXFP4 vocabulary head, 32768 x
    2048 int4) at full size, in the launch configuration the benchmark times
    (m = 1) and at m = 4: 512 sampled rows plus the first and last ones
    against the oracle (dequantized rows, fp64 products)."""
    cfg = synth.DENSE[name]
    arrs = synth.dense_matrix(cfg, 0)
    x, xbits = synth.hidden_batch(cfg, range(m))
    banner(f"qgemv dense {name} m={m}")
    if cfg.fmt == "mxfp4":
        qw = mx_weight(*arrs, dev)
    else:
        qw = i4_weight(*arrs, cfg.group, dev)
    y = to_np(bdg.qgemv(qw, dev_t(xbits, dev).view(torch.bfloat16)))   # bf16 input, as benchmarked
    rows = np.unique(np.concatenate([[0, cfg.n - 1], np.random.default_rng(cfg.base).integers(0, cfg.n, 512)]))
    if cfg.fmt == "mxfp4":
        w = formats.mxfp4_dequant(arrs[0][rows], arrs[1][rows])
    else:
        w = formats.int4g_dequant(arrs[0][rows], arrs[1][rows], arrs[2][rows], cfg.group)
    y_ref, den = ogemv.gemv(w, x)
    assert np.all(np.isfinite(y))
    assert_close(y[:, rows], y_ref, den, f"qgemv {name}")


@pytest.mark.parametrize("n,k", [(1, 32), (3, 96), (7, 288), (37, 768), (130, 2048), (65, 2880),
                                 (33, 5760), (9, 8192), (5, 1056)])
@pytest.mark.parametrize("fmt", ["mxfp4", "int4g"])
def test_qgemv_shapes(dev, n, k, fmt):
    group = 32 if (fmt == "mxfp4" or k % 64) else 64
    seed = n * 10007 + k
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    x = rng.standard_normal((3, k)).astype(np.float32)
    banner(f"qgemv {fmt} n={n} k={k} m=3")
    if fmt == "mxfp4":
        scales = rng.integers(118, 131, (n, k // 32), dtype=np.uint8)
        w = formats.mxfp4_dequant(codes, scales)
        qw = mx_weight(codes, scales, dev)
    else:
        g = k // group
        scales = synth.fp16_bits_of(rng.uniform(0.005, 0.02, (n, g)))
        zeros = rng.integers(0, 256, (n, (g + 1) // 2), dtype=np.uint8)
        w = formats.int4g_dequant(codes, scales, zeros, group)
        qw = i4_weight(codes, scales, zeros, group, dev)
    y = to_np(bdg.qgemv(qw, dev_t(x, dev)))
    y_ref, den = ogemv.gemv(w, x)
    assert_close(y, y_ref, den, f"qgemv {fmt} {n}x{k}")


def test_qgemv_integer_exact(dev):
    # scale 2^0 and integer x: every partial sum is a multiple of 0.5 below 2^24,
    # so any summation order is exact
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 256, (2880, 1440), dtype=np.uint8)
    scales = np.full((2880, 90), 127, dtype=np.uint8)
    x = rng.integers(-2, 3, 2880).astype(np.float32)
    y = to_np(bdg.qgemv(mx_weight(codes, scales, dev), dev_t(x, dev)))
    y_ref, _ = ogemv.gemv(formats.mxfp4_dequant(codes, scales), x)
    assert np.array_equal(y.astype(np.float64), y_ref)


def test_qgemv_onehot_columns(dev):
    rng = np.random.default_rng(8)
    codes = rng.integers(0, 256, (96, 1440), dtype=np.uint8)
    scales = rng.integers(110, 140, (96, 90), dtype=np.uint8)
    w = formats.mxfp4_dequant(codes, scales)
    qw = mx_weight(codes, scales, dev)
    cols = [0, 31, 32, 1439, 2879]
    x = np.zeros((len(cols), 2880), dtype=np.float32)
    for i, c in enumerate(cols):
        x[i, c] = 1.0
    y = to_np(bdg.qgemv(qw, dev_t(x, dev)))
    for i, c in enumerate(cols):
        assert np.array_equal(y[i], w[:, c])      # value equality (a sum's zero sign is free)


def test_qgemv_bf16_x_equals_f32_x(dev):
    cfg = synth.CONFIGS["gemv_2880"]
    codes, scales = synth.gemv_matrix(cfg, 0)
    vals, bits = synth.hidden(synth.CONFIGS["gptoss20b_layer"], 5)
    qw = mx_weight(codes, scales, dev)
    y_bf = bdg.qgemv(qw, dev_t(bits, dev).view(torch.bfloat16))
    y_f = bdg.qgemv(qw, dev_t(vals, dev))
    assert torch.equal(y_bf, y_f)


def test_qgemv_m16_and_repeatable(dev):
    cfg = synth.CONFIGS["gemv_2880"]
    codes, scales = synth.gemv_matrix(cfg, 2)
    x = np.stack([synth.hidden(cfg, t)[0] for t in range(16)])
    qw = mx_weight(codes, scales, dev)
    y1 = bdg.qgemv(qw, dev_t(x, dev))
    y2 = torch.full_like(y1, float("nan"))
    bdg.qgemv(qw, dev_t(x, dev), out=y2)          # rerun into a dirty buffer
    assert torch.equal(y1, y2)
    y_ref, den = ogemv.gemv(formats.mxfp4_dequant(codes, scales), x)
    assert_close(to_np(y1), y_ref, den, "qgemv m=16")


def test_qgemv_rejects_bad_args(dev):
    codes = torch.zeros((4, 16), dtype=torch.uint8, device=dev)
    scales = torch.zeros((4, 1), dtype=torch.uint8, device=dev)
    qw = bdg.QWeight("mxfp4", codes, scales)
    x = torch.zeros((17, 32), device=dev)
    with pytest.raises(Exception):
        bdg.qgemv(qw, x)                          # m > 16
    with pytest.raises(ValueError):
        bdg.qgemv(qw, torch.zeros(64, device=dev))


# ---------------------------------------------------------------- router

@pytest.mark.parametrize("E,k,H,norm", [(32, 4, 2880, False), (128, 8, 2048, True),
                                        (128, 4, 2880, True), (7, 7, 64, False), (300, 32, 512, True)])
def test_router_topk(dev, E, k, H, norm):
    cfg = synth.MoEConfig(name="r", base=700 + E, fmt="mxfp4", n_layers=1, hidden=H, inter=64,
                          n_experts=E, top_k=k)
    w_r, _, _ = synth.router(cfg, 0)
    b = synth.random_input(E, (E,)) if E == 300 else None
    x = np.stack([synth.hidden(cfg, t)[0] for t in range(5)]) * 3.0
    banner(f"moe_router_topk E={E} k={k} H={H} norm={norm}")
    idx, wts, logits = bdg.moe_router_topk(dev_t(x, dev), dev_t(w_r, dev),
                                           dev_t(b, dev) if b is not None else None, k,
                                           rmsnorm=norm)
    idx, wts, logits = to_np(idx), to_np(wts), to_np(logits)
    xin = omoe.rmsnorm(x) if norm else x.astype(np.float64)
    ref, scale = omoe.router_logits(w_r, xin, b)
    assert np.all(np.abs(logits - ref) <= ROUTER_REL * scale + 1e-30)
    # exact top-k on the GPU's own fp32 logits
    o_idx, o_w = omoe.topk_softmax(logits.astype(np.float64), k)
    assert np.array_equal(idx, o_idx)
    assert np.max(np.abs(wts - o_w)) <= WEIGHT_ABS
    # end to end vs the oracle's fp64 logits, modulo the near-tie band
    for t in range(x.shape[0]):
        ok, _, msg = omoe.check_routing(ref[t], scale[t], idx[t], k)
        assert ok, msg


@pytest.mark.parametrize("m,norm", [(64, False), (203, True), (1500, True), (4100, False), (4100, True)])
def test_router_topk_many_tokens(dev, m, norm):
    """Many tokens in one call (m = 64 and 203: blocks of one token; 1500:
    of 4; 4100: of 16, the last one ragged): logits, picks and weights must
    equal those of one-token calls bit for bit (the same sums in the same
    order), and the logits the oracle's within the router tolerance."""
    E, k, H = 32, 4, 2880
    cfg = synth.MoEConfig(name="r", base=760, fmt="mxfp4", n_layers=1, hidden=H, inter=64, n_experts=E, top_k=k)
    w_r, _, _ = synth.router(cfg, 0)
    x = np.stack([synth.hidden(cfg, t)[0] for t in range(m)])
    banner(f"moe_router_topk many tokens m={m} norm={norm}")
    xt, wt = dev_t(x, dev), dev_t(w_r, dev)
    idx, wts, logits = (to_np(a) for a in bdg.moe_router_topk(xt, wt, None, k, rmsnorm=norm))
    for t in sorted({0, 1, 5, 15, 16, 63, m // 2 + 7, m - 2, m - 1}):
        i1, w1, l1 = (to_np(a) for a in bdg.moe_router_topk(xt[t:t + 1].contiguous(), wt, None, k, rmsnorm=norm))
        assert np.array_equal(f32_bits(l1[0]), f32_bits(logits[t]))
        assert np.array_equal(i1[0], idx[t]) and np.array_equal(f32_bits(w1[0]), f32_bits(wts[t]))
    xin = omoe.rmsnorm(x) if norm else x.astype(np.float64)
    ref, scale = omoe.router_logits(w_r, xin)
    assert np.all(np.abs(logits - ref) <= ROUTER_REL * scale + 1e-30)


def test_router_ties_lower_index(dev):
    E, H = 16, 64
    w_r = np.zeros((E, H), dtype=np.float32)
    w_r[5] = 1.0 / 64
    w_r[9] = 1.0 / 64           # experts 5 and 9 tie, everything else 0
    x = np.ones((1, H), dtype=np.float32)
    idx, wts, logits = bdg.moe_router_topk(dev_t(x, dev), dev_t(w_r, dev), None, 4)
    assert list(to_np(idx)[0]) == [5, 9, 0, 1]
    e1 = np.exp(np.float32(-1.0))
    np.testing.assert_allclose(to_np(wts)[0], np.array([1, 1, e1, e1]) / (2 + 2 * e1), atol=1e-7)


@pytest.mark.parametrize("E,k", [(16, 4), (128, 8), (300, 32), (1024, 32)])
def test_router_topk_ties_nan_inf(dev, E, k):
    """Logits made of the bias alone (zero router rows) from a tiny value set:
    long runs of equal logits, -inf and NaN.  Picks must come out in
    descending order with ties to the lower index; NaN ranks as -inf, and
    more than k logits are finite, so neither is ever picked."""
    H = 64
    rng = np.random.default_rng(E)
    b = rng.choice(np.array([2.0, 1.0, 1.0, 0.5, 0.5, -np.inf, np.nan], dtype=np.float32), size=E)
    b[rng.choice(E, size=k + 1, replace=False)] = 0.25     # at least k+1 finite logits
    w_r = np.zeros((E, H), dtype=np.float32)
    x = synth.random_input(E, (3, H))
    banner(f"moe_router_topk ties/nan/inf E={E} k={k}")
    idx, wts, logits = bdg.moe_router_topk(dev_t(x, dev), dev_t(w_r, dev), dev_t(b, dev), k)
    idx, wts = to_np(idx), to_np(wts)
    finite = np.where(np.isnan(b), -np.inf, b).astype(np.float64)
    o_idx, o_w = omoe.topk_softmax(np.tile(finite, (3, 1)), k)
    assert np.array_equal(idx, o_idx)
    assert np.max(np.abs(wts - o_w)) <= WEIGHT_ABS
