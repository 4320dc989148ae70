"""GPU parity of the large-M path: MXFP8 activation quantization (bit-exact
against the oracle) and the MXFP4 x MXFP8 product on the MX-scaled matrix
cores (within a tolerance relative to sum |W| |xq|).

All calls go through the C ABI of libbdg (via the ctypes binding).
"""

import numpy as np
import pytest
import torch

import bit_dequant_gemv_amd as bdg
import synth
from oracle import mxq

from bit_dequant_gemv_amd._lib import BdgError
from helpers import banner, to_np

pytestmark = pytest.mark.gpu

# The MX-scaled MFMA adds the 64 products of one instruction at reduced
# internal precision: a single instruction on random FP4 x FP8 data showed
# errors up to 1.02e-4 of its sum |products| (against ~1e-7 for fp32
# accumulation).  Chained over K / 64 instructions (fp32 accumulator) the
# error stays within the same fraction of the whole sum |W| |xq|, so the
# product is held to 4e-4 of it (a 4x margin) and to cosine >= 0.9999.
MX_REL_TOL = 4e-4
MX_COS_TOL = 0.9999


def dev_t(a, dev):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(dev)


def quantize_dev(x, dev, bf16=False):
    if bf16:
        bits = synth.bf16_bits_of(x)
        xt = dev_t(bits, dev).view(torch.bfloat16)
    else:
        xt = dev_t(np.asarray(x, dtype=np.float32), dev)
    c, s = bdg.mxfp8_quantize(xt)
    return to_np(c), to_np(s)


def block_cases(rng):
    """Rows of 32-element blocks that reach every branch of the conversion."""
    vals = mxq.e4m3_value(np.arange(0x7F))
    rows = []
    for X in (-20, -8, 0, 3):
        mids = (vals[:-1] + vals[1:]) / 2                   # every tie, in one binade set
        for i in range(0, len(mids), 31):
            blk = np.zeros(32)
            blk[0] = 448.0                                   # fixes X
            part = mids[i:i + 31]
            blk[1:1 + len(part)] = part * rng.choice([-1, 1], len(part))
            rows.append(blk * 2.0 ** X)
    sat = np.array([511.9, 464.0, 463.99, 480.0, -500.0, 448.0] + [1.0] * 26)   # saturation
    rows.append(sat)
    rows.append(np.zeros(32))
    rows.append(-np.zeros(32))
    tiny = np.zeros(32)
    tiny[:4] = [2.0 ** -140, -2.0 ** -135, 1e-39, -1e-42]   # subnormal amax
    rows.append(tiny)
    # subnormal range: j * 2^-10 for j = 1..31 (odd j are ties between
    # neighbouring multiples of 2^-9), with the block scale fixed at 2^-2
    sub = np.arange(32) * 2.0 ** -10
    sub[0] = 448.0
    rows.append(sub * 2.0 ** -2)
    return np.stack(rows)


def test_mxfp8_quantize_special_blocks(dev):
    rng = np.random.default_rng(1)
    x = block_cases(rng).astype(np.float32)      # both sides quantize these fp32 values
    banner(f"mxfp8_quantize special blocks {x.shape}")
    c, s = quantize_dev(x, dev)
    oc, os_ = mxq.mxfp8_quantize(x)
    assert np.array_equal(s, os_)
    assert np.array_equal(c, oc), np.argwhere(c != oc)[:8]


def test_mxfp8_quantize_non_finite(dev):
    x = np.zeros((3, 64), dtype=np.float32)
    x[0, 5] = np.nan
    x[1, 40] = np.inf
    x[2, :] = np.linspace(-3, 3, 64)
    banner("mxfp8_quantize non-finite blocks")
    c, s = quantize_dev(x, dev)
    oc, os_ = mxq.mxfp8_quantize(x)
    assert np.array_equal(s, os_) and np.array_equal(c, oc)
    assert s[0, 0] == 255 and s[0, 1] == 0 and s[1, 1] == 255


@pytest.mark.parametrize("m,k", [(1, 32), (3, 96), (17, 2880), (64, 2048), (300, 5760)])
@pytest.mark.parametrize("bf16", [False, True])
def test_mxfp8_quantize_random(dev, m, k, bf16):
    rng = np.random.default_rng(m * 131 + k)
    # per-row magnitudes over many binades
    x = (rng.standard_normal((m, k)) * np.exp(rng.uniform(-12, 12, (m, 1)))).astype(np.float32)
    if bf16:
        x = synth.bf16_to_f32(synth.bf16_bits_of(x))
    banner(f"mxfp8_quantize m={m} k={k} bf16={bf16}")
    c, s = quantize_dev(x, dev, bf16)
    oc, os_ = mxq.mxfp8_quantize(x)
    assert np.array_equal(s, os_)
    assert np.array_equal(c, oc), np.argwhere(c != oc)[:8]


def mx_weight(codes, scales, dev):
    return bdg.QWeight("mxfp4", dev_t(codes, dev), dev_t(scales, dev))


def check_gemm(y, yref, den, what):
    rel = float(np.max(np.abs(y - yref) / np.maximum(den, 1e-30)))
    a, b = y.ravel().astype(np.float64), yref.ravel()
    cos = float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b) + 1e-300))
    banner(f"{what}: max |err| / den {rel:.3e}, cosine {cos:.9f}")
    assert np.all(np.isfinite(y))
    assert rel <= MX_REL_TOL, f"{what}: {rel:.3e}"
    assert cos >= MX_COS_TOL, f"{what}: cosine {cos}"


@pytest.mark.parametrize("n,m,k", [(32, 32, 64), (64, 1, 32), (33, 5, 96), (100, 37, 2880), (130, 129, 2048),
                                   (257, 70, 4096)])
def test_mx_gemm_shapes(dev, n, m, k):
    """Ragged rows, tokens and K (an odd number of 32-blocks) against the
    oracle's product of the same quantized activations."""
    rng = np.random.default_rng(n * 7 + m * 11 + k)
    wc = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    ws = rng.integers(118, 129, (n, k // 32), dtype=np.uint8)
    x = rng.standard_normal((m, k)).astype(np.float32)
    banner(f"mx_gemm n={n} m={m} k={k}")
    c, s = quantize_dev(x, dev)
    oc, os_ = mxq.mxfp8_quantize(x)
    assert np.array_equal(c, oc) and np.array_equal(s, os_)
    y = to_np(bdg.mx_gemm(mx_weight(wc, ws, dev), dev_t(c, dev), dev_t(s, dev)))
    yref, den = mxq.mx_gemm(wc, ws, oc, os_)
    check_gemm(y, yref, den, f"mx_gemm {n}x{k} m={m}")


def test_mx_gemm_one_hot(dev):
    """A one-hot activation row picks one weight column exactly: each output
    is a single product (no rounding anywhere)."""
    n, k = 64, 128
    rng = np.random.default_rng(9)
    wc = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    ws = rng.integers(120, 127, (n, k // 32), dtype=np.uint8)
    x = np.zeros((k, k), dtype=np.float32)
    np.fill_diagonal(x, 1.0)
    c, s = quantize_dev(x, dev)
    oc, os_ = mxq.mxfp8_quantize(x)
    assert np.array_equal(c, oc) and np.array_equal(s, os_)
    y = to_np(bdg.mx_gemm(mx_weight(wc, ws, dev), dev_t(c, dev), dev_t(s, dev)))
    yref, _ = mxq.mx_gemm(wc, ws, oc, os_)
    assert np.array_equal(y, yref.astype(np.float32))


def test_mx_gemm_expert_shape_full(dev):
    """A gpt-oss expert's gate_up (5760 x 2880 MXFP4) over 512 tokens, the
    prefill configuration the benchmark times: 64 sampled tokens x all rows."""
    cfg = synth.CONFIGS["gptoss20b_layer"]
    w = synth.expert_weights(cfg, 0, 0)["gu"]
    m = 512
    x = synth.hidden_batch(cfg, range(m))[0]
    banner("mx_gemm 5760x2880 m=512")
    xt = dev_t(synth.bf16_bits_of(x), dev).view(torch.bfloat16)
    c, s = bdg.mxfp8_quantize(xt)
    y = to_np(bdg.mx_gemm(mx_weight(*w, dev), c, s))
    c, s = to_np(c), to_np(s)
    toks = np.random.default_rng(2).choice(m, 64, replace=False)
    oc, os_ = mxq.mxfp8_quantize(x[toks])
    assert np.array_equal(c[toks], oc) and np.array_equal(s[toks], os_)
    yref, den = mxq.mx_gemm(*w, oc, os_)
    check_gemm(y[toks], yref, den, "mx_gemm expert shape")


def test_mx_rejects_bad_args(dev):
    w = mx_weight(np.zeros((32, 32), dtype=np.uint8), np.full((32, 2), 127, dtype=np.uint8), dev)
    c = torch.zeros((4, 64), dtype=torch.uint8, device=dev)
    with pytest.raises(ValueError):
        bdg.mx_gemm(w, c, torch.zeros((4, 1), dtype=torch.uint8, device=dev))
    with pytest.raises(BdgError):
        bdg.mxfp8_quantize(torch.zeros((2, 48), dtype=torch.float32, device=dev))
