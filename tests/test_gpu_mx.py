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
from synth import device as sdev

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


def test_mx_gemm_wide_blocks_ragged(dev):
    """Enough tiles for the 128-token blocks (17 row tiles x 32 token tiles on
    256 CUs): ragged rows and tokens and a partial last K stage (K = 160,
    five 32-blocks), every output against the oracle."""
    n, m, k = 4100, 3970, 160
    rng = np.random.default_rng(77)
    wc = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    ws = rng.integers(118, 129, (n, k // 32), dtype=np.uint8)
    x = rng.standard_normal((m, k)).astype(np.float32)
    c, s = quantize_dev(x, dev)
    w = mx_weight(wc, ws, dev)
    w.stage_mx_scales()
    banner(f"mx_gemm wide blocks n={n} m={m} k={k}")
    y = to_np(bdg.mx_gemm(w, dev_t(c, dev), dev_t(s, dev)))
    yref, den = mxq.mx_gemm(wc, ws, c, s)
    check_gemm(y, yref, den, "mx_gemm wide blocks")


def test_mx_gemm_benchmark_size(dev):
    """The benchmarked dense product at full size: a gpt-oss expert's gate_up
    (5760 x 2880 MXFP4, scale words staged once) over 4096 tokens, in the
    launch configuration the benchmark times (128-token blocks); 64 sampled
    tokens x all rows against the oracle."""
    cfg = synth.CONFIGS["gptoss20b_layer"]
    w = synth.expert_weights(cfg, 0, 0)["gu"]
    m = 4096
    x = synth.hidden_batch(cfg, range(m))[0]
    banner("mx_gemm 5760x2880 m=4096")
    xt = dev_t(synth.bf16_bits_of(x), dev).view(torch.bfloat16)
    c, s = bdg.mxfp8_quantize(xt)
    qw = mx_weight(*w, dev)
    qw.stage_mx_scales()
    y = to_np(bdg.mx_gemm(qw, c, s))
    c, s = to_np(c), to_np(s)
    toks = np.random.default_rng(3).choice(m, 64, replace=False)
    oc, os_ = mxq.mxfp8_quantize(x[toks])
    assert np.array_equal(c[toks], oc) and np.array_equal(s[toks], os_)
    yref, den = mxq.mx_gemm(*w, oc, os_)
    check_gemm(y[toks], yref, den, "mx_gemm benchmark size")


def test_mx_rejects_bad_args(dev):
    w = mx_weight(np.zeros((32, 32), dtype=np.uint8), np.full((32, 2), 127, dtype=np.uint8), dev)
    c = torch.zeros((4, 64), dtype=torch.uint8, device=dev)
    with pytest.raises(ValueError):
        bdg.mx_gemm(w, c, torch.zeros((4, 1), dtype=torch.uint8, device=dev))
    xb = torch.zeros((2, 48), dtype=torch.float32, device=dev)
    with pytest.raises(ValueError):
        bdg.mxfp8_quantize(xb)                    # the binding refuses k % 32 != 0
    from bit_dequant_gemv_amd import _lib
    import ctypes
    cb = torch.zeros((2, 48), dtype=torch.uint8, device=dev)
    assert _lib.load().mxfp8_quantize(ctypes.c_void_p(xb.data_ptr()), _lib.BDG_F32, 2, 48,
                                      ctypes.c_void_p(cb.data_ptr()), ctypes.c_void_p(cb.data_ptr()),
                                      None) == _lib.BDG_E_INVALID   # and so does the library


@pytest.mark.parametrize("E,n,k", [(1, 37, 96), (3, 70, 2880), (2, 256, 4096), (2, 21, 4224), (1, 40, 8192)])
def test_mx_stage_scales_layout(dev, E, n, k):
    """mx_stage_scales against its layout written out: word [e][s][r] holds
    row r's scale bytes of K blocks 4s .. 4s+3 (byte q = block 4s + q), 127
    past K (K = 96: 3 blocks, one padded byte; 2880: 90 blocks, two; 4224:
    33 stages, two chunks of the staging kernel's 32, the last of one; 8192:
    the largest K, 64 stages)."""
    rng = np.random.default_rng(E * 1000 + n + k)
    kb, S = k // 32, (k // 32 + 3) // 4
    sc = rng.integers(0, 256, (E, n, kb), dtype=np.uint8)
    codes = np.zeros((E, n, k // 2), dtype=np.uint8)
    if E == 1:
        w = bdg.QWeight("mxfp4", dev_t(codes[0], dev), dev_t(sc[0], dev))
    else:
        w = bdg.QWeight("mxfp4", dev_t(codes, dev), dev_t(sc, dev))
    w.stage_mx_scales()
    got = to_np(w.scale_words).view(np.uint8).reshape(E, S, n, 4)
    want = np.full((E, S, n, 4), 127, dtype=np.uint8)
    for s_ in range(S):
        for q in range(4):
            if 4 * s_ + q < kb:
                want[:, s_, :, q] = sc[:, :, 4 * s_ + q]
    assert np.array_equal(got, want)


@pytest.mark.parametrize("n,m,k", [(33, 5, 96), (100, 37, 2880), (257, 70, 4096), (70, 40, 4224), (70, 40, 8192)])
def test_mx_gemm_staged_scale_words(dev, n, m, k):
    """Weights with their stage-major scale copy staged once give the same
    product, bit for bit, as the per-call staging (and the oracle's)."""
    rng = np.random.default_rng(n * 13 + m * 5 + k)
    wc = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    ws = rng.integers(118, 129, (n, k // 32), dtype=np.uint8)
    x = rng.standard_normal((m, k)).astype(np.float32)
    c, s = quantize_dev(x, dev)
    w = mx_weight(wc, ws, dev)
    y0 = bdg.mx_gemm(w, dev_t(c, dev), dev_t(s, dev)).clone()
    w.stage_mx_scales()
    banner(f"mx_gemm with staged scale words n={n} m={m} k={k}")
    y1 = bdg.mx_gemm(w, dev_t(c, dev), dev_t(s, dev))
    assert torch.equal(y0, y1)
    yref, den = mxq.mx_gemm(wc, ws, c, s)
    check_gemm(to_np(y1), yref, den, f"mx_gemm staged {n}x{k} m={m}")


# ---------------------------------------------------------------- grouped prefill layer

# Checking the layer.  h is computed on the matrix cores (sums at reduced
# precision, within MX_REL_TOL of their sum |terms| as the mx_gemm tests hold
# every MX product to) and then quantized to MXFP8, so an element of h near a
# rounding boundary - or a block maximum near a power of two - can take the
# neighbouring code on the GPU: the quantized h is not unique.  The test
# derives how far it may move and checks three things:
# (1) every GPU code of h lies within the requantization spread of the
#     oracle's own (mxq.mxfp8_requant_spread: the worst case over every h'
#     within the error bound herr of the float64 h), and the codes equal the
#     oracle's rounding almost everywhere;
# (2) teacher forcing: the oracle's down product and combine on the GPU's
#     validated codes, y within the matrix cores' product error MX_LAYER_TOL
#     of den = sum_j w_j |W_d| |hq|;
# (3) end to end against the oracle's own quantization: |y - y_o| <=
#     sum_j w_j |W_d| spread_j (h codes that may differ) + MX_REL_TOL sum_j
#     w_j |W_d| (|hq_o| + spread_j) (the GPU's down product) + the router
#     weight error times |d|, plus fp32 rounding of the combine.
# herr: |dg| <= T gd_g, |du| <= T gd_u (T = MX_REL_TOL, gd = sum |xq| |w|),
# carried through h = silu(g) u with |silu'| <= 1.1 and |silu''| <= 0.5:
# |dh| <= |silu'(g)| |u| dg + |silu(g)| du + 0.5 |u| dg^2 + 1.1 dg du.
MX_LAYER_TOL = 5e-4
W_ERR = 1e-5            # router weights (fp32 softmax) vs the oracle's float64


def _h_error_bound(gu, gd, inter):
    g, u = gu[:, :inter], gu[:, inter:]
    dg, du = MX_REL_TOL * gd[:, :inter], MX_REL_TOL * gd[:, inter:]
    sig = 1.0 / (1.0 + np.exp(-g))
    d1 = np.abs(sig * (1.0 + g * (1.0 - sig)))
    return d1 * np.abs(u) * dg + np.abs(g * sig) * du + 0.5 * np.abs(u) * dg * dg + 1.1 * dg * du


def _prefill_case(dev, name, E, k, H, I, m, base, sample=None, staged=False):
    """sample: check the h codes and outputs of this many seeded tokens
    (routing, weights and grouping of every token are always checked).
    staged: the weights' stage-major scale words made once beforehand (as
    the benchmark does) instead of by the call."""
    from oracle import formats, moe as omoe
    cfg = synth.MoEConfig(name=name, base=base, fmt="mxfp4", n_layers=1, hidden=H, inter=I, n_experts=E,
                          top_k=k, norm=False, m=m)
    layer = sdev.upload_layer(cfg, 0, dev)
    if staged:
        layer["gate_up"].stage_mx_scales()
        layer["down"].stage_mx_scales()
    x, xv = sdev.hidden_device(cfg, range(m), dev)
    banner(f"moe_prefill_mx {name} E={E} k={k} H={H} I={I} m={m}{' staged scale words' if staged else ''}")
    ws = torch.empty(bdg.prefill_workspace_bytes(m, H, I, E, k), dtype=torch.uint8, device=dev)
    y, idx, wts = bdg.moe_prefill_mx(layer, E, k, x, workspace=ws)
    torch.cuda.synchronize()
    views = {n: to_np(v) for n, v in bdg.prefill_workspace_views(ws, m, H, I, E, k).items()}
    y, idx, wts = to_np(y), to_np(idx), to_np(wts)
    w_r, b_r, _ = synth.router(cfg, 0)
    # routing of every token (fp64 logits, near-tie band), its weights and the grouping
    logits, scale = omoe.router_logits(w_r, xv, b_r)
    for t in range(m):
        ok, _, msg = omoe.check_routing(logits[t], scale[t], idx[t], k)
        assert ok, f"token {t}: {msg}"
    w_o = np.stack([omoe.softmax_over(logits[t], idx[t]) for t in range(m)])
    assert np.max(np.abs(wts - w_o)) <= W_ERR
    oc, os_ = mxq.mxfp8_quantize(xv)
    assert np.array_equal(views["xq"], oc) and np.array_equal(views["xq_scales"], os_)
    pick_row = views["pick_row"]
    assert np.array_equal(np.sort(pick_row), np.arange(m * k))
    assert np.array_equal(views["row_src"][pick_row], np.repeat(np.arange(m), k))
    if sample is None or sample >= m:
        toks_chk = np.arange(m)
    else:
        toks_chk = np.sort(np.random.default_rng(base).choice(m, sample, replace=False))
    sel = np.zeros(m, dtype=bool)
    sel[toks_chk] = True

    def get_packed(e):
        wts_e = synth.expert_weights(cfg, 0, e)
        return wts_e["gu"], wts_e["dn"]
    xq = mxq.mxfp8_dequant64(oc, os_)
    mc = len(toks_chk)
    pos = np.full(m, -1)
    pos[toks_chk] = np.arange(mc)
    y_tf, den_tf = np.zeros((mc, H)), np.zeros((mc, H))
    y_o, bound = np.zeros((mc, H)), np.zeros((mc, H))
    n_codes = n_diff = 0
    for e in np.unique(idx[toks_chk]):
        (gc, gs), (dc, ds) = get_packed(int(e))
        w_gu = formats.mxfp4_dequant64(gc, gs)
        w_d = formats.mxfp4_dequant64(dc, ds)
        toks, slots = np.nonzero((idx == e) & sel[:, None])
        gu = xq[toks] @ w_gu.T
        gd = np.abs(xq[toks]) @ np.abs(w_gu).T
        h = omoe.swiglu(gu, I)
        herr = _h_error_bound(gu, gd, I)
        hc_o, hs_o = mxq.mxfp8_quantize(h)
        hq_o = mxq.mxfp8_dequant64(hc_o, hs_o)
        spread = mxq.mxfp8_requant_spread(h, herr)
        rows = pick_row[toks * k + slots]
        hc_g, hs_g = views["hq"][rows], views["hq_scales"][rows]
        hq_g = mxq.mxfp8_dequant64(hc_g, hs_g)
        bad = np.abs(hq_g - hq_o) > spread
        assert not bad.any(), (f"expert {e}: {int(bad.sum())} h codes outside the requantization spread")
        n_codes += hc_g.size
        n_diff += int(np.count_nonzero(hc_g != hc_o))
        wt_g = wts[toks, slots][:, None].astype(np.float64)
        wt_o = w_o[toks, slots][:, None]
        abs_wd = np.abs(w_d)
        d_o = hq_o @ w_d.T
        p = pos[toks]
        np.add.at(y_tf, p, wt_o * (hq_g @ w_d.T))
        np.add.at(den_tf, p, np.abs(wt_o) * (np.abs(hq_g) @ abs_wd.T))
        np.add.at(y_o, p, wt_o * d_o)
        np.add.at(bound, p, np.abs(wt_g) * (spread @ abs_wd.T)
                  + MX_REL_TOL * np.abs(wt_g) * ((np.abs(hq_o) + spread) @ abs_wd.T)
                  + W_ERR * np.abs(d_o) + 1e-6 * np.abs(wt_g) * (np.abs(hq_o) @ abs_wd.T))
    frac = n_diff / n_codes
    yc = y[toks_chk].astype(np.float64)
    rel = float(np.max(np.abs(yc - y_tf) / np.maximum(den_tf, 1e-30)))
    cos = float(yc.ravel() @ y_tf.ravel() / (np.linalg.norm(yc) * np.linalg.norm(y_tf)))
    e2e = float(np.max(np.abs(yc - y_o) / np.maximum(bound, 1e-30)))
    banner(f"moe_prefill_mx {name}: {mc} tokens checked; h codes differing from the oracle's rounding "
           f"{frac:.2e}; y vs teacher-forced {rel:.3e} of den (cosine {cos:.9f}); end to end "
           f"{e2e:.3f} of the derived bound")
    assert frac <= 0.01
    assert np.all(np.isfinite(y))
    assert rel <= MX_LAYER_TOL and cos >= 0.99999
    assert e2e <= 1.0, f"end-to-end error {e2e:.3f} x the derived bound"


@pytest.mark.parametrize("m", [1, 37, 300])
def test_moe_prefill_small(dev, m):
    """Ragged token tiles, experts with no picks (m = 1) and several tiles."""
    _prefill_case(dev, "prefill_small", 8, 2, 256, 128, m, 2100 + m)


def test_moe_prefill_many_picks(dev):
    """More picks (4200 tokens x top-4 = 16,800) than the grouping kernel
    assembles in LDS, so it takes its looped path; outputs of 256 sampled
    tokens."""
    _prefill_case(dev, "prefill_many_picks", 16, 4, 256, 128, 4200, 2150, sample=256)


def test_moe_prefill_heavy_sharing(dev):
    """Every token on both experts: 300 grouped rows per expert (3 token tiles)."""
    _prefill_case(dev, "prefill_share", 2, 2, 384, 160, 300, 2200)


def test_moe_prefill_gptoss_layer(dev):
    """The gpt-oss-20B layer shape (32 experts, top-4, 2880 x 2880) over 512
    tokens, the weights' scale words staged once."""
    _prefill_case(dev, "prefill_20b", 32, 4, 2880, 2880, 512, 2300, staged=True)


def test_moe_prefill_benchmark_size(dev):
    """The benchmarked prefill workload at full size: the bare gpt-oss-20B
    layer over 4096 tokens, in the launch configuration the benchmark times
    (the weights' scale words staged once).  Routing, weights and grouping of
    all 4096 tokens; h codes and outputs of 384 sampled tokens."""
    pc = synth.PREFILL["gptoss20b_prefill"]
    _prefill_case(dev, "prefill_20b_4096", 32, 4, 2880, 2880, pc.m, pc.base, sample=384, staged=True)


def test_moe_prefill_staged_scale_words_bit_identical(dev):
    """The same layer with its weights' scale words staged once and staged by
    the call: identical outputs, routing weights and picks (H = 320 and
    I = 224 leave the last K stage of both products partial)."""
    cfg = synth.MoEConfig(name="pf_staged", base=2400, fmt="mxfp4", n_layers=1, hidden=320, inter=224,
                          n_experts=8, top_k=2, norm=False, m=150)
    layer = sdev.upload_layer(cfg, 0, dev)
    x, _ = sdev.hidden_device(cfg, range(cfg.m), dev)
    ws = torch.empty(bdg.prefill_workspace_bytes(cfg.m, 320, 224, 8, 2), dtype=torch.uint8, device=dev)
    banner("moe_prefill_mx staged vs per-call scale words")
    out0 = [t.clone() for t in bdg.moe_prefill_mx(layer, 8, 2, x, workspace=ws)]
    layer["gate_up"].stage_mx_scales()
    layer["down"].stage_mx_scales()
    out1 = bdg.moe_prefill_mx(layer, 8, 2, x, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(out1[0]).all()
    for a, b in zip(out0, out1):
        assert torch.equal(a, b)


def test_moe_prefill_rejects_bad_args(dev):
    cfg = synth.MoEConfig(name="bad", base=1, fmt="mxfp4", n_layers=1, hidden=64, inter=32, n_experts=4,
                          top_k=2, norm=False, m=2)
    layer = sdev.upload_layer(cfg, 0, dev)
    x, _ = sdev.hidden_device(cfg, range(2), dev)
    small = torch.empty(16, dtype=torch.uint8, device=dev)
    with pytest.raises(ValueError):                # the binding checks the size first
        bdg.moe_prefill_mx(layer, 4, 2, x, workspace=small)
    with pytest.raises((ValueError, BdgError)):
        bdg.moe_prefill_mx(layer, 4, 5, x)         # k > E
    # the library itself rejects a short workspace before any launch
    import ctypes
    from bit_dequant_gemv_amd import _lib
    desc = _lib.LayerDesc()
    desc.w_router = layer["w_router"].data_ptr()
    desc.b_router = None
    desc.gate_up = layer["gate_up"].qmat()
    desc.down = layer["down"].qmat()
    y = torch.empty((2, 64), dtype=torch.float32, device=dev)
    idx = torch.empty((2, 2), dtype=torch.int32, device=dev)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    assert _lib.load().moe_prefill_mx(ctypes.byref(desc), 4, 2, p(x), _lib.BDG_BF16, 2, p(y), p(idx), p(y),
                                      p(small), 16, None) == _lib.BDG_E_INVALID
