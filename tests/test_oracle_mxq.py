"""Pins of the MXFP8 activation quantizer in oracle/mxq.py.

Each check is fixed by something other than the oracle's own code: the OFP8
table's named values, a brute-force nearest-value search written here over
all 127 non-negative finite E4M3 values, closed forms of the shared-scale
rule, and the spec's error bound for round-to-nearest.
"""

import os

import numpy as np
import pytest

from oracle import mxq

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_e4m3():
    rows = []
    for line in open(os.path.join(GOLDEN, "e4m3_ocp_ofp8.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        code, val = line.split()
        rows.append((int(code, 16), float(val)))
    return rows


def test_e4m3_named_values():
    for code, val in _golden_e4m3():
        got = mxq.e4m3_value(code)
        if np.isnan(val):
            assert np.isnan(got), hex(code)
        else:
            assert got == val and np.signbit(got) == np.signbit(val), hex(code)


def test_e4m3_bit_construction():
    # every code from its fields, written out independently: (-1)^s 2^(e-7) (1 + m/8),
    # e = 0: (-1)^s 2^-6 (m/8)
    for code in range(256):
        s, e, m = code >> 7, (code >> 3) & 0xF, code & 7
        if e == 15 and m == 7:
            assert np.isnan(mxq.e4m3_value(code))
            continue
        mag = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
        assert mxq.e4m3_value(code) == (-mag if s else mag)


def _brute_round(v):
    """Nearest non-negative E4M3 value by scanning all 127 of them; a tie
    takes the even code; beyond 448 saturate."""
    vals = [(c, mxq.e4m3_value(c)) for c in range(0x7F)]
    a = abs(v)
    if a >= 448.0:
        c = 0x7E
    else:
        best = min(abs(a - val) for _, val in vals)
        cands = [c for c, val in vals if abs(a - val) == best]
        c = [x for x in cands if x % 2 == 0][0] if len(cands) > 1 else cands[0]
    return c | (0x80 if np.signbit(v) else 0)


def test_e4m3_round_brute_force():
    rng = np.random.default_rng(7)
    vals = mxq.e4m3_value(np.arange(0x7F))
    mids = (vals[:-1] + vals[1:]) / 2                    # every tie
    samples = np.concatenate([
        vals, -vals, mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
        rng.uniform(-512, 512, 400), rng.uniform(-0.02, 0.02, 400), rng.uniform(-4, 4, 400),
        [448.0, 463.99, 464.0, 464.01, 500.0, 511.9, -480.0, 2 ** -10, -2 ** -10, 2 ** -10 * 1.0001, 1e-30, -1e-30],
    ])
    got = mxq.e4m3_round(samples)
    want = np.array([_brute_round(v) for v in samples], dtype=np.uint8)
    assert np.array_equal(got, want)


def test_scale_closed_form():
    # amax in [2^j, 2^(j+1)) -> X = j - 8, scale byte j - 8 + 127
    for j in (-20, -9, -1, 0, 1, 7, 8, 20, 100):
        for f in (1.0, 1.5, 1.999):
            x = np.zeros((1, 32))
            x[0, 5] = -f * 2.0 ** j
            _, s = mxq.mxfp8_quantize(x)
            assert s[0, 0] == j - 8 + 127
    # clamps: tiny amax -> byte 0; zero block -> byte 0 and zero codes
    x = np.zeros((2, 32))
    x[0, 0] = 2.0 ** -140
    c, s = mxq.mxfp8_quantize(x)
    assert s[0, 0] == 0 and s[1, 0] == 0 and not c[1].any()


def test_exact_blocks_round_trip():
    # a block whose elements are E4M3 values times 2^X, with amax in [256, 448] * 2^X
    rng = np.random.default_rng(3)
    vals = mxq.e4m3_value(np.arange(0x7F))
    for X in (-30, -8, 0, 5):
        codes = rng.integers(0, 0x7F, 32)
        codes[0] = 0x78 + rng.integers(0, 7)               # 256 .. 448
        sign = rng.integers(0, 2, 32)
        x = np.where(sign == 1, -vals[codes], vals[codes]) * 2.0 ** X
        c, s = mxq.mxfp8_quantize(x[None, :])
        assert s[0, 0] == X + 127
        assert np.array_equal(c[0] & 0x7F, codes)
        assert np.array_equal(mxq.mxfp8_dequant64(c, s)[0], x)


def test_error_bound():
    # round to nearest with 3 mantissa bits: |x - q| <= 2^-4 |x| in the normal
    # range of the block, <= 2^(X-10) below it
    rng = np.random.default_rng(11)
    x = rng.standard_normal((64, 256)) * np.exp(rng.uniform(-8, 8, (64, 1)))
    c, s = mxq.mxfp8_quantize(x)
    q = mxq.mxfp8_dequant64(c, s)
    X = np.repeat(s.astype(np.int64) - 127, 32, axis=1)
    # (values in [448, 512) * 2^X saturate: their error is |x| - 448 * 2^X)
    sat = np.abs(x) >= 448.0 * 2.0 ** X
    normal = (np.abs(x) >= 2.0 ** (X - 6)) & ~sat
    assert np.all(np.abs(x - q)[normal] <= 2.0 ** -4 * np.abs(x)[normal])
    sub = np.abs(x) < 2.0 ** (X - 6)
    assert np.all(np.abs(x - q)[sub] <= 2.0 ** (X[sub] - 10))
    assert np.all(np.abs(q)[sat] == 448.0 * 2.0 ** X[sat])
    # amax never saturates by more than the top quantum: |q| <= 448 * 2^X
    assert np.all(np.abs(q) <= 448.0 * 2.0 ** X)


def test_signs_and_non_finite():
    x = np.zeros((3, 32))
    x[0, :] = -0.0
    x[0, 1] = 1.0
    x[1, 3] = np.nan
    x[2, 7] = -np.inf
    c, s = mxq.mxfp8_quantize(x)
    assert c[0, 0] == 0x80 and c[0, 2] == 0x80            # -0.0 keeps its sign
    assert s[1, 0] == 255 and np.all(c[1] == 0x7F)
    assert s[2, 0] == 255 and np.all(c[2] == 0x7F)


@pytest.mark.parametrize("k", [32, 96, 2880])
def test_quantize_shapes(k):
    rng = np.random.default_rng(k)
    x = rng.standard_normal((5, k)).astype(np.float32)
    c, s = mxq.mxfp8_quantize(x)
    assert c.shape == (5, k) and s.shape == (5, k // 32) and c.dtype == np.uint8


def test_mx_gemm_brute_force():
    # tiny shapes by explicit loops over the decoded element values
    from oracle import formats
    rng = np.random.default_rng(5)
    n, m, k = 3, 2, 64
    wc = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    ws = rng.integers(120, 130, (n, k // 32), dtype=np.uint8)
    xc, xs = mxq.mxfp8_quantize(rng.standard_normal((m, k)))
    y, den = mxq.mx_gemm(wc, ws, xc, xs)
    for i in range(m):
        for j in range(n):
            acc = 0.0
            dd = 0.0
            for kk in range(k):
                nib = (wc[j, kk // 2] >> (4 * (kk % 2))) & 15
                w = formats.e2m1_value(nib) * 2.0 ** (int(ws[j, kk // 32]) - 127)
                xv = mxq.e4m3_value(xc[i, kk]) * 2.0 ** (int(xs[i, kk // 32]) - 127)
                acc += w * xv
                dd += abs(w * xv)
            assert y[i, j] == pytest.approx(acc, rel=1e-12, abs=1e-12)
            assert den[i, j] == pytest.approx(dd, rel=1e-12)


def _layer_case(seed, m=6, E=4, k=2, H=64, I=32):
    from oracle import formats
    rng = np.random.default_rng(seed)
    w_r = rng.standard_normal((E, H)) * 0.3
    packed = []
    for e in range(E):
        gu = (rng.integers(0, 256, (2 * I, H // 2), dtype=np.uint8), rng.integers(120, 127, (2 * I, H // 32), dtype=np.uint8))
        dn = (rng.integers(0, 256, (H, I // 2), dtype=np.uint8), rng.integers(120, 127, (H, I // 32), dtype=np.uint8))
        packed.append((gu, dn))
    x = rng.standard_normal((m, H))

    def get_packed(e):
        return packed[e]

    def get_deq(e):
        (gc, gs), (dc, ds) = packed[e]
        return formats.mxfp4_dequant64(gc, gs), formats.mxfp4_dequant64(dc, ds)
    return x, w_r, packed, get_packed, get_deq, k


def test_moe_layer_mx_close_to_unquantized():
    # MXFP8 keeps 3 mantissa bits: the quantized layer stays near the exact one
    # (same routing: both route on the unquantized x)
    from oracle import moe as omoe
    x, w_r, _, get_packed, get_deq, k = _layer_case(21)
    q = mxq.moe_layer_mx(x, w_r, get_packed, k)
    ref = omoe.moe_layer(x, w_r, get_deq, k)
    assert np.array_equal(q["idx"], ref["idx"])
    rel = np.max(np.abs(q["y"] - ref["y"]) / ref["den"])
    cos = np.dot(q["y"].ravel(), ref["y"].ravel()) / (np.linalg.norm(q["y"]) * np.linalg.norm(ref["y"]))
    assert rel < 0.25 and cos > 0.99
    assert not np.allclose(q["y"], ref["y"])          # the quantization is really applied


def test_moe_layer_mx_linear_in_down_scale():
    # raising every down-matrix E8M0 scale by one doubles each d exactly (the
    # quantized h does not depend on the down weights), so y doubles exactly
    x, w_r, packed, get_packed, _, k = _layer_case(22)
    q1 = mxq.moe_layer_mx(x, w_r, get_packed, k)
    packed2 = [(gu, (dc, ds + 1)) for gu, (dc, ds) in packed]
    q2 = mxq.moe_layer_mx(x, w_r, lambda e: packed2[e], k)
    assert np.array_equal(q2["y"], 2 * q1["y"])


def test_moe_layer_mx_single_expert():
    # k = E = 1: every token's output is its own expert product, weight 1
    from oracle import formats, moe as omoe
    x, w_r, packed, get_packed, _, _ = _layer_case(23, E=1)
    q = mxq.moe_layer_mx(x, w_r[:1], get_packed, 1)
    (gc, gs), (dc, ds) = packed[0]
    xq = mxq.mxfp8_dequant64(*mxq.mxfp8_quantize(x))
    for t in range(x.shape[0]):
        h = omoe.swiglu(formats.mxfp4_dequant64(gc, gs) @ xq[t], dc.shape[1] * 2)
        hq = mxq.mxfp8_dequant64(*mxq.mxfp8_quantize(h[None, :]))[0]
        assert np.allclose(q["y"][t], formats.mxfp4_dequant64(dc, ds) @ hq, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- requantization spread

def _spread_cases():
    rng = np.random.default_rng(23)
    cases = []
    h = rng.standard_normal((3, 64))
    cases.append((h, np.abs(h) * 1e-3 + 1e-4))
    # block maxima just under and just over a power of two: the scale can flip
    h = rng.uniform(-1, 1, (2, 64))
    h[0, 5] = 2.0 - 1e-6
    h[0, 40] = -(4.0 + 1e-6)
    h[1, 0] = 0.5
    cases.append((h, np.full(h.shape, 1e-5)))
    # elements on rounding midpoints of their block's scale (448 fixes X = 0)
    mids = (mxq.e4m3_value(np.arange(0x7E)) + mxq.e4m3_value(np.arange(1, 0x7F))) / 2
    h = np.zeros((1, 32))
    h[0, 0] = 448.0
    h[0, 1:] = mids[::4][:31]
    cases.append((h, np.full(h.shape, 1e-9)))
    return cases


def pin_requant_spread(mq):
    rng = np.random.default_rng(29)
    attained = False
    for h, herr in _spread_cases():
        sp = mq.mxfp8_requant_spread(h, herr)
        hq = mxq.mxfp8_dequant64(*mxq.mxfp8_quantize(h))
        assert np.array_equal(mq.mxfp8_requant_spread(h, 0.0), np.zeros_like(h))
        for i in range(600):
            u = rng.choice([-1.0, 1.0], h.shape) if i % 2 else rng.uniform(-1, 1, h.shape)
            hp = h + herr * u
            d = np.abs(mxq.mxfp8_dequant64(*mxq.mxfp8_quantize(hp)) - hq)
            assert np.all(d <= sp), f"requantization moved {np.max(d - sp):.3e} past the spread"
            attained |= bool(np.any((d == sp) & (sp > 0)))
    assert attained, "the spread is never reached (not a worst case)"


def test_requant_spread_brute_force():
    """The spread bounds every quantization of a perturbed h in the box, and
    some perturbation reaches it."""
    pin_requant_spread(mxq)


def _spread_fixed_scale(h, herr):
    # takes the scale of h itself only: misses codes re-quantized at a flipped scale
    h = np.atleast_2d(np.asarray(h, np.float64))
    herr = np.broadcast_to(np.asarray(herr, np.float64), h.shape)
    hc, hs = mxq.mxfp8_quantize(h)
    sc = np.repeat(np.ldexp(1.0, hs.astype(np.int64) - 127), 32, axis=1)
    hq = mxq.mxfp8_dequant64(hc, hs)
    lo = mxq.e4m3_value(mxq.e4m3_round((h - herr) / sc)) * sc
    hi = mxq.e4m3_value(mxq.e4m3_round((h + herr) / sc)) * sc
    return np.maximum(np.abs(lo - hq), np.abs(hi - hq))


def test_requant_spread_planted_fixed_scale_is_caught():
    class Planted:
        mxfp8_requant_spread = staticmethod(_spread_fixed_scale)
    with pytest.raises(AssertionError):
        pin_requant_spread(Planted)
