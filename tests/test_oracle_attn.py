"""Pins of the decode-attention oracle in oracle/attn.py.

Each check is fixed by something other than the oracle's own formulas:
YaRN's ramp by the rotation counts that define it, plain RoPE as its factor-1
case, the rotation by complex multiplication, bf16 rounding by torch's
conversion, attention by torch's scaled_dot_product_attention in float64
(sinks as an extra zero-valued key with an additive mask, windows as a band
mask written here), a closed form for identical keys, a pure-Python loop on a
tiny case, and the page's statement that a 128-token window changes nothing
below 128 tokens.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attn

GPTOSS = dict(head_dim=64, theta=150000.0, factor=32.0, orig_ctx=4096, beta_fast=32.0, beta_slow=1.0)
OTHER = dict(head_dim=128, theta=10000.0, factor=8.0, orig_ctx=2048, beta_fast=32.0, beta_slow=1.0)


def _rng(seed):
    return np.random.default_rng(seed)


# ---- YaRN frequencies ----

def test_yarn_factor_one_is_plain_rope():
    for d, base in ((64, 10000.0), (128, 500000.0)):
        inv, scale = attn.yarn_inv_freq(d, base, 1.0, 4096, 32.0, 1.0)
        want = np.exp(-np.arange(d // 2) * (2.0 / d) * math.log(base))
        np.testing.assert_allclose(inv, want, rtol=1e-14)
        assert scale == 1.0


def pin_yarn_regions(p, A=attn):
    d, base, s, L = p["head_dim"], p["theta"], p["factor"], p["orig_ctx"]
    inv, _ = A.yarn_inv_freq(**p)
    theta_i = base ** (-2.0 * np.arange(d // 2) / d)
    turns = L * theta_i / (2 * math.pi)           # rotations over the original context
    fast = turns >= p["beta_fast"]
    slow = turns <= p["beta_slow"]
    assert fast.any() and slow.any() and (~fast & ~slow).any()
    np.testing.assert_allclose(inv[fast], theta_i[fast], rtol=1e-15)
    np.testing.assert_allclose(inv[slow], theta_i[slow] / s, rtol=1e-15)
    mid = ~fast & ~slow
    assert np.all(inv[mid] < theta_i[mid]) and np.all(inv[mid] > theta_i[mid] / s)
    assert np.all(np.diff(inv) < 0)


def pin_yarn_ramp(p, A=attn):
    # the weight of the original frequency falls linearly in the index; the
    # two ends of the ramp sit where the rotation count equals beta_fast and
    # beta_slow
    d, base, s, L = p["head_dim"], p["theta"], p["factor"], p["orig_ctx"]
    inv, _ = A.yarn_inv_freq(**p)
    theta_i = base ** (-2.0 * np.arange(d // 2) / d)
    w = (inv - theta_i / s) / (theta_i - theta_i / s)
    inner = np.nonzero((w > 0) & (w < 1))[0]
    assert inner.size >= 3
    np.testing.assert_allclose(np.diff(w[inner], 2), 0.0, atol=1e-12)
    slope = w[inner[1]] - w[inner[0]]
    lo = inner[0] + (1.0 - w[inner[0]]) / slope         # index where w = 1
    hi = inner[0] - w[inner[0]] / slope                 # index where w = 0
    turns_at = lambda x: L * base ** (-2.0 * x / d) / (2 * math.pi)
    assert turns_at(lo) == pytest.approx(p["beta_fast"], rel=1e-9)
    assert turns_at(hi) == pytest.approx(p["beta_slow"], rel=1e-9)


def test_yarn_truncate_rounds_the_ramp_ends_outward():
    p = dict(GPTOSS, truncate=True)
    inv, _ = attn.yarn_inv_freq(**p)
    d, base, s = p["head_dim"], p["theta"], p["factor"]
    theta_i = base ** (-2.0 * np.arange(d // 2) / d)
    w = (inv - theta_i / s) / (theta_i - theta_i / s)
    # gpt-oss: rotation counts cross 32 between index 8 and 9 and 1 between 17 and 18
    assert np.all(w[:9] == 1.0) and np.all(w[18:] == 0.0)
    np.testing.assert_allclose(np.diff(w[8:19]), -0.1, atol=1e-12)


def pin_attention_scaling(A=attn):
    for s, want in ((1.0, 1.0), (0.5, 1.0), (math.exp(10.0), 2.0), (math.exp(5.0), 1.5)):
        _, scale = A.yarn_inv_freq(64, 10000.0, s, 4096, 32.0, 1.0)
        assert scale == pytest.approx(want, rel=1e-15)


# ---- rotation ----

def pin_rotation_complex(A=attn):
    r = _rng(1)
    d = 64
    inv32, a32 = A.rope_constants(**GPTOSS)
    x = r.standard_normal((5, 3, d)).astype(np.float32)
    pos = r.integers(0, 200000, size=(5, 3))
    got = A.rotate64(x, pos, inv32, a32)
    z = (x[..., :32] + 1j * x[..., 32:].astype(np.float64)) * \
        np.exp(1j * pos[..., None] * inv32.astype(np.float64)) * float(a32)
    np.testing.assert_allclose(got[..., :32], z.real, rtol=0, atol=1e-12)
    np.testing.assert_allclose(got[..., 32:], z.imag, rtol=0, atol=1e-12)
    # the table's columns are the same phasor
    tab = A.rope_table(inv32, a32, pos[:, 0])
    ph = np.exp(1j * pos[:, 0, None] * inv32.astype(np.float64)) * float(a32)
    np.testing.assert_allclose(tab[:, :32], ph.real, rtol=0, atol=2e-7)
    np.testing.assert_allclose(tab[:, 32:], ph.imag, rtol=0, atol=2e-7)


def test_rotation_keeps_relative_position():
    r = _rng(2)
    inv32, _ = attn.rope_constants(**GPTOSS)
    q, k = r.standard_normal((2, 64))
    for m, n, shift in ((5, 3, 97), (4000, 10, 123456), (7, 7, 31)):
        a = attn.rotate64(q, m, inv32, 1.0) @ attn.rotate64(k, n, inv32, 1.0)
        b = attn.rotate64(q, m + shift, inv32, 1.0) @ attn.rotate64(k, n + shift, inv32, 1.0)
        assert a == pytest.approx(b, rel=1e-9, abs=1e-9)
    # position 0 is the identity scaled by the attention scaling
    np.testing.assert_allclose(attn.rotate64(q, 0, inv32, 1.5), 1.5 * q, rtol=1e-15)


def test_rotation_in_fp32_is_within_two_ulps():
    r = _rng(3)
    inv32, a32 = attn.rope_constants(**GPTOSS)
    x = r.standard_normal((50, 8, 64)).astype(np.float32)
    pos = r.integers(0, 131072, size=50)
    rows = attn.rope_table(inv32, a32, pos)
    got = attn.rotate_f32(x, np.broadcast_to(rows[:, None, :], x.shape)).astype(np.float64)
    want = attn.rotate64(x, np.broadcast_to(pos[:, None], x.shape[:2]), inv32, a32)
    mag = np.abs(x[..., :32]).astype(np.float64) + np.abs(x[..., 32:])
    tol = 4 * 2.0 ** -24 * float(a32) * np.concatenate([mag, mag], axis=-1)
    assert np.all(np.abs(got - want) <= tol)


def pin_round_bf16(A=attn):
    r = _rng(4)
    x = np.concatenate([
        r.standard_normal(20000).astype(np.float32),
        (r.standard_normal(2000) * 1e-30).astype(np.float32),
        (r.standard_normal(2000) * 1e30).astype(np.float32),
        # exact ties between two bf16 neighbours (odd and even mantissas)
        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(2 + 2 ** -7), 3 * 2 ** -130], dtype=np.float32),
        np.array([0.0, -0.0], dtype=np.float32),
    ])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = A.round_bf16(x)
    assert np.array_equal(got, want)
    assert got[-6] == 1.0 and got[-5] == 1 + 2 ** -6


# ---- attention ----

def _sdpa(q_rot, kc, vc, pos, window, sm_scale, sinks=None):
    """torch's scaled_dot_product_attention, float64 on the CPU, with a band
    mask for the window and an extra zero key / value carrying the sink."""
    m, hq, d = q_rot.shape
    hkv, n, _ = kc.shape
    rep = hq // hkv
    K = torch.from_numpy(np.repeat(kc, rep, axis=0))          # [hq][n][d]
    V = torch.from_numpy(np.repeat(vc, rep, axis=0))
    Q = torch.from_numpy(np.transpose(q_rot, (1, 0, 2)).copy())  # [hq][m][d]
    j = np.arange(n)[None, :]
    p = np.asarray(pos)[:, None]
    allowed = (j <= p) & ((j > p - window) if window else True)
    mask = np.where(allowed, 0.0, -np.inf)[None].repeat(hq, 0)  # [hq][m][n]
    if sinks is not None:
        K = torch.cat([K, torch.zeros(hq, 1, d, dtype=K.dtype)], 1)
        V = torch.cat([V, torch.zeros(hq, 1, d, dtype=V.dtype)], 1)
        col = np.broadcast_to(np.asarray(sinks, dtype=np.float64)[:, None, None], (hq, m, 1))
        mask = np.concatenate([mask, col], axis=2)
    out = torch.nn.functional.scaled_dot_product_attention(
        Q, K, V, attn_mask=torch.from_numpy(np.ascontiguousarray(mask)), scale=sm_scale)
    return np.transpose(out.numpy(), (1, 0, 2))


def _case(seed, m=3, hq=8, hkv=2, d=16, n=37):
    r = _rng(seed)
    q = r.standard_normal((m, hq, d))
    kc = r.standard_normal((hkv, n, d))
    vc = r.standard_normal((hkv, n, d))
    pos = np.arange(n - m, n)
    sinks = r.standard_normal(hq) * 2
    return q, kc, vc, pos, sinks


def pin_attention_sdpa(window, with_sinks, A=attn):
    q, kc, vc, pos, sinks = _case(10 + window)
    s = sinks if with_sinks else None
    got = A.attention(q, kc, vc, pos, window, 0.25, s)
    want = _sdpa(q, kc, vc, pos, window, 0.25, s)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_window_changes_nothing_below_its_length():
    q, kc, vc, _, sinks = _case(20, m=4, n=128)
    pos = np.array([0, 50, 126, 127])
    full = attn.attention(q, kc, vc, pos, 0, 0.125, sinks)
    win = attn.attention(q, kc, vc, pos, 128, 0.125, sinks)
    assert np.array_equal(full, win)
    q2, kc2, vc2, _, _ = _case(21, m=1, n=140)
    pos2 = np.array([139])
    assert not np.allclose(attn.attention(q2, kc2, vc2, pos2, 0, 0.125),
                           attn.attention(q2, kc2, vc2, pos2, 128, 0.125))


def test_identical_keys_closed_form():
    r = _rng(30)
    d, n = 8, 11
    k_row = r.standard_normal(d)
    kc = np.broadcast_to(k_row, (1, n, d)).copy()
    vc = r.standard_normal((1, n, d))
    q = r.standard_normal((1, 2, d))
    sinks = np.array([0.7, -3.0])
    got = attn.attention(q, kc, vc, [n - 1], 0, 0.3, sinks)
    for h in range(2):
        s0 = 0.3 * (q[0, h] @ k_row)
        want = vc[0].sum(0) * math.exp(s0) / (n * math.exp(s0) + math.exp(sinks[h]))
        np.testing.assert_allclose(got[0, h], want, rtol=1e-13)


def test_tiny_case_by_loops():
    r = _rng(31)
    hq, hkv, d, n = 4, 2, 4, 6
    q = r.standard_normal((2, hq, d))
    kc = r.standard_normal((hkv, n, d))
    vc = r.standard_normal((hkv, n, d))
    sinks = r.standard_normal(hq)
    pos, window = [4, 5], 3
    got = attn.attention(q, kc, vc, pos, window, 0.5, sinks)
    for t in range(2):
        for h in range(hq):
            g = h // (hq // hkv)
            keys = [j for j in range(n) if pos[t] - window < j <= pos[t]]
            sc = [0.5 * sum(q[t, h, i] * kc[g, j, i] for i in range(d)) for j in keys]
            den = sum(math.exp(x) for x in sc) + math.exp(sinks[h])
            for i in range(d):
                num = sum(math.exp(x) * vc[g, j, i] for x, j in zip(sc, keys))
                assert got[t, h, i] == pytest.approx(num / den, rel=1e-12, abs=1e-14)


@pytest.mark.parametrize("cache_dtype", ["bf16", "f32"])
def test_chunk_of_tokens_equals_token_by_token(cache_dtype):
    r = _rng(40)
    hq, hkv, d, cap, pos0, m = 8, 2, 64, 64, 20, 5
    inv32, a32 = attn.rope_constants(**GPTOSS)
    kc = attn.store_value(r.standard_normal((hkv, cap, d)).astype(np.float32), cache_dtype)
    vc = attn.store_value(r.standard_normal((hkv, cap, d)).astype(np.float32), cache_dtype)
    q = r.standard_normal((m, hq, d)).astype(np.float32)
    k = r.standard_normal((m, hkv, d)).astype(np.float32)
    v = r.standard_normal((m, hkv, d)).astype(np.float32)
    sinks = r.standard_normal(hq)
    o, kc1, vc1 = attn.decode_step(q, k, v, kc, vc, cache_dtype, pos0, inv32, a32, 8, 0.125, sinks)
    kc2, vc2 = kc, vc
    for t in range(m):
        o_t, kc2, vc2 = attn.decode_step(q[t:t + 1], k[t:t + 1], v[t:t + 1], kc2, vc2, cache_dtype,
                                         pos0 + t, inv32, a32, 8, 0.125, sinks)
        np.testing.assert_allclose(o[t], o_t[0], rtol=1e-13, atol=1e-14)
    assert np.array_equal(kc1, kc2) and np.array_equal(vc1, vc2)
    # untouched positions keep their values; new ones hold the rounded rotation
    assert np.array_equal(kc1[:, :pos0], kc[:, :pos0]) and np.array_equal(kc1[:, pos0 + m:], kc[:, pos0 + m:])
    if cache_dtype == "bf16":
        assert np.array_equal(attn.round_bf16(kc1[:, pos0:pos0 + m].astype(np.float32)),
                              kc1[:, pos0:pos0 + m])


def test_output_bound_covers_a_float32_evaluation():
    r = _rng(50)
    hq, hkv, d, n = 16, 2, 64, 3000
    q = r.standard_normal((2, hq, d)) * 1.3
    kc = r.standard_normal((hkv, n, d))
    vc = r.standard_normal((hkv, n, d))
    pos = np.array([n - 2, n - 1])
    sinks = r.standard_normal(hq)
    exact = attn.attention(q, kc, vc, pos, 0, 0.125, sinks)
    bound = attn.output_bound(q, kc, vc, pos, 0, 0.125)
    # a float32 evaluation in another order (numpy's pairwise sums)
    rep = hq // hkv
    o32 = np.zeros_like(exact)
    for t in range(2):
        for h in range(hq):
            kk = kc[h // rep, :pos[t] + 1].astype(np.float32)
            vv = vc[h // rep, :pos[t] + 1].astype(np.float32)
            s = np.float32(0.125) * (kk @ q[t, h].astype(np.float32))
            top = max(s.max(), np.float32(sinks[h]))
            e = np.exp(s - top)
            o32[t, h] = (e @ vv) / (e.sum() + np.exp(np.float32(sinks[h]) - top))
    err = np.abs(o32 - exact).max(axis=2)
    assert np.all(err <= bound)
    assert np.all(bound < 1e-3)
    # the bound is a worst case; a float32 evaluation lands far inside it
    vmax = np.abs(vc).max()
    assert err.max() <= 2e-5 * vmax


# ---- the pins as tests ----

@pytest.mark.parametrize("p", [GPTOSS, OTHER], ids=["gptoss", "other"])
def test_yarn_regions_follow_rotation_counts(p):
    pin_yarn_regions(p)


@pytest.mark.parametrize("p", [GPTOSS, OTHER], ids=["gptoss", "other"])
def test_yarn_ramp_is_linear_between_the_correction_dims(p):
    pin_yarn_ramp(p)


def test_attention_scaling():
    pin_attention_scaling()


def test_rotation_is_a_complex_multiplication():
    pin_rotation_complex()


def test_round_bf16_matches_torch():
    pin_round_bf16()


@pytest.mark.parametrize("window", [0, 5, 36, 200])
@pytest.mark.parametrize("with_sinks", [False, True])
def test_attention_matches_sdpa(window, with_sinks):
    pin_attention_sdpa(window, with_sinks)


# ---- planted mistakes: each plausible slip in the oracle fails a pin ----

class NS:
    def __init__(self, base, **over):
        for name in dir(base):
            if not name.startswith("__"):
                setattr(self, name, getattr(base, name))
        for k, v in over.items():
            setattr(self, k, v)


def _rotate_interleaved(x, pos, inv_freq32, scale32):
    x = np.asarray(x, dtype=np.float64)
    f = np.asarray(inv_freq32, dtype=np.float32).astype(np.float64)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * f
    a = float(np.float32(scale32))
    c, s = np.cos(ang) * a, np.sin(ang) * a
    x1, x2 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x1 * c - x2 * s
    out[..., 1::2] = x2 * c + x1 * s
    return out


def _rotate_sign(x, pos, inv_freq32, scale32):
    return attn.rotate64(x, -np.asarray(pos), inv_freq32, scale32)


def _table_swapped(inv_freq32, scale32, positions):
    t = attn.rope_table(inv_freq32, scale32, positions)
    half = t.shape[1] // 2
    return np.concatenate([t[:, half:], t[:, :half]], axis=1)


def _yarn_reversed(head_dim, theta, factor, orig_ctx, beta_fast, beta_slow, truncate=False):
    inv, sc = attn.yarn_inv_freq(head_dim, theta, factor, orig_ctx, beta_fast, beta_slow, truncate)
    base = np.power(float(theta), -2.0 * np.arange(head_dim // 2) / head_dim)
    keep = (inv - base / factor) / (base - base / factor)
    return base / factor * keep + base * (1.0 - keep), sc


def _yarn_log2(head_dim, theta, factor, orig_ctx, beta_fast, beta_slow, truncate=False):
    i = np.arange(head_dim // 2, dtype=np.float64)
    base = np.power(float(theta), -2.0 * i / head_dim)
    lo = head_dim * math.log2(orig_ctx / (beta_fast * 2 * math.pi)) / (2 * math.log(theta))
    hi = head_dim * math.log2(orig_ctx / (beta_slow * 2 * math.pi)) / (2 * math.log(theta))
    lo, hi = max(lo, 0.0), min(hi, head_dim - 1.0)
    keep = 1.0 - np.clip((i - lo) / (hi - lo), 0.0, 1.0)
    return base / factor * (1.0 - keep) + base * keep, 0.1 * math.log(factor) + 1.0


def _yarn_scale_log10(head_dim, theta, factor, orig_ctx, beta_fast, beta_slow, truncate=False):
    inv, _ = attn.yarn_inv_freq(head_dim, theta, factor, orig_ctx, beta_fast, beta_slow, truncate)
    return inv, (0.1 * math.log10(factor) + 1.0 if factor > 1 else 1.0)


def _bf16_truncate(x32):
    u = np.asarray(x32, dtype=np.float32).view(np.uint32) & np.uint32(0xFFFF0000)
    return u.view(np.float32).astype(np.float64)


def _attention_variant(kind):
    def f(q_rot, k_cache, v_cache, pos_q, window, sm_scale, sinks=None):
        q_rot = np.asarray(q_rot, dtype=np.float64)
        m, hq, d = q_rot.shape
        hkv = k_cache.shape[0]
        o = np.zeros((m, hq, d))
        for t in range(m):
            p = int(pos_q[t])
            lo = (max(0, p - window) if kind == "window" else max(0, p - window + 1)) if window else 0
            for h in range(hq):
                g = h % hkv if kind == "gqa" else h // (hq // hkv)
                kk, vv = k_cache[g, lo:p + 1], v_cache[g, lo:p + 1]
                sc = (1.0 if kind == "scale" else sm_scale) * (kk @ q_rot[t, h])
                top = sc.max() if sinks is None else max(sc.max(), float(sinks[h]))
                e = np.exp(sc - top)
                if sinks is None or kind == "nosink":
                    den = e.sum()
                else:
                    den = e.sum() + math.exp(float(sinks[h]) - top)
                num = e @ vv
                if kind == "sinkvalue" and sinks is not None:
                    num = num + math.exp(float(sinks[h]) - top) * vv.mean(axis=0)
                o[t, h] = num / den
        return o
    return f


@pytest.mark.parametrize("which", [
    "interleaved", "sin_sign", "table_swapped", "yarn_reversed", "yarn_log2", "scale_log10", "bf16_truncate",
    "window_off_by_one", "gqa_modulo", "no_score_scale", "sink_dropped", "sink_has_value",
])
def test_planted_mistake_is_caught(which):
    with pytest.raises(AssertionError):
        if which == "interleaved":
            pin_rotation_complex(NS(attn, rotate64=_rotate_interleaved))
        elif which == "sin_sign":
            pin_rotation_complex(NS(attn, rotate64=_rotate_sign))
        elif which == "table_swapped":
            pin_rotation_complex(NS(attn, rope_table=_table_swapped))
        elif which == "yarn_reversed":
            pin_yarn_regions(GPTOSS, NS(attn, yarn_inv_freq=_yarn_reversed))
        elif which == "yarn_log2":
            pin_yarn_ramp(GPTOSS, NS(attn, yarn_inv_freq=_yarn_log2))
        elif which == "scale_log10":
            pin_attention_scaling(NS(attn, yarn_inv_freq=_yarn_scale_log10))
        elif which == "bf16_truncate":
            pin_round_bf16(NS(attn, round_bf16=_bf16_truncate))
        elif which == "window_off_by_one":
            pin_attention_sdpa(5, True, NS(attn, attention=_attention_variant("window")))
        elif which == "gqa_modulo":
            pin_attention_sdpa(0, False, NS(attn, attention=_attention_variant("gqa")))
        elif which == "no_score_scale":
            pin_attention_sdpa(0, False, NS(attn, attention=_attention_variant("scale")))
        elif which == "sink_dropped":
            pin_attention_sdpa(0, True, NS(attn, attention=_attention_variant("nosink")))
        elif which == "sink_has_value":
            pin_attention_sdpa(36, True, NS(attn, attention=_attention_variant("sinkvalue")))
