"""Pins for the oracle's GEMV, routing, SwiGLU experts, combine and stack.

Every pin compares the oracle with something other than itself: brute force
by Python loops or exact integer arithmetic, closed forms, identities that
hold for any correct implementation, and compositions of the smaller parts.
Planted-mistake tests at the end check that the pins catch plausible bugs.
"""

import math

import numpy as np
import pytest

import synth
from oracle import formats, gemv, moe


# ---------------------------------------------------------------- GEMV

def pin_gemv_onehot(gm):
    rng = np.random.default_rng(5)
    w = rng.standard_normal((7, 64)).astype(np.float32)       # non-square: catches W^T
    for c in (0, 13, 63):
        x = np.zeros(64)
        x[c] = 1.0
        y, den = gm.gemv(w, x)
        assert np.array_equal(y, w[:, c].astype(np.float64))
        assert np.array_equal(den, np.abs(w[:, c]).astype(np.float64))


def pin_gemv_integer_exact(gm):
    # e8m0 = 127 (scale 1): W entries are multiples of 0.5, x integers in [-2, 2];
    # 2*y is then an exact integer computed with Python ints.
    codes = synth.random_input(11, (5, 48), "bytes")
    scales = np.full((5, 3), 127, dtype=np.uint8)
    w = formats.mxfp4_dequant(codes, scales)
    x = synth.random_input(12, (2, 96), "int", -2, 2)
    y, den = gm.gemv(w, x.astype(np.float64))
    w2 = [[int(round(2 * float(v))) for v in row] for row in w]
    for m in range(2):
        for r in range(5):
            exact2 = sum(w2[r][c] * int(x[m, c]) for c in range(96))
            abs2 = sum(abs(w2[r][c]) * abs(int(x[m, c])) for c in range(96))
            assert y[m, r] * 2 == exact2 and den[m, r] * 2 == abs2


def pin_gemv_bruteforce(gm):
    for n, k in ((1, 32), (3, 32), (4, 64)):
        w = synth.random_input(20 + n, (n, k))
        x = synth.random_input(30 + k, (k,))
        y, den = gm.gemv(w, x)
        yl, denl = gemv.gemv_loops(w, x)
        assert np.allclose(y, yl, rtol=1e-13, atol=1e-13)
        assert np.allclose(den, denl, rtol=1e-13, atol=0)


def test_gemv_onehot_columns():
    pin_gemv_onehot(gemv)


def test_gemv_integer_exact():
    pin_gemv_integer_exact(gemv)


def test_gemv_bruteforce_tiny():
    pin_gemv_bruteforce(gemv)


# ---------------------------------------------------------------- router

def brute_topk(row, k):
    keyed = sorted(range(len(row)), key=lambda e: (-row[e], e))
    return keyed[:k]


def pin_topk(mm):
    rng = np.random.default_rng(3)
    for trial in range(50):
        E = int(rng.integers(2, 40))
        k = int(rng.integers(1, E + 1))
        row = np.round(rng.standard_normal(E), 1)       # rounding forces ties
        idx, w = mm.topk_softmax(row[None, :], k)
        assert list(idx[0]) == brute_topk(list(row), k)
        sel = np.array([row[e] for e in idx[0]])
        ex = [math.exp(v - max(sel)) for v in sel]
        assert np.allclose(w[0], [v / sum(ex) for v in ex], rtol=1e-14)
    # ties go to the lower index
    idx, w = mm.topk_softmax(np.array([[1.0, 3.0, 3.0, 2.0]]), 2)
    assert list(idx[0]) == [1, 2] and np.allclose(w[0], [0.5, 0.5])
    idx, w = mm.topk_softmax(np.array([[1.0, 3.0, 3.0, 2.0]]), 3)
    d = 2.0 + math.exp(-1.0)
    assert list(idx[0]) == [1, 2, 3]
    assert np.allclose(w[0], [1 / d, 1 / d, math.exp(-1.0) / d], rtol=1e-15)
    # all equal -> 0..k-1 with weights 1/k; k = E -> a permutation
    idx, w = mm.topk_softmax(np.zeros((1, 8)), 5)
    assert list(idx[0]) == [0, 1, 2, 3, 4] and np.allclose(w, 0.2)
    row = rng.standard_normal((1, 16))
    idx, _ = mm.topk_softmax(row, 16)
    assert sorted(idx[0]) == list(range(16))


def pin_softmax_identities(mm):
    rng = np.random.default_rng(4)
    row = rng.standard_normal((1, 32)) * 3
    idx, w = mm.topk_softmax(row, 4)
    assert abs(w.sum() - 1.0) < 1e-15
    idx2, w2 = mm.topk_softmax(row + 123.25, 4)         # shift invariance
    assert np.array_equal(idx, idx2) and np.allclose(w, w2, rtol=1e-12)
    # equals the full softmax renormalised over the chosen k
    full = np.exp(row[0] - row[0].max())
    full /= full.sum()
    ren = full[idx[0]] / full[idx[0]].sum()
    assert np.allclose(w[0], ren, rtol=1e-13)


def pin_router_logits(mm):
    w_r = synth.random_input(40, (6, 40))
    x = synth.random_input(41, (3, 40))
    b = synth.random_input(42, (6,))
    lg, sc = mm.router_logits(w_r, x, b)
    for m in range(3):
        for e in range(6):
            exact = sum(float(w_r[e, h]) * float(x[m, h]) for h in range(40)) + float(b[e])
            assert abs(lg[m, e] - exact) < 1e-12
            assert abs(sc[m, e] - sum(abs(float(w_r[e, h]) * float(x[m, h]))
                                      for h in range(40))) < 1e-12


def test_topk_bruteforce_and_ties():
    pin_topk(moe)


def test_softmax_identities():
    pin_softmax_identities(moe)


def test_router_logits_loops():
    pin_router_logits(moe)


def pin_check_routing(mm):
    row = np.array([0.0, 5.0, 4.0, 4.0 - 1e-9, 1.0])
    scale = np.full(5, 10.0)
    assert mm.check_routing(row, scale, [1, 2], 2)[0]
    ok, ties, _ = mm.check_routing(row, scale, [1, 3], 2)       # in band: accepted
    assert ok and ties == 1
    assert not mm.check_routing(row, scale, [1, 4], 2)[0]        # outside band
    assert not mm.check_routing(row, scale, [2, 1], 2)[0]        # wrong order
    # a list that drops a clear winner for two near-tied losers is wrong:
    # expert 2 (logit 4) is left out although it beats the kept expert 4 by 1
    row = np.array([0.0, 5.0, 4.0, 3.0, 3.0 - 1e-9])
    scale = np.full(5, 10.0)
    assert mm.check_routing(row, scale, [1, 2, 3], 3)[0]
    assert mm.check_routing(row, scale, [1, 2, 4], 3) == (True, 1, "")
    assert not mm.check_routing(row, scale, [1, 3, 4], 3)[0]
    # dropping the largest logit, with the rest in band, is wrong too
    row = np.array([10.0, 5.0, 4.0, 3.0, 3.0 + 1e-9])
    assert not mm.check_routing(row, scale, [1, 2, 4, 3], 4)[0]
    assert mm.check_routing(row, scale, [0, 1, 2, 4], 4)[0]
    # indices must name experts: negative (Python would wrap) and >= E fail
    assert not mm.check_routing(row, scale, [0, 1, 2, -1], 4)[0]
    assert not mm.check_routing(row, scale, [0, 1, 2, 5], 4)[0]
    # wrong length and duplicates fail
    assert not mm.check_routing(row, scale, [0, 1, 2], 4)[0]
    assert not mm.check_routing(row, scale, [0, 1, 1, 2], 4)[0]
    # brute force: on random logits with planted near ties, the checker agrees
    # with the definition "no left-out expert beats a kept one beyond the band,
    # order descending up to the band" taken over every k-subset and order
    import itertools
    rng = np.random.default_rng(17)
    for trial in range(60):
        n_exp, k = 6, 3
        lg = np.round(rng.standard_normal(n_exp), 1)
        if trial % 2:
            lg[rng.integers(n_exp)] = lg[rng.integers(n_exp)] + 1e-9
        sc = np.full(n_exp, 10.0)
        band = 1e-6 * 10.0
        for cand in itertools.permutations(range(n_exp), k):
            beats = any(lg[u] - lg[c] > band for u in range(n_exp) if u not in cand
                        for c in cand)
            inv = any(lg[b] - lg[a] > band for a, b in zip(cand[:-1], cand[1:]))
            assert mm.check_routing(lg, sc, list(cand), k)[0] == (not beats and not inv), \
                (lg, cand)


def test_check_routing_band():
    pin_check_routing(moe)


# ---------------------------------------------------------------- SwiGLU / expert

def pin_silu(mm):
    assert mm.silu(np.array([0.0]))[0] == 0.0
    v = mm.silu(np.array([-1000.0, 1000.0, 1.0, -1.0, 2.0]))
    assert not np.any(np.isnan(v))
    assert v[0] == 0.0 and np.signbit(v[0])                     # -1000 * tiny = -0.0
    assert v[1] == 1000.0
    assert abs(v[2] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    assert abs(v[3] - (-1.0) / (1.0 + math.exp(1.0))) < 1e-16
    assert abs(v[4] - 2.0 / (1.0 + math.exp(-2.0))) < 1e-15


def pin_expert_hand(mm):
    # W_gu rows: g0 = [1, 0], u0 = [0, 2]; W_d = [[3], [-1]]; x = [2, 0.5]
    # g = 2, u = 1, h = silu(2) = 2 / (1 + e^-2), d = [3h, -h]
    w_gu = np.array([[1.0, 0.0], [0.0, 2.0]])
    w_d = np.array([[3.0], [-1.0]])
    d, h, den = mm.expert_ffn(w_gu, w_d, np.array([2.0, 0.5]))
    hv = 2.0 / (1.0 + math.exp(-2.0))
    assert abs(h[0] - hv) < 1e-15
    assert np.allclose(d, [3 * hv, -hv], rtol=1e-15)
    assert np.allclose(den, [3 * hv, hv], rtol=1e-15)
    # g / u order: swapping the rows changes the result
    d2, _, _ = mm.expert_ffn(w_gu[::-1], w_d, np.array([2.0, 0.5]))
    assert not np.allclose(d, d2)


def small_layer(seed=0, E=6, H=64, I=32, fmt="mxfp4"):
    cfg = synth.MoEConfig(name="t", base=900 + seed, fmt=fmt, n_layers=2, hidden=H,
                          inter=I, n_experts=E, top_k=2, group=64 if fmt == "int4g" else 32)
    return cfg


def dequant_expert(cfg, layer, e):
    wts = synth.expert_weights(cfg, layer, e)
    if cfg.fmt == "mxfp4":
        return formats.mxfp4_dequant(*wts["gu"]), formats.mxfp4_dequant(*wts["dn"])
    return (formats.int4g_dequant(*wts["gu"], cfg.group),
            formats.int4g_dequant(*wts["dn"], cfg.group))


def pin_layer_composition(mm):
    cfg = small_layer()
    w_r, _, _ = synth.router(cfg, 0)
    x, _ = synth.hidden_batch(cfg, range(3))
    get = lambda e: dequant_expert(cfg, 0, e)
    res = mm.moe_layer(x, w_r, get, 2)
    for t in range(3):
        want = np.zeros(cfg.hidden)
        for j, e in enumerate(res["idx"][t]):
            wg, wd = get(int(e))
            g = wg[:cfg.inter].astype(np.float64) @ x[t]
            u = wg[cfg.inter:].astype(np.float64) @ x[t]
            h = g / (1 + np.exp(-g)) * u
            want += res["w"][t, j] * (wd.astype(np.float64) @ h)
        assert np.allclose(res["y"][t], want, rtol=1e-12, atol=1e-9)
    # k = 1: weight exactly 1, output = the single expert
    res1 = mm.moe_layer(x, w_r, get, 1)
    assert np.all(res1["w"] == 1.0)
    d, _, _ = mm.expert_ffn(*get(int(res1["idx"][0, 0])), x[0])
    assert np.array_equal(res1["y"][0], d)


def pin_zero_expert(mm):
    # an expert whose codes are all 0 contributes exactly 0
    H, I = 64, 32
    zero_gu = formats.mxfp4_dequant(np.zeros((2 * I, H // 2), np.uint8),
                                    np.full((2 * I, H // 32), 127, np.uint8))
    zero_dn = formats.mxfp4_dequant(np.zeros((H, I // 2), np.uint8),
                                    np.full((H, I // 32), 127, np.uint8))
    d, h, den = mm.expert_ffn(zero_gu, zero_dn, synth.random_input(7, (H,)))
    assert np.all(d == 0) and np.all(h == 0) and np.all(den == 0)


def pin_linear_in_down(mm):
    cfg = small_layer(1)
    wg, wd = dequant_expert(cfg, 0, 0)
    x = synth.random_input(8, (cfg.hidden,))
    d1, _, _ = mm.expert_ffn(wg, wd, x)
    d2, _, _ = mm.expert_ffn(wg, 2.0 * wd.astype(np.float64), x)
    assert np.array_equal(2.0 * d1, d2)


def pin_rmsnorm(mm):
    x = np.full(10, 3.0)
    assert np.allclose(mm.rmsnorm(x), 3.0 / math.sqrt(9.0 + 1e-5), rtol=1e-15)
    r = synth.random_input(9, (4, 100)).astype(np.float64) * 7
    n = mm.rmsnorm(r)
    ms = np.mean(r * r, axis=1)
    assert np.allclose(np.mean(n * n, axis=1), ms / (ms + 1e-5), rtol=1e-13)


def pin_stack_composition(mm):
    cfg = small_layer(2)
    layers = []
    for l in range(2):
        w_r, _, _ = synth.router(cfg, l)
        layers.append((w_r, None, (lambda l: (lambda e: dequant_expert(cfg, l, e)))(l)))
    x, _ = synth.hidden_batch(cfg, range(2))
    results, out = mm.moe_stack(x, layers, 2)
    cur = x.astype(np.float64)
    for l, (w_r, _, get) in enumerate(layers):
        xn = cur / np.sqrt(np.mean(cur * cur, axis=1, keepdims=True) + 1e-5)
        single = mm.moe_layer(xn, w_r, get, 2)            # bare layer on normed input
        cur = cur + single["y"]
    assert np.allclose(out, cur, rtol=1e-12, atol=1e-9)


def test_silu_values():
    pin_silu(moe)


def test_expert_hand_worked():
    pin_expert_hand(moe)


def test_layer_composition():
    pin_layer_composition(moe)


def test_zero_expert():
    pin_zero_expert(moe)


def test_linear_in_down():
    pin_linear_in_down(moe)


def test_rmsnorm_closed_form():
    pin_rmsnorm(moe)


def test_stack_composition():
    pin_stack_composition(moe)


def test_int4_layer_runs():
    cfg = small_layer(3, fmt="int4g", H=128, I=64)
    w_r, _, _ = synth.router(cfg, 0)
    x, _ = synth.hidden_batch(cfg, range(2))
    res = moe.moe_layer(x, w_r, lambda e: dequant_expert(cfg, 0, e), 2)
    assert np.all(np.isfinite(res["y"]))


def test_teacher_forcing_adopts_in_band_choice():
    cfg = small_layer(4)
    w_r, _, _ = synth.router(cfg, 0)
    # make experts 0 and 1 exact ties for every input
    w_r = w_r.copy()
    w_r[1] = w_r[0]
    x = np.abs(synth.hidden_batch(cfg, range(1))[0]) * 0 + 1.0
    get = lambda e: dequant_expert(cfg, 0, e)
    res = moe.moe_layer(x, w_r, get, 2)
    own = list(res["idx"][0])
    assert own[:2] == [0, 1] or 0 in own
    # a forced order that swaps the tied pair is adopted; a far-off choice raises
    forced = np.array([[1, 0]]) if own == [0, 1] else None
    if forced is not None:
        r2 = moe.moe_layer(x, w_r, get, 2, forced_idx=forced)
        assert list(r2["idx"][0]) == [1, 0] and r2["ties"] >= 1
    far = [e for e in range(cfg.n_experts) if e not in own][-1]
    with pytest.raises(AssertionError):
        moe.moe_layer(x, w_r, get, 2, forced_idx=np.array([[own[0], far]]))


# ---------------------------------------------------------------- planted mistakes

class NS:
    def __init__(self, base, **over):
        for name in dir(base):
            if not name.startswith("__"):
                setattr(self, name, getattr(base, name))
        for k, v in over.items():
            setattr(self, k, v)


def _gemv_transposed(w, x):
    w = np.asarray(w, np.float64)
    x = np.asarray(x, np.float64)
    wt = w.T[:w.shape[0], :w.shape[1]] if w.shape[0] >= w.shape[1] else np.resize(w.T, w.shape)
    return gemv.gemv(wt, x)


def _gemv_no_abs_den(w, x):
    y, _ = gemv.gemv(w, x)
    return y, np.abs(y)


def _topk_ties_high(logits, k):
    logits = np.atleast_2d(np.asarray(logits, np.float64))
    idx = np.argsort(-logits[:, ::-1], axis=1, kind="stable")
    idx = logits.shape[1] - 1 - idx[:, :k]
    return idx, np.stack([moe.softmax_over(logits[m], idx[m]) for m in range(len(idx))])


def _topk_full_softmax(logits, k):
    logits = np.atleast_2d(np.asarray(logits, np.float64))
    idx = moe.topk_order(logits, k)
    full = np.exp(logits - logits.max(axis=1, keepdims=True))
    full /= full.sum(axis=1, keepdims=True)
    return idx, np.take_along_axis(full, idx, axis=1)


def _ffn_gu_swapped(w_gu, w_d, xin):
    w_gu = np.asarray(w_gu, np.float64)
    inter = np.asarray(w_d).shape[1]
    return moe.expert_ffn(np.concatenate([w_gu[inter:], w_gu[:inter]]), w_d, xin)


def _silu_sign(g):
    g = np.asarray(g, np.float64)
    return g * moe.sigmoid(-g)


def _rmsnorm_no_eps(x, eps=0.0):
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True))


def _router_dropped_term(w_r, xin, bias=None):
    lg, sc = moe.router_logits(w_r, xin, None)
    return lg, sc


def _check_routing_kth_only(logits_row, scale_row, idx_gpu, k, rel=moe.NEAR_TIE_REL):
    # compares each pick the oracle did not make with the oracle's k-th pick
    # only, so a list that drops a larger logit passes
    own = list(moe.topk_order(np.asarray(logits_row)[None, :], k)[0])
    idx_gpu = [int(e) for e in idx_gpu]
    if own == idx_gpu:
        return True, 0, ""
    if len(set(idx_gpu)) != k:
        return False, 0, "dup"
    for e in idx_gpu:
        if e not in own and not moe.near_tie(logits_row, scale_row, e, own[-1], rel):
            return False, 0, "band"
    for a, b in zip(idx_gpu[:-1], idx_gpu[1:]):
        if logits_row[a] < logits_row[b] and not moe.near_tie(logits_row, scale_row, a, b, rel):
            return False, 0, "order"
    return True, 1, ""


def _check_routing_no_range(logits_row, scale_row, idx_gpu, k, rel=moe.NEAR_TIE_REL):
    # negative indices wrap in Python indexing and pass unnoticed
    idx = [int(e) % len(logits_row) for e in idx_gpu]
    return moe.check_routing(logits_row, scale_row, idx, k, rel)


@pytest.mark.parametrize("which", [
    "gemv_T", "gemv_den", "ties_high", "full_softmax", "gu_swap", "silu_sign",
    "norm_eps", "router_bias", "routing_kth_only", "routing_no_range",
])
def test_planted_mistake_is_caught(which):
    with pytest.raises(AssertionError):
        if which == "gemv_T":
            pin_gemv_onehot(NS(gemv, gemv=_gemv_transposed))
        elif which == "gemv_den":
            pin_gemv_integer_exact(NS(gemv, gemv=_gemv_no_abs_den))
        elif which == "ties_high":
            pin_topk(NS(moe, topk_softmax=_topk_ties_high))
        elif which == "full_softmax":
            pin_softmax_identities(NS(moe, topk_softmax=_topk_full_softmax))
        elif which == "gu_swap":
            pin_expert_hand(NS(moe, expert_ffn=_ffn_gu_swapped))
        elif which == "silu_sign":
            pin_silu(NS(moe, silu=_silu_sign))
        elif which == "norm_eps":
            pin_rmsnorm(NS(moe, rmsnorm=_rmsnorm_no_eps))
        elif which == "router_bias":
            pin_router_logits(NS(moe, router_logits=_router_dropped_term))
        elif which == "routing_kth_only":
            pin_check_routing(NS(moe, check_routing=_check_routing_kth_only))
        elif which == "routing_no_range":
            pin_check_routing(NS(moe, check_routing=_check_routing_no_range))


def test_comparison_helpers_pinned():
    """The helpers every parity check ends in, against hand-worked values:
    max_rel_err is max |y - ref| / den with den = 0 demanding an exact match
    (inf otherwise) and NaN never passing a tolerance; cosine is the angle's
    cosine (1 for two zero vectors)."""
    y_ref = np.array([1.0, -2.0, 4.0])
    assert moe.max_rel_err(y_ref, y_ref, np.ones(3)) == 0.0
    # |0.5| / 2 = 0.25 beats |0.1| / 1 and |0| / 4
    assert moe.max_rel_err([1.1, -2.0, 4.5], y_ref, [1.0, 4.0, 2.0]) == pytest.approx(0.25)
    assert moe.max_rel_err([1.1, -2.0, 4.0], y_ref, [1.0, 0.0, 1.0]) == pytest.approx(0.1)
    assert moe.max_rel_err([1.0, -2.5, 4.0], y_ref, [1.0, 0.0, 1.0]) == np.inf
    r = moe.max_rel_err([1.0, np.nan, 4.0], y_ref, np.ones(3))
    assert not (r <= 1e30)
    assert moe.max_rel_err([], [], []) == 0.0
    assert moe.cosine([1.0, 0.0], [3.0, 0.0]) == pytest.approx(1.0)
    assert moe.cosine([1.0, 0.0], [-2.0, 0.0]) == pytest.approx(-1.0)
    assert moe.cosine([1.0, 0.0], [0.0, 5.0]) == pytest.approx(0.0)
    assert moe.cosine([1.0, 0.0], [1.0, 1.0]) == pytest.approx(1.0 / np.sqrt(2.0))
    assert moe.cosine([[1.0, 2.0], [3.0, 4.0]], [1.0, 2.0, 3.0, 4.0]) == pytest.approx(1.0)
    assert moe.cosine([0.0, 0.0], [0.0, 0.0]) == 1.0
