"""Shared helpers for the GPU parity tests (comparison rules, case banners)."""

import sys

import numpy as np

from oracle import moe as omoe

REL_TOL = 1e-4          # max |y - yref| / (|W| . |x|)
COS_TOL = 0.99999       # cosine(y, yref)
ROUTER_REL = 1e-6       # |logit - ref| <= 1e-6 * sum |W_r x|
WEIGHT_ABS = 1e-6       # router weights vs softmax of the GPU's own logits


def banner(msg):
    """Name the GPU case on the real stdout before it runs (survives capture)."""
    sys.__stdout__.write(f"[gpu-case] {msg}\n")
    sys.__stdout__.flush()


def f32_bits(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32)).view(np.uint32)


def assert_bit_exact(got, want):
    got = np.asarray(got, dtype=np.float32)
    want = np.asarray(want, dtype=np.float32)
    assert got.shape == want.shape
    gn, wn = np.isnan(got), np.isnan(want)
    assert np.array_equal(gn, wn), f"NaN positions differ: {np.argwhere(gn != wn)[:5]}"
    gb, wb = f32_bits(got)[~gn], f32_bits(want)[~wn]
    bad = np.nonzero(gb != wb)[0]
    assert bad.size == 0, f"{bad.size} mismatches, first at flat {bad[:5]}: {gb[bad[:5]]} vs {wb[bad[:5]]}"


def assert_close(y, y_ref, den, what=""):
    rel = omoe.max_rel_err(y, y_ref, den)
    cos = omoe.cosine(y, y_ref)
    assert rel <= REL_TOL, f"{what}: max rel err {rel:.3e} > {REL_TOL}"
    assert cos >= COS_TOL, f"{what}: cosine {cos:.8f} < {COS_TOL}"
    return rel, cos


def to_np(t):
    return t.detach().cpu().numpy()
