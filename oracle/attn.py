"""Decode attention of a gpt-oss layer: YaRN rotary embedding, a KV cache,
learned per-head attention sinks, and full or sliding-window causal attention.

TEST INFRASTRUCTURE (see ``oracle/__init__``).

What the pages fix ("Sovereign gpt-oss-20B (MXFP4) on Apple Silicon"):
learned per-head attention sinks are the second of the port's two new kernels
(section 1) and carry the attention (section 4: without them the layer-0
attention cosine drops to about 0.55); the sliding window holds 128 tokens and
changes nothing until a sequence is longer than that (sections 3 and 4); the
YaRN inverse frequencies and attention scaling were reproduced (section 3).
They print no formula, so the readings below are taken, each the plainest
one the rest supports:

* YaRN (Peng, Quesnelle, Fan, Shippole 2023, "YaRN: Efficient Context Window
  Extension of Large Language Models"), in the form the Hugging Face golden
  the page compares against uses: base frequencies theta_i = base^(-2i/D) for
  i < D/2; a dimension turns r_i = L * theta_i / (2 pi) times over the
  original context L; the continuous index at which r_i equals a count r is
  c(r) = D ln(L / (2 pi r)) / (2 ln base); between lo = c(beta_fast) and
  hi = c(beta_slow) (clamped to [0, D-1]; rounded outward when `truncate`)
  the weight of the original frequency falls linearly in the index from 1 to
  0; the frequency is theta_i * w_i + (theta_i / s) * (1 - w_i).  The
  attention scaling is 0.1 ln s + 1 (1 when s <= 1), applied to both the
  query and the key rotation (so logits carry its square).
* Rotation pairs dimension i with i + D/2 (the two halves of a head), as a
  complex multiplication of (x_i + j x_{i+D/2}) by the scaled unit phasor of
  angle p * f_i at position p.
* A sink is one learned logit per query head that joins the softmax over the
  keys and carries a zero value vector.
* A query at position p attends keys at positions max(0, p - W + 1) .. p
  with a window of W keys (W = 0: all of 0 .. p).  Queries use grouped KV
  heads: query head h reads KV head h // (Hq / Hkv).
* Scores are (q . k) / sqrt(D) unless a scale is given (gpt-oss: 1/8).

Cache entries are a rounding decision (fp32 rotation, then bf16 for a bf16
cache), so they are computed here in the precision the kernel takes that
decision in: inverse frequencies and attention scale as fp32 constants, the
angle p * f_i exact in fp64, cos / sin of it times the scale rounded once to
fp32, then x_i c - x_{i+D/2} s and x_{i+D/2} c + x_i s in fp32 with each
product and the sum rounded separately (no fused multiply-add), then
round-to-nearest-even to bf16.  Everything else (the query rotation, scores,
softmax, the weighted sum of values) is float64.
"""

import math

import numpy as np


def yarn_inv_freq(head_dim, theta, factor, orig_ctx, beta_fast, beta_slow, truncate=False):
    """YaRN inverse frequencies [head_dim/2] and the attention scaling, float64."""
    half = head_dim // 2
    i = np.arange(half, dtype=np.float64)
    base_freq = np.power(float(theta), -2.0 * i / head_dim)
    if factor <= 1.0:
        return base_freq, 1.0

    def corr_dim(n_rot):
        return head_dim * math.log(orig_ctx / (n_rot * 2.0 * math.pi)) / (2.0 * math.log(theta))

    lo, hi = corr_dim(beta_fast), corr_dim(beta_slow)
    if truncate:
        lo, hi = math.floor(lo), math.ceil(hi)
    lo, hi = max(lo, 0.0), min(hi, float(head_dim - 1))
    if lo == hi:
        hi += 0.001
    keep = 1.0 - np.clip((i - lo) / (hi - lo), 0.0, 1.0)
    inv = (base_freq / factor) * (1.0 - keep) + base_freq * keep
    return inv, 0.1 * math.log(factor) + 1.0


def rope_constants(head_dim, theta, factor, orig_ctx, beta_fast, beta_slow, truncate=False):
    """(inv_freq fp32 [D/2], attention scale fp32): the constants the rotation uses."""
    inv, scale = yarn_inv_freq(head_dim, theta, factor, orig_ctx, beta_fast, beta_slow, truncate)
    return inv.astype(np.float32), np.float32(scale)


def rope_table(inv_freq32, scale32, positions):
    """[len(positions)][D] fp32: cos(p f_i) * a in columns i < D/2, sin(p f_i) * a
    in columns D/2 + i, each rounded once to fp32 from float64."""
    f = np.asarray(inv_freq32, dtype=np.float32).astype(np.float64)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * f[None, :]
    a = float(np.float32(scale32))
    c = (np.cos(ang) * a).astype(np.float32)
    s = (np.sin(ang) * a).astype(np.float32)
    return np.concatenate([c, s], axis=1)


def rotate64(x, pos, inv_freq32, scale32):
    """Float64 rotation of x [..., D] at position(s) pos (broadcast over the
    leading axes: pos has x's shape without the last axis)."""
    x = np.asarray(x, dtype=np.float64)
    half = x.shape[-1] // 2
    f = np.asarray(inv_freq32, dtype=np.float32).astype(np.float64)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * f
    a = float(np.float32(scale32))
    c, s = np.cos(ang) * a, np.sin(ang) * a
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def rotate_f32(x32, table_rows):
    """Kernel-precision rotation of x32 [..., D] (fp32) with table rows [..., D]
    from ``rope_table`` (same leading shape): fp32 products and sums, each
    rounded separately."""
    x = np.asarray(x32, dtype=np.float32)
    t = np.asarray(table_rows, dtype=np.float32)
    half = x.shape[-1] // 2
    c, s = t[..., :half], t[..., half:]
    x1, x2 = x[..., :half], x[..., half:]
    o1 = np.subtract(np.multiply(x1, c), np.multiply(x2, s))
    o2 = np.add(np.multiply(x2, c), np.multiply(x1, s))
    return np.concatenate([o1, o2], axis=-1).astype(np.float32)


def round_bf16(x32):
    """fp32 values rounded to the nearest bf16 value (8 significant bits),
    ties to even, returned as float64.  Finite inputs only."""
    x = np.asarray(x32, dtype=np.float32).astype(np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("round_bf16 takes finite values")
    _, e = np.frexp(x)                      # |x| in [2^(e-1), 2^e)
    q = np.ldexp(1.0, np.maximum(e - 8, -133))   # bf16 quantum of that binade
    return np.rint(x / q) * q


def store_value(x32, cache_dtype):
    """Value a cache of dtype 'bf16' or 'f32' holds for the fp32 value x32."""
    if cache_dtype == "bf16":
        return round_bf16(x32)
    if cache_dtype == "f32":
        return np.asarray(x32, dtype=np.float32).astype(np.float64)
    raise ValueError(cache_dtype)


def attention(q_rot, k_cache, v_cache, pos_q, window, sm_scale, sinks=None):
    """o [M][Hq][D] float64 for queries q_rot [M][Hq][D] at positions pos_q [M]
    over caches [Hkv][n][D] (values), window W (0 = full), optional sinks [Hq]."""
    q_rot = np.asarray(q_rot, dtype=np.float64)
    k_cache = np.asarray(k_cache, dtype=np.float64)
    v_cache = np.asarray(v_cache, dtype=np.float64)
    m, hq, d = q_rot.shape
    hkv = k_cache.shape[0]
    group = hq // hkv
    o = np.zeros((m, hq, d))
    for t in range(m):
        p = int(pos_q[t])
        lo = max(0, p - window + 1) if window else 0
        for h in range(hq):
            kk = k_cache[h // group, lo:p + 1]
            vv = v_cache[h // group, lo:p + 1]
            s = sm_scale * (kk @ q_rot[t, h])
            top = s.max() if sinks is None else max(s.max(), float(sinks[h]))
            e = np.exp(s - top)
            den = e.sum() + (0.0 if sinks is None else math.exp(float(sinks[h]) - top))
            o[t, h] = (e @ vv) / den
    return o


def decode_step(q, k, v, k_cache, v_cache, cache_dtype, pos0, inv_freq32, scale32, window,
                sm_scale, sinks=None):
    """One attention step for m new tokens at positions pos0 .. pos0 + m - 1.

    q [m][Hq][D], k and v [m][Hkv][D] fp32 (projection outputs, before the
    rotation); k_cache, v_cache [Hkv][cap][D] float64 values of the cache
    (positions below pos0 hold earlier tokens).  The new keys are rotated and
    stored, the new values stored, then every new token attends its window.
    Returns (o [m][Hq][D] float64, k_cache, v_cache) with the caches updated
    (copies).
    """
    q = np.asarray(q, dtype=np.float32)
    k = np.asarray(k, dtype=np.float32)
    v = np.asarray(v, dtype=np.float32)
    m = q.shape[0]
    pos = pos0 + np.arange(m)
    kc = np.array(k_cache, dtype=np.float64, copy=True)
    vc = np.array(v_cache, dtype=np.float64, copy=True)
    rows = rope_table(inv_freq32, scale32, pos)                    # [m][D]
    k_rot = rotate_f32(k, np.broadcast_to(rows[:, None, :], k.shape))
    kc[:, pos0:pos0 + m] = np.transpose(store_value(k_rot, cache_dtype), (1, 0, 2))
    vc[:, pos0:pos0 + m] = np.transpose(store_value(v, cache_dtype), (1, 0, 2))
    q_rot = rotate64(q, np.broadcast_to(pos[:, None], q.shape[:2]), inv_freq32, scale32)
    o = attention(q_rot, kc, vc, pos, window, sm_scale, sinks)
    return o, kc, vc


def output_bound(q_rot, k_cache, v_cache, pos_q, window, sm_scale, n_split_max=4096):
    """Per (token, head) bound on |o_fp32 - o_exact| for an fp32 evaluation
    of ``attention``: a score error of at most (D + 3) u sm sum|q||k| (u =
    2^-24; dot product, scale, base change) plus 8 u for exp and division
    changes each weight by a relative 2 * that, and summing weighted values in
    a tree of depth <= 2 log2(n) + 8 adds (depth) u; all times max |v| of the
    window.  Returns an array [M][Hq]."""
    q_rot = np.asarray(q_rot, dtype=np.float64)
    k_cache = np.asarray(k_cache, dtype=np.float64)
    v_cache = np.asarray(v_cache, dtype=np.float64)
    u = 2.0 ** -24
    m, hq, d = q_rot.shape
    hkv = k_cache.shape[0]
    group = hq // hkv
    b = np.zeros((m, hq))
    for t in range(m):
        p = int(pos_q[t])
        lo = max(0, p - window + 1) if window else 0
        n = p + 1 - lo
        depth = 2 * math.ceil(math.log2(max(n, 2))) + 8
        for h in range(hq):
            kk = np.abs(k_cache[h // group, lo:p + 1])
            vmax = np.abs(v_cache[h // group, lo:p + 1]).max()
            smax = sm_scale * (kk @ np.abs(q_rot[t, h])).max()
            e_s = (d + 3) * u * smax + 8 * u
            b[t, h] = (4.0 * e_s + depth * u) * vmax
    return b
