"""MX quantization of activations (MXFP8 E4M3) and the MX-scaled product.

TEST INFRASTRUCTURE (see ``oracle/__init__``).

The pages name grouped-expert GEMM over the active experts as the lever left
untried ("Sovereign gpt-oss-20B (MXFP4) on Apple Silicon", section 5) and fp8
/ grouped-expert GEMM as what lies beyond the single-stream floor ("Amortizing
the per-token host-sync setup tax in fused all-layer q4 decode", section 5).
They print no activation format, so the reading taken is the OCP
Microscaling Formats (MX) v1.0 one for MXFP8:

* an element is FP8 E4M3 - 1 sign bit, 4 exponent bits with bias 7, 3
  mantissa bits; exponent field 0 is subnormal (m * 2^-9); the pattern
  S.1111.111 is NaN, so the largest finite magnitude is 448 (there is no
  infinity);
* a block of 32 contiguous K-elements of one row shares an E8M0 scale 2^X.

Quantization of one block x[0..31] (the spec's conversion, with the open
points read as stated):

1. amax = max |x_i|.  If amax is NaN or infinite the block is not finite:
   scale byte 255 (NaN) and every element code 0x7F (NaN).
2. X = floor(log2(amax)) - 8, 8 being the exponent of E4M3's largest normal
   (448 = 1.75 * 2^8); for amax = 0, X = -127.  X is clamped to [-127, 127];
   the scale byte is X + 127.
3. Each element v_i = x_i / 2^X is rounded to the nearest E4M3 value, ties to
   the even code, and magnitudes at or above 448 saturate to 448 (v can reach
   just under 512).  The sign is kept, so -0.0 and negative values that round
   to zero give the code 0x80.

Everything here is float64 and value-domain: the rounding is done by finding
the quantum of v's binade and rounding v / quantum with ``np.rint`` (round
half to even), not by manipulating bit patterns.
"""

import numpy as np

from .formats import e8m0_value

E4M3_MAX = 448.0
E4M3_EMAX = 8          # exponent of the largest normal
E4M3_EMIN = -6         # exponent of the smallest normal
E4M3_MBITS = 3
MX_BLOCK = 32


def e4m3_value(code):
    """Value(s) of FP8 E4M3 code(s) 0..255 in float64; NaN for S.1111.111."""
    code = np.asarray(code, dtype=np.int64)
    sign = (code >> 7) & 1
    e = (code >> 3) & 15
    m = code & 7
    mag = np.where(e == 0, m * 2.0 ** (E4M3_EMIN - E4M3_MBITS),
                   np.ldexp(1.0 + m / 8.0, e - 7)).astype(np.float64)
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


def floor_log2(a):
    """floor(log2 a) for finite a > 0, exactly (from the binary exponent)."""
    _, p = np.frexp(np.asarray(a, dtype=np.float64))
    return p.astype(np.int64) - 1


# code of each non-negative finite E4M3 value (codes 0x00..0x7E are increasing)
_POS_CODES = np.arange(0x7F)
_POS_VALUES = e4m3_value(_POS_CODES)


def e4m3_round(v):
    """Round float64 values to E4M3 codes: nearest, ties to even code,
    saturating at +-448 (step 3 of the block conversion above)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    # the quantum of a's binade: 2^(E - 3) for normals, 2^-9 below 2^-6;
    # E = floor(log2 a) exactly, from frexp (a = f * 2^p, f in [0.5, 1))
    e = floor_log2(np.where(a > 0, a, 1.0))
    e = np.clip(e, E4M3_EMIN, E4M3_EMAX)
    quantum = np.ldexp(1.0, (e - E4M3_MBITS).astype(np.int64))
    q = np.rint(a / quantum) * quantum          # np.rint: round half to even
    q = np.minimum(q, E4M3_MAX)                  # saturate (also catches rounding up past 448)
    code = np.searchsorted(_POS_VALUES, q)       # exact: q is an E4M3 value
    if not np.all(_POS_VALUES[np.minimum(code, 0x7E)] == q):
        raise AssertionError("rounded value is not an E4M3 value")
    return (code | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


def mxfp8_quantize(x):
    """Quantize rows of x (float [m][k], k % 32 == 0) to MXFP8 E4M3.

    Returns (codes uint8 [m][k], scales uint8 [m][k/32]).
    """
    x = np.asarray(x, dtype=np.float64)
    if x.ndim == 1:
        x = x[None, :]
    m, k = x.shape
    if k % MX_BLOCK:
        raise ValueError("MXFP8: k must be a multiple of 32")
    blocks = x.reshape(m, k // MX_BLOCK, MX_BLOCK)
    amax = np.max(np.abs(blocks), axis=2)
    finite = np.isfinite(amax)
    xexp = np.where(amax > 0, floor_log2(np.where(finite & (amax > 0), amax, 1.0)) - E4M3_EMAX, -127)
    xexp = np.clip(xexp, -127, 127).astype(np.int64)
    scales = np.where(finite, xexp + 127, 255).astype(np.uint8)
    v = blocks / np.ldexp(1.0, xexp)[:, :, None]
    v = np.where(finite[:, :, None], v, 0.0)
    codes = e4m3_round(v)
    codes = np.where(finite[:, :, None], codes, 0x7F).astype(np.uint8)
    return codes.reshape(m, k), scales


def mxfp8_dequant64(codes, scales):
    """float64 values of an MXFP8 tensor (codes [m][k], scales [m][k/32])."""
    codes = np.asarray(codes, dtype=np.uint8)
    m, k = codes.shape
    s = np.repeat(e8m0_value(scales), MX_BLOCK, axis=1)
    return e4m3_value(codes) * s


def mx_gemm(w_codes, w_scales, x_codes, x_scales):
    """y[m][n] = sum_k W[n][k] * xq[m][k] for MXFP4 weights W and MXFP8
    activations xq, both dequantized exactly to float64, plus the normaliser
    den[m][n] = sum_k |W[n][k]| |xq[m][k]| (the GEMV definition with the
    quantized activations in place of x)."""
    from .formats import mxfp4_dequant64
    from .gemv import gemv
    return gemv(mxfp4_dequant64(w_codes, w_scales), mxfp8_dequant64(x_codes, x_scales))


def moe_layer_mx(x, w_r, get_expert_packed, k, bias=None, forced_idx=None):
    """A bare MoE layer (no norm, no residual) evaluated the large-M way.

    Routing is the oracle's own (``oracle.moe``: logits of x, top-k, softmax
    over the chosen k; ``forced_idx`` adopts a GPU choice only inside the
    near-tie band).  Then, per pick (t, j) of expert e:
      xq = MXFP8(x[t])                      (the activation quantizer above)
      [g; u] = W_gu[e] . xq,  h = silu(g) * u
      hq = MXFP8(h)                         (h quantized along the intermediate axis)
      d = W_d[e] . hq
    and y[t] = sum_j w[t][j] d_{t,j}, all in float64.
    den[t] = sum_j w[t][j] |W_d| . |hq| normalises the error of y[t].

    get_expert_packed : e -> ((gu_codes, gu_scales), (dn_codes, dn_scales)).
    """
    from . import moe as omoe
    from .formats import mxfp4_dequant64
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    m = x.shape[0]
    logits, scale = omoe.router_logits(w_r, x, bias)
    idx, w = omoe.topk_softmax(logits, k)
    ties = 0
    if forced_idx is not None:
        forced_idx = np.atleast_2d(np.asarray(forced_idx))
        for t in range(m):
            ok, n_ties, msg = omoe.check_routing(logits[t], scale[t], forced_idx[t], k)
            if not ok:
                raise AssertionError(f"token {t}: {msg}")
            if n_ties:
                ties += n_ties
                idx[t] = forced_idx[t]
                w[t] = omoe.softmax_over(logits[t], idx[t])
    xc, xs = mxfp8_quantize(x)
    xq = mxfp8_dequant64(xc, xs)
    y = np.zeros_like(x)
    den = np.zeros_like(x)
    for e in np.unique(idx):
        (gc, gs), (dc, ds) = get_expert_packed(int(e))
        w_gu = mxfp4_dequant64(gc, gs)
        w_d = mxfp4_dequant64(dc, ds)
        inter = w_d.shape[1]
        toks, slots = np.nonzero(idx == e)          # a token picks an expert at most once
        gu = xq[toks] @ w_gu.T
        h = omoe.swiglu(gu, inter)
        hc, hs = mxfp8_quantize(h)
        hq = mxfp8_dequant64(hc, hs)
        wt = w[toks, slots][:, None]
        y[toks] += wt * (hq @ w_d.T)
        den[toks] += np.abs(wt) * (np.abs(hq) @ np.abs(w_d).T)
    return dict(y=y, den=den, idx=idx, w=w, logits=logits, scale=scale, ties=ties)


def mxfp8_requant_spread(h, herr):
    """Largest change of the MXFP8 quantization of h (rows along the last axis)
    over all h' with |h' - h| <= herr elementwise: spread[i] = max |MXFP8(h')_i
    - MXFP8(h)_i| (dequantized, float64).

    Used where h is computed with a bounded error (here by matrix cores that
    sum at reduced precision) before it is quantized: the quantization of the
    computed h may then differ from the exact h's.  Worst case taken from the
    conversion steps above:
    * a block's amax' lies in [max_i (|h_i| - herr_i)+, max_i (|h_i| + herr_i)],
      so its exponent X' takes every value floor_log2 gives on that range;
    * at a fixed X', rounding to nearest (any tie rule) with saturation is
      monotone, so an element's code lies between the codes of
      (h_i - herr_i) / 2^X' and (h_i + herr_i) / 2^X'.
    Finite inputs only.
    """
    h = np.atleast_2d(np.asarray(h, dtype=np.float64))
    herr = np.broadcast_to(np.asarray(herr, dtype=np.float64), h.shape)
    m, k = h.shape
    if k % MX_BLOCK:
        raise ValueError("MXFP8: k must be a multiple of 32")
    hc, hs = mxfp8_quantize(h)
    hq = mxfp8_dequant64(hc, hs).reshape(m, k // MX_BLOCK, MX_BLOCK)
    hb = h.reshape(m, k // MX_BLOCK, MX_BLOCK)
    eb = herr.reshape(m, k // MX_BLOCK, MX_BLOCK)
    lo_v, hi_v = hb - eb, hb + eb
    amax_lo = np.max(np.maximum(np.abs(hb) - eb, 0.0), axis=2)
    amax_hi = np.max(np.abs(hb) + eb, axis=2)

    def xexp(a):
        return np.where(a > 0, np.clip(floor_log2(np.where(a > 0, a, 1.0)) - E4M3_EMAX, -127, 127), -127)
    x_lo, x_hi = xexp(amax_lo), xexp(amax_hi)
    spread = np.zeros_like(hb)
    for d in range(int(np.max(x_hi - x_lo)) + 1):
        X = np.minimum(x_lo + d, x_hi)                   # every exponent in [x_lo, x_hi]
        sc = np.ldexp(1.0, X.astype(np.int64))[:, :, None]
        q_lo = e4m3_value(e4m3_round(lo_v / sc)) * sc
        q_hi = e4m3_value(e4m3_round(hi_v / sc)) * sc
        spread = np.maximum(spread, np.maximum(np.abs(q_lo - hq), np.abs(q_hi - hq)))
    return spread.reshape(m, k)
