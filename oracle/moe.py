"""Sparse-MoE expert decode in float64: router top-k, SwiGLU experts, combine.

TEST INFRASTRUCTURE (see ``oracle/__init__``).

What the pages fix, and what is read into them:

* A MoE layer routes each token to its top-k experts and runs, per chosen
  expert, a gate_up GEMV then a down GEMV ("4 sequential experts x 2
  small-block GEMVs" per layer on the gpt-oss page, section 3 Results; top-4
  of 32 experts, hidden = intermediate = 2880, 24 layers for gpt-oss-20B and
  the same expert shape with 128 experts and 36 layers for 120B, same
  section).  Routing runs on the GPU ("GPU top-k path" on the host-sync page,
  section 3).
* The pages print no router or FFN formula.  Readings taken:
  - logits l[e] = sum_h W_r[e][h] x[h] (+ b[e]);
  - the chosen experts are the k largest logits, ties to the lower index;
  - their weights are a softmax over the chosen k logits (identical to a full
    softmax renormalised over the chosen k);
  - the expert FFN is the SiLU-gated SwiGLU: [g; u] = W_gu . x with g the
    first I rows and u the next I rows, h = silu(g) * u, d = W_d . h, no bias,
    no clamp;
  - the layer output is the router-weighted sum of the k expert outputs.
* Layer stacks: a per-layer norm exists in the fused all-layer decode path
  (host-sync page, section 3: per-layer norm/offset buffers).  Read as
  x <- x + MoE(RMSNorm(x)) with unit gain and eps = 1e-5; without a norm the
  residual stream of a random-weight stack overflows fp32 within a few
  layers.  A single layer (no stack) routes x itself and adds no residual.
"""

import numpy as np

RMS_EPS = 1e-5
NEAR_TIE_REL = 1e-6


def rmsnorm(x, eps=RMS_EPS):
    """x / sqrt(mean(x^2) + eps) along the last axis, unit gain, float64."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps)


def router_logits(w_r, xin, bias=None):
    """Router logits l[m][e] = sum_h W_r[e][h] xin[m][h] (+ b[e]) in float64.

    Also returns S[m][e] = sum_h |W_r[e][h] xin[m][h]|, the scale of the
    rounding error any fp32 evaluation of l[m][e] can carry.
    """
    w = np.asarray(w_r, dtype=np.float64)
    x = np.atleast_2d(np.asarray(xin, dtype=np.float64))
    logits = x @ w.T
    scale = np.abs(x) @ np.abs(w).T
    if bias is not None:
        logits = logits + np.asarray(bias, dtype=np.float64)[None, :]
    return logits, scale


def topk_order(logits, k):
    """Indices of the k largest logits per row: descending value, ties -> lower index."""
    logits = np.atleast_2d(np.asarray(logits, dtype=np.float64))
    n_exp = logits.shape[1]
    if not 1 <= k <= n_exp:
        raise ValueError("need 1 <= k <= number of experts")
    # A stable sort of -l keeps equal logits in ascending expert order.
    order = np.argsort(-logits, axis=1, kind="stable")
    return order[:, :k].astype(np.int64)


def softmax_over(logits_row, chosen):
    """Softmax of the chosen logits among themselves (float64)."""
    sel = np.asarray([logits_row[e] for e in chosen], dtype=np.float64)
    ex = np.exp(sel - np.max(sel))
    return ex / np.sum(ex)


def topk_softmax(logits, k):
    """(idx [m][k], w [m][k]): top-k experts and their softmax weights."""
    logits = np.atleast_2d(np.asarray(logits, dtype=np.float64))
    idx = topk_order(logits, k)
    w = np.stack([softmax_over(logits[m], idx[m]) for m in range(logits.shape[0])])
    return idx, w


def sigmoid(g):
    """1 / (1 + exp(-g)), evaluated without overflow for either sign."""
    g = np.asarray(g, dtype=np.float64)
    out = np.empty_like(g)
    pos = g >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-g[pos]))
    e = np.exp(g[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def silu(g):
    g = np.asarray(g, dtype=np.float64)
    return g * sigmoid(g)


def swiglu(gu, inter):
    """h = silu(g) * u with g = gu[:inter], u = gu[inter:2*inter]."""
    gu = np.asarray(gu, dtype=np.float64)
    if gu.shape[-1] != 2 * inter:
        raise ValueError("gate_up output must hold 2*inter rows")
    return silu(gu[..., :inter]) * gu[..., inter:]


def expert_ffn(w_gu, w_d, xin):
    """One expert on one token: returns (d, h, den_d).

    w_gu : [2I][H] dequantized gate_up, w_d : [H][I] dequantized down.
    den_d[i] = sum_k |W_d[i][k]| |h[k]| normalises the error of d[i].
    """
    w_gu = np.asarray(w_gu, dtype=np.float64)
    w_d = np.asarray(w_d, dtype=np.float64)
    inter = w_d.shape[1]
    gu = w_gu @ np.asarray(xin, dtype=np.float64)
    h = swiglu(gu, inter)
    d = w_d @ h
    den_d = np.abs(w_d) @ np.abs(h)
    return d, h, den_d


def near_tie(logits_row, scale_row, a, b, rel=NEAR_TIE_REL):
    """True when experts a and b are within the fp32 rounding band of each other."""
    band = rel * max(scale_row[a], scale_row[b])
    return abs(logits_row[a] - logits_row[b]) <= band


def check_routing(logits_row, scale_row, idx_gpu, k, rel=NEAR_TIE_REL):
    """Validate a GPU top-k list against float64 logits.

    A list is a correct top-k when it names k distinct experts in [0, E),
    no expert it leaves out beats an expert it keeps, and it runs in
    descending order -- each comparison exact outside the near-tie band and
    free inside it (fp32 rounding may decide a near tie either way).
    Returns (ok, n_ties, msg); n_ties counts the decisions taken inside the
    band (picks that differ from the oracle's own, and swapped neighbours).
    """
    logits_row = np.asarray(logits_row, dtype=np.float64)
    n_exp = logits_row.shape[0]
    try:
        idx_gpu = [int(e) for e in idx_gpu]
    except (TypeError, ValueError):
        return False, 0, "GPU top-k holds a non-integer"
    if len(idx_gpu) != k:
        return False, 0, f"GPU top-k holds {len(idx_gpu)} entries, expected {k}"
    for e in idx_gpu:
        if not 0 <= e < n_exp:
            return False, 0, f"expert {e} outside [0, {n_exp})"
    if len(set(idx_gpu)) != k:
        return False, 0, "duplicate expert in GPU top-k"
    own = [int(e) for e in topk_order(logits_row[None, :], k)[0]]
    if own == idx_gpu:
        return True, 0, ""
    kept = set(idx_gpu)
    # every expert left out must not beat any expert kept, up to the band
    for u in range(n_exp):
        if u in kept:
            continue
        for c in idx_gpu:
            if logits_row[u] > logits_row[c] and not near_tie(logits_row, scale_row, u, c, rel):
                return False, 0, f"expert {u} left out although it beats chosen expert {c}"
    ties = sum(1 for e in idx_gpu if e not in own)
    # the order must be descending up to the band
    for a, b in zip(idx_gpu[:-1], idx_gpu[1:]):
        inverted = logits_row[a] < logits_row[b] or (logits_row[a] == logits_row[b] and a > b)
        if inverted and not near_tie(logits_row, scale_row, a, b, rel):
            return False, ties, f"order {a} before {b} violates the logits"
        if inverted:
            ties += 1
    return True, ties, ""


def moe_layer(x, w_r, get_expert, k, bias=None, norm=False, residual=False,
              forced_idx=None, rel=NEAR_TIE_REL):
    """One MoE layer for a batch of tokens, layer-major.

    x          : [m][H] layer input (the residual stream when ``residual``)
    w_r, bias  : router weights [E][H] (and optional bias [E])
    get_expert : callable e -> (W_gu [2I][H], W_d [H][I]) dequantized weights
    norm       : route and feed the experts RMSNorm(x) instead of x
    residual   : output x + combine instead of combine
    forced_idx : optional [m][k] routing to adopt where it differs from the
                 oracle's own choice only inside the near-tie band
                 (teacher forcing); outside the band a mismatch raises.

    Returns a dict with y [m][H], den [m][H], idx, w, logits, scale, ties.
    """
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    m, hid = x.shape
    xin = rmsnorm(x) if norm else x
    logits, scale = router_logits(w_r, xin, bias)
    idx, w = topk_softmax(logits, k)
    ties = 0
    if forced_idx is not None:
        forced_idx = np.atleast_2d(np.asarray(forced_idx))
        for t in range(m):
            ok, n_ties, msg = check_routing(logits[t], scale[t], forced_idx[t], k, rel)
            if not ok:
                raise AssertionError(f"token {t}: {msg}")
            if n_ties:
                ties += n_ties
                idx[t] = forced_idx[t]
                w[t] = softmax_over(logits[t], idx[t])
    y = x.copy() if residual else np.zeros_like(x)
    den = np.abs(x) if residual else np.zeros_like(x)
    for e in np.unique(idx):
        w_gu, w_d = get_expert(int(e))
        for t, j in zip(*np.nonzero(idx == e)):
            d, _, den_d = expert_ffn(w_gu, w_d, xin[t])
            y[t] += w[t, j] * d
            den[t] += w[t, j] * den_d
    return dict(y=y, den=den, idx=idx, w=w, logits=logits, scale=scale,
                ties=ties, xin=xin)


def moe_stack(x, layers, k, forced_idx=None, resid_in=None, rel=NEAR_TIE_REL):
    """Residual stack: for each layer x <- x + MoE(RMSNorm(x)).

    layers     : list of (w_r, bias, get_expert) per layer
    forced_idx : optional [L][m][k] GPU routing, adopted inside the near-tie band
    resid_in   : optional [L][m][H] GPU residual inputs per layer.  When given,
                 layer l runs on resid_in[l] (teacher forcing), so each layer
                 is checked on its own; otherwise the oracle's own residual
                 stream is carried through.

    Returns a list of per-layer result dicts (``moe_layer``) and the output.
    """
    cur = np.atleast_2d(np.asarray(x, dtype=np.float64))
    results = []
    for l, (w_r, bias, get_expert) in enumerate(layers):
        inp = cur if resid_in is None else np.atleast_2d(np.asarray(resid_in[l], np.float64))
        f = None if forced_idx is None else forced_idx[l]
        res = moe_layer(inp, w_r, get_expert, k, bias=bias, norm=True,
                        residual=True, forced_idx=f, rel=rel)
        results.append(res)
        cur = res["y"]
    return results, cur


def max_rel_err(y, y_ref, den):
    """max_i |y_i - yref_i| / den_i (den_i = 0 requires an exact match)."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    den = np.asarray(den, dtype=np.float64)
    diff = np.abs(y - y_ref)
    if np.any((den == 0) & (diff != 0)):
        return np.inf
    with np.errstate(invalid="ignore", divide="ignore"):
        rel = np.where(den > 0, diff / np.where(den > 0, den, 1.0), 0.0)
    return float(np.max(rel)) if rel.size else 0.0


def cosine(a, b):
    a = np.asarray(a, dtype=np.float64).ravel()
    b = np.asarray(b, dtype=np.float64).ravel()
    na = np.linalg.norm(a)
    nb = np.linalg.norm(b)
    if na == 0 and nb == 0:
        return 1.0
    return float(a @ b / (na * nb))
