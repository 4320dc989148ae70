"""Dequant-GEMV, written as dequantize-then-dense-matvec in float64.

TEST INFRASTRUCTURE (see ``oracle/__init__``).

The fused kernel of the TinyTitan tracker (entry D108, "MetalInt4Matmul") is
stated there to equal dequantisation followed by an ordered dense matmul; the
cooperative MXFP4 GEMV of the gpt-oss page (section 4 Ablations) differs from
the plain one only by re-associating the fp32 sum across blocks.  So the
plain definition of the fused dequant-GEMV is: dequantize W, then y = W . x.
Here that product is taken in float64 (a library matmul), together with the
normaliser den = |W| . |x| that bounds any summation-order error.
"""

import numpy as np


def gemv(w, x):
    """y[m][n] = sum_k W[n][k] * x[m][k] and den[m][n] = sum_k |W[n][k]| |x[m][k]|.

    w : [n][k] (fp32 dequantized weights, or fp64)
    x : [k] or [m][k]
    Returns (y, den) in float64 with x's leading shape.
    """
    w64 = np.asarray(w, dtype=np.float64)
    x64 = np.asarray(x, dtype=np.float64)
    squeeze = x64.ndim == 1
    x2 = x64[None, :] if squeeze else x64
    if x2.shape[1] != w64.shape[1]:
        raise ValueError("x and W disagree on K")
    y = x2 @ w64.T
    den = np.abs(x2) @ np.abs(w64).T
    if squeeze:
        return y[0], den[0]
    return y, den


def gemv_loops(w, x):
    """The same product by explicit Python loops (tiny inputs only).

    Used to pin ``gemv`` by brute force; no library routine is involved.
    """
    w = np.asarray(w, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    n, k = w.shape
    y = [0.0] * n
    den = [0.0] * n
    for r in range(n):
        acc = 0.0
        acc_abs = 0.0
        for c in range(k):
            acc += float(w[r, c]) * float(x[c])
            acc_abs += abs(float(w[r, c])) * abs(float(x[c]))
        y[r] = acc
        den[r] = acc_abs
    return np.array(y), np.array(den)
