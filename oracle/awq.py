"""fp64 oracle for AWQ's per-layer alpha grid search (TEST INFRASTRUCTURE ONLY).

Plain NumPy float64; only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import it.

Sources:

* "GPTQ versus AWQ objectives" (inferenceinterviews.com), "A strong answer",
  AWQ paragraph: s_j = mean|x_j|^alpha, scale W's input channel j up by s_j
  (the activation is scaled down by the same factor elsewhere), round to
  nearest, and grid-search the single exponent alpha per layer on the
  calibration output error; no reconstruction, no backprop.
* "A Comprehensive Analysis of Post-Training Quantization Strategies for Large
  Language Models: GPTQ, AWQ and GGUF" (uplatz.com), section 3.2: the
  equivalent transform y = (W s)(X / s), then uniform low-bit quantization of
  the scaled matrix.

Readings: every channel is scaled (first page), s is not normalised (the error
is invariant to a global rescale of s), mean|x_j| is floored at 1e-12 times
its maximum so a dead channel cannot produce s = 0, the error is
||X (W - What)^T||^2 computed from dW directly, and ties in the grid go to the
smallest alpha (first argmin).
"""
from __future__ import annotations

import numpy as np

from .gptq import rtn

MEAN_ABS_FLOOR = 1e-12


def channel_mean_abs(X):
    """m_j = mean over calibration rows of |x_ij|, floored at 1e-12 * max m."""
    X = np.asarray(X, dtype=np.float64)
    m = np.mean(np.abs(X), axis=0)
    return np.maximum(m, MEAN_ABS_FLOOR * np.max(m))


def awq_quantize(W, s, bits: int, g: int):
    """RTN of W diag(s); returns (codes, scales, What) with What = Q(W s)/s."""
    W = np.asarray(W, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    Ws = W * s[None, :]
    codes, scales = rtn(Ws, bits, g)
    n = W.shape[1]
    g_idx = np.arange(n) // g
    What = (codes * scales[:, g_idx]) / s[None, :]
    return codes, scales, What


def awq_search(W, X, alphas, bits: int = 4, g: int = 128):
    """Grid search of alpha on the calibration output error.

    Returns dict(alpha, index, errors[len(alphas)], s, codes, scales, What).
    """
    W = np.asarray(W, dtype=np.float64)
    X = np.asarray(X, dtype=np.float64)
    m = channel_mean_abs(X)
    errors = np.zeros(len(alphas), dtype=np.float64)
    for i, a in enumerate(alphas):
        s = m ** float(a)
        _, _, What = awq_quantize(W, s, bits, g)
        E = X @ (W - What).T
        errors[i] = np.sum(E * E)
    best = int(np.argmin(errors))
    s = m ** float(alphas[best])
    codes, scales, What = awq_quantize(W, s, bits, g)
    return {"alpha": float(alphas[best]), "index": best, "errors": errors, "s": s,
            "codes": codes, "scales": scales, "What": What, "m": m}


def awq_gptq_layer(W, H0, d, s, bits: int = 4, g: int = 128, damp: float = 0.01, act_order: bool = False):
    """AWQ's scaling first, GPTQ's rounding after ("GPTQ versus AWQ
    objectives", "A strong answer": the two compose).

    With X' = X diag(s)^-1 and W' = W diag(s) the layer output is unchanged;
    GPTQ then runs on the scaled layer as on any layer: H0' = X'^T X' =
    diag(s)^-1 H0 diag(s)^-1, its fp64 column sums of squares d' = d / s^2,
    and the damping is taken on H0'. Returns gptq_layer's dict for the
    scaled layer (codes / scales quantize W') plus "What_orig" = What' / s,
    the weights the original activations see.
    """
    from .gptq import gptq_layer
    W = np.asarray(W, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    H0 = np.asarray(H0, dtype=np.float64)
    Ws = W * s[None, :]
    Hs = H0 / np.outer(s, s)
    ds = None if d is None else np.asarray(d, dtype=np.float64) / (s * s)
    res = gptq_layer(Ws, Hs, ds, bits=bits, g=g, damp=damp, act_order=act_order)
    res["What_orig"] = res["What"] / s[None, :]
    return res
