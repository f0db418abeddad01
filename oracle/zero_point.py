"""fp64 oracle for GPTQ / RTN with asymmetric (zero-point) groups
(TEST INFRASTRUCTURE ONLY; only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import it).

Sources:

* "A Comprehensive Analysis of Post-Training Quantization Strategies for Large
  Language Models: GPTQ, AWQ and GGUF" (uplatz.com), section 2.2: grouped
  quantization gives every group its own quantization parameters, a scale
  and a zero-point; section 2 opening: GPTQ also serves 3-bit and 2-bit.
* "GPTQ versus AWQ objectives" (inferenceinterviews.com), "A strong answer":
  the column loop itself (group parameters from the current, error-updated
  weights at the group's first column; round to nearest; error over U_jj fed
  to the later columns through row j of U), unchanged but for the grid.

Reading of "scale and zero-point" (the pages give no formula): the affine
grid w ~ (code - zero) * scale with codes 0 .. 2^bits - 1. Per row and group,
lo = min(0, min w), hi = max(0, max w) over the group's current weights (0 is
kept in the range so that it stays exactly representable), scale =
(hi - lo) / (2^bits - 1), zero = round_half_even(-lo / scale) and code =
clip(round_half_even(w / scale) + zero, 0, 2^bits - 1). A group whose weights
are all 0 gets scale 0, zero 0 and code 0.
"""
from __future__ import annotations

import numpy as np


def maxq(bits: int) -> int:
    """Largest code of the unsigned grid: 2^bits - 1."""
    return 2 ** bits - 1


def group_params(Wg, bits: int):
    """(scale, zero) per row of a group's current weights Wg [rows, cols]."""
    Wg = np.asarray(Wg, dtype=np.float64)
    lo = np.minimum(Wg.min(axis=1), 0.0)
    hi = np.maximum(Wg.max(axis=1), 0.0)
    scale = (hi - lo) / maxq(bits)
    zero = np.zeros_like(scale)
    live = scale != 0.0
    zero[live] = np.round(-lo[live] / scale[live])
    return scale, zero


def nearest_code(w, scale, zero, bits: int):
    """clip(round_half_even(w / scale) + zero, 0, maxq); scale 0 gives code 0."""
    code = np.zeros_like(w, dtype=np.float64)
    live = scale != 0.0
    code[live] = np.round(w[live] / scale[live]) + zero[live]
    return np.clip(code, 0, maxq(bits))


def dequantize(codes, scales, zeros, g_idx):
    """What[r, c] = (codes[r, c] - zeros[r, g_idx[c]]) * scales[r, g_idx[c]]."""
    gi = np.asarray(g_idx)
    codes = np.asarray(codes, dtype=np.float64)
    return (codes - np.asarray(zeros, dtype=np.float64)[:, gi]) * np.asarray(scales, dtype=np.float64)[:, gi]


def gptq_columns(W, U, bits: int, g: int):
    """The column loop with zero-point groups; returns (codes, scales, zeros,
    err), all in processing order."""
    Wc = np.array(W, dtype=np.float64, copy=True)
    U = np.asarray(U, dtype=np.float64)
    out, n = Wc.shape
    ngroups = (n + g - 1) // g
    codes = np.zeros((out, n), dtype=np.int64)
    scales = np.zeros((out, ngroups))
    zeros = np.zeros((out, ngroups))
    err = np.zeros((out, n))
    for grp in range(ngroups):
        g0, g1 = grp * g, min(n, (grp + 1) * g)
        scale, zero = group_params(Wc[:, g0:g1], bits)
        scales[:, grp] = scale
        zeros[:, grp] = zero
        for j in range(g0, g1):
            c = nearest_code(Wc[:, j], scale, zero, bits)
            codes[:, j] = c.astype(np.int64)
            e = (Wc[:, j] - (c - zero) * scale) / U[j, j]
            err[:, j] = e
            Wc[:, j + 1:] -= e[:, None] * U[j, j + 1:][None, :]
    return codes, scales, zeros, err


def rtn(W, bits: int, g: int):
    """Zero-point group round-to-nearest, no feedback: (codes, scales, zeros)."""
    W = np.asarray(W, dtype=np.float64)
    out, n = W.shape
    ngroups = (n + g - 1) // g
    codes = np.zeros((out, n), dtype=np.int64)
    scales = np.zeros((out, ngroups))
    zeros = np.zeros((out, ngroups))
    for grp in range(ngroups):
        g0, g1 = grp * g, min(n, (grp + 1) * g)
        scale, zero = group_params(W[:, g0:g1], bits)
        scales[:, grp] = scale
        zeros[:, grp] = zero
        for j in range(g0, g1):
            codes[:, j] = nearest_code(W[:, j], scale, zero, bits).astype(np.int64)
    return codes, scales, zeros


def gptq_layer(W, H0, d=None, bits: int = 4, g: int = 128, damp: float = 0.01, act_order: bool = False):
    """GPTQ with zero-point groups on a precomputed H0: the same stages as the
    symmetric layer (damping, optional act-order, U, the loop), returning
    codes in the original column order with g_idx, scales and zeros."""
    from .gptq import damped, act_order_permutation, inverse_upper_factor
    W = np.asarray(W, dtype=np.float64)
    H, lam = damped(H0, damp)
    n = W.shape[1]
    if d is None:
        d = np.diag(np.asarray(H0, dtype=np.float64))
    perm = act_order_permutation(d) if act_order else np.arange(n, dtype=np.int64)
    U = inverse_upper_factor(H[np.ix_(perm, perm)])
    codes_p, scales, zeros, err = gptq_columns(W[:, perm], U, bits, g)
    codes = np.empty_like(codes_p)
    codes[:, perm] = codes_p
    g_idx = np.empty(n, dtype=np.int64)
    g_idx[perm] = np.arange(n) // g
    What = dequantize(codes, scales, zeros, g_idx)
    dW = W - What
    return {
        "codes": codes, "scales": scales, "zeros": zeros, "g_idx": g_idx, "perm": perm,
        "U": U, "lambda": lam, "err": err,
        "sum_err2": float(np.sum(err * err)), "dW_fro2": float(np.sum(dW * dW)), "What": What,
    }
