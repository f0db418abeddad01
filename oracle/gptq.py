"""fp64 oracle for GPTQ layer quantization (TEST INFRASTRUCTURE ONLY).

Plain, slow, obviously-correct NumPy in float64. Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it; the product path never does, and it shares no code with the HIP
library.

Sources (cited by page title and section):

* "GPTQ versus AWQ objectives" (inferenceinterviews.com), "A strong answer":
  the layer objective ||X W^T - X What^T||^2, the proxy Hessian X^T X, the 1%
  mean-diagonal damping, the upper Cholesky factor of H^-1, and the
  column-by-column loop (group scale at each group start from the current,
  error-updated weights; round to nearest; clip to [-qmax-1, qmax]; error
  divided by U_jj pushed onto the later columns through row j of U).
* same page, "What interviewers probe next": act-order (columns in decreasing
  Hessian diagonal) and the purpose of damping.
* "A Comprehensive Analysis of Post-Training Quantization Strategies for Large
  Language Models: GPTQ, AWQ and GGUF" (uplatz.com), section 2.1 (layer-wise
  objective), 2.2 (group size, act-order) and 2.3 (GPTQ equals Babai's
  nearest-plane algorithm on the lattice defined by the Hessian).

Readings where the pages are silent:

* H = X^T X without the factor 2 or a 1/N (codes are invariant to H -> cH
  because the damping is relative);
* rounding is half-to-even (NumPy's round); a group whose max |w| is 0 gets
  scale 0 and code 0;
* a last group shorter than g is its own group;
* the act-order key is d_j = sum_i x_ij^2 in float64, ties broken by the lower
  column index (stable sort).
"""
from __future__ import annotations

import numpy as np


def qmax(bits: int) -> int:
    """Largest positive code of a symmetric signed grid: 2^(bits-1) - 1."""
    return 2 ** (bits - 1) - 1


def hessian_nbytes(n: int) -> int:
    """Bytes of an fp32 [n, n] proxy Hessian (page sizes it for Llama 3.3 70B)."""
    return n * n * 4


# ---------------------------------------------------------------- stage 1 ---

def proxy_hessian(X, chunk_rows: int = 2048):
    """H0 = X^T X and d_j = sum_i x_ij^2, both float64.

    Accumulated over row chunks (the calibration set is streamed). The upper
    triangle is mirrored so H0 is exactly symmetric.
    """
    X = np.asarray(X)
    n = X.shape[1]
    H0 = np.zeros((n, n), dtype=np.float64)
    d = np.zeros(n, dtype=np.float64)
    for r0 in range(0, X.shape[0], chunk_rows):
        xc = np.asarray(X[r0:r0 + chunk_rows], dtype=np.float64)
        H0 += xc.T @ xc
        d += np.sum(xc * xc, axis=0)
    upper = np.triu(H0)
    H0 = upper + np.triu(upper, 1).T
    return H0, d


def damped(H0, damp: float):
    """H = H0 + lambda I with lambda = damp * mean(diag H0). Returns (H, lambda)."""
    H0 = np.asarray(H0, dtype=np.float64)
    lam = float(damp) * float(np.mean(np.diag(H0)))
    return H0 + lam * np.eye(H0.shape[0]), lam


def act_order_permutation(d):
    """perm[k] = original column processed k-th: decreasing d, ties by index."""
    d = np.asarray(d, dtype=np.float64)
    return np.argsort(-d, kind="stable").astype(np.int64)


# ---------------------------------------------------------------- stage 2 ---

def inverse_upper_factor(H):
    """Upper-triangular U with positive diagonal and U^T U = H^-1.

    "GPTQ versus AWQ objectives", "A strong answer": the loop reads U, the
    upper Cholesky factor of H^-1 (the page forms it by inverting H, taking
    the lower Cholesky factor and transposing). That factor is
    unique, and it is also the inverse of the Cholesky factor of H taken in
    reversed index order: if H = R R^T with R upper triangular, then
    U = R^-1 gives U^T U = R^-T R^-1 = (R R^T)^-1 = H^-1. Reversing both
    indices (J H J, J the exchange matrix) turns R into an ordinary lower
    Cholesky factor L = J R J, so U = J L^-1 J: one LAPACK Cholesky and one
    triangular inverse, with no explicit H^-1 (a third of the work, which is
    what lets the oracle factor a 28672^2 Hessian).
    """
    from scipy.linalg import lapack

    A = np.asfortranarray(np.asarray(H, dtype=np.float64)[::-1, ::-1])
    L, info = lapack.dpotrf(A, lower=1, clean=1, overwrite_a=1)
    if info != 0:
        raise np.linalg.LinAlgError(f"H is not positive definite (LAPACK potrf info {info})")
    del A
    Linv, info = lapack.dtrtri(L, lower=1, overwrite_c=1)
    if info != 0:
        raise np.linalg.LinAlgError(f"singular Cholesky factor (LAPACK trtri info {info})")
    del L
    return np.ascontiguousarray(Linv[::-1, ::-1])


# ---------------------------------------------------------------- stage 3 ---

def _nearest_code(w, scale, q):
    """Round w/scale half-to-even, clip to [-q-1, q]; scale 0 gives code 0."""
    code = np.zeros_like(w)
    live = scale != 0.0
    code[live] = np.round(w[live] / scale[live])
    return np.clip(code, -q - 1, q)


def gptq_columns(W, U, bits: int, g: int):
    """The column-by-column error-feedback loop, in the order the page gives.

    Walks groups of g columns; at a group's first column the per-row scale is
    max |W_cur| over that group's columns divided by qmax, where W_cur already
    carries the feedback of every earlier column. Each column is rounded and
    clipped; its error over U_jj is subtracted from all later columns through
    row j of U.

    Returns (codes [out, n] int64, scales [out, ngroups] float64,
    err [out, n] float64) in processing order.
    """
    Wc = np.array(W, dtype=np.float64, copy=True)
    U = np.asarray(U, dtype=np.float64)
    out, n = Wc.shape
    q = qmax(bits)
    ngroups = (n + g - 1) // g
    codes = np.zeros((out, n), dtype=np.int64)
    scales = np.zeros((out, ngroups), dtype=np.float64)
    err = np.zeros((out, n), dtype=np.float64)
    for grp in range(ngroups):
        g0, g1 = grp * g, min(n, (grp + 1) * g)
        scale = np.max(np.abs(Wc[:, g0:g1]), axis=1) / q
        scales[:, grp] = scale
        for j in range(g0, g1):
            c = _nearest_code(Wc[:, j], scale, q)
            codes[:, j] = c.astype(np.int64)
            e = (Wc[:, j] - c * scale) / U[j, j]
            err[:, j] = e
            Wc[:, j + 1:] -= e[:, None] * U[j, j + 1:][None, :]
    return codes, scales, err


def rtn(W, bits: int, g: int):
    """Plain group round-to-nearest: no feedback. Returns (codes, scales)."""
    W = np.asarray(W, dtype=np.float64)
    out, n = W.shape
    q = qmax(bits)
    ngroups = (n + g - 1) // g
    codes = np.zeros((out, n), dtype=np.int64)
    scales = np.zeros((out, ngroups), dtype=np.float64)
    for grp in range(ngroups):
        g0, g1 = grp * g, min(n, (grp + 1) * g)
        scale = np.max(np.abs(W[:, g0:g1]), axis=1) / q
        scales[:, grp] = scale
        for j in range(g0, g1):
            codes[:, j] = _nearest_code(W[:, j], scale, q).astype(np.int64)
    return codes, scales


def dequantize(codes, scales, g_idx):
    """What[r, c] = codes[r, c] * scales[r, g_idx[c]]."""
    codes = np.asarray(codes, dtype=np.float64)
    return codes * np.asarray(scales, dtype=np.float64)[:, np.asarray(g_idx)]


def gptq_layer(W, H0, d=None, bits: int = 4, g: int = 128, damp: float = 0.01,
               act_order: bool = False, U=None):
    """Whole GPTQ layer on a precomputed H0 (and the fp64 key d for act-order).

    Stages: damping; optional act-order permutation of H's rows/columns and
    W's columns; U; the column loop; codes back in the original column order
    with g_idx[c] = (position of column c in processing order) // g.
    A caller may pass ``U`` (already in the processing basis) to skip stage 2.
    """
    W = np.asarray(W, dtype=np.float64)
    H, lam = damped(H0, damp)
    n = W.shape[1]
    if d is None:
        d = np.diag(np.asarray(H0, dtype=np.float64))
    perm = act_order_permutation(d) if act_order else np.arange(n, dtype=np.int64)
    Hp = H[np.ix_(perm, perm)]
    Wp = W[:, perm]
    if U is None:
        U = inverse_upper_factor(Hp)
    codes_p, scales, err = gptq_columns(Wp, U, bits, g)
    codes = np.empty_like(codes_p)
    codes[:, perm] = codes_p
    g_idx = np.empty(n, dtype=np.int64)
    g_idx[perm] = np.arange(n) // g
    What = dequantize(codes, scales, g_idx)
    dW = W - What
    return {
        "codes": codes, "scales": scales, "g_idx": g_idx, "perm": perm,
        "U": U, "lambda": lam, "err": err,
        "sum_err2": float(np.sum(err * err)),
        "dW_fro2": float(np.sum(dW * dW)),
        "What": What,
    }


# ---------------------------------------------------------------- metrics ---

def output_error(X, W, What):
    """||X W^T - X What^T||_F^2, the objective both methods share ("A strong
    answer": the layer-wise output reconstruction error)."""
    X = np.asarray(X, dtype=np.float64)
    dW = np.asarray(W, dtype=np.float64) - np.asarray(What, dtype=np.float64)
    E = X @ dW.T
    return float(np.sum(E * E))


def output_energy(X, W):
    """||X W^T||_F^2: the energy of the layer output the objective above is
    measured against (denominator of the relative output error)."""
    X = np.asarray(X, dtype=np.float64)
    Y = X @ np.asarray(W, dtype=np.float64).T
    return float(np.sum(Y * Y))


def quadratic_error(H0, W, What):
    """tr(dW H0 dW^T): equals output_error when H0 = X^T X."""
    dW = np.asarray(W, dtype=np.float64) - np.asarray(What, dtype=np.float64)
    return float(np.sum((dW @ np.asarray(H0, dtype=np.float64)) * dW))
