"""Pins of the fp64 oracle against facts fixed outside the oracle itself.

Each ``check_*`` takes an implementation namespace ``impl`` (the real
``oracle`` package, or a copy with a planted mistake) and raises
AssertionError when the implementation disagrees with what the pages or the
mathematics fix: hand-derived worked examples under tests/golden/, closed
forms, identities, special cases that reduce to a simpler routine, and a
textbook algorithm written independently (Babai's nearest plane).
"""
from __future__ import annotations

import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------- helpers ---

def spd(n, seed, cond_spread=1.0, corr=0.3):
    """A random SPD matrix with correlated off-diagonals."""
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((3 * n, n))
    A = A + corr * rng.standard_normal((3 * n, 1))      # shared factor -> correlation
    A = A * np.exp(cond_spread * rng.standard_normal(n))[None, :]
    return A.T @ A


def reverse_cholesky(H):
    """R upper with H = R R^T (flip, lower Cholesky, flip back)."""
    J = np.eye(H.shape[0])[::-1]
    Lf = np.linalg.cholesky(J @ H @ J)
    return J @ Lf @ J


def textbook_cholesky_lower(A):
    """Cholesky-Banachiewicz in plain Python loops (tiny sizes only)."""
    n = len(A)
    L = [[0.0] * n for _ in range(n)]
    for i in range(n):
        for j in range(i + 1):
            s = sum(L[i][k] * L[j][k] for k in range(j))
            if i == j:
                L[i][j] = (A[i][i] - s) ** 0.5
            else:
                L[i][j] = (A[i][j] - s) / L[j][j]
    return np.array(L)


def babai_nearest_plane(basis_rows, target):
    """Babai's nearest-plane algorithm (textbook form).

    basis_rows[k] is b_{k+1}; Gram-Schmidt runs in index order and the
    coefficients are decided from the last basis vector to the first.
    Returns the integer coefficient vector c with lattice point sum c_k b_k.
    """
    B = np.asarray(basis_rows, dtype=np.float64)
    n = B.shape[0]
    Bs = np.zeros_like(B)
    for k in range(n):
        v = B[k].copy()
        for i in range(k):
            v -= (B[k] @ Bs[i]) / (Bs[i] @ Bs[i]) * Bs[i]
        Bs[k] = v
    t = np.asarray(target, dtype=np.float64).copy()
    c = np.zeros(n)
    for k in range(n - 1, -1, -1):
        c[k] = np.round((t @ Bs[k]) / (Bs[k] @ Bs[k]))
        t -= c[k] * B[k]
    return c


# ------------------------------------------------------------------ pins ---

def check_rtn_hand(impl):
    gd = load_golden("rtn_hand.json")
    W = np.array(gd["W"])
    for bits, key in ((4, "bits4"), (2, "bits2")):
        codes, scales = impl.rtn(W, bits, gd["g"])
        assert np.array_equal(codes, np.array(gd[key]["codes"])), (bits, codes)
        assert np.allclose(scales, np.array(gd[key]["scales"]), rtol=0, atol=1e-15)


def check_gptq_hand(impl):
    gd = load_golden("gptq_hand.json")
    for case in gd["cases"]:
        U = np.array(case["U"])
        H = np.linalg.inv(U.T @ U)
        if "H_by_hand" in case:
            assert np.allclose(H, np.array(case["H_by_hand"]), atol=1e-9)
        W = np.array(case["W"])
        res = impl.gptq_layer(W, H, None, bits=case["bits"], g=case["g"], damp=0.0)
        assert np.allclose(res["U"], U, atol=1e-9), res["U"]
        assert np.array_equal(res["codes"], np.array(case["codes"])), (case["name"], res["codes"])
        assert np.allclose(res["scales"], np.array(case["scales"]), atol=1e-9), res["scales"]
        assert np.allclose(res["err"], np.array(case["err"]), atol=1e-9), res["err"]


def check_damping_hand(impl):
    gd = load_golden("small_hand.json")["damping"]
    H, lam = impl.damped(np.array(gd["H0"]), gd["damp"])
    assert abs(lam - gd["lambda"]) < 1e-15
    assert np.allclose(np.diag(H), gd["diag"], rtol=0, atol=1e-14)
    off = H - np.diag(np.diag(H))
    H0 = np.array(gd["H0"])
    assert np.array_equal(off, H0 - np.diag(np.diag(H0)))


def check_act_order_hand(impl):
    gd = load_golden("small_hand.json")["act_order"]
    perm = impl.act_order_permutation(np.array(gd["d"]))
    assert list(perm) == gd["perm"]
    # g_idx through the layer: diagonal H0 = diag(d), so the loop is RTN
    W = np.array([[0.5, -0.25, 0.125, 1.0]])
    res = impl.gptq_layer(W, np.diag(gd["d"]), np.array(gd["d"]), bits=4, g=gd["g"], damp=0.01,
                          act_order=True)
    assert list(res["g_idx"]) == gd["g_idx"]
    assert list(res["perm"]) == gd["perm"]


def check_hessian_bruteforce(impl):
    rng = np.random.default_rng(11)
    X = rng.standard_normal((7, 4))
    H0, d = impl.proxy_hessian(X, chunk_rows=3)
    for i in range(4):
        assert abs(d[i] - sum(X[k, i] ** 2 for k in range(7))) < 1e-12
        for j in range(4):
            ref = sum(X[k, i] * X[k, j] for k in range(7))
            assert abs(H0[i, j] - ref) < 1e-12, (i, j)
    assert np.array_equal(H0, H0.T)


def check_hessian_orthogonal(impl):
    """X = Hadamard(8) diag(c): columns orthogonal, H0 = 8 diag(c^2) exactly."""
    Hd = np.array([[1.0]])
    for _ in range(3):
        Hd = np.block([[Hd, Hd], [Hd, -Hd]])
    c = np.array([0.5, 1.0, 2.0, 0.25, 4.0, 1.5, 3.0, 0.125])
    H0, d = impl.proxy_hessian(Hd * c[None, :], chunk_rows=3)
    assert np.array_equal(H0, np.diag(8.0 * c * c))
    assert np.array_equal(d, 8.0 * c * c)


def check_hessian_chunking(impl):
    rng = np.random.default_rng(5)
    X = rng.standard_normal((300, 12))
    a, da = impl.proxy_hessian(X, chunk_rows=1)
    b, db = impl.proxy_hessian(X, chunk_rows=1000)
    assert np.allclose(a, b, rtol=1e-13, atol=1e-12)
    assert np.allclose(da, db, rtol=1e-13)
    w = np.linalg.eigvalsh(b)
    assert w.min() >= -1e-10 * w.max()


def check_inverse_factor_closed_form(impl):
    """2x2: U^T U = H^-1 by hand."""
    a, b, c = 5.0, 1.5, 2.0
    det = a * c - b * b
    u11 = np.sqrt(c / det)
    u12 = -b / (det * u11)
    u22 = np.sqrt(a / det - u12 * u12)
    U = impl.inverse_upper_factor(np.array([[a, b], [b, c]]))
    assert np.allclose(U, [[u11, u12], [0.0, u22]], rtol=1e-13, atol=1e-15)


def check_inverse_factor_identity(impl):
    for n, seed in ((6, 1), (40, 2), (128, 3)):
        H = spd(n, seed)
        U = impl.inverse_upper_factor(H)
        assert np.array_equal(U, np.triu(U))
        assert np.all(np.diag(U) > 0)
        assert np.max(np.abs(U.T @ U @ H - np.eye(n))) <= 1e-10
        # the page's own route: invert H, lower Cholesky factor of the
        # inverse, transpose (a different computation of the same unique factor)
        Upage = np.linalg.cholesky(np.linalg.inv(H)).T
        assert np.allclose(U, Upage, rtol=1e-9, atol=1e-11 * np.abs(U).max())
    # brute-force Cholesky (plain loops) on the flipped matrix
    H = spd(5, 9)
    J = np.eye(5)[::-1]
    R = J @ textbook_cholesky_lower((J @ H @ J).tolist()) @ J
    assert np.allclose(impl.inverse_upper_factor(H), np.linalg.inv(R), rtol=1e-11, atol=1e-13)


def check_diagonal_H_is_rtn(impl):
    rng = np.random.default_rng(3)
    W = rng.standard_normal((9, 20))
    for H0 in (np.eye(20) * 3.7, np.diag(np.exp(rng.standard_normal(20)))):
        res = impl.gptq_layer(W, H0, None, bits=4, g=8, damp=0.01)
        codes, scales = impl.rtn(W, 4, 8)
        assert np.array_equal(res["codes"], codes)
        assert np.allclose(res["scales"], scales, rtol=1e-14, atol=0)


def check_babai_identity(impl):
    """sum err^2 = tr(dW H dW^T) for the damped H, for any rounding choices."""
    rng = np.random.default_rng(4)
    for n, g, bits in ((24, 8, 4), (30, 16, 3), (17, 5, 2)):
        H0 = spd(n, 10 + n)
        W = rng.standard_normal((6, n))
        res = impl.gptq_layer(W, H0, None, bits=bits, g=g, damp=0.01)
        H, lam = impl.damped(H0, 0.01)
        dW = W - res["What"]
        quad = float(np.sum((dW @ H) * dW))
        assert abs(res["sum_err2"] - quad) <= 1e-9 * quad, (res["sum_err2"], quad)
        # free calibration objective: tr(dW H0 dW^T) = sum err^2 - lambda ||dW||^2
        q0 = float(np.sum((dW @ H0) * dW))
        assert abs(res["sum_err2"] - lam * res["dW_fro2"] - q0) <= 1e-9 * q0
        # nearest-plane bound holds when no code sits on the clip edge
        edge = (res["codes"] == -(2 ** (bits - 1)))
        if not edge.any():
            U = res["U"]
            s = res["scales"][:, np.arange(n) // g]
            bound = np.sum(s * s / (4.0 * np.diag(U)[None, :] ** 2), axis=1)
            per_row = np.sum(res["err"] ** 2, axis=1)
            assert np.all(per_row <= bound * (1 + 1e-12))


def check_babai_equivalence(impl):
    """One group, no clipping: GPTQ codes = Babai nearest plane on the lattice
    generated by the rows of R (H = R R^T), decided from column 0 onward."""
    rng = np.random.default_rng(8)
    for n in (2, 3, 4, 5, 6):
        H0 = spd(n, 100 + n, cond_spread=0.7, corr=0.8)
        H, _ = impl.damped(H0, 0.0)
        R = reverse_cholesky(H)
        for _ in range(4):
            w = rng.standard_normal(n)
            w[0] = 10.0                      # the max sits in column 0: no clip at 8 bits
            res = impl.gptq_layer(w[None, :], H0, None, bits=8, g=n, damp=0.0)
            s = res["scales"][0, 0]
            basis = R[::-1]                  # b_1 = r_{n-1}, ..., b_n = r_0
            c = babai_nearest_plane(basis, (w / s) @ R)
            q = c[::-1]
            assert np.array_equal(res["codes"][0], q.astype(np.int64)), (n, res["codes"][0], q)


def check_grid_and_invariances(impl):
    rng = np.random.default_rng(6)
    n = 32
    H0 = spd(n, 77)
    W = rng.standard_normal((5, n))
    for bits in (2, 3, 4):
        res = impl.gptq_layer(W, H0, None, bits=bits, g=8, damp=0.01)
        q = 2 ** (bits - 1) - 1
        assert res["codes"].min() >= -q - 1 and res["codes"].max() <= q
        What = res["What"]
        ratio = What / res["scales"][:, np.arange(n) // 8]
        assert np.allclose(ratio, np.round(ratio), atol=1e-9)
        # first group's scale comes from the untouched weights
        assert np.allclose(res["scales"][:, 0], np.abs(W[:, :8]).max(1) / q, rtol=1e-15)
        # H -> cH and positive row scaling of W leave codes unchanged
        res2 = impl.gptq_layer(W * np.array([[2.0], [0.5], [4.0], [1.0], [8.0]]), H0 * 3.0, None,
                               bits=bits, g=8, damp=0.01)
        assert np.array_equal(res["codes"], res2["codes"])


def check_gptq_beats_rtn_correlated(impl):
    """Empirical (not a theorem): with correlated inputs GPTQ's calibration
    error is well below RTN's."""
    rng = np.random.default_rng(12)
    n, N = 64, 512
    base = rng.standard_normal((N, 8))
    X = base @ rng.standard_normal((8, n)) + 0.3 * rng.standard_normal((N, n))
    W = rng.standard_normal((16, n))
    H0, d = impl.proxy_hessian(X)
    res = impl.gptq_layer(W, H0, d, bits=4, g=32, damp=0.01)
    codes, scales = impl.rtn(W, 4, 32)
    Wr = impl.dequantize(codes, scales, np.arange(n) // 32)
    e_g = impl.output_error(X, W, res["What"])
    e_r = impl.output_error(X, W, Wr)
    assert e_g < 0.8 * e_r, (e_g, e_r)
    assert abs(impl.quadratic_error(H0, W, res["What"]) - e_g) <= 1e-9 * e_g


def check_act_order_matches_permuted_problem(impl):
    """act-order = natural order on the column-permuted problem, un-permuted."""
    rng = np.random.default_rng(13)
    n = 24
    X = rng.standard_normal((100, n)) * np.exp(rng.standard_normal(n))[None, :]
    W = rng.standard_normal((4, n))
    H0, d = impl.proxy_hessian(X)
    res = impl.gptq_layer(W, H0, d, bits=4, g=8, damp=0.01, act_order=True)
    perm = np.argsort(-d, kind="stable")
    assert np.array_equal(res["perm"], perm)
    assert np.all(np.diff(d[perm]) <= 0)
    ref = impl.gptq_layer(W[:, perm], H0[np.ix_(perm, perm)], d[perm], bits=4, g=8, damp=0.01)
    assert np.array_equal(res["codes"][:, perm], ref["codes"])
    assert np.allclose(res["scales"], ref["scales"], rtol=1e-14)


def check_awq(impl):
    gd = load_golden("small_hand.json")["awq_mean_abs"]
    assert np.allclose(impl.channel_mean_abs(np.array(gd["X"])), gd["m"], rtol=0, atol=1e-15)
    rng = np.random.default_rng(14)
    n = 64
    X = rng.standard_normal((200, n)) * np.exp(rng.standard_normal(n))[None, :]
    W = rng.standard_normal((8, n))
    alphas = [0.0, 0.25, 0.5, 0.75]
    r = impl.awq_search(W, X, alphas, bits=4, g=32)
    # alpha = 0 is plain RTN
    codes, scales = impl.rtn(W, 4, 32)
    What0 = impl.dequantize(codes, scales, np.arange(n) // 32)
    assert abs(r["errors"][0] - impl.output_error(X, W, What0)) <= 1e-12 * r["errors"][0]
    # the choice is the first argmin of the grid
    assert r["index"] == int(np.argmin(r["errors"]))
    # each error equals tr(dW H0 dW^T)
    H0, _ = impl.proxy_hessian(X)
    for a, e in zip(alphas, r["errors"]):
        _, _, What = impl.awq_quantize(W, impl.channel_mean_abs(X) ** a, 4, 32)
        assert abs(impl.quadratic_error(H0, W, What) - e) <= 1e-9 * e
    # weights change only by rounding: (What * s) / scale is integral
    ratio = (r["What"] * r["s"][None, :]) / r["scales"][:, np.arange(n) // 32]
    assert np.allclose(ratio, np.round(ratio), atol=1e-9)
    # global rescale of s (here of the activations' magnitude) changes nothing
    r2 = impl.awq_search(W, X * 7.3, alphas, bits=4, g=32)
    assert r2["index"] == r["index"]
    assert np.allclose(r2["errors"] / (7.3 ** 2), r["errors"], rtol=1e-9)


def check_hessian_sizes(impl):
    gd = load_golden("small_hand.json")["hessian_sizes"]
    for n, printed, precision in gd["cases"]:
        assert abs(impl.hessian_nbytes(n) - printed) <= precision / 2, (n, impl.hessian_nbytes(n))


def check_pack_hand(impl):
    gd = load_golden("pack_hand.json")["pack"]
    words = impl.pack_int4(np.array(gd["codes"]))
    assert words.dtype == np.uint32
    assert np.array_equal(words.astype(np.int64), np.array(gd["words"], dtype=np.int64))
    assert np.array_equal(impl.unpack_int4(words, 8), np.array(gd["codes"]))


def check_pack_roundtrip(impl):
    """Every nibble value at every position survives pack -> unpack."""
    vals = np.arange(-8, 8)
    codes = np.stack([np.roll(vals, s)[:16] for s in range(16)])       # [16, 16]: each value at each column
    assert np.array_equal(impl.unpack_int4(impl.pack_int4(codes), 16), codes)
    rng = np.random.default_rng(21)
    c = rng.integers(-8, 8, size=(7, 40))
    assert np.array_equal(impl.unpack_int4(impl.pack_int4(c), 40), c)


def check_pack_zero_point(impl):
    """Zero-point codes (0..15) pack as plain nibbles and dequantize with their zero."""
    codes = np.array([[0, 15, 7, 8, 1, 14, 3, 12]])
    words = impl.pack_int4(codes)
    # nibbles 0, F, 7, 8, 1, E, 3, C -> 0xC3E187F0
    assert int(words[0, 0]) == 0xC3E187F0
    assert np.array_equal(impl.unpack_int4(words, 8, signed=False), codes)
    zeros = np.array([[7.0]])
    What = impl.dequantize_packed(words, np.array([[0.5]]), np.zeros(8, dtype=int), 8, zeros=zeros)
    assert np.array_equal(What, (codes - 7.0) * 0.5)


def check_dequant_g_idx_hand(impl):
    gd = load_golden("pack_hand.json")["dequant_g_idx"]
    packed = impl.pack_int4(np.array(gd["codes"]))
    What = impl.dequantize_packed(packed, np.array(gd["scales"]), np.array(gd["g_idx"]), 8)
    assert np.array_equal(What, np.array(gd["What"]))
    assert not np.array_equal(What, np.array(gd["What_ignoring_g_idx"]))
    # same as dequantizing in processing order and un-permuting
    perm = np.array(gd["perm"])
    codes = np.array(gd["codes"])
    proc = impl.dequantize(codes[:, perm], np.array(gd["scales"]), np.arange(8) // gd["g"])
    assert np.array_equal(What[:, perm], proc)


def check_awq_gptq(impl):
    """AWQ scaling then GPTQ ("the two compose"): pinned by its definition
    through the activations (X' = X / s), by s = 1 (plain GPTQ), by a diagonal
    H (GPTQ is RTN, so the composition is AWQ's RTN) and by a global rescale
    of s."""
    rng = np.random.default_rng(31)
    n, N = 32, 400
    base = rng.standard_normal((N, 6))
    X = (base @ rng.standard_normal((6, n)) + 0.5 * rng.standard_normal((N, n))) * np.exp(rng.standard_normal(n))
    W = rng.standard_normal((6, n))
    H0, d = impl.proxy_hessian(X)
    s = impl.channel_mean_abs(X) ** 0.5
    for act_order in (False, True):
        res = impl.awq_gptq_layer(W, H0, d, s, bits=3, g=8, damp=0.01, act_order=act_order)
        # definition: GPTQ on the scaled layer, its Hessian built from X / s
        Hs, ds = impl.proxy_hessian(X / s[None, :])
        ref = impl.gptq_layer(W * s[None, :], Hs, ds, bits=3, g=8, damp=0.01, act_order=act_order)
        assert np.array_equal(res["codes"], ref["codes"])
        assert np.allclose(res["scales"], ref["scales"], rtol=1e-12)
        assert np.array_equal(res["perm"], ref["perm"])
        assert np.allclose(res["What_orig"], ref["What"] / s[None, :], rtol=1e-12)
        # the objective in the original basis equals the scaled layer's
        e_orig = impl.output_error(X, W, res["What_orig"])
        e_scaled = impl.output_error(X / s[None, :], W * s[None, :], res["What"])
        assert abs(e_orig - e_scaled) <= 1e-9 * e_orig
    # s = 1: plain GPTQ
    one = impl.awq_gptq_layer(W, H0, d, np.ones(n), bits=4, g=8, damp=0.01)
    plain = impl.gptq_layer(W, H0, d, bits=4, g=8, damp=0.01)
    assert np.array_equal(one["codes"], plain["codes"])
    # diagonal H: no feedback, so the composition is AWQ's RTN of W diag(s)
    Hdiag = np.diag(np.diag(H0))
    dg = impl.awq_gptq_layer(W, Hdiag, np.diag(H0), s, bits=4, g=8, damp=0.01)
    c_awq, sc_awq, What_awq = impl.awq_quantize(W, s, 4, 8)
    assert np.array_equal(dg["codes"], c_awq)
    assert np.allclose(dg["What_orig"], What_awq, rtol=1e-12)
    # a global rescale of s changes nothing the original activations see
    r1 = impl.awq_gptq_layer(W, H0, d, s, bits=4, g=8, damp=0.01)
    r2 = impl.awq_gptq_layer(W, H0, d, 3.7 * s, bits=4, g=8, damp=0.01)
    assert np.array_equal(r1["codes"], r2["codes"])
    assert np.allclose(r1["What_orig"], r2["What_orig"], rtol=1e-12)


def check_zero_point(impl):
    """Zero-point groups: hand-worked grid, diagonal H => RTN, the loop
    identity, the grid itself, and GPTQ below RTN on correlated inputs."""
    gd = load_golden("zero_point_hand.json")["rtn"]
    W = np.array(gd["W"])
    codes, scales, zeros = impl.zp_rtn(W, gd["bits"], gd["g"])
    assert np.array_equal(codes, np.array(gd["codes"]))
    assert np.allclose(scales, gd["scales"], rtol=1e-15, atol=0)
    assert np.array_equal(zeros, np.array(gd["zeros"]))
    assert np.allclose(impl.zp_dequantize(codes, scales, zeros, np.zeros(4, dtype=int)), gd["What"], rtol=1e-15)
    rng = np.random.default_rng(41)
    n, N = 48, 500
    base = rng.standard_normal((N, 6))
    X = base @ rng.standard_normal((6, n)) + 0.3 * rng.standard_normal((N, n))
    Wr = rng.standard_normal((7, n)) + 0.4          # off-centre weights: the zero-point matters
    H0, d = impl.proxy_hessian(X)
    for bits in (2, 3, 4):
        # diagonal H: no feedback, so GPTQ is RTN
        dg = impl.zp_gptq_layer(Wr, np.diag(np.diag(H0)), None, bits=bits, g=16, damp=0.01)
        rc, rs, rz = impl.zp_rtn(Wr, bits, 16)
        assert np.array_equal(dg["codes"], rc)
        assert np.array_equal(dg["zeros"], rz)
        res = impl.zp_gptq_layer(Wr, H0, d, bits=bits, g=16, damp=0.01)
        q = 2 ** bits - 1
        assert res["codes"].min() >= 0 and res["codes"].max() <= q
        assert res["zeros"].min() >= 0 and res["zeros"].max() <= q
        # the loop identity: sum err^2 = tr(dW (H0 + lambda I) dW^T)
        Hd = H0 + res["lambda"] * np.eye(n)
        dW = Wr - res["What"]
        assert abs(res["sum_err2"] - float(np.sum((dW @ Hd) * dW))) <= 1e-9 * res["sum_err2"]
        # GPTQ's calibration error below RTN's (empirical, large margin here)
        What_r = impl.zp_dequantize(rc, rs, rz, np.arange(n) // 16)
        assert impl.output_error(X, Wr, res["What"]) < 0.9 * impl.output_error(X, Wr, What_r)
    # act-order: the permuted problem in natural order
    res = impl.zp_gptq_layer(Wr, H0, d, bits=3, g=16, damp=0.01, act_order=True)
    perm = np.argsort(-d, kind="stable")
    ref = impl.zp_gptq_layer(Wr[:, perm], H0[np.ix_(perm, perm)], d[perm], bits=3, g=16, damp=0.01)
    assert np.array_equal(res["codes"][:, perm], ref["codes"])


def check_output_energy_hand(impl):
    """||X W^T||^2 and ||X (W - What)^T||^2 on the hand-worked values of
    tests/golden/output_energy_hand.json, and by brute-force loops."""
    gd = load_golden("output_energy_hand.json")
    X, W, What = (np.array(gd[k], dtype=np.float64) for k in ("X", "W", "What"))
    assert impl.output_energy(X, W) == gd["energy"]
    assert impl.output_error(X, W, What) == gd["error"]
    rng = np.random.default_rng(17)
    for rows, out, n in ((5, 3, 4), (4, 4, 4), (3, 6, 2)):
        X = rng.standard_normal((rows, n))
        W = rng.standard_normal((out, n))
        What = W + 0.1 * rng.standard_normal((out, n))
        e = f = 0.0
        for i in range(rows):
            for o in range(out):
                y = sum(X[i, j] * W[o, j] for j in range(n))
                yq = sum(X[i, j] * What[o, j] for j in range(n))
                e += y * y
                f += (y - yq) * (y - yq)
        assert abs(impl.output_energy(X, W) - e) <= 1e-12 * e
        assert abs(impl.output_error(X, W, What) - f) <= 1e-12 * f


ALL_CHECKS = [
    check_rtn_hand, check_gptq_hand, check_damping_hand, check_act_order_hand,
    check_hessian_bruteforce, check_hessian_orthogonal, check_hessian_chunking,
    check_inverse_factor_closed_form, check_inverse_factor_identity, check_diagonal_H_is_rtn,
    check_babai_identity, check_babai_equivalence, check_grid_and_invariances,
    check_gptq_beats_rtn_correlated, check_act_order_matches_permuted_problem, check_awq,
    check_hessian_sizes, check_pack_hand, check_pack_roundtrip, check_dequant_g_idx_hand, check_awq_gptq,
    check_zero_point, check_pack_zero_point, check_output_energy_hand,
]
