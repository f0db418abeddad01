"""Plant plausible mistakes in copies of the oracle (on the CPU) and show that
at least one pin fails for each: the pins are strong enough to catch them."""
import types

import numpy as np
import pytest

import oracle
import oracle.gptq as og
from oracle_pins import ALL_CHECKS


def _namespace(**overrides):
    ns = types.SimpleNamespace(**{k: getattr(oracle, k) for k in oracle.__all__})
    for k, v in overrides.items():
        setattr(ns, k, v)
    return ns


def _columns_factory(sign=1.0, divide_by_ujj=True, scale_from_original=False, rounding=np.round,
                     update_row_of_u=True):
    def gptq_columns(W, U, bits, g):
        W0 = np.array(W, dtype=np.float64)
        Wc = W0.copy()
        U = np.asarray(U, dtype=np.float64)
        out, n = Wc.shape
        q = og.qmax(bits)
        ng = (n + g - 1) // g
        codes = np.zeros((out, n), dtype=np.int64)
        scales = np.zeros((out, ng))
        err = np.zeros((out, n))
        for grp in range(ng):
            g0, g1 = grp * g, min(n, (grp + 1) * g)
            src = W0 if scale_from_original else Wc
            scale = np.max(np.abs(src[:, g0:g1]), axis=1) / q
            scales[:, grp] = scale
            for j in range(g0, g1):
                c = np.zeros(out)
                live = scale != 0
                c[live] = rounding(Wc[live, j] / scale[live])
                c = np.clip(c, -q - 1, q)
                codes[:, j] = c
                e = Wc[:, j] - c * scale
                if divide_by_ujj:
                    e = e / U[j, j]
                err[:, j] = e
                row = U[j, j + 1:] if update_row_of_u else U[j + 1:, j]
                Wc[:, j + 1:] -= sign * e[:, None] * row[None, :]
        return codes, scales, err
    return gptq_columns


def _layer_with(columns=None, factor=None, damped=None, perm=None):
    def gptq_layer(W, H0, d=None, bits=4, g=128, damp=0.01, act_order=False, U=None):
        saved = (og.gptq_columns, og.inverse_upper_factor, og.damped, og.act_order_permutation)
        try:
            if columns is not None:
                og.gptq_columns = columns
            if factor is not None:
                og.inverse_upper_factor = factor
            if damped is not None:
                og.damped = damped
            if perm is not None:
                og.act_order_permutation = perm
            return saved_layer(W, H0, d, bits, g, damp, act_order, U)
        finally:
            og.gptq_columns, og.inverse_upper_factor, og.damped, og.act_order_permutation = saved
    return gptq_layer


saved_layer = og.gptq_layer


def _lower_factor(H):
    return np.linalg.cholesky(np.linalg.inv(H))          # forgot the transpose


def _factor_not_reversed(H):
    L = np.linalg.cholesky(np.asarray(H, dtype=np.float64))   # H = L L^T in natural order
    return np.linalg.inv(L).T                                 # upper, but U^T U = (L^T L)^-1


def _no_damp(H0, damp):
    return np.asarray(H0, dtype=np.float64).copy(), 0.0


def _damp_sum(H0, damp):
    H0 = np.asarray(H0, dtype=np.float64)
    lam = damp * float(np.sum(np.diag(H0)))              # sum instead of mean
    return H0 + lam * np.eye(H0.shape[0]), lam


def _ascending(d):
    return np.argsort(np.asarray(d), kind="stable")      # increasing instead of decreasing


def _ties_reversed(d):
    n = len(d)
    return np.lexsort((-np.arange(n), -np.asarray(d, dtype=np.float64)))   # ties: higher index first


def _hessian_no_mirror(X, chunk_rows=2048):
    X = np.asarray(X, dtype=np.float64)
    H0 = X.T @ X
    d = np.sum(X * X, axis=0)
    return H0 + np.triu(H0, 1) * 1e-3, d                 # asymmetric junk in the upper part


def _rtn_floor(W, bits, g):
    W = np.asarray(W, dtype=np.float64)
    out, n = W.shape
    q = og.qmax(bits)
    ng = (n + g - 1) // g
    codes = np.zeros((out, n), dtype=np.int64)
    scales = np.zeros((out, ng))
    for grp in range(ng):
        g0, g1 = grp * g, min(n, (grp + 1) * g)
        s = np.max(np.abs(W[:, g0:g1]), axis=1) / q
        scales[:, grp] = s
        with np.errstate(invalid="ignore", divide="ignore"):
            c = np.where(s[:, None] != 0, np.trunc(W[:, g0:g1] / s[:, None]), 0)
        codes[:, g0:g1] = np.clip(c, -q - 1, q)
    return codes, scales


def _awq_channels_reversed(X):
    return np.mean(np.abs(np.asarray(X, dtype=np.float64)), axis=0)[::-1]


def _awq_rms(X):
    X = np.asarray(X, dtype=np.float64)
    return np.sqrt(np.mean(X * X, axis=0))                # root-mean-square instead of mean |x|


def _pack_reversed(codes):
    """nibbles in the opposite order inside each word"""
    codes = np.asarray(codes, dtype=np.int64)
    out, n = codes.shape
    words = np.zeros((out, n // 8), dtype=np.uint64)
    for w in range(n // 8):
        for k in range(8):
            words[:, w] |= ((codes[:, 8 * w + k] & 0xF).astype(np.uint64)) << np.uint64(4 * (7 - k))
    return words.astype(np.uint32)


def _unpack_unsigned(packed, n, signed=True):
    """nibbles read as unsigned (no sign extension)"""
    packed = np.asarray(packed, dtype=np.uint64)
    codes = np.zeros((packed.shape[0], n), dtype=np.int64)
    for w in range(n // 8):
        for k in range(8):
            codes[:, 8 * w + k] = ((packed[:, w] >> np.uint64(4 * k)) & np.uint64(0xF)).astype(np.int64)
    return codes


def _dequant_ignores_g_idx(packed, scales, g_idx, n, zeros=None):
    """group taken as column // g (processing order assumed), g_idx unused"""
    scales = np.asarray(scales, dtype=np.float64)
    g = -(-n // scales.shape[1])
    gi = np.arange(n) // g
    codes = oracle.unpack_int4(packed, n, signed=zeros is None).astype(np.float64)
    if zeros is not None:
        codes = codes - np.asarray(zeros, dtype=np.float64)[:, gi]
    return codes * scales[:, gi]


def _awq_gptq_factory(h_scale="inverse", w_scale="mul", rescale_d=True, unscale=True):
    def awq_gptq_layer(W, H0, d, s, bits=4, g=128, damp=0.01, act_order=False):
        W = np.asarray(W, dtype=np.float64)
        s = np.asarray(s, dtype=np.float64)
        H0 = np.asarray(H0, dtype=np.float64)
        Ws = W * s[None, :] if w_scale == "mul" else W / s[None, :]
        Hs = H0 / np.outer(s, s) if h_scale == "inverse" else H0 * np.outer(s, s)
        ds = None if d is None else (np.asarray(d) / (s * s) if rescale_d else np.asarray(d))
        res = oracle.gptq_layer(Ws, Hs, ds, bits=bits, g=g, damp=damp, act_order=act_order)
        res["What_orig"] = res["What"] / s[None, :] if unscale else res["What"]
        return res
    return awq_gptq_layer


def _zp_dequant_no_zero(codes, scales, zeros, g_idx):
    gi = np.asarray(g_idx)
    return np.asarray(codes, dtype=np.float64) * np.asarray(scales, dtype=np.float64)[:, gi]


def _zp_params_without_origin(Wg, bits):
    Wg = np.asarray(Wg, dtype=np.float64)
    lo, hi = Wg.min(axis=1), Wg.max(axis=1)
    scale = (hi - lo) / (2 ** bits - 1)
    zero = np.zeros_like(scale)
    live = scale != 0
    zero[live] = np.round(-lo[live] / scale[live])
    return scale, zero


def _zp_params_floor(Wg, bits):
    Wg = np.asarray(Wg, dtype=np.float64)
    lo, hi = np.minimum(Wg.min(axis=1), 0.0), np.maximum(Wg.max(axis=1), 0.0)
    scale = (hi - lo) / (2 ** bits - 1)
    zero = np.zeros_like(scale)
    live = scale != 0
    zero[live] = np.floor(-lo[live] / scale[live])
    return scale, zero


def _zp_with_params(params):
    import oracle.zero_point as zpm

    def rtn(W, bits, g):
        saved = zpm.group_params
        zpm.group_params = params
        try:
            return zpm.rtn(W, bits, g)
        finally:
            zpm.group_params = saved

    def layer(*a, **k):
        saved = zpm.group_params
        zpm.group_params = params
        try:
            return zpm.gptq_layer(*a, **k)
        finally:
            zpm.group_params = saved
    return dict(zp_rtn=rtn, zp_gptq_layer=layer, zp_group_params=params)


def _energy_untransposed(X, W):
    Y = np.asarray(X, dtype=np.float64) @ np.asarray(W, dtype=np.float64)   # X W instead of X W^T
    return float(np.sum(Y * Y))


def _energy_unsquared(X, W):
    Y = np.asarray(X, dtype=np.float64) @ np.asarray(W, dtype=np.float64).T
    return float(np.sum(np.abs(Y)))                                      # |y| summed, not y^2


def _error_untransposed(X, W, What):
    dW = np.asarray(W, dtype=np.float64) - np.asarray(What, dtype=np.float64)
    E = np.asarray(X, dtype=np.float64) @ dW
    return float(np.sum(E * E))


MUTANTS = {
    "feedback sign flipped": dict(gptq_layer=_layer_with(columns=_columns_factory(sign=-1.0))),
    "error not divided by U_jj": dict(gptq_layer=_layer_with(columns=_columns_factory(divide_by_ujj=False))),
    "scale from original W": dict(gptq_layer=_layer_with(columns=_columns_factory(scale_from_original=True))),
    "floor instead of round": dict(gptq_layer=_layer_with(columns=_columns_factory(rounding=np.floor))),
    "column of U instead of row": dict(gptq_layer=_layer_with(columns=_columns_factory(update_row_of_u=False))),
    "lower factor (no transpose)": dict(gptq_layer=_layer_with(factor=_lower_factor),
                                        inverse_upper_factor=_lower_factor),
    "factor without the index reversal": dict(gptq_layer=_layer_with(factor=_factor_not_reversed),
                                              inverse_upper_factor=_factor_not_reversed),
    "damping dropped": dict(gptq_layer=_layer_with(damped=_no_damp), damped=_no_damp),
    "damping by sum not mean": dict(gptq_layer=_layer_with(damped=_damp_sum), damped=_damp_sum),
    "act-order ascending": dict(gptq_layer=_layer_with(perm=_ascending), act_order_permutation=_ascending),
    "hessian not symmetric": dict(proxy_hessian=_hessian_no_mirror),
    "rtn truncates": dict(rtn=_rtn_floor),
    "act-order ties reversed": dict(gptq_layer=_layer_with(perm=_ties_reversed),
                                    act_order_permutation=_ties_reversed),
    "awq channels reversed": dict(channel_mean_abs=_awq_channels_reversed),
    "awq rms instead of mean abs": dict(channel_mean_abs=_awq_rms),
    "int4 nibbles reversed": dict(pack_int4=_pack_reversed),
    "int4 unpack without sign": dict(unpack_int4=_unpack_unsigned),
    "dequant ignores g_idx": dict(dequantize_packed=_dequant_ignores_g_idx),
    "awq+gptq: H scaled by s s": dict(awq_gptq_layer=_awq_gptq_factory(h_scale="direct")),
    "awq+gptq: W divided by s": dict(awq_gptq_layer=_awq_gptq_factory(w_scale="div")),
    "awq+gptq: act-order key not rescaled": dict(awq_gptq_layer=_awq_gptq_factory(rescale_d=False)),
    "awq+gptq: 1/s not applied": dict(awq_gptq_layer=_awq_gptq_factory(unscale=False)),
    "zero-point: zero not subtracted": dict(zp_dequantize=_zp_dequant_no_zero),
    "zero-point: range without the origin": _zp_with_params(_zp_params_without_origin),
    "zero-point: zero floored": _zp_with_params(_zp_params_floor),
    "output energy: X W instead of X W^T": dict(output_energy=_energy_untransposed),
    "output energy: not squared": dict(output_energy=_energy_unsquared),
    "output error: X dW instead of X dW^T": dict(output_error=_error_untransposed),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    impl = _namespace(**MUTANTS[name])
    failures = []
    for check in ALL_CHECKS:
        try:
            check(impl)
        except (AssertionError, np.linalg.LinAlgError, ValueError, FloatingPointError):
            failures.append(check.__name__)
    assert failures, f"no pin caught the planted mistake: {name}"


def test_real_oracle_passes_every_pin():
    impl = _namespace()
    for check in ALL_CHECKS:
        check(impl)
