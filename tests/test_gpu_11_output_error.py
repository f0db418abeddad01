"""GPU: layer_output_error — ||X (W - What)^T||^2 and ||X W^T||^2 of a
quantized layer ("GPTQ versus AWQ objectives", "A strong answer": the
objective and its normaliser) — against the oracle's output_error /
output_energy, in fp64 on the same What.

Tolerance: relative 1e-4 on both sums. With bf16 X the library multiplies
W and W - What split into a bf16 high part and a bf16 residual (about 16
significant bits, relative error <= 2^-17 per element) on the bf16 MFMA
with fp32 accumulation; with fp32 X it runs the fp32 MFMA GEMM. Either way
the sums of squares are within ~1e-5 of the fp64 values at these sizes.
"""
import math

import numpy as np
import pytest
import torch

import inputs
import oracle
from gpu_util import announce, to64, zeros_h, progress

pytestmark = pytest.mark.gpu
TOL = 1e-4


def _check(res, X64, W64, What):
    e_ref = oracle.output_error(X64, W64, What)
    y_ref = oracle.output_energy(X64, W64)
    e, y = res
    assert abs(e - e_ref) <= TOL * e_ref, (e, e_ref)
    assert abs(y - y_ref) <= TOL * y_ref, (y, y_ref)
    progress(f"[oracle] error {e:.8g} vs {e_ref:.8g}, energy {y:.8g} vs {y_ref:.8g}", flush=True)


@pytest.mark.parametrize("out,n,rows,g,dtype", [
    (256, 512, 2048, 128, "bf16"),
    (200, 776, 1000, 64, "bf16"),        # in not a multiple of 32: register-staged GEMM, ragged tiles
    (96, 256, 5000, 32, "f32"),          # fp32 X in two row chunks (4096 + 904)
])
def test_synthetic_codes(gpu, out, n, rows, g, dtype):
    from post_int4_weight_amd import api
    announce(f"layer_output_error synthetic codes out={out} n={n} rows={rows} g={g} {dtype}")
    W, X = inputs.custom(out, n, rows, out + n, dtype, gpu)
    rng = np.random.default_rng(out * 7 + n)
    ng = math.ceil(n / g)
    codes = rng.integers(-8, 8, size=(out, n), dtype=np.int8)
    scales = (rng.random((out, ng)) * 0.02 + 1e-3).astype(np.float32)
    g_idx = rng.integers(0, ng, size=n, dtype=np.int32)
    res = api.layer_output_error(X, W, torch.from_numpy(codes).to(gpu), torch.from_numpy(scales).to(gpu),
                                 g_idx=torch.from_numpy(g_idx).to(gpu), group_size=g)
    _check(res, to64(X.cpu()), to64(W.cpu()), oracle.dequantize(codes, scales.astype(np.float64), g_idx))


def test_gptq_act_order(gpu):
    from post_int4_weight_amd import api
    announce("layer_output_error on a GPTQ act-order result (bf16)")
    W, X = inputs.custom(320, 1024, 4096, 17, "bf16", gpu)
    H, d = zeros_h(1024, gpu)
    api.hessian_accumulate(H, d, X)
    r = api.gptq_quantize_layer(W, H, d, bits=4, group_size=128, act_order=True)
    res = api.layer_output_error(X, W, r["codes"], r["scales"], g_idx=r["g_idx"], group_size=128)
    What = oracle.dequantize(r["codes"].cpu().numpy(), r["scales"].cpu().double().numpy(), r["g_idx"].cpu().numpy())
    _check(res, to64(X.cpu()), to64(W.cpu()), What)
    # the loop's own objective (stats) is the same quantity computed another way
    assert abs(r["stats"]["objective"] - res[0]) <= 2e-3 * res[0]


def test_zero_point_fp32(gpu):
    from post_int4_weight_amd import api
    announce("layer_output_error on a zero-point GPTQ result (fp32 X and W)")
    W, X = inputs.custom(128, 512, 3000, 23, "f32", gpu)
    W = W + 0.02
    H, d = zeros_h(512, gpu)
    api.hessian_accumulate(H, d, X)
    r = api.gptq_quantize_layer_zp(W, H, d, bits=3, group_size=64)
    res = api.layer_output_error(X, W, r["codes"], r["scales"], g_idx=r["g_idx"], zeros=r["zeros"], group_size=64)
    What = oracle.zp_dequantize(r["codes"].cpu().numpy(), r["scales"].cpu().double().numpy(),
                                r["zeros"].cpu().numpy(), r["g_idx"].cpu().numpy())
    _check(res, to64(X.cpu()), to64(W.cpu()), What)


def test_awq_scales(gpu):
    from post_int4_weight_amd import api
    announce("layer_output_error on an AWQ result (s applied, bf16)")
    W, X = inputs.custom(256, 1024, 2048, 31, "bf16", gpu)
    a = api.awq_search_alpha(W, X, [0.0, 0.25, 0.5], bits=4, group_size=128)
    res = api.layer_output_error(X, W, a["codes"], a["scales"], s=a["s"], group_size=128)
    gi = np.arange(1024) // 128
    What = oracle.dequantize(a["codes"].cpu().numpy(), a["scales"].cpu().double().numpy(), gi) / \
        a["s"].cpu().double().numpy()[None, :]
    _check(res, to64(X.cpu()), to64(W.cpu()), What)
    # the search's own error at the chosen alpha is the same quantity
    best = [0.0, 0.25, 0.5].index(a["alpha"])
    assert abs(a["errors"][best] - res[0]) <= 1e-3 * res[0]


def test_group_index_out_of_range_is_nan(gpu):
    from post_int4_weight_amd import api
    announce("layer_output_error with a group index out of range")
    W, X = inputs.custom(64, 256, 512, 3, "bf16", gpu)
    codes = torch.zeros(64, 256, dtype=torch.int8, device=gpu)
    scales = torch.ones(64, 2, dtype=torch.float32, device=gpu)
    g_idx = torch.zeros(256, dtype=torch.int32, device=gpu)
    g_idx[5] = 2
    e, y = api.layer_output_error(X, W, codes, scales, g_idx=g_idx, group_size=128)
    assert math.isnan(e) and math.isfinite(y) and y > 0
