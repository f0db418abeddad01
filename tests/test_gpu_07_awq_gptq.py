"""GPU: AWQ's scaling composed with GPTQ (awq_gptq_quantize_layer) against the
oracle's awq_gptq_layer, on the same seeded layers and the same fp32 s.

Tolerances as for GPTQ: >= 99% identical codes, scales relative Frobenius
error <= 1e-4, g_idx / perm exact, relative output error (original basis)
within 1% of the oracle's. With s = 1 the call must reproduce
gptq_quantize_layer bit for bit (the scaled inputs are then exact copies).
"""
import numpy as np
import pytest
import torch

import inputs
import oracle
from gpu_util import announce, code_match, rel_fro, to64, zeros_h, progress

pytestmark = pytest.mark.gpu


def _layer(gpu, out, n, rows, seed, dtype):
    from post_int4_weight_amd import api
    W, X = inputs.custom(out, n, rows, seed, dtype, gpu)
    H, d = zeros_h(n, gpu)
    api.hessian_accumulate(H, d, X)
    torch.cuda.synchronize()
    return W, X, H, d


@pytest.mark.parametrize("out,n,rows,bits,alpha,act_order,dtype", [
    (256, 512, 2048, 4, 0.5, False, "f32"),
    (384, 1024, 8192, 3, 0.5, True, "bf16"),
    (200, 768, 4096, 4, 0.25, False, "bf16"),
])
def test_awq_gptq_vs_oracle(gpu, out, n, rows, bits, alpha, act_order, dtype):
    from post_int4_weight_amd import api
    announce(f"awq+gptq out={out} n={n} rows={rows} bits={bits} alpha={alpha} act_order={act_order} {dtype}")
    W, X, H, d = _layer(gpu, out, n, rows, out + n, dtype)
    X64 = to64(X.cpu())
    s32 = (oracle.channel_mean_abs(X64) ** alpha).astype(np.float32)
    s = torch.from_numpy(s32).to(gpu)
    res = api.awq_gptq_quantize_layer(W, H, d, s, bits=bits, group_size=128, damp=0.01, act_order=act_order)
    torch.cuda.synchronize()
    H0, d0 = oracle.proxy_hessian(X64)
    ref = oracle.awq_gptq_layer(to64(W.cpu()), H0, d0, s32.astype(np.float64), bits=bits, g=128, damp=0.01,
                                act_order=act_order)
    codes = res["codes"].cpu().numpy()
    assert code_match(codes, ref["codes"]) >= 0.99
    assert rel_fro(res["scales"].cpu().double().numpy(), ref["scales"]) <= 1e-4
    assert np.array_equal(res["g_idx"].cpu().numpy(), ref["g_idx"])
    if act_order:
        assert np.array_equal(res["perm"].cpu().numpy(), ref["perm"])
    What = oracle.dequantize(codes, res["scales"].cpu().double().numpy(), res["g_idx"].cpu().numpy())
    What_orig = What / s32.astype(np.float64)[None, :]
    W64 = to64(W.cpu())
    den = oracle.output_energy(X64, W64)
    e_gpu = oracle.output_error(X64, W64, What_orig) / den
    e_ref = oracle.output_error(X64, W64, ref["What_orig"]) / den
    assert abs(e_gpu - e_ref) <= 0.01 * e_ref, (e_gpu, e_ref)
    # stats[3] is the calibration error in the original basis
    obj = oracle.output_error(X64, W64, What_orig)
    assert abs(res["stats"]["objective"] - obj) <= 2e-3 * obj
    progress(f"[oracle] relative output error {e_gpu:.5g} vs {e_ref:.5g}; codes "
          f"{100 * code_match(codes, ref['codes']):.3f}% equal", flush=True)


def test_unit_scales_reproduce_gptq(gpu):
    from post_int4_weight_amd import api
    announce("awq+gptq with s = 1 against gptq_quantize_layer")
    W, X, H, d = _layer(gpu, 192, 512, 4096, 9, "bf16")
    one = torch.ones(512, device=gpu)
    a = api.awq_gptq_quantize_layer(W, H, d, one, bits=4, group_size=128, act_order=True)
    b = api.gptq_quantize_layer(W, H, d, bits=4, group_size=128, act_order=True)
    torch.cuda.synchronize()
    assert torch.equal(a["codes"], b["codes"])
    assert torch.equal(a["scales"], b["scales"])
    assert torch.equal(a["g_idx"], b["g_idx"])


def test_composition_after_awq_search(gpu):
    """The pipeline the page describes: AWQ's alpha search picks s, then GPTQ
    rounds the scaled layer; on the calibration rows the composition's error
    is below AWQ's RTN at the same s (the feedback only removes error)."""
    from post_int4_weight_amd import api
    announce("awq search then awq+gptq")
    W, X, H, d = _layer(gpu, 256, 1024, 4096, 17, "bf16")
    alphas = [0.05 * i for i in range(20)]
    r = api.awq_search_alpha(W, X, alphas, bits=3, group_size=128)
    comp = api.awq_gptq_quantize_layer(W, H, d, r["s"], bits=3, group_size=128)
    torch.cuda.synchronize()
    s64 = r["s"].cpu().double().numpy()
    X64, W64 = to64(X.cpu()), to64(W.cpu())
    What_c = oracle.dequantize(comp["codes"].cpu().numpy(), comp["scales"].cpu().double().numpy(),
                               comp["g_idx"].cpu().numpy()) / s64[None, :]
    What_a = oracle.dequantize(r["codes"].cpu().numpy(), r["scales"].cpu().double().numpy(),
                               np.arange(1024) // 128) / s64[None, :]
    e_c = oracle.output_error(X64, W64, What_c)
    e_a = oracle.output_error(X64, W64, What_a)
    progress(f"[check] calibration error: AWQ {e_a:.5g}, AWQ then GPTQ {e_c:.5g}", flush=True)
    assert e_c < e_a
