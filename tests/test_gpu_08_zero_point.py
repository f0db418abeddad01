"""GPU: GPTQ with zero-point groups (gptq_quantize_layer_zp) against the
oracle (oracle/zero_point.py), and zero-point INT4 storage.

Tolerances as for the symmetric grid: >= 99% identical codes and zero-points,
scales relative Frobenius error <= 1e-4, the first group's scales and
zero-points (untouched weights) exact up to fp32 rounding, g_idx / perm
exact, relative output error within 1% of the oracle's. A diagonal H (no
feedback) must give the oracle's zero-point RTN bit for bit.
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
    W = (W.float() + 0.02).to(W.dtype)          # off-centre weights: the zero-point matters
    H, d = zeros_h(n, gpu)
    api.hessian_accumulate(H, d, X)
    torch.cuda.synchronize()
    return W, X, H, d


@pytest.mark.parametrize("out,n,rows,bits,g,act_order,dtype", [
    (256, 512, 2048, 4, 128, False, "f32"),
    (320, 1024, 8192, 3, 128, True, "bf16"),
    (200, 776, 4096, 2, 64, False, "bf16"),
    (128, 512, 4096, 7, 256, True, "bf16"),
])
def test_zero_point_vs_oracle(gpu, out, n, rows, bits, g, act_order, dtype):
    from post_int4_weight_amd import api
    announce(f"zero-point gptq out={out} n={n} bits={bits} g={g} act_order={act_order} {dtype}")
    W, X, H, d = _layer(gpu, out, n, rows, out + 3 * n, dtype)
    res = api.gptq_quantize_layer_zp(W, H, d, bits=bits, group_size=g, damp=0.01, act_order=act_order)
    torch.cuda.synchronize()
    X64, W64 = to64(X.cpu()), to64(W.cpu())
    H0, d0 = oracle.proxy_hessian(X64)
    ref = oracle.zp_gptq_layer(W64, H0, d0, bits=bits, g=g, damp=0.01, act_order=act_order)
    codes = res["codes"].cpu().numpy()
    zeros = res["zeros"].cpu().numpy()
    scales = res["scales"].cpu().double().numpy()
    q = 2 ** bits - 1
    assert codes.min() >= 0 and codes.max() <= q and zeros.min() >= 0 and zeros.max() <= q
    assert code_match(codes, ref["codes"]) >= 0.99
    assert code_match(zeros, ref["zeros"]) >= 0.99
    assert np.array_equal(zeros[:, 0], ref["zeros"][:, 0])                 # first group: untouched W
    assert np.allclose(scales[:, 0], ref["scales"][:, 0], rtol=1e-6, atol=0)
    assert rel_fro(scales, ref["scales"]) <= 1e-4
    assert np.array_equal(res["g_idx"].cpu().numpy(), ref["g_idx"])
    if act_order:
        assert np.array_equal(res["perm"].cpu().numpy(), ref["perm"])
    What = oracle.zp_dequantize(codes, scales, zeros, res["g_idx"].cpu().numpy())
    den = oracle.output_energy(X64, W64)
    e_gpu = oracle.output_error(X64, W64, What) / den
    e_ref = oracle.output_error(X64, W64, ref["What"]) / den
    assert abs(e_gpu - e_ref) <= 0.01 * e_ref, (e_gpu, e_ref)
    # the loop identity on the device's own outputs
    Hd = H0 + res["stats"]["lambda"] * np.eye(n)
    dW = W64 - What
    quad = float(np.sum((dW @ Hd) * dW))
    assert abs(res["stats"]["sum_err2"] - quad) <= 1e-3 * quad
    progress(f"[oracle] relative output error {e_gpu:.5g} vs {e_ref:.5g}; codes "
          f"{100 * code_match(codes, ref['codes']):.3f}% equal", flush=True)

    if bits <= 4:
        packed = api.pack_int4(res["codes"], bits=bits)
        torch.cuda.synchronize()
        words = oracle.pack_int4(codes)
        assert np.array_equal(packed.cpu().numpy().view(np.uint32), words)
        Wd = api.dequantize_int4(packed, res["scales"], res["g_idx"], n, group_size=g, zeros=res["zeros"])
        torch.cuda.synchronize()
        ref_d = oracle.dequantize_packed(words, scales, res["g_idx"].cpu().numpy(), n, zeros=zeros)
        assert np.array_equal(Wd.cpu().numpy(), ref_d.astype(np.float32))


def test_zero_point_diagonal_h_is_rtn(gpu):
    from post_int4_weight_amd import api
    announce("zero-point gptq with diagonal H against zero-point RTN")
    W, X, H, d = _layer(gpu, 96, 256, 2048, 5, "f32")
    Hdiag = torch.diag(torch.diagonal(H)).contiguous()
    res = api.gptq_quantize_layer_zp(W, Hdiag, d, bits=3, group_size=64, damp=0.01)
    torch.cuda.synchronize()
    c, s, z = oracle.zp_rtn(to64(W.cpu()), 3, 64)
    assert np.array_equal(res["codes"].cpu().numpy(), c)
    assert np.array_equal(res["zeros"].cpu().numpy(), z)
    assert np.allclose(res["scales"].cpu().double().numpy(), s, rtol=1e-6, atol=0)
