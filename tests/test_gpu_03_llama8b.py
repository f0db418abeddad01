"""GPU parity on the Llama-8B-shaped q_proj: W [4096, 4096] bf16, X [32768,
4096] bf16 (16 sequences x 2048 tokens), 4-bit, g = 128, damp = 0.01, with
and without act-order.

The oracle computes H, U and, on a fixed subset of 256 output rows (rows are
independent given U, so a subset is exact), the column loop. Criteria: H
relative Frobenius error <= 1e-5, U <= 1e-4, >= 99% of the subset's codes
identical, relative output error of the subset within 1% of the oracle's,
identical act-order permutation.
"""
import numpy as np
import pytest
import torch

import inputs
import oracle
from gpu_util import announce, code_match, rel_fro, relative_output_error, to64, zeros_h

pytestmark = pytest.mark.gpu

ROWS = np.arange(0, 4096, 16)     # 256-row subset


@pytest.fixture(scope="module")
def layer8b(gpu):
    from post_int4_weight_amd import api
    cfg = inputs.CONFIGS["llama8b_q_proj"]
    announce("llama8b_q_proj: generate + hessian")
    W, X, _ = inputs.layer(cfg, device=gpu)
    H, d = zeros_h(cfg.inp, gpu)
    api.hessian_accumulate(H, d, X)
    torch.cuda.synchronize()
    Xh = X.cpu()
    H0, d0 = oracle.proxy_hessian(to64(Xh), chunk_rows=4096)
    return cfg, W, X, H, d, H0, d0


def test_hessian_8b(layer8b):
    cfg, W, X, H, d, H0, d0 = layer8b
    Hg = H.cpu().double().numpy()
    assert np.array_equal(Hg, Hg.T)
    assert rel_fro(Hg, H0) <= 1e-5
    assert np.max(np.abs(d.cpu().numpy() - d0) / d0) <= 1e-12


@pytest.mark.parametrize("act_order", [False, True])
def test_gptq_8b(layer8b, act_order):
    from post_int4_weight_amd import api
    cfg, W, X, H, d, H0, d0 = layer8b
    announce(f"llama8b_q_proj gptq act_order={act_order}")
    res = api.gptq_quantize_layer(W, H, d, bits=4, group_size=128, damp=0.01, act_order=act_order)
    U, perm, lam = api.gptq_inverse_factor(H, d, damp=0.01, act_order=act_order)
    torch.cuda.synchronize()
    Hd, lam0 = oracle.damped(H0, 0.01)
    assert abs(lam - lam0) <= 1e-12 * lam0
    p = oracle.act_order_permutation(d0) if act_order else np.arange(cfg.inp)
    if act_order:
        assert np.array_equal(perm.cpu().numpy(), p)
        assert np.array_equal(res["perm"].cpu().numpy(), p)
    Uref = oracle.inverse_upper_factor(Hd[np.ix_(p, p)])
    assert rel_fro(U.cpu().double().numpy(), Uref) <= 1e-4
    Wsub = to64(W[ROWS.tolist()].cpu())
    ref = oracle.gptq_layer(Wsub, H0, d0, bits=4, g=128, damp=0.01, act_order=act_order, U=Uref)
    codes = res["codes"].cpu().numpy()[ROWS]
    assert code_match(codes, ref["codes"]) >= 0.99
    assert np.array_equal(res["g_idx"].cpu().numpy(), ref["g_idx"])
    What = oracle.dequantize(codes, res["scales"].cpu().double().numpy()[ROWS], ref["g_idx"])
    e_gpu = relative_output_error(H0, Wsub, What)
    e_ref = relative_output_error(H0, Wsub, ref["What"])
    assert abs(e_gpu - e_ref) <= 0.01 * e_ref, (e_gpu, e_ref)
