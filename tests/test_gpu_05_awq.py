"""GPU parity of AWQ's alpha grid search against the fp64 oracle.

Criteria: the same alpha is chosen (or, if not, the oracle's own error at the
GPU's alpha is within 1e-4 relative of its minimum: a near-tie), every
per-alpha error within 1e-4 relative of the oracle's, and >= 99% of the codes
of W diag(s) identical at the chosen alpha.
"""
import numpy as np
import pytest
import torch

import inputs
import oracle
from gpu_util import announce, code_match, to64, progress

pytestmark = pytest.mark.gpu


def _compare(res, ref, alphas):
    errs = np.array(res["errors"])
    assert np.all(np.abs(errs - ref["errors"]) <= 1e-4 * ref["errors"]), (errs, ref["errors"])
    ia = alphas.index(res["alpha"]) if res["alpha"] in alphas else int(np.argmin(np.abs(np.array(alphas) - res["alpha"])))
    assert ia == ref["index"] or ref["errors"][ia] <= (1 + 1e-4) * ref["errors"][ref["index"]]
    if ia == ref["index"]:
        assert code_match(res["codes"].cpu().numpy(), ref["codes"]) >= 0.99
        assert np.allclose(res["s"].cpu().double().numpy(), ref["s"], rtol=1e-6)


# n = 1056 (a multiple of 32, not of 64) takes the 32-deep ring of the direct
# kernel; 520 the register-staged kernel; 1024 the 64-deep ring. Group sizes
# 32..512 take the batched 8-columns-per-lane search kernel (ragged last
# groups at n = 520, 1056, 776, 1096), g = 24 the one-wave-per-group one.
@pytest.mark.parametrize("dtype,out,n,rows,g", [("f32", 256, 512, 2048, 128), ("bf16", 300, 1024, 1000, 128),
                                                ("bf16", 128, 520, 700, 128), ("bf16", 260, 1056, 600, 128),
                                                ("bf16", 201, 776, 500, 32), ("bf16", 96, 1536, 400, 512),
                                                ("bf16", 130, 1096, 300, 64), ("bf16", 70, 960, 300, 24)])
def test_awq_small(gpu, dtype, out, n, rows, g):
    from post_int4_weight_amd import api
    announce(f"awq {dtype} out={out} n={n} rows={rows} g={g}")
    W, X = inputs.custom(out, n, rows, seed=out + rows, dtype=dtype)
    alphas = list(inputs.AWQ_ALPHAS)
    res = api.awq_search_alpha(W.to(gpu), X.to(gpu), alphas, bits=4, group_size=g)
    torch.cuda.synchronize()
    ref = oracle.awq_search(to64(W), to64(X), alphas, bits=4, g=g)
    _compare(res, ref, alphas)


def test_awq_llama70b_q_proj(gpu):
    """The pages-shaped AWQ case: config llama70b_qkv_proj's W and its first
    4096 calibration rows, 20 alphas in {0, 0.05, ..., 0.95}."""
    from post_int4_weight_amd import api
    cfg = inputs.CONFIGS["llama70b_qkv_proj"]
    announce("awq llama70b q_proj 8192x8192, 4096 rows, 20 alphas")
    W, X, _ = inputs.layer(cfg, device=gpu, rows=inputs.AWQ_CAL_ROWS)
    alphas = list(inputs.AWQ_ALPHAS)
    res = api.awq_search_alpha(W, X, alphas, bits=4, group_size=128)
    torch.cuda.synchronize()
    # the oracle's grid search (oracle.awq_search), one alpha at a time so
    # the long fp64 evaluation reports its progress
    W64, X64 = to64(W.cpu()), to64(X.cpu())
    m = oracle.channel_mean_abs(X64)
    errors = []
    for a in alphas:
        _, _, What = oracle.awq_quantize(W64, m ** a, 4, 128)
        errors.append(oracle.output_error(X64, W64, What))
        progress(f"[oracle] alpha {a:.2f}: error {errors[-1]:.6e}", flush=True)
    errors = np.array(errors)
    best = int(np.argmin(errors))
    s = m ** alphas[best]
    codes, _, _ = oracle.awq_quantize(W64, s, 4, 128)
    ref = {"errors": errors, "index": best, "codes": codes, "s": s}
    _compare(res, ref, alphas)
