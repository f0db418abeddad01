"""GPU: the toy layer of "GPTQ versus AWQ objectives" ("A strong answer", the
output-MSE table under a distribution shift), through the library's entry
points: RTN (the AWQ search with the single exponent 0), GPTQ (4-bit,
g = 128, damp 0.01) and AWQ with alpha = 0.25, all calibrated on one sample
and evaluated on it, on a fresh sample of the same distribution and on one
whose four outlier channels moved.

The page's values come from its own synthetic draw and are not reproduced
(the recipe here is in inputs.toy_layer); what is checked is (a) each GPU
error against the oracle's within 1% and (b) the qualitative ordering the
page reports: AWQ < GPTQ < RTN on the calibration sample and the fresh
in-distribution sample, RTN < AWQ < GPTQ once the outliers move.
"""
import numpy as np
import pytest
import torch

import inputs
import oracle
from gpu_util import announce, zeros_h, progress

pytestmark = pytest.mark.gpu


def test_toy_table_ordering(gpu):
    from post_int4_weight_amd import api
    announce("toy layer: RTN / GPTQ / AWQ(0.25) under an outlier shift")
    W, Xc, Xh, Xm = inputs.toy_layer(device=gpu)
    n, out = W.shape[1], W.shape[0]
    H, d = zeros_h(n, gpu)
    api.hessian_accumulate(H, d, Xc)
    gq = api.gptq_quantize_layer(W, H, d, bits=4, group_size=128, damp=0.01)
    rt = api.awq_search_alpha(W, Xc, [0.0], bits=4, group_size=128)
    aw = api.awq_search_alpha(W, Xc, [0.25], bits=4, group_size=128)
    torch.cuda.synchronize()
    gi = np.arange(n) // 128
    W64 = W.cpu().double().numpy()
    dq = lambda r: oracle.dequantize(r["codes"].cpu().numpy(), r["scales"].cpu().double().numpy(),
                                     r["g_idx"].cpu().numpy() if "g_idx" in r else gi)
    What = {"RTN": dq(rt) / rt["s"].cpu().double().numpy()[None, :],
            "GPTQ": dq(gq),
            "AWQ": dq(aw) / aw["s"].cpu().double().numpy()[None, :]}
    Xs = {name: x.cpu().double().numpy() for name, x in (("calibration", Xc), ("same", Xh), ("moved", Xm))}
    # oracle on the same inputs
    Xc64 = Xs["calibration"]
    H0, d0 = oracle.proxy_hessian(Xc64)
    rc, rs = oracle.rtn(W64, 4, 128)
    ref = {"RTN": oracle.dequantize(rc, rs, gi),
           "GPTQ": oracle.gptq_layer(W64, H0, d0, bits=4, g=128, damp=0.01)["What"],
           "AWQ": oracle.awq_search(W64, Xc64, [0.25], bits=4, g=128)["What"]}
    mse = {}
    for sname, X in Xs.items():
        for m in ("RTN", "GPTQ", "AWQ"):
            e = oracle.output_error(X, W64, What[m]) / (X.shape[0] * out)
            e_ref = oracle.output_error(X, W64, ref[m]) / (X.shape[0] * out)
            assert abs(e - e_ref) <= 0.01 * e_ref, (sname, m, e, e_ref)
            mse[sname, m] = e
        progress(f"[toy] {sname:12s} RTN {mse[sname, 'RTN']:.4f}  GPTQ {mse[sname, 'GPTQ']:.4f}  "
              f"AWQ {mse[sname, 'AWQ']:.4f}", flush=True)
    for sname in ("calibration", "same"):
        assert mse[sname, "AWQ"] < mse[sname, "GPTQ"] < mse[sname, "RTN"], sname
    assert mse["moved", "RTN"] < mse["moved", "AWQ"] < mse["moved", "GPTQ"]
