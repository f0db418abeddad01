"""hessian_accumulate_noalloc against hessian_accumulate (the entry point with
a workspace) on the same inputs, through the C ABI: two calls in a row, the
second with a smaller input, so the fixed scratch carries the first call's
contents into the second. Bar: H relative Frobenius error <= 1e-5 and exactly
symmetric, d relative error <= 1e-12 per entry (the sums differ only in the
order of fp32 adds across row chunks)."""
import numpy as np
import pytest
import torch

import inputs
from gpu_util import announce, rel_fro, zeros_h

pytestmark = pytest.mark.gpu


def _both(api, X, n, gpu):
    H0, d0 = zeros_h(n, gpu)
    api.hessian_accumulate(H0, d0, X)
    H1, d1 = zeros_h(n, gpu)
    api.hessian_accumulate_noalloc(H1, d1, X)
    torch.cuda.synchronize()
    return H0, d0, H1, d1


def _check(H0, d0, H1, d1):
    a = H1.cpu().double().numpy()
    b = H0.cpu().double().numpy()
    assert np.array_equal(a, a.T)
    assert rel_fro(a, b) <= 1e-5, rel_fro(a, b)
    dd0, dd1 = d0.cpu().numpy(), d1.cpu().numpy()
    assert np.max(np.abs(dd1 - dd0) / np.maximum(np.abs(dd0), 1e-300)) <= 1e-12


def test_noalloc_two_calls_second_smaller(gpu):
    from post_int4_weight_amd import api
    # first call: in = 8192, 9000 bf16 rows -> chunks of a few thousand rows
    # (the scratch holds about 4000 at this width), the last one ragged
    announce("hessian_accumulate_noalloc call 1: in=8192 rows=9000 bf16")
    _, X = inputs.custom(4, 8192, 9000, seed=31, dtype="bf16", device=gpu, outlier_frac=0.005, outlier_mult=50.0)
    _check(*_both(api, X, 8192, gpu))
    del X
    # second call, smaller: in = 996 as a view with row stride 1000 (not a
    # multiple of 8: the scalar transpose and the separate sums), 1500 rows;
    # then in = 512 with 700 rows
    announce("hessian_accumulate_noalloc call 2: in=996 (row stride 1000) rows=1500 bf16")
    _, X = inputs.custom(4, 1000, 1500, seed=32, dtype="bf16", device=gpu)
    _check(*_both(api, X[:, :996], 996, gpu))
    announce("hessian_accumulate_noalloc call 3: in=512 rows=700 bf16")
    _, X = inputs.custom(4, 512, 700, seed=33, dtype="bf16", device=gpu)
    _check(*_both(api, X, 512, gpu))


def test_noalloc_is_additive_and_rejects_oversize(gpu):
    from post_int4_weight_amd import api
    announce("hessian_accumulate_noalloc: additivity over row chunks, empty input, oversize in")
    _, X = inputs.custom(4, 2048, 4100, seed=34, dtype="bf16", device=gpu)
    H0, d0 = zeros_h(2048, gpu)
    api.hessian_accumulate(H0, d0, X)
    H1, d1 = zeros_h(2048, gpu)
    api.hessian_accumulate_noalloc(H1, d1, X[:1500])
    api.hessian_accumulate_noalloc(H1, d1, X[1500:1500])     # rows = 0: no-op
    api.hessian_accumulate_noalloc(H1, d1, X[1500:])
    torch.cuda.synchronize()
    _check(H0, d0, H1, d1)
    big = torch.empty(1, 262144, dtype=torch.bfloat16, device=gpu)
    Hbig = torch.empty(4, 4, dtype=torch.float32, device=gpu)   # never touched: rejected first
    with pytest.raises(api.PTQError) as ei:
        api._check(api._lib.hessian_accumulate_noalloc(api._ptr(Hbig), None, 262144, api._ptr(big), 0, 1, 262144,
                                                       api._stream()))
    assert ei.value.name == "PTQ_EINVAL" and "too large" in str(ei.value)
