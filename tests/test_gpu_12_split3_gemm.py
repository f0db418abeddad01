"""GPU: the fp32 GEMM run on the bf16 MFMA from three-term bf16 splits of
its operands (the large GEMMs of the U recursion), through its test hook,
against fp64 products.

Every operand layout, triangle mode and upper_only, on ragged shapes spanning
several 256-wide tiles, with beta 0 and 1 and alpha +-1. Tolerance: relative
Frobenius error <= 1e-5, the fp32 GEMM's own bar, and within 4x the error
the fp32 MFMA GEMM makes on the same product (the split keeps 24 significant
bits of each operand and every term product down to 2^-16 relative).
"""
import numpy as np
import pytest
import torch

from gpu_util import announce, rel_fro

pytestmark = pytest.mark.gpu


def _pad4(t, gpu):
    r, c = t.shape
    out = torch.zeros(r, (c + 3) // 4 * 4)
    out[:, :c] = t
    return out.to(gpu)


@pytest.mark.parametrize("M,N,K", [(600, 520, 1000), (300, 260, 300), (5, 9, 3), (37, 4, 36), (256, 256, 64),
                                   (1100, 700, 2100)])
@pytest.mark.parametrize("la,lb", [(0, 0), (0, 1), (1, 0), (1, 1)])
def test_split3_layouts(gpu, M, N, K, la, lb):
    from post_int4_weight_amd import api
    announce(f"gemm_f32_split3 M={M} N={N} K={K} la={la} lb={lb}")
    g = torch.Generator().manual_seed(M * 1000 + N + K)
    A = torch.randn(M, K, generator=g)
    B = torch.randn(K, N, generator=g)
    C0 = torch.randn(M, N, generator=g)
    Ad = _pad4(A if la == 0 else A.T.contiguous(), gpu)
    Bd = _pad4(B if lb == 0 else B.T.contiguous(), gpu)
    ref = A.double() @ B.double()
    for beta_one, alpha in ((0, 1.0), (1, -1.0)):
        want = (alpha * ref + (C0.double() if beta_one else 0)).numpy()
        C = _pad4(C0, gpu)
        api._test_gemm_f32_split3(Ad, Bd, C, M, N, K, la, lb, alpha=alpha, beta_one=beta_one)
        C32 = _pad4(C0, gpu)
        api._test_gemm_f32(Ad, Bd, C32, M, N, K, la, lb, alpha=alpha, beta_one=beta_one)
        torch.cuda.synchronize()
        e = rel_fro(C[:, :N].cpu().double().numpy(), want)
        e32 = rel_fro(C32[:, :N].cpu().double().numpy(), want)
        assert e < 1e-5 and e <= 4 * e32 + 1e-9, (e, e32)


@pytest.mark.parametrize("beta_one", [0, 1])
def test_split3_large_ragged(gpu, beta_one):
    """A product of 33 x 17 output tiles with ragged edges on both sides and a
    depth that is not a multiple of 64."""
    from post_int4_weight_amd import api
    M, N, K = 8200, 4100, 100
    announce(f"gemm_f32_split3 large ragged M={M} N={N} K={K} beta_one={beta_one}")
    g = torch.Generator().manual_seed(11 + beta_one)
    A = torch.randn(M, K, generator=g)
    B = torch.randn(N, K, generator=g)
    C0 = torch.randn(M, N, generator=g)
    C = _pad4(C0, gpu)
    api._test_gemm_f32_split3(_pad4(A, gpu), _pad4(B, gpu), C, M, N, K, 0, 1, alpha=-1.0, beta_one=beta_one)
    torch.cuda.synchronize()
    want = (-(A.double() @ B.double().T) + (C0.double() if beta_one else 0)).numpy()
    assert rel_fro(C[:, :N].cpu().double().numpy(), want) < 1e-5


# n = 2100: nine 256-wide tile columns, the last ragged, so the products
# with a triangular B take the whole-column deal over the XCDs; C starts as
# NaN, so a tile left out shows
@pytest.mark.parametrize("n,m", [(640, 544), (2100, 300)])
@pytest.mark.parametrize("tri", [1, 2, 3])
def test_split3_triangles(gpu, tri, n, m):
    from post_int4_weight_amd import api
    announce(f"gemm_f32_split3 triangle mode {tri} n={n} m={m}")
    g = torch.Generator().manual_seed(tri)
    T = torch.triu(torch.randn(n, n, generator=g))
    if tri == 1:      # C[n, m] = T[n, n] X[n, m], A upper
        X = torch.randn(n, m, generator=g)
        A, B, la, lb, M, N, K = T, X, 0, 0, n, m, n
        ref = T.double() @ X.double()
    elif tri == 2:    # C[m, n] = X[m, n] T[n, n], B upper (k <= j)
        X = torch.randn(m, n, generator=g)
        A, B, la, lb, M, N, K = X, T, 0, 0, m, n, n
        ref = X.double() @ T.double()
    else:             # C[m, n] = X[m, n] T^T, B stored [N][K] upper (k >= j)
        X = torch.randn(m, n, generator=g)
        A, B, la, lb, M, N, K = X, T, 0, 1, m, n, n
        ref = X.double() @ T.double().T
    C = torch.full((M, N), float("nan"), device=gpu)
    api._test_gemm_f32_split3(A.to(gpu), B.to(gpu), C, M, N, K, la, lb, tri=tri)
    torch.cuda.synchronize()
    assert rel_fro(C.cpu().double().numpy(), ref.numpy()) < 1e-5


@pytest.mark.parametrize("k", [50, 640])
def test_split3_upper_only_same_operand(gpu, k):
    """C -= P P^T on tiles on or above the diagonal (A and B one matrix: split once)."""
    from post_int4_weight_amd import api
    announce(f"gemm_f32_split3 upper_only k={k}")
    n = 600
    g = torch.Generator().manual_seed(7)
    P = torch.randn(n, k, generator=g)
    C0 = torch.randn(n, n, generator=g)
    C = C0.clone().to(gpu)
    Pd = _pad4(P, gpu)
    api._test_gemm_f32_split3(Pd, Pd, C, n, n, k, 0, 1, alpha=-1.0, beta_one=1, upper_only=1)
    torch.cuda.synchronize()
    ref = C0.double() - P.double() @ P.double().T
    got = C.cpu().double()
    for ti in range(3):
        for tj in range(3):
            blk = (slice(256 * ti, min(n, 256 * ti + 256)), slice(256 * tj, min(n, 256 * tj + 256)))
            if ti <= tj:
                assert rel_fro(got[blk].numpy(), ref[blk].numpy()) < 1e-5
            else:
                assert torch.equal(got[blk], C0.double()[blk])


def test_split3_special_values(gpu):
    """Exact small integers stay exact; a NaN operand row gives NaN in that row only."""
    from post_int4_weight_amd import api
    announce("gemm_f32_split3 exact integers and NaN propagation")
    g = torch.Generator().manual_seed(3)
    A = torch.randint(-50, 50, (300, 200), generator=g).float()
    B = torch.randint(-50, 50, (200, 280), generator=g).float()
    C = torch.zeros(300, 280, device=gpu)
    api._test_gemm_f32_split3(A.to(gpu), B.to(gpu), C, 300, 280, 200, 0, 0)
    torch.cuda.synchronize()
    assert torch.equal(C.cpu(), A @ B)
    A[7, 3] = float("nan")
    api._test_gemm_f32_split3(A.to(gpu), B.to(gpu), C, 300, 280, 200, 0, 0)
    torch.cuda.synchronize()
    Cc = C.cpu()
    assert torch.isnan(Cc[7]).all() and not torch.isnan(Cc[torch.arange(300) != 7]).any()
