"""GPU: the MFMA building blocks on their own, against fp64 references.

The fp32 GEMM (stages 2 and 3) through its test hook, every operand layout
and triangle mode, on ragged shapes spanning several 128-wide tiles; the bf16
X^T X path through hessian_accumulate on ragged shapes, split-K and several
row chunks.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import announce, rel_fro, to64, zeros_h

pytestmark = pytest.mark.gpu


# below 1024 tiles of 128 x 128 the direct kernel runs 64 x 64 tiles; (4200, 4100, 64) has 1089
@pytest.mark.parametrize("M,N,K", [(200, 130, 77), (128, 128, 16), (300, 260, 300), (5, 9, 3), (260, 388, 1000),
                                   (37, 4, 36), (1700, 1540, 200), (4200, 4100, 64)])
@pytest.mark.parametrize("la,lb", [(0, 0), (0, 1), (1, 0), (1, 1)])
def test_gemm_f32_layouts(gpu, M, N, K, la, lb):
    from post_int4_weight_amd import api
    announce(f"gemm_f32 M={M} N={N} K={K} la={la} lb={lb}")
    g = torch.Generator().manual_seed(M * 1000 + N + K)
    A = torch.randn(M, K, generator=g)
    B = torch.randn(K, N, generator=g)
    C0 = torch.randn(M, N, generator=g)

    def pad4(t):
        r, c = t.shape
        c4 = (c + 3) // 4 * 4
        out = torch.zeros(r, c4)
        out[:, :c] = t
        return out.to(gpu)
    Ad = pad4(A if la == 0 else A.T.contiguous())
    Bd = pad4(B if lb == 0 else B.T.contiguous())
    ref = A.double() @ B.double()
    for beta_one, alpha in ((0, 1.0), (1, -1.0)):
        C = pad4(C0)
        api._test_gemm_f32(Ad, Bd, C, M, N, K, la, lb, alpha=alpha, beta_one=beta_one)
        torch.cuda.synchronize()
        want = alpha * ref + (C0.double() if beta_one else 0)
        got = C[:, :N].cpu().double()
        assert rel_fro(got.numpy(), want.numpy()) < 1e-5


@pytest.mark.parametrize("n,m", [(384, 272), (2048, 1100)])
@pytest.mark.parametrize("tri", [1, 2, 3])
def test_gemm_f32_triangles(gpu, tri, n, m):
    from post_int4_weight_amd import api
    announce(f"gemm_f32 triangle mode {tri} n={n} m={m}")
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
    C = torch.zeros(M, N, device=gpu)
    api._test_gemm_f32(A.to(gpu), B.to(gpu), C, M, N, K, la, lb, tri=tri)
    torch.cuda.synchronize()
    assert rel_fro(C.cpu().double().numpy(), ref.numpy()) < 1e-5


# (n1, n2): the recursion's small levels (one launch, 64 x 64 tiles), ragged
# sizes, a depth past the short ring, and a pair whose two products take
# different tile sizes (4200: 128 x 128 tiles for the update; two launches)
@pytest.mark.parametrize("n1,n2", [(128, 128), (256, 256), (1024, 1024), (200, 332), (256, 2048), (4200, 200)])
def test_gemm_f32_pair(gpu, n1, n2):
    """The U recursion's H11 -= R12 R12^T (upper tiles) and T = R12 U22 (U22 upper) in one launch: bit for bit
    the two separate launches, and both against fp64."""
    from post_int4_weight_amd import api
    announce(f"gemm_f32 pair n1={n1} n2={n2}")
    g = torch.Generator().manual_seed(n1 * 7 + n2)
    R = torch.randn(n1, n2, generator=g)
    Uu = torch.triu(torch.randn(n2, n2, generator=g))
    H0 = torch.randn(n1, n1, generator=g)
    Rd, Ud = R.to(gpu), Uu.to(gpu)
    outs = []
    for paired in (True, False):
        H = H0.clone().to(gpu)
        T = torch.full((n1, n2), float("nan"), device=gpu)
        syrk = dict(A=Rd, B=Rd, C=H, M=n1, N=n1, K=n2, alpha=-1.0, beta_one=1, upper_only=1)
        tprod = dict(A=Rd, B=Ud, C=T, M=n1, N=n2, K=n2, tri=2)
        if paired:
            api._test_gemm_f32_pair(syrk, tprod)
        else:
            api._test_gemm_f32(Rd, Rd, H, n1, n1, n2, 0, 1, alpha=-1.0, beta_one=1, upper_only=1)
            api._test_gemm_f32(Rd, Ud, T, n1, n2, n2, 0, 0, tri=2)
        torch.cuda.synchronize()
        outs.append((H.cpu(), T.cpu()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    Hg, Tg = outs[0]
    want_t = R.double() @ Uu.double()
    assert rel_fro(Tg.double().numpy(), want_t.numpy()) < 1e-5
    want_h = H0.double() - R.double() @ R.double().T
    up = np.triu(np.ones((n1, n1), dtype=bool))
    assert rel_fro(Hg.double().numpy()[up], want_h.numpy()[up]) < 1e-5


@pytest.mark.parametrize("n", [300, 1800])
@pytest.mark.parametrize("k", [50, 64])
def test_gemm_f32_upper_only(gpu, k, n):
    """Every entry on or above the diagonal is updated; 128-blocks below it are untouched."""
    from post_int4_weight_amd import api
    announce(f"gemm_f32 upper_only k={k} n={n}")
    g = torch.Generator().manual_seed(7)
    P = torch.randn(n, k, generator=g)
    C0 = torch.randn(n, n, generator=g)
    C = C0.clone().to(gpu)
    Pd = torch.zeros(n, (k + 3) // 4 * 4)
    Pd[:, :k] = P
    Pd = Pd.to(gpu)
    api._test_gemm_f32(Pd, Pd, C, n, n, k, 0, 1, alpha=-1.0, beta_one=1, upper_only=1)
    torch.cuda.synchronize()
    ref = C0.double() - P.double() @ P.double().T
    got = C.cpu().double()
    nb = (n + 127) // 128
    for ti in range(nb):
        for tj in range(nb):
            blk = (slice(128 * ti, min(n, 128 * ti + 128)), slice(128 * tj, min(n, 128 * tj + 128)))
            if ti < tj:
                assert rel_fro(got[blk].numpy(), ref[blk].numpy()) < 1e-5
            elif ti == tj:
                up = np.triu(np.ones(got[blk].shape, dtype=bool))
                assert rel_fro(got[blk].numpy()[up], ref[blk].numpy()[up]) < 1e-5
            else:
                assert torch.equal(got[blk], C0.double()[blk])


@pytest.mark.parametrize("rows,n,dtype", [(1000, 520, "bf16"), (2048, 512, "f32"), (3000, 2056, "bf16"),
                                          (32768, 1024, "bf16"), (70000, 256, "bf16"), (40000, 640, "bf16"),
                                          (64, 8, "bf16"), (1500, 300, "bf16")])     # in % 8 != 0: scalar transpose
def test_hessian_vs_oracle(gpu, rows, n, dtype):
    """H relative Frobenius error <= 1e-5, exact symmetry, d to fp64 rounding."""
    import inputs
    from post_int4_weight_amd import api
    announce(f"hessian rows={rows} n={n} {dtype}")
    W, X = inputs.custom(8, n, rows, seed=rows + n, dtype=dtype, device="cpu")
    Xd = X.to(gpu)
    if n % 8:
        # rows padded to 16 bytes (the ABI's ldx rule); in % 8 != 0 takes the scalar transpose
        Xp = torch.zeros(rows, (n + 7) // 8 * 8, dtype=Xd.dtype, device=gpu)
        Xp[:, :n] = Xd
        Xd = Xp[:, :n]
    H, d = zeros_h(n, gpu)
    api.hessian_accumulate(H, d, Xd)
    torch.cuda.synchronize()
    H0, d0 = oracle.proxy_hessian(to64(X))
    Hg = H.cpu().double().numpy()
    assert np.array_equal(Hg, Hg.T)
    assert rel_fro(Hg, H0) <= 1e-5
    assert np.max(np.abs(d.cpu().numpy() - d0) / d0) <= 1e-12


@pytest.mark.parametrize("rows", [3000, 70000])
def test_hessian_large_n(gpu, rows):
    """n = 12544 (49 tile rows of 256: ten rounds of tiles, the last tile
    column a single one): blocks of H in the last tile column, on the
    diagonal and inside, against the oracle, with one chunk of rows and with
    two (the second adds onto the first and writes the mirror); H exactly
    symmetric; d to fp64 rounding."""
    import inputs
    from post_int4_weight_amd import api
    n = 12544
    announce(f"hessian large n rows={rows} n={n}")
    W, X = inputs.custom(8, n, rows, seed=rows, dtype="bf16", device="cpu")
    H, d = zeros_h(n, gpu)
    api.hessian_accumulate(H, d, X.to(gpu))
    torch.cuda.synchronize()
    assert torch.equal(H, H.T)
    X64 = to64(X)
    for (r0, c0) in ((8192, 12288), (12288, 12288), (0, 256), (4096, 8192)):
        Xa, Xb = X64[:, r0:r0 + 256], X64[:, c0:c0 + 256]
        ref = Xa.T @ Xb
        got = H[r0:r0 + 256, c0:c0 + 256].cpu().double().numpy()
        assert rel_fro(got, ref) <= 1e-5, (r0, c0)
    d0 = np.sum(X64 * X64, axis=0)
    assert np.max(np.abs(d.cpu().numpy() - d0) / d0) <= 1e-12


def test_hessian_is_additive(gpu):
    """Two calls on two halves equal one call on the whole (chunked streaming)."""
    import inputs
    from post_int4_weight_amd import api
    announce("hessian additive")
    _, X = inputs.custom(8, 1024, 4096, seed=3, dtype="bf16", device="cpu")
    Xd = X.to(gpu)
    H1, d1 = zeros_h(1024, gpu)
    api.hessian_accumulate(H1, d1, Xd[:2048])
    api.hessian_accumulate(H1, d1, Xd[2048:])
    H2, d2 = zeros_h(1024, gpu)
    api.hessian_accumulate(H2, d2, Xd)
    torch.cuda.synchronize()
    assert rel_fro(H1.cpu().double().numpy(), H2.cpu().double().numpy()) < 1e-6
    H0, _ = oracle.proxy_hessian(to64(X))
    assert rel_fro(H1.cpu().double().numpy(), H0) <= 1e-5


def test_hessian_empty_and_deterministic(gpu):
    import inputs
    from post_int4_weight_amd import api
    announce("hessian empty + determinism")
    _, X = inputs.custom(8, 2048, 4096, seed=9, dtype="bf16", device="cpu")
    Xd = X.to(gpu)
    H, d = zeros_h(2048, gpu)
    H += 1.5
    api.hessian_accumulate(H, d, Xd[:0])
    torch.cuda.synchronize()
    assert torch.all(H == 1.5)
    Ha, da = zeros_h(2048, gpu)
    Hb, db = zeros_h(2048, gpu)
    api.hessian_accumulate(Ha, da, Xd)
    api.hessian_accumulate(Hb, db, Xd)
    torch.cuda.synchronize()
    assert torch.equal(Ha, Hb) and torch.equal(da, db)
