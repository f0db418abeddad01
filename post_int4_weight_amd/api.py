"""ctypes binding of libptq.so — argument marshalling only.

Every function takes torch tensors that already live on the GPU, passes their
device pointers, sizes and torch's current HIP stream to the C entry point of
the same name (include/ptq.h), and raises PTQError on a non-OK status. Output
tensors may be passed in (no allocation) or are allocated here with
torch.empty; workspaces likewise. Nothing here computes: there is no CPU or
PyTorch fallback, and a missing library is an ImportError.
"""
from __future__ import annotations

import ctypes
import os

import torch

PTQ_BF16 = 0
PTQ_F32 = 1

_STATUS = {0: "PTQ_OK", 1: "PTQ_EINVAL", 2: "PTQ_ENOTPD", 3: "PTQ_ENONFINITE", 4: "PTQ_EWORKSPACE",
           5: "PTQ_EHIP"}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libptq.so")


class PTQError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status
        self.name = _STATUS.get(status, str(status))


def library_path() -> str:
    return _LIB_PATH


def _load() -> ctypes.CDLL:
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with `python post_int4_weight_amd/build.py`")
    lib = ctypes.CDLL(_LIB_PATH)
    i64, i32, sz, vp, dbl = ctypes.c_int64, ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_double
    fp = ctypes.POINTER(ctypes.c_float)
    dp = ctypes.POINTER(ctypes.c_double)
    sig = {
        "ptq_last_error": (ctypes.c_char_p, []),
        "ptq_status_string": (ctypes.c_char_p, [i32]),
        "ptq_abi_version": (i32, []),
        "ptq_profile_enable": (i32, [ctypes.c_uint]),
        "ptq_profile_read": (i32, [i32, dp, ctypes.POINTER(i64)]),
        "ptq_profile_flops": (i32, [i32, dp]),
        "hessian_workspace_bytes": (sz, [i64, i64]),
        "hessian_accumulate": (i32, [vp, vp, i64, vp, i32, i64, i64, vp, sz, vp]),
        "hessian_accumulate_noalloc": (i32, [vp, vp, i64, vp, i32, i64, i64, vp]),
        "gptq_factor_workspace_bytes": (sz, [i64]),
        "gptq_inverse_factor": (i32, [vp, vp, i64, dbl, i32, vp, vp, dp, vp, sz, vp]),
        "gptq_columns_workspace_bytes": (sz, [i64, i64, i32]),
        "gptq_quantize_columns": (i32, [vp, i32, i64, i64, i64, vp, vp, i32, i32, i32, vp, vp, vp, dp, vp, sz, vp]),
        "gptq_workspace_bytes": (sz, [i64, i64, i32]),
        "gptq_quantize_layer": (i32, [vp, i32, i64, i64, i64, vp, vp, i32, i32, dbl, i32, i32, vp, vp, vp, vp, dp,
                                      vp, sz, vp]),
        "awq_workspace_bytes": (sz, [i64, i64, i64, i32]),
        "ptq_test_gemm_f32": (i32, [i64, i64, i64, vp, i64, i32, vp, i64, i32, vp, i64, ctypes.c_float, i32, i32,
                                    i32, vp]),
        "awq_search_alpha": (i32, [vp, i32, i64, i64, i64, vp, i32, i64, i64, fp, i32, i32, i32, fp, dp, vp, vp, vp,
                                   vp, sz, vp]),
        "pack_int4": (i32, [vp, i64, i64, i32, vp, vp]),
        "awq_gptq_quantize_layer_workspace_bytes": (sz, [i64, i64, i32]),
        "awq_gptq_quantize_layer": (i32, [vp, i32, i64, i64, i64, vp, vp, vp, i32, i32, dbl, i32, i32, vp, vp, vp, vp,
                                          dp, vp, sz, vp]),
        "dequantize_int4": (i32, [vp, vp, vp, vp, i64, i64, i32, i32, vp, i64, vp]),
        "gptq_quantize_layer_zp": (i32, [vp, i32, i64, i64, i64, vp, vp, i32, i32, dbl, i32, i32, vp, vp, vp, vp, vp,
                                         dp, vp, sz, vp]),
        "layer_output_error_workspace_bytes": (sz, [i64, i64, i64, i32]),
        "ptq_test_gemm_f32_pair": (i32, [i64, i64, i64, vp, i64, vp, i64, vp, i64, ctypes.c_float, i32, i32, i32,
                                         i64, i64, i64, vp, i64, vp, i64, vp, i64, ctypes.c_float, i32, i32, i32,
                                         vp]),
        "ptq_test_gemm_f32_split3_workspace_bytes": (sz, [i64, i64, i64]),
        "ptq_test_gemm_f32_split3": (i32, [i64, i64, i64, vp, i64, i32, vp, i64, i32, vp, i64, ctypes.c_float, i32,
                                           i32, i32, vp, sz, vp]),
        "layer_output_error": (i32, [vp, i32, i64, i64, vp, i32, i64, i64, i64, vp, vp, vp, vp, vp, i32, dp, vp, sz,
                                     vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()


def _check(status: int):
    if status != 0:
        raise PTQError(status, _lib.ptq_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return PTQ_BF16
    if t.dtype == torch.float32:
        return PTQ_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def _workspace(nbytes: int, device, given):
    if given is not None:
        return given, given.numel() * given.element_size()
    if nbytes == 0:
        return None, 0
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


def _rowmajor(t: torch.Tensor, name: str):
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D row-major tensor")
    return t.stride(0)


# ------------------------------------------------------------- profiling ---

PROFILE_KERNELS = {"xtx_gemm": 0, "factor_gemm": 1, "factor_base": 2, "block_loop": 3, "trail_gemm": 4,
                   "awq_gemm": 5, "inner_gemm": 6, "split3_gemm": 7}


def profile_enable(kernels=()):
    """Bracket later launches of the named kernel classes with hipEvents."""
    mask = 0
    for k in kernels:
        mask |= 1 << PROFILE_KERNELS[k]
    _check(_lib.ptq_profile_enable(mask))


def profile_read(kernel: str):
    """(total_ms, launches) of the recorded launches of one kernel class."""
    tot = ctypes.c_double(0.0)
    cnt = ctypes.c_int64(0)
    _check(_lib.ptq_profile_read(PROFILE_KERNELS[kernel], ctypes.byref(tot), ctypes.byref(cnt)))
    return tot.value, cnt.value


def profile_flops(kernel: str) -> float:
    """MFMA flops executed by the recorded launches of one kernel class."""
    f = ctypes.c_double(0.0)
    _check(_lib.ptq_profile_flops(PROFILE_KERNELS[kernel], ctypes.byref(f)))
    return f.value


# ---------------------------------------------------------------- stage 1 ---

def hessian_workspace_bytes(n: int, rows: int) -> int:
    return int(_lib.hessian_workspace_bytes(n, rows))


def hessian_accumulate(H: torch.Tensor, d: torch.Tensor | None, X: torch.Tensor, workspace=None):
    """H (+)= X^T X (fp32 [n, n]), d (+)= column sums of squares (fp64 [n])."""
    n = H.shape[0]
    ldx = _rowmajor(X, "X")
    ws, wsb = _workspace(hessian_workspace_bytes(n, X.shape[0]), X.device, workspace)
    _check(_lib.hessian_accumulate(_ptr(H), _ptr(d), n, _ptr(X), _dtype_code(X), X.shape[0], ldx, _ptr(ws), wsb,
                                   _stream()))
    return H, d


def hessian_accumulate_noalloc(H: torch.Tensor, d: torch.Tensor | None, X: torch.Tensor):
    """hessian_accumulate_noalloc (include/ptq.h): the same sums with the
    library's fixed device scratch instead of a workspace (allocates nothing)."""
    n = H.shape[0]
    ldx = _rowmajor(X, "X")
    _check(_lib.hessian_accumulate_noalloc(_ptr(H), _ptr(d), n, _ptr(X), _dtype_code(X), X.shape[0], ldx,
                                           _stream()))
    return H, d


# ---------------------------------------------------------------- stage 2 ---

def gptq_factor_workspace_bytes(n: int) -> int:
    return int(_lib.gptq_factor_workspace_bytes(n))


def gptq_inverse_factor(H, d=None, damp=0.01, act_order=False, U=None, perm=None, workspace=None):
    """Upper factor U of (P (H + lambda I) P^T)^-1; returns (U, perm, lambda)."""
    n = H.shape[0]
    if U is None:
        U = torch.empty(n, n, dtype=torch.float32, device=H.device)
    if perm is None and act_order:
        perm = torch.empty(n, dtype=torch.int32, device=H.device)
    ws, wsb = _workspace(gptq_factor_workspace_bytes(n), H.device, workspace)
    lam = ctypes.c_double(0.0)
    _check(_lib.gptq_inverse_factor(_ptr(H), _ptr(d), n, float(damp), int(bool(act_order)), _ptr(U), _ptr(perm),
                                    ctypes.byref(lam), _ptr(ws), wsb, _stream()))
    return U, perm, lam.value


# ---------------------------------------------------------------- stage 3 ---

def gptq_columns_workspace_bytes(out: int, n: int, block_size: int = 128) -> int:
    return int(_lib.gptq_columns_workspace_bytes(out, n, block_size))


def _alloc_codes(W, n, g, codes, scales, g_idx):
    out = W.shape[0]
    dev = W.device
    if codes is None:
        codes = torch.empty(out, n, dtype=torch.int8, device=dev)
    if scales is None:
        scales = torch.empty(out, (n + g - 1) // g, dtype=torch.float32, device=dev)
    if g_idx is None:
        g_idx = torch.empty(n, dtype=torch.int32, device=dev)
    return codes, scales, g_idx


def gptq_quantize_columns(W, U, perm=None, bits=4, group_size=128, block_size=128, codes=None, scales=None,
                          g_idx=None, workspace=None):
    """The column loop given U; returns (codes, scales, g_idx, stats[4])."""
    out, n = W.shape
    ldw = _rowmajor(W, "W")
    codes, scales, g_idx = _alloc_codes(W, n, group_size, codes, scales, g_idx)
    ws, wsb = _workspace(gptq_columns_workspace_bytes(out, n, block_size), W.device, workspace)
    stats = (ctypes.c_double * 4)()
    _check(_lib.gptq_quantize_columns(_ptr(W), _dtype_code(W), out, n, ldw, _ptr(U), _ptr(perm), bits, group_size,
                                      block_size, _ptr(codes), _ptr(scales), _ptr(g_idx), stats, _ptr(ws), wsb,
                                      _stream()))
    return codes, scales, g_idx, list(stats)


# ------------------------------------------------------------ stages 2+3 ---

def gptq_workspace_bytes(out: int, n: int, block_size: int = 128) -> int:
    return int(_lib.gptq_workspace_bytes(out, n, block_size))


def gptq_quantize_layer(W, H, d=None, bits=4, group_size=128, damp=0.01, act_order=False, block_size=128,
                        codes=None, scales=None, g_idx=None, perm=None, workspace=None):
    """Whole GPTQ layer from the undamped H; returns dict(codes, scales, g_idx, perm, stats)."""
    out, n = W.shape
    ldw = _rowmajor(W, "W")
    codes, scales, g_idx = _alloc_codes(W, n, group_size, codes, scales, g_idx)
    if perm is None:
        perm = torch.empty(n, dtype=torch.int32, device=W.device)
    ws, wsb = _workspace(gptq_workspace_bytes(out, n, block_size), W.device, workspace)
    stats = (ctypes.c_double * 4)()
    _check(_lib.gptq_quantize_layer(_ptr(W), _dtype_code(W), out, n, ldw, _ptr(H), _ptr(d), bits, group_size,
                                    float(damp), int(bool(act_order)), block_size, _ptr(codes), _ptr(scales),
                                    _ptr(g_idx), _ptr(perm), stats, _ptr(ws), wsb, _stream()))
    return {"codes": codes, "scales": scales, "g_idx": g_idx, "perm": perm,
            "stats": {"sum_err2": stats[0], "lambda": stats[1], "dW_fro2": stats[2], "objective": stats[3]}}


# ---------------------------------------------------------------- stage 4 ---

def awq_workspace_bytes(out: int, n: int, rows: int, n_alpha: int) -> int:
    return int(_lib.awq_workspace_bytes(out, n, rows, n_alpha))


def awq_search_alpha(W, X, alphas, bits=4, group_size=128, s=None, codes=None, scales=None, workspace=None):
    """AWQ grid search; returns dict(alpha, errors, s, codes, scales)."""
    out, n = W.shape
    rows = X.shape[0]
    ldw = _rowmajor(W, "W")
    ldx = _rowmajor(X, "X")
    na = len(alphas)
    al = (ctypes.c_float * na)(*[float(a) for a in alphas])
    dev = W.device
    if s is None:
        s = torch.empty(n, dtype=torch.float32, device=dev)
    if codes is None:
        codes = torch.empty(out, n, dtype=torch.int8, device=dev)
    if scales is None:
        scales = torch.empty(out, (n + group_size - 1) // group_size, dtype=torch.float32, device=dev)
    ws, wsb = _workspace(awq_workspace_bytes(out, n, rows, na), dev, workspace)
    best = ctypes.c_float(0.0)
    errs = (ctypes.c_double * na)()
    _check(_lib.awq_search_alpha(_ptr(W), _dtype_code(W), out, n, ldw, _ptr(X), _dtype_code(X), rows, ldx, al, na,
                                 bits, group_size, ctypes.byref(best), errs, _ptr(s), _ptr(codes), _ptr(scales),
                                 _ptr(ws), wsb, _stream()))
    return {"alpha": best.value, "errors": list(errs), "s": s, "codes": codes, "scales": scales}


# ------------------------------------------- composition and INT4 storage ---

def gptq_quantize_layer_zp(W, H, d=None, bits=4, group_size=128, damp=0.01, act_order=False, block_size=128,
                           codes=None, scales=None, zeros=None, g_idx=None, perm=None, workspace=None):
    """gptq_quantize_layer_zp (include/ptq.h): GPTQ with zero-point groups; codes in [0, 2^bits - 1]."""
    out, n = W.shape
    ldw = _rowmajor(W, "W")
    codes, scales, g_idx = _alloc_codes(W, n, group_size, codes, scales, g_idx)
    if zeros is None:
        zeros = torch.empty(out, (n + group_size - 1) // group_size, dtype=torch.int8, device=W.device)
    if perm is None:
        perm = torch.empty(n, dtype=torch.int32, device=W.device)
    ws, wsb = _workspace(gptq_workspace_bytes(out, n, block_size), W.device, workspace)
    stats = (ctypes.c_double * 4)()
    _check(_lib.gptq_quantize_layer_zp(_ptr(W), _dtype_code(W), out, n, ldw, _ptr(H), _ptr(d), bits, group_size,
                                       float(damp), int(bool(act_order)), block_size, _ptr(codes), _ptr(scales),
                                       _ptr(zeros), _ptr(g_idx), _ptr(perm), stats, _ptr(ws), wsb, _stream()))
    return {"codes": codes, "scales": scales, "zeros": zeros, "g_idx": g_idx, "perm": perm,
            "stats": {"sum_err2": stats[0], "lambda": stats[1], "dW_fro2": stats[2], "objective": stats[3]}}


def awq_gptq_quantize_layer(W, H, d, s, bits=4, group_size=128, damp=0.01, act_order=False, block_size=128,
                            codes=None, scales=None, g_idx=None, perm=None, workspace=None):
    """awq_gptq_quantize_layer (include/ptq.h): GPTQ on W diag(s) with the Hessian of X diag(s)^-1."""
    out, n = W.shape
    ldw = _rowmajor(W, "W")
    codes, scales, g_idx = _alloc_codes(W, n, group_size, codes, scales, g_idx)
    if perm is None:
        perm = torch.empty(n, dtype=torch.int32, device=W.device)
    ws, wsb = _workspace(int(_lib.awq_gptq_quantize_layer_workspace_bytes(out, n, block_size)), W.device, workspace)
    stats = (ctypes.c_double * 4)()
    _check(_lib.awq_gptq_quantize_layer(_ptr(W), _dtype_code(W), out, n, ldw, _ptr(H), _ptr(d), _ptr(s), bits,
                                        group_size, float(damp), int(bool(act_order)), block_size, _ptr(codes),
                                        _ptr(scales), _ptr(g_idx), _ptr(perm), stats, _ptr(ws), wsb, _stream()))
    return {"codes": codes, "scales": scales, "g_idx": g_idx, "perm": perm,
            "stats": {"sum_err2": stats[0], "lambda": stats[1], "dW_fro2": stats[2], "objective": stats[3]}}


def pack_int4(codes: torch.Tensor, bits: int = 4, packed=None):
    """pack_int4 (include/ptq.h): int8 codes [out, in] -> int32 words [out, in/8]
    (uint32 bit patterns; torch has no uint32 arithmetic, so int32 holds them)."""
    out, n = codes.shape
    if codes.dtype != torch.int8 or codes.stride(1) != 1 or codes.stride(0) != n:
        raise ValueError("codes must be a contiguous int8 [out, in] tensor")
    if packed is None:
        packed = torch.empty(out, n // 8, dtype=torch.int32, device=codes.device)
    _check(_lib.pack_int4(_ptr(codes), out, n, bits, _ptr(packed), _stream()))
    return packed


def dequantize_int4(packed: torch.Tensor, scales: torch.Tensor, g_idx, n: int, group_size: int = 128,
                    out_dtype=torch.float32, What=None, zeros=None):
    """dequantize_int4 (include/ptq.h): What[r][c] = code * scales[r][g_idx[c]] (g_idx None: c // group_size);
    with zeros, unsigned codes and What = (code - zero) * scale."""
    out = packed.shape[0]
    if What is None:
        What = torch.empty(out, n, dtype=out_dtype, device=packed.device)
    ldo = _rowmajor(What, "What") if out > 0 else n
    _check(_lib.dequantize_int4(_ptr(packed), _ptr(scales), _ptr(g_idx), _ptr(zeros), out, n, group_size,
                                _dtype_code(What), _ptr(What), ldo, _stream()))
    return What


# ------------------------------------------------------------ evaluation ---

def layer_output_error_workspace_bytes(out: int, n: int, rows: int, x_dtype: int) -> int:
    return int(_lib.layer_output_error_workspace_bytes(out, n, rows, x_dtype))


def layer_output_error(X, W, codes, scales, g_idx=None, zeros=None, s=None, group_size=128, workspace=None):
    """layer_output_error (include/ptq.h): (||X (W - What)^T||^2, ||X W^T||^2) with
    What = (codes - zeros[g_idx]) * scales[g_idx] / s."""
    out, n = W.shape
    rows = X.shape[0]
    ldw = _rowmajor(W, "W")
    ldx = _rowmajor(X, "X")
    if codes.dtype != torch.int8 or not codes.is_contiguous() or tuple(codes.shape) != (out, n):
        raise ValueError("codes must be a contiguous int8 [out, in] tensor")
    xd = _dtype_code(X)
    ws, wsb = _workspace(layer_output_error_workspace_bytes(out, n, rows, xd), W.device, workspace)
    res = (ctypes.c_double * 2)()
    _check(_lib.layer_output_error(_ptr(X), xd, rows, ldx, _ptr(W), _dtype_code(W), out, n, ldw, _ptr(codes),
                                   _ptr(scales), _ptr(g_idx), _ptr(zeros), _ptr(s), group_size, res, _ptr(ws), wsb,
                                   _stream()))
    return res[0], res[1]


# ------------------------------------------------------------- test hook ---

def _test_gemm_f32(A, B, C, M, N, K, layout_a, layout_b, alpha=1.0, beta_one=0, tri=0, upper_only=0):
    """ptq_test_gemm_f32 (include/ptq_testing.h): the fp32 MFMA GEMM alone."""
    _check(_lib.ptq_test_gemm_f32(M, N, K, _ptr(A), A.stride(0), layout_a, _ptr(B), B.stride(0), layout_b, _ptr(C),
                                  C.stride(0), float(alpha), int(beta_one), int(tri), int(upper_only), _stream()))
    return C


def _test_gemm_f32_pair(p0, p1):
    """ptq_test_gemm_f32_pair (include/ptq_testing.h): two products in one launch, the first with B stored
    [N][K], the second with B row-major [K][N]. Each pi is a dict with A, B, C, M, N, K and optionally alpha,
    beta_one, tri, upper_only."""
    def args(p):
        return (p["M"], p["N"], p["K"], _ptr(p["A"]), p["A"].stride(0), _ptr(p["B"]), p["B"].stride(0), _ptr(p["C"]),
                p["C"].stride(0), float(p.get("alpha", 1.0)), int(p.get("beta_one", 0)), int(p.get("tri", 0)),
                int(p.get("upper_only", 0)))
    _check(_lib.ptq_test_gemm_f32_pair(*args(p0), *args(p1), _stream()))


def _test_gemm_f32_split3(A, B, C, M, N, K, layout_a, layout_b, alpha=1.0, beta_one=0, tri=0, upper_only=0):
    """ptq_test_gemm_f32_split3 (include/ptq_testing.h): the same product on the bf16 MFMA from split operands."""
    ws, wsb = _workspace(int(_lib.ptq_test_gemm_f32_split3_workspace_bytes(M, N, K)), C.device, None)
    _check(_lib.ptq_test_gemm_f32_split3(M, N, K, _ptr(A), A.stride(0), layout_a, _ptr(B), B.stride(0), layout_b,
                                         _ptr(C), C.stride(0), float(alpha), int(beta_one), int(tri),
                                         int(upper_only), _ptr(ws), wsb, _stream()))
    return C
