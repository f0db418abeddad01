"""C ABI checks that need no GPU: the library loads, exports every function
include/ptq.h declares, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in sorted(os.listdir(os.path.join(ROOT, "include")))
           if f.endswith(".h")]


def _declared_functions():
    src = "\n".join(open(h).read() for h in HEADERS)
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_][a-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while", "for")))


def test_header_lists_the_entry_points():
    names = _declared_functions()
    for n in ("hessian_accumulate", "gptq_inverse_factor", "gptq_quantize_columns", "gptq_quantize_layer",
              "awq_search_alpha", "ptq_last_error", "ptq_test_gemm_f32", "pack_int4", "dequantize_int4",
              "awq_gptq_quantize_layer", "gptq_quantize_layer_zp", "layer_output_error"):
        assert n in names


def test_library_exports_every_declared_symbol():
    from post_int4_weight_amd import api
    lib = ctypes.CDLL(api.library_path())
    missing = [n for n in _declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


@pytest.fixture(scope="module")
def lib():
    from post_int4_weight_amd import api
    return api._lib


def _err(lib):
    return lib.ptq_last_error().decode()


def test_status_strings(lib):
    assert lib.ptq_status_string(0) == b"PTQ_OK"
    assert lib.ptq_status_string(2) == b"PTQ_ENOTPD"
    assert lib.ptq_abi_version() >= 1


def test_hessian_validation(lib):
    fake = ctypes.c_void_p(1 << 20)      # never dereferenced: validation fails first
    assert lib.hessian_accumulate(None, None, 0, None, 0, 0, 0, None, 0, None) == 1
    assert "in = 0" in _err(lib)
    assert lib.hessian_accumulate(fake, None, 6, fake, 0, 10, 8, None, 0, None) == 1    # in % 4
    assert lib.hessian_accumulate(fake, None, 8, fake, 7, 10, 8, None, 0, None) == 1    # dtype
    assert lib.hessian_accumulate(fake, None, 16, fake, 0, 10, 8, None, 0, None) == 1   # ldx < in
    assert lib.hessian_accumulate(fake, None, 16, fake, 0, -1, 16, None, 0, None) == 1  # rows < 0
    assert lib.hessian_accumulate(None, None, 16, fake, 0, 4, 16, None, 0, None) == 1   # H NULL
    assert lib.hessian_accumulate(fake, None, 16, None, 0, 4, 16, None, 0, None) == 1   # X NULL
    mis = ctypes.c_void_p((1 << 20) + 4)
    assert lib.hessian_accumulate(mis, None, 16, fake, 0, 4, 16, None, 0, None) == 1    # misaligned
    # rows == 0 is a no-op that touches nothing
    assert lib.hessian_accumulate(fake, None, 16, None, 0, 0, 16, None, 0, None) == 0


def test_factor_validation(lib):
    fake = ctypes.c_void_p(1 << 20)
    lam = ctypes.c_double()
    ws = lib.gptq_factor_workspace_bytes(64)
    assert ws > 0
    assert lib.gptq_inverse_factor(fake, None, 64, -0.1, 0, fake, None, ctypes.byref(lam), fake, ws, None) == 1
    assert lib.gptq_inverse_factor(fake, None, 64, float("nan"), 0, fake, None, ctypes.byref(lam), fake, ws, None) == 1
    assert lib.gptq_inverse_factor(fake, None, 64, 0.01, 2, fake, None, ctypes.byref(lam), fake, ws, None) == 1
    assert lib.gptq_inverse_factor(fake, None, 64, 0.01, 1, fake, None, ctypes.byref(lam), fake, ws, None) == 1
    assert "perm" in _err(lib)
    assert lib.gptq_inverse_factor(fake, None, 64, 0.01, 0, fake, None, ctypes.byref(lam), fake, 16, None) == 4


def test_columns_and_layer_validation(lib):
    fake = ctypes.c_void_p(1 << 20)
    st = (ctypes.c_double * 4)()
    ws = lib.gptq_workspace_bytes(32, 256, 128)
    base = dict(W=fake, wt=0, out=32, n=256, ldw=256, H=fake, d=None, bits=4, g=128, damp=0.01, ao=0, blk=128)

    def call(**kw):
        a = dict(base, **kw)
        return lib.gptq_quantize_layer(a["W"], a["wt"], a["out"], a["n"], a["ldw"], a["H"], a["d"], a["bits"],
                                       a["g"], a["damp"], a["ao"], a["blk"], fake, fake, fake, fake, st, fake, ws,
                                       None)
    assert call(bits=1) == 1
    assert call(bits=9) == 1
    assert call(g=96) == 1          # neither divides the other
    assert call(g=4) == 1           # divides 128 but not a multiple of 8
    assert call(blk=96) == 1
    assert call(n=250, ldw=256) == 1  # in % 8
    assert call(ldw=200) == 1
    assert call(damp=-1.0) == 1
    assert call(ao=3) == 1
    assert call(out=-1) == 1
    assert call(W=None) == 1
    assert call(H=None) == 1
    assert lib.gptq_quantize_layer(fake, 0, 32, 256, 256, fake, None, 4, 128, 0.01, 0, 128, fake, fake, fake, fake,
                                   st, fake, 64, None) == 4  # workspace too small


def test_awq_validation(lib):
    fake = ctypes.c_void_p(1 << 20)
    al = (ctypes.c_float * 2)(0.0, 0.5)
    best = ctypes.c_float()
    ws = lib.awq_workspace_bytes(32, 256, 64, 2)
    assert ws > 0
    args = lambda **k: dict(dict(out=32, n=256, rows=64, na=2, bits=4, g=128), **k)

    def call(**k):
        a = args(**k)
        return lib.awq_search_alpha(fake, 0, a["out"], a["n"], 256, fake, 0, a["rows"], 256, al, a["na"], a["bits"],
                                    a["g"], ctypes.byref(best), None, fake, fake, fake, fake, ws, None)
    assert call(rows=0) == 1
    assert call(na=0) == 1
    assert call(na=65) == 1
    assert call(bits=12) == 1
    assert call(g=0) == 1
    assert call(n=250) == 1


def test_int4_storage_validation(lib):
    fake = ctypes.c_void_p(1 << 20)
    assert lib.pack_int4(fake, 4, 12, 4, fake, None) == 1          # in not a multiple of 8
    assert lib.pack_int4(fake, 4, 16, 5, fake, None) == 1          # 5-bit codes do not fit a nibble
    assert lib.pack_int4(None, 4, 16, 4, fake, None) == 1
    assert lib.pack_int4(ctypes.c_void_p((1 << 20) + 4), 4, 16, 4, fake, None) == 1   # misaligned
    assert "pack_int4" in _err(lib)
    assert lib.pack_int4(None, 0, 16, 4, None, None) == 0          # empty: nothing to do

    def deq(**k):
        a = dict(dict(out=4, n=16, g=8, dt=1, ldo=16, packed=fake, scales=fake, what=fake), **k)
        return lib.dequantize_int4(a["packed"], a["scales"], None, None, a["out"], a["n"], a["g"], a["dt"],
                                   a["what"], a["ldo"], None)
    assert deq(n=12) == 1
    assert deq(g=0) == 1
    assert deq(dt=7) == 1
    assert deq(ldo=12) == 1
    assert deq(ldo=20) == 1                                       # not a multiple of 8
    assert deq(scales=None) == 1
    assert "dequantize_int4" in _err(lib)


def test_awq_gptq_validation(lib):
    fake = ctypes.c_void_p(1 << 20)
    st = (ctypes.c_double * 4)()
    ws = lib.awq_gptq_quantize_layer_workspace_bytes(32, 256, 128)
    assert ws > 0

    def call(**k):
        a = dict(dict(out=32, n=256, s=fake, bits=4, g=128, damp=0.01, ao=0, blk=128, ws=ws, H=fake), **k)
        return lib.awq_gptq_quantize_layer(fake, 0, a["out"], a["n"], 256, a["H"], None, a["s"], a["bits"], a["g"],
                                           a["damp"], a["ao"], a["blk"], fake, fake, fake, fake, st, fake, a["ws"],
                                           None)
    assert call(s=None) == 1
    assert call(H=None) == 1
    assert call(bits=9) == 1
    assert call(damp=-1.0) == 1
    assert call(ao=2) == 1
    assert call(blk=96) == 1
    assert call(n=250) == 1
    assert call(ws=64) == 4
    assert "awq_gptq_quantize_layer" in _err(lib)


def test_zero_point_validation(lib):
    fake = ctypes.c_void_p(1 << 20)
    st = (ctypes.c_double * 4)()

    def call(**k):
        a = dict(dict(bits=4, zeros=fake, g=128), **k)
        return lib.gptq_quantize_layer_zp(fake, 0, 32, 256, 256, fake, None, a["bits"], a["g"], 0.01, 0, 128, fake,
                                          fake, a["zeros"], fake, fake, st, fake, 64, None)
    assert call(bits=8) == 1          # codes 0..255 do not fit int8
    assert call(bits=1) == 1
    assert call(zeros=None) == 1
    assert call(g=0) == 1
    assert call() == 4                # workspace too small
    assert "gptq_quantize_layer_zp" in _err(lib)


def test_output_error_validation(lib):
    fake = ctypes.c_void_p(1 << 20)
    res = (ctypes.c_double * 2)()
    ws = lib.layer_output_error_workspace_bytes(32, 256, 64, 0)
    assert ws > 0 and lib.layer_output_error_workspace_bytes(32, 256, 64, 1) > 0
    assert lib.layer_output_error_workspace_bytes(0, 256, 64, 0) == 0
    assert lib.layer_output_error_workspace_bytes(32, 256, 64, 7) == 0

    def call(out=32, n=256, rows=64, xd=0, wd=0, g=128, ldx=256, ldw=256, codes=fake, r=res, wsb=ws, w=fake):
        return lib.layer_output_error(fake, xd, rows, ldx, fake, wd, out, n, ldw, codes, fake, None, None, None, g, r,
                                      w, wsb, None)
    assert call(rows=0) == 1
    assert call(out=0) == 1
    assert call(n=250, ldx=256, ldw=256) == 1        # in not a multiple of 8
    assert call(xd=3) == 1
    assert call(g=0) == 1
    assert call(ldx=100) == 1
    assert call(codes=None) == 1
    assert call(r=None) == 1
    assert "layer_output_error" in _err(lib)
    assert call(wsb=ws - 1) == 4                      # PTQ_EWORKSPACE
    assert call(w=None) == 4


def test_noalloc_rejects_oversize_before_any_hip_call(lib):
    fake = ctypes.c_void_p(1 << 20)      # never dereferenced: validation fails first
    # bf16 X with in = 262144: a 64-row chunk's transposed copy exceeds the fixed scratch
    assert lib.hessian_accumulate_noalloc(fake, None, 262144, fake, 0, 1, 262144, None) == 1
    assert "too large" in _err(lib)
    assert lib.hessian_accumulate_noalloc(fake, None, 6, fake, 0, 10, 8, None) == 1     # in % 4
    assert lib.hessian_accumulate_noalloc(None, None, 16, fake, 0, 4, 16, None) == 1    # H NULL
