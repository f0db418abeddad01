"""fp64 / integer oracle for INT4 storage of the codes (TEST INFRASTRUCTURE ONLY).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import it.

Sources:

* "GPTQ versus AWQ objectives" (inferenceinterviews.com), opening question
  and "A strong answer": both methods store INT4 weights with group scales;
* same page, "What interviewers probe next" and "Common mistakes": with
  act-order the groups follow the processing order, so the stored model
  needs a group index per column, and a dequantizer that ignores it applies
  the wrong scales to valid-looking weights.

The pages fix no bit layout. Reading (shared with the HIP path): eight codes
per 32-bit word along the input dimension, code 8w + k of a row in bits
4k .. 4k + 3 of word w, as a two's-complement nibble (INT3 codes use the same
nibbles). Dequantization is code * scale[row, g_idx[col]].
"""
from __future__ import annotations

import numpy as np


def pack_int4(codes):
    """codes int [out, n], n % 8 == 0 -> uint32 [out, n / 8]. Codes of a
    symmetric grid lie in [-8, 7] (two's-complement nibbles), those of a
    zero-point grid in [0, 15] (plain nibbles); both store their low 4 bits."""
    codes = np.asarray(codes, dtype=np.int64)
    out, n = codes.shape
    if n % 8:
        raise ValueError("the input dimension must be a multiple of 8")
    if codes.size and (codes.min() < -8 or codes.max() > 15 or (codes.min() < 0 and codes.max() > 7)):
        raise ValueError("codes must lie in [-8, 7] or in [0, 15] to fit a 4-bit nibble")
    words = np.zeros((out, n // 8), dtype=np.uint64)
    for w in range(n // 8):
        for k in range(8):
            words[:, w] |= ((codes[:, 8 * w + k] & 0xF).astype(np.uint64)) << np.uint64(4 * k)
    return words.astype(np.uint32)


def unpack_int4(packed, n: int, signed: bool = True):
    """Inverse of pack_int4: uint32 [out, n / 8] -> int64 codes [out, n]
    (two's-complement nibbles, or plain ones with signed=False)."""
    packed = np.asarray(packed, dtype=np.uint64)
    out = packed.shape[0]
    codes = np.zeros((out, n), dtype=np.int64)
    for w in range(n // 8):
        for k in range(8):
            nib = ((packed[:, w] >> np.uint64(4 * k)) & np.uint64(0xF)).astype(np.int64)
            codes[:, 8 * w + k] = np.where(nib >= 8, nib - 16, nib) if signed else nib
    return codes


def dequantize_packed(packed, scales, g_idx, n: int, zeros=None):
    """What[r, c] = code(r, c) * scales[r, g_idx[c]] in float64; with zeros
    (zero-point grid) the nibbles are plain and What = (code - zero) * scale."""
    gi = np.asarray(g_idx)
    codes = unpack_int4(packed, n, signed=zeros is None).astype(np.float64)
    if zeros is not None:
        codes = codes - np.asarray(zeros, dtype=np.float64)[:, gi]
    return codes * np.asarray(scales, dtype=np.float64)[:, gi]
