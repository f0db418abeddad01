"""GPU: INT4 storage of the codes (pack_int4) and the g_idx-aware dequantizer
(dequantize_int4) against the oracle (oracle/pack.py), bit for bit.

Codes come from the GPU quantizer itself (act-order and natural order, 4- and
3-bit, a ragged last group), so the check covers the storage contract of the
path's real output: with act-order, dequantizing through g_idx reproduces
code * scale of the processing-order groups, and ignoring g_idx does not.
The fp32 output is the fp32 product code * scale (exact in fp64, so one
rounding); the bf16 output is that fp32 value rounded to nearest even.
"""
import numpy as np
import pytest
import torch

import inputs
import oracle
from gpu_util import announce, zeros_h

pytestmark = pytest.mark.gpu


def _quantized(gpu, out, n, bits, g, act_order, seed):
    from post_int4_weight_amd import api
    W, X = inputs.custom(out, n, 4096, seed, "bf16", gpu)
    H, d = zeros_h(n, gpu)
    api.hessian_accumulate(H, d, X)
    res = api.gptq_quantize_layer(W, H, d, bits=bits, group_size=g, damp=0.01, act_order=act_order)
    torch.cuda.synchronize()
    return W, res


def _u32(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("out,n,bits,g,act_order", [(384, 1024, 4, 128, True), (256, 1000, 4, 128, False),
                                                    (130, 512, 3, 64, True), (64, 256, 2, 32, True)])
def test_pack_and_dequant_match_oracle(gpu, out, n, bits, g, act_order):
    from post_int4_weight_amd import api
    announce(f"int4 storage out={out} n={n} bits={bits} g={g} act_order={act_order}")
    W, res = _quantized(gpu, out, n, bits, g, act_order, seed=out + n)
    codes, scales, g_idx = res["codes"], res["scales"], res["g_idx"]
    packed = api.pack_int4(codes, bits=bits)
    torch.cuda.synchronize()
    ref_words = oracle.pack_int4(codes.cpu().numpy())
    assert np.array_equal(_u32(packed), ref_words)

    gi = g_idx.cpu().numpy()
    ref64 = oracle.dequantize_packed(ref_words, scales.cpu().double().numpy(), gi, n)
    ref32 = ref64.astype(np.float32)
    What = api.dequantize_int4(packed, scales, g_idx, n, group_size=g)
    What_bf16 = api.dequantize_int4(packed, scales, g_idx, n, group_size=g, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert np.array_equal(What.cpu().numpy(), ref32)
    assert torch.equal(What_bf16.cpu(), torch.from_numpy(ref32).to(torch.bfloat16))
    # the same weights as code * scale from the quantizer's own outputs
    assert np.array_equal(ref64, oracle.dequantize(codes.cpu().numpy(), scales.cpu().double().numpy(), gi))

    if act_order:
        # the contract: a dequantizer that ignores g_idx loads other weights
        plain = api.dequantize_int4(packed, scales, None, n, group_size=g)
        torch.cuda.synchronize()
        assert not torch.equal(plain, What)
        # processing order: groups are consecutive runs of g columns
        perm = res["perm"].long().cpu().numpy()
        proc = oracle.dequantize(codes.cpu().numpy()[:, perm], scales.cpu().double().numpy(), np.arange(n) // g)
        assert np.array_equal(ref64[:, perm], proc)
    else:
        plain = api.dequantize_int4(packed, scales, None, n, group_size=g)
        torch.cuda.synchronize()
        assert torch.equal(plain, What)


def test_dequant_bad_group_index_is_nan(gpu):
    from post_int4_weight_amd import api
    announce("int4 dequant: out-of-range group index")
    n, g = 64, 16
    codes = torch.randint(-8, 8, (8, n), dtype=torch.int8, device=gpu)
    scales = torch.rand(8, n // g, device=gpu) + 0.5
    g_idx = (torch.arange(n, device=gpu, dtype=torch.int32) // g)
    g_idx[5] = 99
    g_idx[40] = -1
    What = api.dequantize_int4(api.pack_int4(codes), scales, g_idx, n, group_size=g)
    torch.cuda.synchronize()
    bad = torch.isnan(What)
    assert bad[:, 5].all() and bad[:, 40].all()
    assert int(bad.sum()) == 16
    good = ~bad
    ref = codes.float() * scales[:, (torch.arange(n, device=gpu) // g)]
    assert torch.equal(What[good], ref[good])


def test_pack_row_stride_and_empty(gpu):
    from post_int4_weight_amd import api
    announce("int4 dequant: padded output rows, empty input")
    n, g = 48, 16
    codes = torch.randint(-8, 8, (5, n), dtype=torch.int8, device=gpu)
    scales = torch.rand(5, 3, device=gpu)
    packed = api.pack_int4(codes)
    big = torch.full((5, 64), 7.0, device=gpu)
    api.dequantize_int4(packed, scales, None, n, group_size=g, What=big[:, :n])
    torch.cuda.synchronize()
    ref = codes.float() * scales[:, torch.arange(n, device=gpu) // g]
    assert torch.equal(big[:, :n], ref)
    assert torch.all(big[:, n:] == 7.0)
    empty = api.pack_int4(torch.empty(0, n, dtype=torch.int8, device=gpu))
    assert empty.shape == (0, n // 8)
