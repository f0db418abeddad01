#!/usr/bin/env python3
"""Benchmark: GPTQ quantization of one Llama-70B-shaped down_proj layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Workload (synthetic, seeded; see inputs/): W [8192, 28672] bf16, calibration
X [262144, 28672] bf16 (128 x 2048 tokens, log-normal channel scales, 60% of
entries zeroed), 4-bit, g = 128, damp = 0.01, natural column order, lazy
block 128. X and W are resident in HBM before timing starts.

One step is the whole path: H = X^T X with the fp64 column sums of squares,
damping, U (reversed Cholesky + triangular inverse), the blocked column loop
with its trailing GEMMs, codes / scales / g_idx and the error statistics.
The metric is seconds per layer (lower is better). Printed as one JSON line,
with a roofline entry for the dominant kernel (X^T X on bf16 MFMA, timed per
launch with hipEvents on its stream), a per-stage breakdown from one extra
instrumented step, and the fp64 oracle timed on a bounded sample on the host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "GPTQ s/layer + XᵀX, Cholesky, block-update TFLOP/s (8192×28672 down_proj)"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3       # MI355X fp32 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--bits", type=int, default=4)
    ap.add_argument("--workload", default="llama70b_down_proj")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-breakdown", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="before the steps, run a copy-like elementwise kernel (torch.neg) over 1 GiB of fp32, "
                         "whose FETCH_SIZE / WRITE_SIZE counters calibrate the traffic figures")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                            "xtx_gemm_down_proj_traffic.md")
TRAFFIC_SOURCES = ["post_int4_weight_amd/csrc/gemm_bf16.hip", "post_int4_weight_amd/csrc/tile_order.hpp"]


def kernel_source_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    root = os.path.dirname(os.path.abspath(__file__))
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(root, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per X^T X launch from the committed FETCH_SIZE / WRITE_SIZE
    counter runs, each scaled by the factor a 1 GiB copy-like kernel gave in
    the same run. None when the kernel source changed since they were taken."""
    try:
        kv = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if ":" in line and not line.startswith(("#", "|", " ")):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("source_sha256") != kernel_source_digest():
            return None
        fetch = float(kv["fetch_kib_per_launch"]) * float(kv["copy_fetch_factor"])
        write = float(kv["write_kib_per_launch"]) * float(kv["copy_write_factor"])
        return round((fetch + write) * 1024.0)
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(cfg, W, X, bits):
    """Time the fp64 oracle on a bounded sample of the same layer, scaled by
    exact operation counts to one whole layer."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits

    cores = min(len(os.sched_getaffinity(0)), 16)
    n, o, N = cfg.inp, cfg.out, cfg.rows
    rs, ns, os_ = 1024, 4096, 32
    with threadpool_limits(limits=cores):
        used = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        Xs = X[:rs].float().cpu().numpy().astype(np.float64)
        t0 = time.perf_counter()
        H0, d = oracle.proxy_hessian(Xs)
        t_h = time.perf_counter() - t0
        Hs, _ = oracle.damped(H0[:ns, :ns], 0.01)
        t0 = time.perf_counter()
        U = oracle.inverse_upper_factor(Hs)
        t_u = time.perf_counter() - t0
        Ws = W[:os_, :ns].float().cpu().numpy().astype(np.float64)
        t0 = time.perf_counter()
        oracle.gptq_columns(Ws, U, bits, 128)
        t_l = time.perf_counter() - t0
    est = t_h * (N / rs) + t_u * (n / ns) ** 3 + t_l * (o / os_) * (n / ns) ** 2
    return {
        "value": est, "unit": "s/layer", "cores": used, "kind": "oracle",
        "sample": (f"fp64 NumPy oracle: X^T X on {rs} of {N} rows (x{N / rs:.0f}), inv+Cholesky on a "
                   f"{ns}^2 block (x(n/{ns})^3), column loop on {os_} rows x {ns} columns (x rows, x(n/{ns})^2); "
                   f"measured {t_h:.2f}+{t_u:.2f}+{t_l:.2f} s"),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: the path here is the single-GPU kernel set (--gpus {args.gpus} "
              "is not supported: this build measures one GPU's share at its real shape)", file=sys.stderr)
        sys.exit(2)

    import torch
    import inputs
    from post_int4_weight_amd import api

    dev = torch.device("cuda:0")
    cfg = inputs.CONFIGS[args.workload]
    n, o, N = cfg.inp, cfg.out, cfg.rows
    g, block, bits = 128, 128, args.bits
    print(f"[bench] generating {args.workload}: W [{o}, {n}], X [{N}, {n}] {cfg.dtype}", file=sys.stderr, flush=True)
    W, X, _ = inputs.layer(cfg, device=dev)
    H = torch.empty(n, n, dtype=torch.float32, device=dev)
    d = torch.empty(n, dtype=torch.float64, device=dev)
    codes = torch.empty(o, n, dtype=torch.int8, device=dev)
    scales = torch.empty(o, (n + g - 1) // g, dtype=torch.float32, device=dev)
    g_idx = torch.empty(n, dtype=torch.int32, device=dev)
    perm = torch.empty(n, dtype=torch.int32, device=dev)
    ws_h = torch.empty(api.hessian_workspace_bytes(n, N), dtype=torch.uint8, device=dev)
    ws_g = torch.empty(api.gptq_workspace_bytes(o, n, block), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    def step():
        H.zero_()
        d.zero_()
        api.hessian_accumulate(H, d, X, workspace=ws_h)
        return api.gptq_quantize_layer(W, H, d, bits=bits, group_size=g, damp=0.01, act_order=False,
                                       block_size=block, codes=codes, scales=scales, g_idx=g_idx, perm=perm,
                                       workspace=ws_g)

    for i in range(args.warmup):
        step()
        print(f"[bench] warmup step {i + 1}/{args.warmup} done", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    api.profile_enable(["xtx_gemm"])
    t0 = time.perf_counter()
    for i in range(args.steps):
        res = step()
        print(f"[bench] timed step {i + 1}/{args.steps} done", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    xtx_ms, xtx_launches = api.profile_read("xtx_gemm")
    api.profile_enable([])

    # roofline of the dominant kernel: X^T X tiles, algorithmic flops = rows * n * (n + 1) per launch
    launches_per_step = max(1, xtx_launches // max(1, args.steps))
    rows_per_launch = N / launches_per_step
    flops_per_launch = rows_per_launch * n * (n + 1)
    avg_launch_s = xtx_ms / 1e3 / max(1, xtx_launches)
    # bf16 X: the direct kernel on 256-wide tiles (128-wide below in = 2048);
    # fp32 X goes through the fp32 GEMM, which this field does not cover
    if xtx_launches and n >= 2048:
        kname = "gemm_bf16_nt_direct_kernel<256, 0, 64, 2, 8, 16>"
    elif xtx_launches:
        kname = "gemm_bf16_nt_direct_kernel<128, 0, 64, 2, 4, 32>"
    else:
        kname = None
    achieved = flops_per_launch / avg_launch_s / 1e12 if xtx_launches else None
    roofline = {"bound": "mfma", "achieved": round(achieved, 2) if achieved else None, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4) if achieved else None,
                "traffic": measured_traffic() if args.workload == "llama70b_down_proj" else None,
                "kernel": f"{kname} (X^T X tiles, one launch per 65536-row chunk)" if kname else None,
                "avg_launch_ms": round(avg_launch_s * 1e3, 3) if xtx_launches else None, "launches": xtx_launches}

    breakdown = None
    if not args.no_breakdown:
        breakdown = stage_breakdown(api, torch, cfg, W, X, H, d, codes, scales, g_idx, perm, ws_h, ws_g, bits, g,
                                    block)

    line = {
        "metric": METRIC, "value": round(ms_per_step / 1e3, 4), "unit": "s/layer", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 2),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16+fp32",
        "data": "synthetic",
        "config": {"workload": f"{args.workload} W[{o},{n}] X[{N},{n}] {cfg.dtype}, {bits}-bit g={g} damp=0.01 "
                               f"block={block} natural order", "out": o, "in": n, "calib_rows": N, "bits": bits,
                   "group_size": g, "block_size": block},
        "roofline": roofline,
        "stages": breakdown,
        "stats": res["stats"],
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the fp64 oracle on a host sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(cfg, W, X, bits)
    print(json.dumps(line), flush=True)


def awq_stage(api, torch, dev):
    """AWQ's alpha search on the q/k/v-shaped layer (W [8192, 8192], its first
    4096 calibration rows, the 20-point grid): whole call and error-GEMM time.
    Algorithmic work 20 * 2 * rows * in * out flops; the error GEMM executes
    twice that (dW as a bf16 high part plus residual)."""
    import inputs
    cfg = inputs.CONFIGS["llama70b_qkv_proj"]
    Wq, Xq, _ = inputs.layer(cfg, device=dev, rows=inputs.AWQ_CAL_ROWS)
    alphas = list(inputs.AWQ_ALPHAS)
    ws = torch.empty(api.awq_workspace_bytes(cfg.out, cfg.inp, inputs.AWQ_CAL_ROWS, len(alphas)),
                     dtype=torch.uint8, device=dev)
    api.awq_search_alpha(Wq, Xq, alphas, bits=4, group_size=128, workspace=ws)   # warm
    api.profile_enable(["awq_gemm"])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    api.awq_search_alpha(Wq, Xq, alphas, bits=4, group_size=128, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 1e3
    ms, _ = api.profile_read("awq_gemm")
    api.profile_enable([])
    f = len(alphas) * 2.0 * inputs.AWQ_CAL_ROWS * cfg.inp * cfg.out
    return {"awq_qkv_s": round(t, 4), "awq_tflops": round(f / t / 1e12, 1), "awq_gemm_ms": round(ms, 3),
            "awq_gemm_frac_bf16_peak": round(2 * f / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def stage_breakdown(api, torch, cfg, W, X, H, d, codes, scales, g_idx, perm, ws_h, ws_g, bits, g, block):
    """One extra instrumented step: stage times from torch events on the current
    stream (the library launches on it), kernel-class totals from the library's
    own event records."""
    n, o, N = cfg.inp, cfg.out, cfg.rows
    U = torch.empty(n, n, dtype=torch.float32, device=X.device)
    fws = torch.empty(api.gptq_factor_workspace_bytes(n), dtype=torch.uint8, device=X.device)
    cws = torch.empty(api.gptq_columns_workspace_bytes(o, n, block), dtype=torch.uint8, device=X.device)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    api.profile_enable(list(api.PROFILE_KERNELS))
    H.zero_()
    d.zero_()
    ev[0].record()
    api.hessian_accumulate(H, d, X, workspace=ws_h)
    ev[1].record()
    api.gptq_inverse_factor(H, d, damp=0.01, act_order=False, U=U, workspace=fws)
    ev[2].record()
    api.gptq_quantize_columns(W, U, None, bits=bits, group_size=g, block_size=block, codes=codes, scales=scales,
                              g_idx=g_idx, workspace=cws)
    ev[3].record()
    torch.cuda.synchronize()
    # INT4 storage after the path (not part of the step): pack, then the
    # g_idx-aware dequantizer to bf16; both stream HBM
    packed = api.pack_int4(codes)
    What = torch.empty(o, n, dtype=torch.bfloat16, device=X.device)
    api.dequantize_int4(packed, scales, g_idx, n, group_size=g, What=What)
    ev2 = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev2[0].record()
    api.pack_int4(codes, packed=packed)
    ev2[1].record()
    api.dequantize_int4(packed, scales, g_idx, n, group_size=g, What=What)
    ev2[2].record()
    torch.cuda.synchronize()
    t_pack = ev2[0].elapsed_time(ev2[1]) / 1e3
    t_deq = ev2[1].elapsed_time(ev2[2]) / 1e3
    b_pack = o * n + o * n / 2
    b_deq = o * n / 2 + 4.0 * o * ((n + g - 1) // g) + 4.0 * n + 2.0 * o * n
    t_h = ev[0].elapsed_time(ev[1]) / 1e3
    t_u = ev[1].elapsed_time(ev[2]) / 1e3
    t_c = ev[2].elapsed_time(ev[3]) / 1e3
    kern = {}
    for k in api.PROFILE_KERNELS:
        ms, cnt = api.profile_read(k)
        if cnt:
            kern[k] = {"total_ms": round(ms, 3), "launches": cnt}
    api.profile_enable([])
    awq = awq_stage(api, torch, X.device)
    f_xtx = N * n * (n + 1)
    f_u = 2.0 * n ** 3 / 3.0
    nb = (n + block - 1) // block
    f_trail = sum(2.0 * o * min(block, n - b * block) * max(0, n - (b + 1) * block) for b in range(nb))
    loop_bytes = 9.0 * o * n + 4.0 * n * block
    out = {
        "hessian_s": round(t_h, 4), "factor_s": round(t_u, 4), "columns_s": round(t_c, 4),
        "xtx_tflops": round(f_xtx / t_h / 1e12, 1),
        "factor_tflops": round(f_u / t_u / 1e12, 2),
        "kernels": kern,
        "int4_pack_ms": round(t_pack * 1e3, 4), "int4_pack_frac_hbm": round(b_pack / t_pack / 1e9 / PEAK_HBM_GBS, 4),
        "int4_dequant_bf16_ms": round(t_deq * 1e3, 4),
        "int4_dequant_frac_hbm": round(b_deq / t_deq / 1e9 / PEAK_HBM_GBS, 4),
    }
    out.update(awq)
    if "xtx_gemm" in kern:
        out["xtx_kernel_frac_bf16_peak"] = round(f_xtx / (kern["xtx_gemm"]["total_ms"] / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4)
    # the large factor and trailing products run on the bf16 MFMA from three-term
    # operand splits: their rates are fp32-equivalent (algorithmic fp32 flops
    # over time), which can exceed the fp32 MFMA peak
    if "factor_gemm" in kern:
        out["factor_gemm_tflops_fp32_equiv"] = round(f_u / (kern["factor_gemm"]["total_ms"] / 1e3) / 1e12, 2)
    if "trail_gemm" in kern:
        out["trail_gemm_tflops_fp32_equiv"] = round(f_trail / (kern["trail_gemm"]["total_ms"] / 1e3) / 1e12, 2)
    if "block_loop" in kern:
        t = kern["block_loop"]["total_ms"] / 1e3
        out["block_loop_us_per_block"] = round(t / nb * 1e6, 2)
        out["block_loop_frac_hbm"] = round(loop_bytes / t / 1e9 / PEAK_HBM_GBS, 4)
    return out


if __name__ == "__main__":
    main()
