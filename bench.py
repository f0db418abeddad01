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
instrumented step, the same measurements on the other layer shapes (the
8B q_proj with and without act-order, the 70B q/k/v projection, the
down_proj at 3 bits), AWQ's alpha search with the held-out RTN / AWQ / GPTQ
report, and the fp64 oracle timed on a bounded sample on the host.
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
G, BLOCK, SB_COLS = 128, 128, 2048   # group size, lazy block, lazy super-block of the column stage


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--bits", type=int, default=4)
    ap.add_argument("--workload", default="llama70b_down_proj")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-breakdown", action="store_true",
                    help="skip the instrumented step, the other layer shapes and the AWQ report")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="before the steps, run a copy-like elementwise kernel (torch.neg) over 1 GiB of fp32, "
                         "whose FETCH_SIZE / WRITE_SIZE counters calibrate the traffic figures")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


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


def host_threads() -> int:
    """Host threads for the oracle: every core of this process's affinity set,
    unless OMP_NUM_THREADS names a smaller share (a GPU host that allots a
    fixed CPU share per GPU sets it; the oracle then stays inside that share)."""
    cores = len(os.sched_getaffinity(0))
    try:
        share = int(os.environ.get("OMP_NUM_THREADS", "0"))
    except ValueError:
        share = 0
    return min(cores, share) if share > 0 else cores


def cpu_baseline(cfg, Xs, Ws, bits):
    """Time the fp64 oracle on a bounded sample of the same layer (host copies
    Xs = the first rows of X, Ws = a corner of W), scaled by exact operation
    counts to one whole layer."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits

    threads = host_threads()
    n, o, N = cfg.inp, cfg.out, cfg.rows
    rs, ns = Xs.shape[0], Ws.shape[1]
    os_ = Ws.shape[0]
    with threadpool_limits(limits=threads):
        used = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        t0 = time.perf_counter()
        H0, d = oracle.proxy_hessian(Xs)
        t_h = time.perf_counter() - t0
        Hs, _ = oracle.damped(H0[:ns, :ns], 0.01)
        t0 = time.perf_counter()
        U = oracle.inverse_upper_factor(Hs)
        t_u = time.perf_counter() - t0
        t0 = time.perf_counter()
        oracle.gptq_columns(Ws, U, bits, G)
        t_l = time.perf_counter() - t0
    est = t_h * (N / rs) + t_u * (n / ns) ** 3 + t_l * (o / os_) * (n / ns) ** 2
    return {
        "value": est, "unit": "s/layer", "cores": used, "kind": "oracle",
        "sample": (f"fp64 NumPy/LAPACK oracle on {used} host threads (affinity {len(os.sched_getaffinity(0))} cores, "
                   f"OMP_NUM_THREADS={os.environ.get('OMP_NUM_THREADS', 'unset')}): X^T X on {rs} of {N} rows "
                   f"(x{N / rs:.0f}), U (reversed Cholesky + triangular inverse) on a {ns}^2 block (x(n/{ns})^3), "
                   f"column loop on {os_} rows x {ns} columns (x rows, x(n/{ns})^2); measured "
                   f"{t_h:.2f}+{t_u:.2f}+{t_l:.2f} s"),
    }


# ------------------------------------------------------------ flop counts ---

def flops_xtx(N, n):
    return N * n * (n + 1)                       # one triangle, N rows


def flops_factor(n):
    return 2.0 * n ** 3 / 3.0                     # n^3/3 Cholesky + n^3/3 triangular inverse


def flops_updates(o, n):
    """Block-update flops of the column stage, split into the updates inside
    a 2048-column super-block and the GEMMs past it (same sums, two levels)."""
    inner = past = 0.0
    for s0 in range(0, n, SB_COLS):
        s1 = min(n, s0 + SB_COLS)
        for b0 in range(s0, s1, BLOCK):
            b1 = min(s1, b0 + BLOCK)
            inner += 2.0 * o * (b1 - b0) * (s1 - b1)
        past += 2.0 * o * (s1 - s0) * (n - s1)
    return inner, past


def loop_bytes(o, n):
    return 9.0 * o * n + 4.0 * n * BLOCK


# ----------------------------------------------------------- measurement ---

class Layer:
    """Device buffers of one layer shape and its timed step."""

    def __init__(self, api, torch, cfg, W, X, bits, act_order):
        self.api, self.torch, self.cfg = api, torch, cfg
        self.W, self.X, self.bits, self.act_order = W, X, bits, act_order
        n, o, N = cfg.inp, cfg.out, X.shape[0]
        dev = X.device
        self.H = torch.empty(n, n, dtype=torch.float32, device=dev)
        self.d = torch.empty(n, dtype=torch.float64, device=dev)
        self.codes = torch.empty(o, n, dtype=torch.int8, device=dev)
        self.scales = torch.empty(o, (n + G - 1) // G, dtype=torch.float32, device=dev)
        self.g_idx = torch.empty(n, dtype=torch.int32, device=dev)
        self.perm = torch.empty(n, dtype=torch.int32, device=dev)
        self.ws_h = torch.empty(api.hessian_workspace_bytes(n, N), dtype=torch.uint8, device=dev)
        self.ws_g = torch.empty(api.gptq_workspace_bytes(o, n, BLOCK), dtype=torch.uint8, device=dev)

    def step(self, bits=None):
        api = self.api
        self.H.zero_()
        self.d.zero_()
        api.hessian_accumulate(self.H, self.d, self.X, workspace=self.ws_h)
        return api.gptq_quantize_layer(self.W, self.H, self.d, bits=bits or self.bits, group_size=G, damp=0.01,
                                       act_order=self.act_order, block_size=BLOCK, codes=self.codes,
                                       scales=self.scales, g_idx=self.g_idx, perm=self.perm, workspace=self.ws_g)

    def timed(self, steps, warmup, label):
        torch = self.torch
        for i in range(warmup):
            self.step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            res = self.step()
        torch.cuda.synchronize()
        t = (time.perf_counter() - t0) / steps
        log(f"{label}: {steps} steps, {t * 1e3:.2f} ms/layer")
        return t, res

    def breakdown(self):
        """Two extra steps: stage times from torch events on the current stream
        (the library launches on it) in a step without per-kernel records, then
        kernel-class totals and executed MFMA flops from the library's own
        event records in a second, instrumented step (its hundreds of event
        pairs around small launches would lengthen the stages)."""
        api, torch, cfg = self.api, self.torch, self.cfg
        n, o, N = cfg.inp, cfg.out, self.X.shape[0]
        dev = self.X.device
        U = torch.empty(n, n, dtype=torch.float32, device=dev)
        fws = torch.empty(api.gptq_factor_workspace_bytes(n), dtype=torch.uint8, device=dev)
        cws = torch.empty(api.gptq_columns_workspace_bytes(o, n, BLOCK), dtype=torch.uint8, device=dev)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        kern = {}

        def collect(classes):
            for k in classes:
                ms, cnt = api.profile_read(k)
                if cnt:
                    kern.setdefault(k, {"total_ms": 0.0, "launches": 0, "mfma_flops": 0.0, "by_stage": {}})
                    e = kern[k]
                    e["total_ms"] += ms
                    e["launches"] += cnt
                    e["mfma_flops"] += api.profile_flops(k)

        api.profile_enable([])
        self.H.zero_()
        self.d.zero_()
        ev[0].record()
        api.hessian_accumulate(self.H, self.d, self.X, workspace=self.ws_h)
        ev[1].record()
        api.gptq_inverse_factor(self.H, self.d, damp=0.01, act_order=self.act_order, U=U, perm=self.perm,
                                workspace=fws)
        ev[2].record()
        api.gptq_quantize_columns(self.W, U, self.perm if self.act_order else None, bits=self.bits, group_size=G,
                                  block_size=BLOCK, codes=self.codes, scales=self.scales, g_idx=self.g_idx,
                                  workspace=cws)
        ev[3].record()
        torch.cuda.synchronize()
        t_h = ev[0].elapsed_time(ev[1]) / 1e3
        t_u = ev[1].elapsed_time(ev[2]) / 1e3
        t_c = ev[2].elapsed_time(ev[3]) / 1e3

        self.H.zero_()
        self.d.zero_()
        api.profile_enable(list(api.PROFILE_KERNELS))
        ev[0].record()
        api.hessian_accumulate(self.H, self.d, self.X, workspace=self.ws_h)
        ev[1].record()
        api.gptq_inverse_factor(self.H, self.d, damp=0.01, act_order=self.act_order, U=U, perm=self.perm,
                                workspace=fws)
        ev[2].record()
        torch.cuda.synchronize()
        collect(["xtx_gemm", "factor_gemm", "factor_base"])
        split_factor = (api.profile_read("split3_gemm")[0], api.profile_flops("split3_gemm"))
        api.profile_enable(list(api.PROFILE_KERNELS))
        ev[2].record()
        api.gptq_quantize_columns(self.W, U, self.perm if self.act_order else None, bits=self.bits, group_size=G,
                                  block_size=BLOCK, codes=self.codes, scales=self.scales, g_idx=self.g_idx,
                                  workspace=cws)
        ev[3].record()
        torch.cuda.synchronize()
        collect(["block_loop", "trail_gemm", "inner_gemm"])
        split_cols = (api.profile_read("split3_gemm")[0], api.profile_flops("split3_gemm"))
        api.profile_enable([])
        for e in kern.values():
            e["total_ms"] = round(e["total_ms"], 3)
            if not e["mfma_flops"]:
                del e["mfma_flops"]
            del e["by_stage"]
        f_xtx, f_u = flops_xtx(N, n), flops_factor(n)
        f_inner, f_past = flops_updates(o, n)
        nb = (n + BLOCK - 1) // BLOCK
        out = {
            "hessian_s": round(t_h, 5), "factor_s": round(t_u, 5), "columns_s": round(t_c, 5),
            "xtx_tflops": round(f_xtx / t_h / 1e12, 1),
            "xtx_frac_bf16_peak": round(f_xtx / t_h / 1e12 / PEAK_BF16_TFLOPS, 4),
            "factor_tflops_fp32_equiv": round(f_u / t_u / 1e12, 2),
            "factor_frac_fp32_peak": round(f_u / t_u / 1e12 / PEAK_FP32_TFLOPS, 4),
            "block_update_tflops_fp32_equiv": None, "block_update_frac_fp32_peak": None,
            "kernels": kern,
        }
        if "xtx_gemm" in kern:
            t = kern["xtx_gemm"]["total_ms"] / 1e3
            out["xtx_kernel_tflops"] = round(f_xtx / t / 1e12, 1)
            out["xtx_kernel_frac_bf16_peak"] = round(f_xtx / t / 1e12 / PEAK_BF16_TFLOPS, 4)
        # the split-operand GEMMs execute six bf16 MFMA term products per fp32
        # product: fp32-equivalent rates (algorithmic fp32 flops over time) can
        # exceed the fp32 MFMA peak, so their executed bf16 fraction goes beside
        for tag, (ms, fl) in (("factor", split_factor), ("columns", split_cols)):
            if ms > 0:
                out[f"{tag}_split3_ms"] = round(ms, 3)
                out[f"{tag}_split3_frac_bf16_peak_executed"] = round(fl / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4)
        if "factor_gemm" in kern:
            t = kern["factor_gemm"]["total_ms"] / 1e3
            out["factor_gemm_tflops_fp32_equiv"] = round(f_u / t / 1e12, 2)
        t_tr = kern.get("trail_gemm", {}).get("total_ms", 0.0) / 1e3
        t_in = kern.get("inner_gemm", {}).get("total_ms", 0.0) / 1e3
        if t_tr + t_in > 0:
            r = (f_inner + f_past) / (t_tr + t_in) / 1e12
            out["block_update_tflops_fp32_equiv"] = round(r, 2)
            out["block_update_frac_fp32_peak"] = round(r / PEAK_FP32_TFLOPS, 4)
        if t_tr > 0:
            out["trail_gemm_tflops_fp32_equiv"] = round(f_past / t_tr / 1e12, 2)
        if t_in > 0:
            out["inner_gemm_tflops"] = round(f_inner / t_in / 1e12, 2)
            out["inner_gemm_frac_fp32_peak"] = round(f_inner / t_in / 1e12 / PEAK_FP32_TFLOPS, 4)
        if "block_loop" in kern:
            t = kern["block_loop"]["total_ms"] / 1e3
            out["block_loop_us_per_block"] = round(t / nb * 1e6, 2)
            out["block_loop_frac_hbm"] = round(loop_bytes(o, n) / t / 1e9 / PEAK_HBM_GBS, 4)
        return out


def int4_storage(api, torch, lay):
    """INT4 storage after the path (not part of the step): pack, then the
    g_idx-aware dequantizer to bf16; both stream HBM."""
    o, n = lay.cfg.out, lay.cfg.inp
    packed = api.pack_int4(lay.codes)
    What = torch.empty(o, n, dtype=torch.bfloat16, device=lay.X.device)
    api.dequantize_int4(packed, lay.scales, lay.g_idx, n, group_size=G, What=What)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record()
    api.pack_int4(lay.codes, packed=packed)
    ev[1].record()
    api.dequantize_int4(packed, lay.scales, lay.g_idx, n, group_size=G, What=What)
    ev[2].record()
    torch.cuda.synchronize()
    t_pack = ev[0].elapsed_time(ev[1]) / 1e3
    t_deq = ev[1].elapsed_time(ev[2]) / 1e3
    b_pack = o * n + o * n / 2
    b_deq = o * n / 2 + 4.0 * o * ((n + G - 1) // G) + 4.0 * n + 2.0 * o * n
    return {"int4_pack_ms": round(t_pack * 1e3, 4), "int4_pack_frac_hbm": round(b_pack / t_pack / 1e9 / PEAK_HBM_GBS, 4),
            "int4_dequant_bf16_ms": round(t_deq * 1e3, 4),
            "int4_dequant_frac_hbm": round(b_deq / t_deq / 1e9 / PEAK_HBM_GBS, 4)}


def other_configs(api, torch, dev):
    """The other layer shapes, each timed as whole steps plus one instrumented
    step: the 8B q_proj with and without act-order, the 70B q/k/v projection.
    Returns (results, the q/k/v layer kept for the AWQ report)."""
    import inputs
    res = {}
    keep = None
    for key, act, steps, warm in (("llama8b_q_proj", False, 10, 2), ("llama8b_q_proj", True, 10, 2),
                                  ("llama70b_qkv_proj", False, 5, 1)):
        cfg = inputs.CONFIGS[key]
        name = key + ("_act_order" if act else "")
        log(f"generating {name}: W [{cfg.out}, {cfg.inp}], X [{cfg.rows}, {cfg.inp}] {cfg.dtype}")
        W, X, _ = inputs.layer(cfg, device=dev)
        lay = Layer(api, torch, cfg, W, X, 4, act)
        t, r = lay.timed(steps, warm, name)
        res[name] = {"workload": f"{key} W[{cfg.out},{cfg.inp}] X[{cfg.rows},{cfg.inp}] {cfg.dtype}, 4-bit g={G} "
                                 f"damp=0.01 block={BLOCK} " + ("act-order" if act else "natural order"),
                     "s_per_layer": round(t, 5), "steps": steps, "warmup": warm,
                     "stages": lay.breakdown(), "stats": r["stats"]}
        if key == "llama70b_qkv_proj":
            keep = lay
        del lay, W, X
        torch.cuda.empty_cache()
    return res, keep


def awq_report(api, torch, qkv):
    """AWQ's 20-point alpha search on the q/k/v layer's first 4096 calibration
    rows (call time, error-GEMM time and executed fraction), then the
    held-out report: RTN, AWQ at the searched alpha, GPTQ calibrated on the
    same 4096 rows and GPTQ calibrated on all 262144 rows, each as relative
    output error ||X dW^T||^2 / ||X W^T||^2 and output MSE on the calibration
    rows and on 4096 held-out rows whose channel sigma is redrawn."""
    import inputs
    cfg = qkv.cfg
    W = qkv.W
    n, o = cfg.inp, cfg.out
    rows = inputs.AWQ_CAL_ROWS
    Xc = qkv.X[:rows]
    alphas = list(inputs.AWQ_ALPHAS)
    ws = torch.empty(api.awq_workspace_bytes(o, n, rows, len(alphas)), dtype=torch.uint8, device=W.device)
    api.awq_search_alpha(W, Xc, alphas, bits=4, group_size=G, workspace=ws)   # warm
    api.profile_enable(["awq_gemm"])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    aw = api.awq_search_alpha(W, Xc, alphas, bits=4, group_size=G, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 1e3
    ms, _ = api.profile_read("awq_gemm")
    fl = api.profile_flops("awq_gemm")
    api.profile_enable([])
    f = len(alphas) * 2.0 * rows * n * o
    out = {"workload": f"llama70b_qkv_proj W[{o},{n}], first {rows} calibration rows, {len(alphas)} alphas "
                       f"{alphas[0]}..{alphas[-1]}, 4-bit g={G}",
           "awq_call_s": round(t, 5), "awq_tflops": round(f / t / 1e12, 1), "awq_gemm_ms": round(ms, 3),
           "awq_gemm_frac_bf16_peak_executed": round(fl / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
           "alpha": round(aw["alpha"], 4), "err_per_alpha": [float(e) for e in aw["errors"]]}
    log(f"AWQ search: alpha {aw['alpha']:.2f}, {t * 1e3:.2f} ms")

    rt = api.awq_search_alpha(W, Xc, [0.0], bits=4, group_size=G)
    Hc = torch.zeros(n, n, dtype=torch.float32, device=W.device)
    dc = torch.zeros(n, dtype=torch.float64, device=W.device)
    api.hessian_accumulate(Hc, dc, Xc)
    g_small = api.gptq_quantize_layer(W, Hc, dc, bits=4, group_size=G)
    g_full = api.gptq_quantize_layer(W, qkv.H, qkv.d, bits=4, group_size=G)
    Xh = inputs.awq_heldout(rows, device=W.device)
    methods = {"RTN": (rt["codes"], rt["scales"], None, rt["s"]),
               f"AWQ (alpha {aw['alpha']:.2f})": (aw["codes"], aw["scales"], None, aw["s"]),
               f"GPTQ ({rows} rows)": (g_small["codes"], g_small["scales"], g_small["g_idx"], None),
               f"GPTQ ({cfg.rows} rows)": (g_full["codes"], g_full["scales"], g_full["g_idx"], None)}
    table = {}
    for sname, Xs in (("calibration", Xc), ("held-out, sigma redrawn", Xh)):
        table[sname] = {}
        for m, (c, s, gi, sv) in methods.items():
            err, energy = api.layer_output_error(Xs, W, c, s, g_idx=gi, s=sv, group_size=G)
            table[sname][m] = {"relative": round(err / energy, 7), "mse": err / (Xs.shape[0] * o)}
    out["heldout_table"] = table
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: the path here is the single-GPU kernel set (--gpus {args.gpus} "
              "is not supported: it measures one GPU's share of the work at its real shape)", file=sys.stderr)
        sys.exit(2)

    import torch
    import inputs
    from post_int4_weight_amd import api

    dev = torch.device("cuda:0")
    cfg = inputs.CONFIGS[args.workload]
    n, o, N = cfg.inp, cfg.out, cfg.rows
    bits = args.bits
    log(f"generating {args.workload}: W [{o}, {n}], X [{N}, {n}] {cfg.dtype}")
    W, X, _ = inputs.layer(cfg, device=dev)
    lay = Layer(api, torch, cfg, W, X, bits, False)
    torch.cuda.synchronize()
    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    for i in range(args.warmup):
        lay.step()
        log(f"warmup step {i + 1}/{args.warmup} done")
    torch.cuda.synchronize()
    api.profile_enable(["xtx_gemm"])
    t0 = time.perf_counter()
    for i in range(args.steps):
        res = lay.step()
        log(f"timed step {i + 1}/{args.steps} done")
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

    line = {
        "metric": METRIC, "value": round(ms_per_step / 1e3, 4), "unit": "s/layer", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 2),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16+fp32",
        "data": "synthetic",
        "config": {"workload": f"{args.workload} W[{o},{n}] X[{N},{n}] {cfg.dtype}, {bits}-bit g={G} damp=0.01 "
                               f"block={BLOCK} natural order", "out": o, "in": n, "calib_rows": N, "bits": bits,
                   "group_size": G, "block_size": BLOCK},
        "roofline": roofline,
        "stats": res["stats"],
    }
    # host copies for the CPU baseline before the large buffers go
    Xs = Ws = None
    if not args.no_cpu_baseline:
        Xs = X[:1024].float().cpu().numpy().astype("float64")
        Ws = W[:32, :4096].float().cpu().numpy().astype("float64")

    if not args.no_breakdown:
        stages = lay.breakdown()
        stages.update(int4_storage(api, torch, lay))
        line["stages"] = stages
        other = 3 if bits == 4 else 4
        lay.bits = other
        t, r = lay.timed(3, 1, f"{args.workload} {other}-bit")
        cfgs = {f"{args.workload}_{other}bit": {
            "workload": f"{args.workload} W[{o},{n}] X[{N},{n}] {cfg.dtype}, {other}-bit g={G} damp=0.01 "
                        f"block={BLOCK} natural order",
            "s_per_layer": round(t, 5), "steps": 3, "warmup": 1, "stages": lay.breakdown(), "stats": r["stats"]}}
        del lay, W, X
        torch.cuda.empty_cache()
        more, qkv = other_configs(api, torch, dev)
        cfgs.update(more)
        line["configs"] = cfgs
        line["awq"] = awq_report(api, torch, qkv)
        del qkv
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on a host sample")
        line["cpu_baseline"] = cpu_baseline(cfg, Xs, Ws, bits)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
