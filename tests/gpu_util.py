"""Helpers shared by the GPU parity tests (no quantization arithmetic here)."""
import sys

import numpy as np
import torch


_CONFIG = None   # pytest's config, set by conftest.py


def set_config(config) -> None:
    global _CONFIG
    _CONFIG = config


def progress(msg: str, flush: bool = True) -> None:
    """Print past pytest's output capture, flushed: the long host-side oracle
    steps of the full-size tests report as they go (a run that prints nothing
    for minutes cannot be told from a hung one), and a failing run names its
    case."""
    capman = _CONFIG.pluginmanager.getplugin("capturemanager") if _CONFIG is not None else None
    if capman is not None:
        with capman.global_and_fixture_disabled():
            print(msg, flush=True)
    else:
        print(msg, flush=True)
    sys.stdout.flush()


def announce(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a failing run says which."""
    progress(f"[gpu-case] {msg}")


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_fro(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def code_match(a, b) -> float:
    return float(np.mean(np.asarray(a) == np.asarray(b)))


def zeros_h(n: int, device):
    return (torch.zeros(n, n, dtype=torch.float32, device=device),
            torch.zeros(n, dtype=torch.float64, device=device))


def relative_output_error(H0, W, What) -> float:
    """tr(dW H0 dW^T) / tr(W H0 W^T) (= ||X dW^T||^2 / ||X W^T||^2)."""
    W = np.asarray(W, dtype=np.float64)
    dW = W - np.asarray(What, dtype=np.float64)
    H0 = np.asarray(H0, dtype=np.float64)
    return float(np.sum((dW @ H0) * dW) / np.sum((W @ H0) * W))


def dequant(codes, scales, g_idx) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.float64)
    return codes * np.asarray(scales, dtype=np.float64)[:, np.asarray(g_idx, dtype=np.int64)]
