"""Seeded synthetic layers shaped like the pages' Llama projections.

This module holds random draws only: no quantization arithmetic. It is the one
piece of code that both the fp64 oracle (``oracle/``) and the HIP path
(``post_int4_weight_amd``) are fed from; nothing else is shared between them.

Recipe (the pages give the layer shapes, not the data; see "GPTQ versus AWQ
objectives", "A strong answer", Hessian sizing for Llama 3.3 70B):

* per input channel j, sigma_j ~ LogNormal(0, 1); a set of round(frac * in)
  channels, drawn without replacement, has sigma multiplied by ``outlier_mult``
  (salient channels);
* W[out, in] ~ N(0, 1/in), i.e. std 1/sqrt(in);
* X[rows, in] has X[i, j] = sigma_j * z_ij, z ~ N(0, 1) i.i.d.; with
  ``zero_frac`` > 0 each entry is zeroed independently with that probability
  (post-activation sparsity);
* fp32 -> bf16 by round-to-nearest-even (torch's cast).

X is drawn in 2048-row chunks, each from its own generator seeded by
(seed, chunk index), so any row range can be regenerated on its own and large
calibration sets can be produced on the GPU without a host copy.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch

CHUNK_ROWS = 2048


@dataclass(frozen=True)
class LayerConfig:
    name: str
    out: int
    inp: int
    rows: int
    dtype: str            # "f32" or "bf16" for both W and X
    seed: int
    outlier_frac: float
    outlier_mult: float
    zero_frac: float = 0.0


CONFIGS = {
    # 256 x 512 tiny layer, fp32, 1% x20 outliers, seed 0
    "tiny": LayerConfig("tiny", 256, 512, 2048, "f32", 0, 0.01, 20.0),
    # Llama-8B-shaped q_proj: 16 seqs x 2048 tokens
    "llama8b_q_proj": LayerConfig("llama8b_q_proj", 4096, 4096, 32768, "bf16", 1, 0.01, 20.0),
    # Llama-70B-shaped q/k/v_proj: 128 x 2048 tokens, 0.5% x50 outliers
    "llama70b_qkv_proj": LayerConfig("llama70b_qkv_proj", 8192, 8192, 262144, "bf16", 2, 0.005, 50.0),
    # Llama-70B-shaped down_proj: 60% of activations zeroed
    "llama70b_down_proj": LayerConfig("llama70b_down_proj", 8192, 28672, 262144, "bf16", 3, 0.0, 1.0, 0.6),
}

# AWQ alpha search: config "llama70b_qkv_proj"'s W, its first 4096 calibration
# rows, and a held-out set whose channel sigma is redrawn with this seed.
AWQ_CAL_ROWS = 4096
AWQ_HELDOUT_SEED = 4
AWQ_ALPHAS = tuple(round(0.05 * i, 2) for i in range(20))


def _torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def channel_sigma(inp: int, seed: int, outlier_frac: float, outlier_mult: float) -> np.ndarray:
    """Per-channel activation scale sigma [inp] (float64)."""
    rng = np.random.default_rng([seed, 0])
    sigma = rng.lognormal(0.0, 1.0, inp)
    k = int(round(outlier_frac * inp))
    if k > 0:
        idx = rng.choice(inp, size=k, replace=False)
        sigma[idx] *= outlier_mult
    return sigma


def weights(out: int, inp: int, seed: int, dtype: str = "bf16", device="cpu") -> torch.Tensor:
    """W [out, inp] ~ N(0, 1/inp), drawn on the CPU (reproducible everywhere)."""
    g = torch.Generator(device="cpu").manual_seed(seed * 7919 + 17)
    w = torch.randn(out, inp, generator=g, dtype=torch.float32) * (1.0 / math.sqrt(inp))
    return w.to(_torch_dtype(dtype)).to(device)


def activations(rows: int, sigma: np.ndarray, seed: int, dtype: str = "bf16", device="cpu",
                zero_frac: float = 0.0, row0: int = 0, out: torch.Tensor | None = None) -> torch.Tensor:
    """X [rows, inp] with X[i, j] = sigma_j z_ij, drawn chunk by chunk on ``device``.

    ``row0`` must be a multiple of CHUNK_ROWS; rows [row0, row0 + rows) of the
    same (sigma, seed) stream are produced. Values differ between a CPU and a
    GPU draw (different generators); a test that compares two implementations
    draws once and copies.
    """
    if row0 % CHUNK_ROWS:
        raise ValueError("row0 must be a multiple of CHUNK_ROWS")
    inp = sigma.shape[0]
    dev = torch.device(device)
    sig = torch.tensor(sigma, dtype=torch.float32, device=dev)
    if out is None:
        out = torch.empty(rows, inp, dtype=_torch_dtype(dtype), device=dev)
    c0 = row0 // CHUNK_ROWS
    for c in range((rows + CHUNK_ROWS - 1) // CHUNK_ROWS):
        r = c * CHUNK_ROWS
        nr = min(CHUNK_ROWS, rows - r)
        g = torch.Generator(device=dev).manual_seed((seed + 1) * 1_000_003 + c0 + c)
        z = torch.randn(CHUNK_ROWS, inp, generator=g, dtype=torch.float32, device=dev)
        if zero_frac > 0.0:
            keep = torch.rand(CHUNK_ROWS, inp, generator=g, dtype=torch.float32, device=dev) >= zero_frac
            z = z * keep
        z = z * sig
        out[r:r + nr].copy_(z[:nr])
    return out


def layer(cfg: LayerConfig | str, device="cpu", rows: int | None = None):
    """(W, X, sigma) for a named config; ``rows`` truncates the calibration set."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    sigma = channel_sigma(cfg.inp, cfg.seed, cfg.outlier_frac, cfg.outlier_mult)
    W = weights(cfg.out, cfg.inp, cfg.seed, cfg.dtype, device)
    X = activations(cfg.rows if rows is None else rows, sigma, cfg.seed, cfg.dtype, device, cfg.zero_frac)
    return W, X, sigma


def awq_heldout(rows: int = AWQ_CAL_ROWS, device="cpu") -> torch.Tensor:
    """Held-out activations for the AWQ config: sigma and outlier set redrawn."""
    base = CONFIGS["llama70b_qkv_proj"]
    sigma = channel_sigma(base.inp, AWQ_HELDOUT_SEED, base.outlier_frac, base.outlier_mult)
    return activations(rows, sigma, AWQ_HELDOUT_SEED, base.dtype, device)


def custom(out: int, inp: int, rows: int, seed: int, dtype: str = "f32", device="cpu",
           outlier_frac: float = 0.01, outlier_mult: float = 20.0, zero_frac: float = 0.0):
    """(W, X) of an arbitrary shape with the same recipe (edge-case tests)."""
    sigma = channel_sigma(inp, seed, outlier_frac, outlier_mult)
    W = weights(out, inp, seed, dtype, device)
    X = activations(rows, sigma, seed, dtype, device, zero_frac)
    return W, X


# Toy layer of "GPTQ versus AWQ objectives" ("A strong answer", the table of
# output MSE under a distribution shift): 256 inputs, 128 outputs, correlated
# Gaussian inputs with four outlier channels; a calibration sample, a fresh
# sample of the same distribution, and one whose outliers moved to four other
# channels. The page gives no mixing or outlier strength: here x = z M with
# M = I + 0.5 G / 16 (G standard normal, fixed), outlier channels x10.
TOY_IN, TOY_OUT, TOY_ROWS = 256, 128, 2048
TOY_OUTLIER_MULT = 10.0
TOY_SEED = 11


def toy_layer(device="cpu"):
    """(W [128, 256], X_cal, X_same, X_moved) in float32, drawn on the CPU."""
    rng = np.random.default_rng([TOY_SEED, 0])
    mix = np.eye(TOY_IN) + 0.5 * rng.standard_normal((TOY_IN, TOY_IN)) / math.sqrt(TOY_IN)
    W = rng.standard_normal((TOY_OUT, TOY_IN)) / math.sqrt(TOY_IN)
    ch = rng.choice(TOY_IN, size=8, replace=False)
    ch_cal, ch_moved = ch[:4], ch[4:]

    def sample(stream, channels):
        z = np.random.default_rng([TOY_SEED, stream]).standard_normal((TOY_ROWS, TOY_IN))
        x = z @ mix
        x[:, channels] *= TOY_OUTLIER_MULT
        return torch.tensor(x, dtype=torch.float32, device=device)

    return (torch.tensor(W, dtype=torch.float32, device=device), sample(1, ch_cal), sample(2, ch_cal),
            sample(3, ch_moved))
