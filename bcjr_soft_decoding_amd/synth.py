"""Seeded synthetic inputs for the trellis workloads.

This module draws random numbers and shapes them; it holds none of the method's arithmetic.
It is the only code shared by the CPU oracle's tests and the GPU path's tests and benchmark.

The BCJR-QAT pages quantise LLM weight matrices (Llama-3.2-1B, OLMoE-1B-7B) to about 2 bits
per weight with a trellis code, but print neither a trellis shape nor any workload size, and
no weights are available offline. The workloads below stand in for those layers with Gaussian
matrices of the stated shapes; every row of a matrix is cut into independent length-L chains.
Generator: ``numpy.random.default_rng(seed).standard_normal(..., dtype=float32)`` with seeds
codebook 1000+i, w 2000+i, upstream gradient 3000+i, theta 4000+i, log-Z gradient 5000+i for
workload i.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    n: int            # state bits, S = 2^n
    k: int            # bits per step, K = 2^k successors
    B: int            # sequences
    L: int            # weights per sequence
    temps: tuple      # temperatures the workload is run at
    dense: bool = False
    matrix: tuple | None = None  # (rows, cols) of the weight matrix the chains are cut from
    w_std: float = 1.0
    unit_rms: bool = False
    notes: str = field(default="", compare=False)

    @property
    def S(self) -> int:
        return 1 << self.n


WORKLOADS = {
    1: Workload(1, "tiny-s16", 4, 2, 8, 64, (1.0, 0.3, 0.01),
                notes="S=16, k=2, 8 x 64; brute force on the first 8 steps"),
    2: Workload(2, "s256", 8, 2, 4096, 256, (0.5, 0.1, 0.01),
                notes="S=256, k=2, 4096 x 256, plus Viterbi"),
    3: Workload(3, "llama32-1b-mlp-up-s4096", 12, 2, 65536, 256, (0.1,), matrix=(2048, 8192),
                w_std=0.02, unit_rms=True,
                notes="2048x8192 N(0,0.02^2) rescaled to unit global RMS -> 65536 x 256, S=4096"),
    4: Workload(4, "qtip-s65536", 16, 2, 16384, 256, (0.3, 0.05), matrix=(2048, 2048),
                notes="2048x2048 N(0,1) -> 16384 x 256, S=65536"),
    5: Workload(5, "dense-s256", 8, 8, 1024, 1024, (0.2,), dense=True,
                notes="fully connected S=256, theta N(0,1) [256,256], 1024 x 1024"),
    6: Workload(6, "long-chain-s256", 8, 2, 1, 1 << 20, (0.1,), matrix=(1024, 1024),
                notes="a 1024x1024 N(0,1) matrix quantised as ONE chain of 2^20 steps, S=256; "
                      "the segmented (parallel-in-L) forward"),
}


def _normal(seed: int, shape) -> np.ndarray:
    return np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)


def codebook(i: int) -> np.ndarray:
    """Codebook LUT c(s) ~ N(0,1), fp32 [S]."""
    wl = WORKLOADS[i]
    return _normal(1000 + i, (wl.S,))


def weights(i: int) -> np.ndarray:
    """Weight chains w, fp32 [B, L] (row-major cut of the workload's weight matrix)."""
    wl = WORKLOADS[i]
    if wl.matrix is not None:
        m = _normal(2000 + i, wl.matrix)
        if wl.w_std != 1.0:
            m = (m * np.float32(wl.w_std)).astype(np.float32)
        if wl.unit_rms:
            rms = np.sqrt(np.mean(np.square(m.astype(np.float64))))
            m = (m.astype(np.float64) / rms).astype(np.float32)
        return np.ascontiguousarray(m.reshape(wl.B, wl.L))
    return _normal(2000 + i, (wl.B, wl.L))


def upstream_grad(i: int) -> np.ndarray:
    """Upstream gradient on the soft codeword, fp32 [B, L] ~ N(0,1)."""
    wl = WORKLOADS[i]
    return _normal(3000 + i, (wl.B, wl.L))


def theta(i: int) -> np.ndarray:
    """Dense transition log-potentials, fp32 [S, S] ~ N(0,1)."""
    wl = WORKLOADS[i]
    return _normal(4000 + i, (wl.S, wl.S))


def logz_grad(i: int) -> np.ndarray:
    """Upstream gradient on log Z, fp32 [B] ~ N(0,1) (used only where a test asks for it)."""
    wl = WORKLOADS[i]
    return _normal(5000 + i, (wl.B,))


def normal(seed: int, shape, scale: float = 1.0) -> np.ndarray:
    """Generic seeded N(0, scale^2) fp32 array for ad-hoc test shapes."""
    x = _normal(seed, shape)
    if scale != 1.0:
        x = (x * np.float32(scale)).astype(np.float32)
    return x


def qat_layer(rows: int, cols: int, samples: int, n: int, seed: int = 0):
    """One synthetic linear layer for the annealed-QAT driver, all fp32 numpy:
    float weights W [rows, cols] rescaled to unit RMS, calibration and held-out inputs
    X, Xv [samples, cols], codebook c [2^n] ~ N(0,1).

    Inputs carry per-channel scales exp(0.75 xi), xi ~ N(0,1): a log-normal spread like the
    outlier channels of LLM activations, so the output error weighs weights unequally.
    Seeds 9000+seed (W), 9100+seed (scales), 9200+seed (X), 9300+seed (Xv), 9400+seed (c)."""
    W = _normal(9000 + seed, (rows, cols)).astype(np.float64)
    W = (W / np.sqrt(np.mean(W * W))).astype(np.float32)
    scale = np.exp(0.75 * _normal(9100 + seed, (cols,)).astype(np.float64))
    X = (_normal(9200 + seed, (samples, cols)) * scale).astype(np.float32)
    Xv = (_normal(9300 + seed, (samples, cols)) * scale).astype(np.float32)
    c = _normal(9400 + seed, (1 << n,))
    return W, X, Xv, c
