"""Annealed quantisation-aware training of one linear layer through the soft trellis quantiser.

The loop the method exists for (BCJR-QAT abstract; technical summary, core mechanism and
annealing): the layer's latent weights w are replaced in the forward pass by the soft codeword
w_hat(w; T), the loss is back-propagated through the exact forward-backward gradient, and T is
annealed from T0 towards a small T_end so that the soft codeword crystallises into the hard
(Viterbi) code. The pages' schedule fix (Skip-High-T) starts at T0 = 0.3 rather than 1.0; their
drift-budget condition says the latent weights can leave the PTQ Voronoi basin only when the
cumulative drift eta * N * g_max (step size, number of steps, largest gradient entry) exceeds the
basin radius r_Voronoi, about 1e-3.

Objective (the pages train against end-to-end distillation; no model or data exists here, so
this is the per-layer reconstruction objective on synthetic calibration inputs): with X the
[N, C] inputs of a layer whose float weights are W [R, C],

    loss(w) = || X (w_hat(w) - W)^T ||_F^2 / N,

the squared output error per calibration sample, whose gradient per weight does not shrink
with the layer's size (reports also give it per weight, divided by R C). The layer is cut row-major into trellis chains of L weights; the
optimiser is plain SGD, so every coordinate moves by at most eta * g_max per step. All trellis
work runs in the HIP kernels (``autograd.soft_quantize`` and ``bcjr.viterbi_decode``); torch
supplies the two matmuls of the loss and its gradient.

    python -m bcjr_soft_decoding_amd.qat --rows 2048 --cols 8192 --n 12 --steps 100 --t0 0.3
"""
from __future__ import annotations

import argparse
import json
import time
from dataclasses import dataclass, field

import numpy as np
import torch

from . import autograd, bcjr, synth


@dataclass
class QATConfig:
    n: int = 8             # state bits (S = 2^n)
    k: int = 2             # bits per step (K = 2^k)
    L: int = 256           # weights per chain
    t0: float = 0.3        # initial temperature (Skip-High-T); 1.0 is the naive schedule
    t_end: float = 0.01    # final temperature
    steps: int = 100
    lr: float = 1e-4       # SGD step size eta
    r_voronoi: float = 1e-3
    segmented: bool = False  # parallel-in-L entry points (for long chains, e.g. L = a whole row)

    def check(self):
        if self.steps < 1 or self.L < 1:
            raise ValueError("steps and L must be positive")
        if not (self.t0 > 0 and self.t_end > 0):
            raise ValueError("temperatures must be positive")
        if not bcjr.bcjr_supported(self.n, self.k):
            raise ValueError(f"trellis n={self.n}, k={self.k} is not built")


@dataclass
class QATResult:
    w: torch.Tensor               # trained latent weights [R, C]
    history: list = field(default_factory=list)
    g_max: float = 0.0            # largest |dloss/dw| entry over all steps
    drift_inf: float = 0.0        # max |w - W| after training
    seconds: float = 0.0

    def budget(self, cfg: QATConfig) -> float:
        """eta * N * g_max: an upper bound on drift_inf under SGD."""
        return cfg.lr * cfg.steps * self.g_max


def temperature(cfg: QATConfig, i: int) -> float:
    """Geometric anneal: t0 at step 0, t_end at the last step."""
    if cfg.steps <= 1:
        return cfg.t0
    return cfg.t0 * (cfg.t_end / cfg.t0) ** (i / (cfg.steps - 1))


def recon_loss(w_q, W, X):
    """||X (w_q - W)^T||_F^2 / N for quantised weights w_q [R, C]."""
    d = X @ (w_q - W).t()
    return (d * d).sum() / X.shape[0]


def step(w, W, X, codebook, cfg: QATConfig, T: float):
    """Loss and dloss/dw at the current latent weights (no update)."""
    R, C = W.shape
    wv = w.detach().requires_grad_(True)
    w_hat, _ = autograd.soft_quantize(wv.reshape(-1, cfg.L), codebook, cfg.n, cfg.k, T,
                                      segmented=cfg.segmented)
    loss = recon_loss(w_hat.reshape(R, C), W, X)
    grad, = torch.autograd.grad(loss, wv)
    return loss.detach(), grad


def train(W, X, codebook, cfg: QATConfig, log_every: int = 0) -> QATResult:
    """SGD on the latent weights from w = W through the annealed schedule."""
    cfg.check()
    R, C = W.shape
    if (R * C) % cfg.L:
        raise ValueError("the layer must cut into whole chains of L weights")
    for t, name in ((W, "W"), (X, "X"), (codebook, "codebook")):
        if t.dtype != torch.float32 or not t.is_cuda:
            raise TypeError(f"{name} must be an fp32 CUDA tensor")
    w = W.clone()
    res = QATResult(w=w)
    g_max = torch.zeros((), dtype=torch.float32, device=W.device)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(cfg.steps):
        T = temperature(cfg, i)
        loss, grad = step(w, W, X, codebook, cfg, T)
        g_i = grad.abs().max()
        g_max = torch.maximum(g_max, g_i)
        w.sub_(cfg.lr * grad)
        if log_every and (i % log_every == 0 or i == cfg.steps - 1):
            res.history.append({"step": i, "T": T, "soft_loss": float(loss), "g_max": float(g_i)})
    torch.cuda.synchronize()
    res.seconds = time.perf_counter() - t_start
    res.g_max = float(g_max)
    res.drift_inf = float((w - W).abs().max())
    return res


def hard(w, codebook, cfg: QATConfig):
    """Viterbi (T -> 0) code of the latent weights: states [chains, L] and w_hard [R, C]."""
    states, w_hard = bcjr.viterbi_decode(codebook, w.reshape(-1, cfg.L).contiguous(), cfg.n, cfg.k)
    return states, w_hard.reshape(w.shape)


def synthetic_layer(rows: int, cols: int, samples: int, n: int, seed: int = 0, device="cuda"):
    """``synth.qat_layer`` moved to the device: W, X, Xv, codebook."""
    return tuple(torch.from_numpy(a).to(device) for a in synth.qat_layer(rows, cols, samples, n, seed))


def run(rows: int, cols: int, samples: int, cfg: QATConfig, seed: int = 0, log_every: int = 0):
    """PTQ (Viterbi of W) against annealed QAT started from W, on one synthetic layer."""
    W, X, Xv, c = synthetic_layer(rows, cols, samples, cfg.n, seed)
    ptq_states, ptq_w = hard(W, c, cfg)
    for T in (cfg.t0, cfg.t_end):  # untimed warm-up of both message precisions
        step(W, W, X, c, cfg, T)
    res = train(W, X, c, cfg, log_every)
    qat_states, qat_w = hard(res.w, c, cfg)
    moved = float((qat_states != ptq_states).any(dim=1).float().mean())
    out = {
        "rows": rows, "cols": cols, "samples": samples, "S": 1 << cfg.n, "k": cfg.k, "L": cfg.L,
        "chains": rows * cols // cfg.L, "t0": cfg.t0, "t_end": cfg.t_end, "steps": cfg.steps,
        "lr": cfg.lr, "seed": seed, "segmented": cfg.segmented,
        # output error per weight: recon_loss / (R C)
        "ptq_loss_calib": float(recon_loss(ptq_w, W, X)) / (rows * cols),
        "ptq_loss_heldout": float(recon_loss(ptq_w, W, Xv)) / (rows * cols),
        "qat_loss_calib": float(recon_loss(qat_w, W, X)) / (rows * cols),
        "qat_loss_heldout": float(recon_loss(qat_w, W, Xv)) / (rows * cols),
        "g_max": res.g_max, "drift_inf": res.drift_inf, "drift_budget": res.budget(cfg),
        "budget_exceeds_r_voronoi": res.budget(cfg) > cfg.r_voronoi,
        "chains_with_new_code": moved, "train_seconds": res.seconds,
        "steps_per_s": cfg.steps / res.seconds,
        "state_steps_per_s": cfg.steps * rows * cols * (1 << cfg.n) / res.seconds,
    }
    if log_every:
        out["history"] = res.history
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--rows", type=int, default=512)
    ap.add_argument("--cols", type=int, default=1024)
    ap.add_argument("--samples", type=int, default=2048)
    ap.add_argument("--n", type=int, default=8)
    ap.add_argument("--k", type=int, default=2)
    ap.add_argument("--L", type=int, default=256)
    ap.add_argument("--t0", type=float, nargs="+", default=[0.3, 1.0])
    ap.add_argument("--t-end", type=float, default=0.01)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--lr", type=float, nargs="+", default=[1e-4])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--log-every", type=int, default=0)
    ap.add_argument("--segmented", action="store_true",
                    help="use the parallel-in-L soft quantiser (long chains, e.g. --L = --cols)")
    a = ap.parse_args(argv)
    for lr in a.lr:
        for t0 in a.t0:
            cfg = QATConfig(n=a.n, k=a.k, L=a.L, t0=t0, t_end=a.t_end, steps=a.steps, lr=lr,
                            segmented=a.segmented)
            print(json.dumps(run(a.rows, a.cols, a.samples, cfg, a.seed, a.log_every)), flush=True)


if __name__ == "__main__":
    main()
