"""Plain CPU oracle of the annealed QAT loop -- test infrastructure only.

Only the test suite and the benchmark's CPU-baseline leg may use this module; it shares no
code with the HIP library. It composes the C oracle's soft quantiser (``sparse_forward`` /
``sparse_backward``) with a per-layer reconstruction loss, all in double precision:

  * annealing (BCJR-QAT technical summary, "Annealing"; "Schedule fix (Skip-High-T)"): T goes
    from T0 to a small T_end over the run; the reading taken here is a geometric schedule,
    T_i = T0 (T_end / T0)^(i / (steps - 1));
  * the objective is the pages' per-layer option read as output reconstruction on calibration
    inputs X [N, C] of a layer with float weights W [R, C]:
        loss(w) = sum((X (w_hat(w) - W)^T)^2) / N,
    the squared output error per calibration sample, whose gradient to the soft codeword is
    G = 2 (w_hat - W) (X^T X) / N;
  * the gradient to the latent weights is the soft quantiser's backward applied to G (the
    chain rule; the oracle's backward is the exact gradient of sum(G * w_hat));
  * plain SGD, w <- w - eta * dloss/dw, from w = W; the drift-budget figure ("Drift-budget
    theory") is eta * N * g_max with g_max the largest gradient entry seen.
"""
from __future__ import annotations

import numpy as np

from . import oracle


def temperature(t0: float, t_end: float, steps: int, i: int) -> float:
    if steps <= 1:
        return float(t0)
    return float(t0) * (float(t_end) / float(t0)) ** (i / (steps - 1))


def recon_loss(w_q, W, X) -> float:
    X = np.asarray(X, np.float64)
    d = X @ (np.asarray(w_q, np.float64) - np.asarray(W, np.float64)).T
    return float(np.sum(d * d) / X.shape[0])


def loss_and_grad(w, W, X, codebook, n, k, L, T):
    """(loss, dloss/dw [R, C], w_hat [R, C]) at latent weights w (fp32 as the GPU sees them)."""
    R, C = W.shape
    w32 = np.asarray(w, np.float32)
    f = oracle.sparse_forward(n, k, codebook, w32.reshape(-1, L), T)
    w_hat = f["w_hat"].reshape(R, C)
    X64 = np.asarray(X, np.float64)
    e = w_hat - np.asarray(W, np.float64)
    d = X64 @ e.T                                   # [N, R]
    loss = float(np.sum(d * d) / X64.shape[0])
    G = 2.0 * (d.T @ X64) / X64.shape[0]            # [R, C] = 2 e X^T X / N
    b = oracle.sparse_backward(n, k, codebook, w32.reshape(-1, L), T, G.reshape(-1, L))
    return loss, b["grad_w"].reshape(R, C), w_hat


def train(W, X, codebook, n, k, L, t0, t_end, steps, lr):
    """SGD through the annealed schedule. The latent weights are kept in fp32 between steps,
    as the GPU driver keeps them. Returns (w, g_max, losses)."""
    w = np.array(W, np.float32)
    g_max = 0.0
    losses = []
    for i in range(steps):
        T = temperature(t0, t_end, steps, i)
        loss, g, _ = loss_and_grad(w, W, X, codebook, n, k, L, T)
        g_max = max(g_max, float(np.max(np.abs(g))))
        w = (w.astype(np.float64) - lr * g).astype(np.float32)
        losses.append(loss)
    return w, g_max, losses
