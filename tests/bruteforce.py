"""Exhaustive path enumeration for tiny trellises (numpy, float64) -- an independent pin.

Nothing here runs a forward-backward recursion: every quantity is computed straight from its
definition over the list of all admissible paths (the Boltzmann distribution over trellis paths
of the BCJR-QAT abstract, with path energy sum_t (w_t - c(s_t))^2 [- sum_t theta(s_{t-1}, s_t)]).
"""
from __future__ import annotations

import numpy as np
from scipy.special import logsumexp


def bitshift_paths(n: int, k: int, L: int) -> np.ndarray:
    """All S*K^(L-1) admissible state paths of the bitshift trellis, int64 [P, L]."""
    S, K = 1 << n, 1 << k
    paths = np.arange(S, dtype=np.int64)[:, None]
    for _ in range(1, L):
        prev = paths[:, -1]
        nxt = ((prev[:, None] << k) | np.arange(K, dtype=np.int64)[None, :]) & (S - 1)
        paths = np.concatenate([np.repeat(paths, K, axis=0), nxt.reshape(-1, 1)], axis=1)
    return paths


def dense_paths(S: int, L: int) -> np.ndarray:
    """All S^L paths of the fully connected trellis, int64 [P, L]."""
    grids = np.meshgrid(*[np.arange(S, dtype=np.int64)] * L, indexing="ij")
    return np.stack([g.reshape(-1) for g in grids], axis=1)


def path_log_weights(paths, c, w, T, theta=None):
    """Lambda(path) = -E(path)/T in float64."""
    c64 = np.asarray(c, np.float64)
    w64 = np.asarray(w, np.float64)
    E = ((w64[None, :] - c64[paths]) ** 2).sum(axis=1)
    if theta is not None:
        th = np.asarray(theta, np.float64)
        E = E - th[paths[:, :-1], paths[:, 1:]].sum(axis=1)
    return -E / T


def exact_stats(paths, c, w, T, S, g=None, h=0.0, theta=None):
    """log Z, posteriors, soft codeword and (if g is given) gradients, from the path list.

    Gradients of F = sum_t g_t w_hat_t + h log Z use the exponential-family identities
      dE_p[f]/dx = E_p[df/dx] + Cov_p(f, dLambda/dx),   dlogZ/dx = E_p[dLambda/dx].
    """
    lam = path_log_weights(paths, c, w, T, theta)
    logz = logsumexp(lam)
    p = np.exp(lam - logz)
    L = paths.shape[1]
    c64 = np.asarray(c, np.float64)
    w64 = np.asarray(w, np.float64)
    gamma = np.zeros((L, S))
    for t in range(L):
        gamma[t] = np.bincount(paths[:, t], weights=p, minlength=S)
    cp = c64[paths]                      # [P, L] codeword on each step of each path
    w_hat = (p[:, None] * cp).sum(axis=0)
    out = {"log_z": logz, "gamma": gamma, "w_hat": w_hat, "p": p}
    if g is None:
        return out
    g64 = np.asarray(g, np.float64)
    F = cp @ g64                          # F(path) = sum_t g_t c(s_t)
    EF = p @ F
    # d Lambda / d w_t = -(2/T)(w_t - c(s_t))
    dlam_dw = -(2.0 / T) * (w64[None, :] - cp)
    grad_w = p @ ((F - EF)[:, None] * dlam_dw) + h * (p @ dlam_dw)
    # d Lambda / d c(s) = (2/T) sum_t (w_t - c(s)) 1{s_t = s}
    dlam_dc = np.zeros((paths.shape[0], S))
    for t in range(L):
        np.add.at(dlam_dc, (np.arange(paths.shape[0]), paths[:, t]), (2.0 / T) * (w64[t] - cp[:, t]))
    direct = (g64[:, None] * gamma).sum(axis=0)   # sum_t g_t P(s_t = s)
    grad_c = direct + p @ ((F - EF)[:, None] * dlam_dc) + h * (p @ dlam_dc)
    out.update(grad_w=grad_w, grad_c=grad_c)
    if theta is not None:
        # d Lambda / d theta(s, s') = (1/T) #{t : s_{t-1} = s, s_t = s'}
        cnt = np.zeros((paths.shape[0], S * S))
        idx = paths[:, :-1] * S + paths[:, 1:]
        for t in range(L - 1):
            np.add.at(cnt, (np.arange(paths.shape[0]), idx[:, t]), 1.0 / T)
        grad_theta = p @ ((F - EF)[:, None] * cnt) + h * (p @ cnt)
        out["grad_theta"] = grad_theta.reshape(S, S)
    return out


def fp32_path_energies(paths, c, w):
    """Path energies accumulated left to right in float32: fl(m + fl(fl(w_t - c)^2))."""
    c32 = np.asarray(c, np.float32)
    w32 = np.asarray(w, np.float32)
    d = (w32[0] - c32[paths[:, 0]]).astype(np.float32)
    m = (d * d).astype(np.float32)
    for t in range(1, paths.shape[1]):
        d = (w32[t] - c32[paths[:, t]]).astype(np.float32)
        m = (m + (d * d).astype(np.float32)).astype(np.float32)
    return m
