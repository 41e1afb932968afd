"""Shared helpers of the GPU parity tests (tolerances, case logging, device runs)."""
from __future__ import annotations

import sys

import numpy as np
import torch

from bcjr_soft_decoding_amd import bcjr

# Tolerances stated for the path: rel 1e-4 on the soft codeword and log Z, rel 1e-3 on the
# gradients, in fp32 against the fp64 oracle. Arrays with entries near zero are compared
# normwise per element: |x - ref| <= rtol * max(|ref|, rms(ref)).
RTOL_FWD = 1e-4
RTOL_GRAD = 1e-3


def log_case(msg: str):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def assert_normwise(x, ref, rtol, what=""):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    assert x.shape == ref.shape, (what, x.shape, ref.shape)
    assert np.all(np.isfinite(x)), f"{what}: non-finite values"
    scale = np.maximum(np.abs(ref), np.sqrt(np.mean(ref * ref))) if ref.size else ref
    diff = np.abs(x - ref)
    # an all-zero reference must be matched exactly
    err = np.where(scale > 0, diff / np.where(scale > 0, scale, 1.0), np.where(diff == 0, 0.0, np.inf))
    worst = float(err.max()) if err.size else 0.0
    assert worst <= rtol, f"{what}: worst normwise error {worst:.3e} > {rtol:.1e}"
    return worst


def assert_rel(x, ref, rtol, what=""):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(x - ref) / np.maximum(np.abs(ref), 1e-30)
    worst = float(err.max()) if err.size else 0.0
    assert worst <= rtol, f"{what}: worst relative error {worst:.3e} > {rtol:.1e}"
    return worst


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run_fwd_bwd(n, k, c, w, T, g=None, h=None):
    """One forward (+ backward if g is given) through the C ABI; returns numpy results."""
    cd, wd = dev(c), dev(w)
    w_hat, log_z, saved = bcjr.bcjr_forward(cd, wd, n, k, T)
    out = {"w_hat": w_hat, "log_z": log_z}
    if g is not None:
        gd = dev(g)
        hd = None if h is None else dev(h)
        gw, gc = bcjr.bcjr_backward(cd, wd, n, k, T, saved, gd, hd)
        out.update(grad_w=gw, grad_codebook=gc)
    torch.cuda.synchronize()
    return {key: v.cpu().numpy() for key, v in out.items()}


def assert_refused(n, k, c, w, T, g):
    """A (shape, T) without kernels that meet the tolerances: forward and backward raise
    BCJR_E_UNSUPPORTED before launching anything, and leave their outputs untouched."""
    import pytest

    cd, wd = dev(c), dev(w)
    B, L = w.shape
    w_hat = torch.full_like(wd, 7.0)
    with pytest.raises(bcjr.BcjrError) as e:
        bcjr.bcjr_forward(cd, wd, n, k, T, w_hat=w_hat)
    assert e.value.status == bcjr.BCJR_E_UNSUPPORTED
    saved = torch.zeros(max(bcjr.bcjr_saved_bytes(n, k, B, L), 1), dtype=torch.uint8, device="cuda")
    gc = torch.full_like(cd, 7.0)
    with pytest.raises(bcjr.BcjrError) as e:
        bcjr.bcjr_backward(cd, wd, n, k, T, saved, dev(g), grad_codebook=gc)
    assert e.value.status == bcjr.BCJR_E_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.all(w_hat == 7.0) and torch.all(gc == 7.0)
