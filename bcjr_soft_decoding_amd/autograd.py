"""The soft quantiser as differentiable torch functions over the C ABI.

``soft_quantize(w, codebook, n, k, T)`` returns ``(w_hat, log_z)`` for the bitshift trellis
(2^n states, 2^k branches); ``dense_soft_quantize(w, codebook, theta, T)`` does the same for the
fully connected trellis with transition log-potentials ``theta``. Their backward passes call
``bcjr_backward`` / ``bcjr_dense_backward`` with the upstream gradients of both outputs (the
gradient of sum(g * w_hat) + sum(h * log_z)), so a QAT loop gets exact gradients to the weights,
the codebook and theta. T is a constant here. Every step runs in the HIP kernels; tensors must be
fp32 CUDA tensors and ``w`` has shape [..., L] (leading dimensions are the chains).

``soft_quantize(..., segmented=True)`` uses the segmented entry points (``bcjr_forward_scan`` /
``bcjr_backward_scan``), which parallelise along the chain: the same values for few, very long
chains (S <= 4096), where the ordinary sweeps would leave the device idle.
"""
from __future__ import annotations

import torch

from . import bcjr


def _chains(w):
    L = w.shape[-1]
    return w.contiguous().reshape(-1, L)


class _SoftTrellisQuant(torch.autograd.Function):
    @staticmethod
    def forward(ctx, w, codebook, n, k, T):
        w2 = _chains(w)
        c = codebook.contiguous()
        w_hat, log_z, saved = bcjr.bcjr_forward(c, w2, n, k, T)
        ctx.save_for_backward(w2, c, saved)
        ctx.cfg = (n, k, T, w.shape)
        return w_hat.reshape(w.shape), log_z.reshape(w.shape[:-1])

    @staticmethod
    def backward(ctx, g_what, g_logz):
        w2, c, saved = ctx.saved_tensors
        n, k, T, shape = ctx.cfg
        g = torch.zeros_like(w2) if g_what is None else g_what.contiguous().reshape(w2.shape)
        h = None if g_logz is None else g_logz.contiguous().reshape(-1)
        gw, gc = bcjr.bcjr_backward(c, w2, n, k, T, saved, g, h)
        return gw.reshape(shape), gc, None, None, None


class _DenseSoftTrellisQuant(torch.autograd.Function):
    @staticmethod
    def forward(ctx, w, codebook, theta, T):
        w2 = _chains(w)
        c = codebook.contiguous()
        th = theta.contiguous()
        w_hat, log_z, saved = bcjr.bcjr_dense_forward(th, c, w2, T)
        ctx.save_for_backward(w2, c, th, saved)
        ctx.cfg = (T, w.shape)
        return w_hat.reshape(w.shape), log_z.reshape(w.shape[:-1])

    @staticmethod
    def backward(ctx, g_what, g_logz):
        w2, c, th, saved = ctx.saved_tensors
        T, shape = ctx.cfg
        g = torch.zeros_like(w2) if g_what is None else g_what.contiguous().reshape(w2.shape)
        h = None if g_logz is None else g_logz.contiguous().reshape(-1)
        gw, gc, gt = bcjr.bcjr_dense_backward(th, c, w2, T, saved, g, h)
        return gw.reshape(shape), gc, gt, None


class _SegmentedTrellisQuant(torch.autograd.Function):
    @staticmethod
    def forward(ctx, w, codebook, n, k, T, seg_len):
        w2 = _chains(w)
        c = codebook.contiguous()
        w_hat, log_z = bcjr.bcjr_forward_scan(c, w2, n, k, T, seg_len)
        ctx.save_for_backward(w2, c, w_hat)
        ctx.cfg = (n, k, T, seg_len, w.shape)
        return w_hat.reshape(w.shape), log_z.reshape(w.shape[:-1])

    @staticmethod
    def backward(ctx, g_what, g_logz):
        w2, c, w_hat = ctx.saved_tensors
        n, k, T, seg_len, shape = ctx.cfg
        g = torch.zeros_like(w2) if g_what is None else g_what.contiguous().reshape(w2.shape)
        h = None if g_logz is None else g_logz.contiguous().reshape(-1)
        gw, gc = bcjr.bcjr_backward_scan(c, w2, n, k, T, w_hat, g, h, seg_len)
        return gw.reshape(shape), gc, None, None, None, None


def soft_quantize(w, codebook, n: int, k: int, T: float, segmented: bool = False,
                  seg_len: int = 0):
    """Soft codeword and log Z of every chain of the bitshift trellis; differentiable in w and
    the codebook. ``segmented`` selects the parallel-in-L entry points (segment length
    ``seg_len``, 0 for the default)."""
    if segmented:
        return _SegmentedTrellisQuant.apply(w, codebook, int(n), int(k), float(T), int(seg_len))
    return _SoftTrellisQuant.apply(w, codebook, int(n), int(k), float(T))


def dense_soft_quantize(w, codebook, theta, T: float):
    """Soft codeword and log Z of every chain of the fully connected trellis; differentiable in
    w, the codebook and theta."""
    return _DenseSoftTrellisQuant.apply(w, codebook, theta, float(T))
