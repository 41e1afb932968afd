"""The autograd wrapper: its gradients are the C ABI backward's, and agree with the oracle."""
import numpy as np
import pytest
import torch

import oracle
from bcjr_soft_decoding_amd import autograd, bcjr, synth
from tests.gpu_helpers import RTOL_FWD, RTOL_GRAD, assert_normwise, dev, log_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bcjr.lib()


def test_soft_quantize_backward_matches_abi_and_oracle():
    n, k, T = 6, 2, 0.3
    c = synth.normal(8000, (1 << n,))
    w = synth.normal(8001, (2, 3, 40))  # leading dims are chains
    g = synth.normal(8002, (2, 3, 40))
    h = synth.normal(8003, (2, 3))
    log_case("autograd bitshift n=6 k=2 [2,3,40]")
    wd = dev(w).requires_grad_(True)
    cd = dev(c).requires_grad_(True)
    w_hat, log_z = autograd.soft_quantize(wd, cd, n, k, T)
    assert w_hat.shape == (2, 3, 40) and log_z.shape == (2, 3)
    ((w_hat * dev(g)).sum() + (log_z * dev(h)).sum()).backward()
    torch.cuda.synchronize()
    # same kernels through the ABI directly: bitwise equal
    wh2, lz2, saved = bcjr.bcjr_forward(dev(c), dev(w.reshape(6, 40)), n, k, T)
    gw2, gc2 = bcjr.bcjr_backward(dev(c), dev(w.reshape(6, 40)), n, k, T, saved,
                                  dev(g.reshape(6, 40)), dev(h.reshape(6)))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(w_hat.detach().cpu().numpy().reshape(6, 40), wh2.cpu().numpy())
    np.testing.assert_array_equal(wd.grad.cpu().numpy().reshape(6, 40), gw2.cpu().numpy())
    np.testing.assert_array_equal(cd.grad.cpu().numpy(), gc2.cpu().numpy())
    rb = oracle.sparse_backward(n, k, c, w.reshape(6, 40), T, g.reshape(6, 40), h.reshape(6))
    assert_normwise(wd.grad.cpu().numpy().reshape(6, 40), rb["grad_w"], RTOL_GRAD, "grad_w")
    assert_normwise(cd.grad.cpu().numpy(), rb["grad_codebook"], RTOL_GRAD, "grad_c")


def test_soft_quantize_only_w_hat_used():
    """log Z unused: its upstream gradient is None and the backward takes h = 0."""
    n, k, T = 5, 2, 0.5
    c = synth.normal(8100, (1 << n,))
    w = synth.normal(8101, (4, 30))
    log_case("autograd bitshift, w_hat only")
    wd = dev(w).requires_grad_(True)
    w_hat, _ = autograd.soft_quantize(wd, dev(c), n, k, T)
    (w_hat ** 2).sum().backward()
    torch.cuda.synchronize()
    g = 2.0 * w_hat.detach().cpu().numpy().astype(np.float32)
    rb = oracle.sparse_backward(n, k, c, w, T, g)
    assert_normwise(wd.grad.cpu().numpy(), rb["grad_w"], RTOL_GRAD, "grad_w")


def test_dense_soft_quantize_matches_oracle():
    S, T = 64, 0.4
    theta = synth.normal(8200, (S, S))
    c = synth.normal(8201, (S,))
    w = synth.normal(8202, (5, 33))
    g = synth.normal(8203, (5, 33))
    log_case("autograd dense S=64 [5,33]")
    td = dev(theta).requires_grad_(True)
    cd = dev(c).requires_grad_(True)
    wd = dev(w).requires_grad_(True)
    w_hat, log_z = autograd.dense_soft_quantize(wd, cd, td, T)
    (w_hat * dev(g)).sum().backward()
    torch.cuda.synchronize()
    rf = oracle.dense_forward(theta, c, w, T)
    rb = oracle.dense_backward(theta, c, w, T, g)
    assert_normwise(w_hat.detach().cpu().numpy(), rf["w_hat"], RTOL_FWD, "w_hat")
    assert_normwise(wd.grad.cpu().numpy(), rb["grad_w"], RTOL_GRAD, "grad_w")
    assert_normwise(cd.grad.cpu().numpy(), rb["grad_codebook"], RTOL_GRAD, "grad_c")
    assert_normwise(td.grad.cpu().numpy(), rb["grad_theta"], RTOL_GRAD, "grad_theta")


def test_segmented_soft_quantize_matches_sequential():
    """soft_quantize(segmented=True) on long chains: the same values and gradients as the
    ordinary wrapper (rel 1e-4 / 1e-3), and the oracle's."""
    n, k, T = 8, 2, 0.2
    c = synth.normal(8300, (1 << n,))
    w = synth.normal(8301, (2, 5000))
    g = synth.normal(8302, (2, 5000))
    h = synth.normal(8303, (2,))
    log_case("autograd segmented n=8 [2,5000]")
    outs = []
    for seg in (True, False):
        wd = dev(w).requires_grad_(True)
        cd = dev(c).requires_grad_(True)
        w_hat, log_z = autograd.soft_quantize(wd, cd, n, k, T, segmented=seg, seg_len=128)
        ((w_hat * dev(g)).sum() + (log_z * dev(h)).sum()).backward()
        torch.cuda.synchronize()
        outs.append((w_hat.detach().cpu().numpy(), log_z.detach().cpu().numpy(),
                     wd.grad.cpu().numpy(), cd.grad.cpu().numpy()))
    (a, lz, gw, gc), (a2, lz2, gw2, gc2) = outs
    assert_normwise(a, a2, RTOL_FWD, "w_hat")
    assert_normwise(gw, gw2, RTOL_GRAD, "grad_w")
    assert_normwise(gc, gc2, RTOL_GRAD, "grad_c")
    rb = oracle.sparse_backward(n, k, c, w, T, g, h)
    assert_normwise(gw, rb["grad_w"], RTOL_GRAD, "grad_w vs oracle")
    assert_normwise(gc, rb["grad_codebook"], RTOL_GRAD, "grad_c vs oracle")
