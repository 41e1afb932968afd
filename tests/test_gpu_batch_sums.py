"""Element-wise parity of the gradients that sum over chains (codebook, theta) in full-size
launches, where every persistent block accumulates many chain units into its partial row.

Construction: the upstream gradients g and h are zero on every chain except a sample spread over
the whole batch (so over every iteration of the persistent blocks' loop and over many blocks).
A chain with g = h = 0 has D = 0 and contributes exactly zero to every gradient (its conditional
expectations, centring mean and posterior-weighted sums are exact zeros in the kernels too), so
the launch's codebook (and theta) gradient must equal the oracle's sum over the sampled chains
alone, element by element. The sampled chains' grad_w is compared with the oracle and every other
chain's grad_w must be exactly zero. Also: the narrow (sub-wave and one/two-wave) kernels with
more chains than resident blocks, compared in full."""
import numpy as np
import pytest
import torch

import oracle
from bcjr_soft_decoding_amd import bcjr, synth
from tests.gpu_helpers import RTOL_FWD, RTOL_GRAD, assert_normwise, dev, log_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bcjr.lib()


def _spread_sample(B, count, seed):
    """`count` distinct chains spread over [0, B): one per stratum, at a random offset in it."""
    r = np.random.default_rng(seed)
    edges = np.linspace(0, B, count + 1).astype(np.int64)
    pick = [int(r.integers(edges[i], max(edges[i] + 1, edges[i + 1]))) for i in range(count)]
    pick[0], pick[-1] = 0, B - 1
    return np.array(sorted(set(pick)), np.int64)


def _sparse_zero_g(i, T, count, hist):
    wl = synth.WORKLOADS[i]
    c, w, g_full = synth.codebook(i), synth.weights(i), synth.upstream_grad(i)
    B, L = w.shape
    sample = _spread_sample(B, count, 9100 + i)
    g = np.zeros_like(g_full)
    g[sample] = g_full[sample]
    log_case(f"zero-g batch sum workload {i} ({wl.name}) B={B} L={L} T={T} history={hist} "
             f"sampled={len(sample)}")
    cd, wd = dev(c), dev(w)
    wf = bcjr.workspace(wl.n, wl.k, B, L, bcjr.FWD_CKPT if hist == "ckpt" else bcjr.FWD)
    wb = bcjr.workspace(wl.n, wl.k, B, L, bcjr.BWD_CKPT if hist == "ckpt" else bcjr.BWD)
    w_hat, log_z, saved = bcjr.bcjr_forward(cd, wd, wl.n, wl.k, T, ws=wf)
    del wf
    gw, gc = bcjr.bcjr_backward(cd, wd, wl.n, wl.k, T, saved, dev(g), ws=wb)
    torch.cuda.synchronize()
    del wb
    gw, gc = gw.cpu().numpy(), gc.cpu().numpy()
    rest = np.ones(B, bool)
    rest[sample] = False
    assert np.count_nonzero(gw[rest]) == 0, "a chain with zero upstream gradient has nonzero grad_w"
    ws_ = w[sample]
    rb = oracle.sparse_backward(wl.n, wl.k, c, ws_, T, g[sample])
    assert_normwise(gw[sample], rb["grad_w"], RTOL_GRAD, "grad_w (sampled chains)")
    assert_normwise(gc, rb["grad_codebook"], RTOL_GRAD, "grad_codebook (whole launch vs the sample)")


def test_workload3_codebook_gradient_elementwise_full_launch():
    """The Llama-MLP workload (65536 x 256, S = 4096, T = 0.1), the benchmark's launch: 64
    sampled chains carry the upstream gradient."""
    _sparse_zero_g(3, 0.1, 64, "full")


def test_workload3_codebook_gradient_elementwise_checkpointed():
    _sparse_zero_g(3, 0.1, 32, "ckpt")


@pytest.mark.parametrize("T", synth.WORKLOADS[4].temps)
def test_workload4_codebook_gradient_elementwise_full_launch(T):
    """S = 65536 (16384 x 256, 1024-lane chains): 12 sampled chains."""
    _sparse_zero_g(4, T, 12, "full")


@pytest.mark.parametrize("n,B,L,T,hist", [
    (12, 2500, 12, 0.1, "full"),   # one/two waves per chain; 2500 > the resident blocks
    (12, 2500, 12, 0.1, "ckpt"),
    (8, 70000, 6, 0.3, "full"),    # 16 / 8 chains per wave; 70000 / 8 units > 8192 slots
    (8, 70000, 6, 0.3, "ckpt"),
    (8, 40000, 7, 0.005, "full"),  # fp64 messages
])
def test_narrow_kernels_more_chains_than_blocks(n, B, L, T, hist):
    """Every block loops over several chain units and accumulates their codebook gradient in
    its partial row; compared in full with the oracle."""
    c = synth.normal(9200 + n, (1 << n,))
    w = synth.normal(9300 + n + L, (B, L))
    g = synth.normal(9400 + n + L, (B, L))
    h = synth.normal(9500 + n, (B,))
    log_case(f"narrow many units n={n} B={B} L={L} T={T} history={hist}")
    cd, wd = dev(c), dev(w)
    wf = bcjr.workspace(n, 2, B, L, bcjr.FWD_CKPT if hist == "ckpt" else bcjr.FWD)
    wb = bcjr.workspace(n, 2, B, L, bcjr.BWD_CKPT if hist == "ckpt" else bcjr.BWD)
    w_hat, log_z, saved = bcjr.bcjr_forward(cd, wd, n, 2, T, ws=wf)
    gw, gc = bcjr.bcjr_backward(cd, wd, n, 2, T, saved, dev(g), dev(h), ws=wb)
    torch.cuda.synchronize()
    ref = oracle.sparse_forward(n, 2, c, w, T)
    rb = oracle.sparse_backward(n, 2, c, w, T, g, h)
    assert_normwise(w_hat.cpu().numpy(), ref["w_hat"], RTOL_FWD, "w_hat")
    # short chains: log Z lies near zero for some, compared normwise over the batch
    assert_normwise(log_z.cpu().numpy(), ref["log_z"], RTOL_FWD, "log_z")
    assert_normwise(gw.cpu().numpy(), rb["grad_w"], RTOL_GRAD, "grad_w")
    assert_normwise(gc.cpu().numpy(), rb["grad_codebook"], RTOL_GRAD, "grad_codebook")


def _dense_zero_g(theta, c, w, g_full, T, sample):
    B, L = w.shape
    g = np.zeros_like(g_full)
    g[sample] = g_full[sample]
    wh, lz, sv = bcjr.bcjr_dense_forward(dev(theta), dev(c), dev(w), T)
    gw, gc, gt = bcjr.bcjr_dense_backward(dev(theta), dev(c), dev(w), T, sv, dev(g))
    torch.cuda.synchronize()
    gw, gc, gt = gw.cpu().numpy(), gc.cpu().numpy(), gt.cpu().numpy()
    rest = np.ones(B, bool)
    rest[sample] = False
    assert np.count_nonzero(gw[rest]) == 0, "a chain with zero upstream gradient has nonzero grad_w"
    rb = oracle.dense_backward(theta, c, w[sample], T, g[sample])
    assert_normwise(gw[sample], rb["grad_w"], RTOL_GRAD, "grad_w (sampled chains)")
    assert_normwise(gc, rb["grad_codebook"], RTOL_GRAD, "grad_codebook (whole launch vs the sample)")
    assert_normwise(gt, rb["grad_theta"], RTOL_GRAD, "grad_theta (whole launch vs the sample)")


def test_workload5_dense_batch_gradients_elementwise_full_launch():
    """Workload 5 (1024 x 1024, S = 256, T = 0.2) in the benchmark's launch: the codebook and
    theta gradients of the whole launch against the oracle's sum over 8 sampled chains."""
    wl = synth.WORKLOADS[5]
    theta, c, w, g = synth.theta(5), synth.codebook(5), synth.weights(5), synth.upstream_grad(5)
    sample = _spread_sample(wl.B, 8, 9105)
    log_case(f"zero-g dense workload 5 sampled={list(sample)}")
    _dense_zero_g(theta, c, w, g, wl.temps[0], sample)


def test_dense_more_chains_than_sweep_blocks():
    """B = 4500 chains, more than the sweeps' 1024 persistent blocks of 4 chains: every block
    accumulates several units into its codebook-gradient partials; compared in full."""
    S, B, L, T = 64, 4500, 10, 0.3
    theta = synth.normal(9600, (S, S))
    c = synth.normal(9601, (S,))
    w = synth.normal(9602, (B, L))
    g = synth.normal(9603, (B, L))
    h = synth.normal(9604, (B,))
    log_case(f"dense many units S={S} B={B} L={L}")
    wh, lz, sv = bcjr.bcjr_dense_forward(dev(theta), dev(c), dev(w), T)
    gw, gc, gt = bcjr.bcjr_dense_backward(dev(theta), dev(c), dev(w), T, sv, dev(g), dev(h))
    torch.cuda.synchronize()
    ref = oracle.dense_forward(theta, c, w, T)
    rb = oracle.dense_backward(theta, c, w, T, g, h)
    assert_normwise(wh.cpu().numpy(), ref["w_hat"], RTOL_FWD, "w_hat")
    assert_normwise(lz.cpu().numpy(), ref["log_z"], RTOL_FWD, "log_z")
    assert_normwise(gw.cpu().numpy(), rb["grad_w"], RTOL_GRAD, "grad_w")
    assert_normwise(gc.cpu().numpy(), rb["grad_codebook"], RTOL_GRAD, "grad_codebook")
    assert_normwise(gt.cpu().numpy(), rb["grad_theta"], RTOL_GRAD, "grad_theta")
