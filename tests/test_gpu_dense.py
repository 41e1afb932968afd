"""GPU parity of the dense (fully connected) trellis path, through the C ABI, against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from bcjr_soft_decoding_amd import bcjr, synth
from tests.gpu_helpers import RTOL_FWD, RTOL_GRAD, assert_normwise, assert_rel, dev, log_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bcjr.lib()  # raises if the HIP library is missing: no fallback


def run_dense(theta, c, w, T, g=None, h=None):
    td, cd, wd = dev(theta), dev(c), dev(w)
    w_hat, log_z, saved = bcjr.bcjr_dense_forward(td, cd, wd, T)
    out = {"w_hat": w_hat, "log_z": log_z}
    if g is not None:
        gw, gc, gt = bcjr.bcjr_dense_backward(td, cd, wd, T, saved, dev(g),
                                              None if h is None else dev(h))
        out.update(grad_w=gw, grad_codebook=gc, grad_theta=gt)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def compare_dense(theta, c, w, T, g=None, h=None, tag=""):
    S = c.shape[0]
    log_case(f"{tag} dense S={S} B={w.shape[0]} L={w.shape[1]} T={T} grad={g is not None} "
             f"h={h is not None}")
    got = run_dense(theta, c, w, T, g, h)
    ref = oracle.dense_forward(theta, c, w, T)
    assert_normwise(got["w_hat"], ref["w_hat"], RTOL_FWD, f"{tag} w_hat")
    assert_rel(got["log_z"], ref["log_z"], RTOL_FWD, f"{tag} log_z")
    if g is not None:
        rb = oracle.dense_backward(theta, c, w, T, g, h)
        assert_normwise(got["grad_w"], rb["grad_w"], RTOL_GRAD, f"{tag} grad_w")
        assert_normwise(got["grad_codebook"], rb["grad_codebook"], RTOL_GRAD, f"{tag} grad_c")
        assert_normwise(got["grad_theta"], rb["grad_theta"], RTOL_GRAD, f"{tag} grad_theta")
    return got


def _case(S, B, L, seed):
    theta = synth.normal(seed, (S, S))
    c = synth.normal(seed + 1, (S,))
    w = synth.normal(seed + 2, (B, L))
    g = synth.normal(seed + 3, (B, L))
    h = synth.normal(seed + 4, (B,))
    return theta, c, w, g, h


# Every built S; B = 6 (one full block of 4 chains and a ragged one), L = 45 (two LDS chunks of
# per-step scalars with a ragged tail, odd so the two-step unrolled loop ends on a half step).
@pytest.mark.parametrize("S", [32, 64, 128, 256])
@pytest.mark.parametrize("T", [0.2, 1.0])
def test_dense_sizes(S, T):
    theta, c, w, g, h = _case(S, 6, 45, 7000 + S)
    compare_dense(theta, c, w, T, g, h, f"S{S}")


@pytest.mark.parametrize("T", [0.1, 5.0])
def test_dense_temperature_range(T):
    theta, c, w, g, h = _case(64, 5, 40, 7100)
    compare_dense(theta, c, w, T, g, h, "trange")


@pytest.mark.parametrize("B,L", [(1, 1), (1, 2), (3, 1), (4, 64), (9, 33)])
def test_dense_edge_shapes(B, L):
    theta, c, w, g, h = _case(32, B, L, 7200 + 10 * B + L)
    got = compare_dense(theta, c, w, 0.5, g, h, f"edge{B}x{L}")
    if L == 1:
        # no transition is taken: the theta gradient vanishes
        assert np.all(got["grad_theta"] == 0.0)


def test_dense_empty_batch():
    S = 64
    theta = dev(synth.normal(7300, (S, S)))
    c = dev(synth.normal(7301, (S,)))
    w = torch.empty((0, 16), dtype=torch.float32, device="cuda")
    log_case("dense B=0")
    w_hat, log_z, saved = bcjr.bcjr_dense_forward(theta, c, w, 0.3)
    gc = torch.full((S,), 7.0, device="cuda")
    gt = torch.full((S, S), 7.0, device="cuda")
    bcjr.bcjr_dense_backward(theta, c, w, 0.3, saved, torch.empty_like(w), None,
                             torch.empty_like(w), gc, gt, ws=torch.empty(16, dtype=torch.uint8,
                                                                         device="cuda"))
    torch.cuda.synchronize()
    assert torch.all(gc == 0) and torch.all(gt == 0)


def test_dense_equals_bitshift_when_theta_masks_edges():
    """theta = 0 on the bitshift edges and far below elsewhere: the dense path computes the
    bitshift trellis (n = 5, k = 2), checked against the bitshift oracle."""
    n, k = 5, 2
    S, K = 1 << n, 1 << k
    theta = np.full((S, S), -1.0e4, np.float32)
    for s in range(S):
        for b in range(K):
            theta[s, ((s << k) | b) & (S - 1)] = 0.0
    c = synth.normal(7400, (S,))
    w = synth.normal(7401, (5, 50))
    g = synth.normal(7402, (5, 50))
    T = 0.3
    log_case("dense masked to bitshift n=5 k=2")
    got = run_dense(theta, c, w, T, g)
    ref = oracle.sparse_forward(n, k, c, w, T)
    rb = oracle.sparse_backward(n, k, c, w, T, g)
    assert_normwise(got["w_hat"], ref["w_hat"], RTOL_FWD, "w_hat")
    assert_rel(got["log_z"], ref["log_z"], RTOL_FWD, "log_z")
    assert_normwise(got["grad_w"], rb["grad_w"], RTOL_GRAD, "grad_w")
    assert_normwise(got["grad_codebook"], rb["grad_codebook"], RTOL_GRAD, "grad_c")


def test_dense_workload5_prefix():
    """Workload 5 (S=256, theta ~ N(0,1), T=0.2) at its full length L=1024, first 6 chains."""
    wl = synth.WORKLOADS[5]
    theta, c = synth.theta(5), synth.codebook(5)
    w, g, h = synth.weights(5)[:6], synth.upstream_grad(5)[:6], synth.logz_grad(5)[:6]
    compare_dense(theta, c, w, wl.temps[0], g, h, "wl5-prefix")


def test_dense_workload5_full_sampled():
    """Workload 5 at full size (1024 x 1024) in the launch configuration the benchmark times:
    sampled chains against the oracle one by one; the batch sums checked against the sum of
    the same path over disjoint sub-batches, and the log Z gradient identities."""
    wl = synth.WORKLOADS[5]
    theta, c, w, g = synth.theta(5), synth.codebook(5), synth.weights(5), synth.upstream_grad(5)
    T = wl.temps[0]
    log_case("wl5 full 1024x1024")
    got = run_dense(theta, c, w, T, g)
    sample = [0, 513, 1023]
    ref = oracle.dense_forward(theta, c, w[sample], T)
    rb = oracle.dense_backward(theta, c, w[sample], T, g[sample])
    assert_normwise(got["w_hat"][sample], ref["w_hat"], RTOL_FWD, "w_hat sampled")
    assert_rel(got["log_z"][sample], ref["log_z"], RTOL_FWD, "log_z sampled")
    assert_normwise(got["grad_w"][sample], rb["grad_w"], RTOL_GRAD, "grad_w sampled")
    # batch sums = sums over four disjoint sub-batches (each a separate launch)
    gc = np.zeros_like(got["grad_codebook"], dtype=np.float64)
    gt = np.zeros_like(got["grad_theta"], dtype=np.float64)
    for i in range(4):
        part = run_dense(theta, c, w[256 * i:256 * (i + 1)], T, g[256 * i:256 * (i + 1)])
        gc += part["grad_codebook"]
        gt += part["grad_theta"]
    assert_normwise(got["grad_codebook"], gc, 1e-4, "grad_c vs sub-batch sum")
    assert_normwise(got["grad_theta"], gt, 1e-4, "grad_theta vs sub-batch sum")
    # g = 0, h = 1: dF/dw = (2/T)(w_hat - w) and sum(dF/dtheta) = B (L - 1) / T exactly
    B, L = w.shape
    hz = run_dense(theta, c, w, T, np.zeros_like(g), np.ones((B,), np.float32))
    assert_normwise(hz["grad_w"], (2.0 / T) * (got["w_hat"].astype(np.float64) - w), 1e-4,
                    "grad_w of log Z")
    assert_rel(hz["grad_theta"].astype(np.float64).sum(), B * (L - 1) / T, 1e-4,
               "sum of grad_theta of log Z")


def test_dense_deterministic():
    theta, c, w, g, h = _case(128, 9, 40, 7500)
    log_case("dense determinism")
    a = run_dense(theta, c, w, 0.4, g, h)
    b = run_dense(theta, c, w, 0.4, g, h)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


@pytest.mark.parametrize("T", [0.099, 0.05, 0.02])
def test_dense_below_01_refused(T):
    """The linear-domain dense path drops states whose weight falls below 2^-126 of a step's
    best; at unit-scale inputs that breaks its tolerances below T = 0.1 (ŵ off by 4e-3 at
    T = 0.05, whole steps underflowing to NaN below 0.03 on workload-5 shapes). Those
    temperatures are refused with BCJR_E_UNSUPPORTED, nothing is enqueued and the outputs keep
    their contents."""
    S, B, L = 64, 3, 20
    theta, c, w, g, h = _case(S, B, L, 7600)
    log_case(f"dense refused T={T}")
    wh = torch.full((B, L), 7.0, device="cuda")
    with pytest.raises(bcjr.BcjrError) as e:
        bcjr.bcjr_dense_forward(dev(theta), dev(c), dev(w), T, w_hat=wh)
    assert e.value.status == bcjr.BCJR_E_UNSUPPORTED
    saved = torch.zeros(bcjr.bcjr_dense_saved_bytes(S, B, L), dtype=torch.uint8, device="cuda")
    gt = torch.full((S, S), 7.0, device="cuda")
    with pytest.raises(bcjr.BcjrError) as e:
        bcjr.bcjr_dense_backward(dev(theta), dev(c), dev(w), T, saved, dev(g), grad_theta=gt)
    assert e.value.status == bcjr.BCJR_E_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.all(wh == 7.0) and torch.all(gt == 7.0)


def test_dense_workload5_at_the_threshold():
    """T = 0.1, the lowest temperature the dense path accepts, on workload-5 shapes (S = 256,
    L = 1024, first 6 chains) against the oracle."""
    theta, c = synth.theta(5), synth.codebook(5)
    w, g, h = synth.weights(5)[:6], synth.upstream_grad(5)[:6], synth.logz_grad(5)[:6]
    compare_dense(theta, c, w, 0.1, g, h, "wl5-threshold")
