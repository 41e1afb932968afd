"""The annealed QAT driver (bcjr_soft_decoding_amd.qat) against the oracle's loop
(oracle/qat.py): one step's loss and latent-weight gradient, a short annealed run, and the
drift-budget behaviour on a larger seeded layer."""
import numpy as np
import pytest
import torch

import oracle
from oracle import qat as oqat
from bcjr_soft_decoding_amd import bcjr, qat, synth
from tests.gpu_helpers import RTOL_FWD, RTOL_GRAD, assert_normwise, assert_rel, dev, log_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bcjr.lib()


@pytest.mark.parametrize("n,R,C,N,T", [(8, 8, 1024, 512, 0.3), (8, 8, 1024, 512, 0.05),
                                       (8, 4, 768, 256, 1.0), (12, 2, 512, 256, 0.1),
                                       (4, 3, 96, 64, 0.3)])
def test_step_matches_oracle(n, R, C, N, T):
    L = 256 if C % 256 == 0 else 32
    log_case(f"qat step n={n} R={R} C={C} N={N} L={L} T={T}")
    W, X, _, c = synth.qat_layer(R, C, N, n, seed=1)
    rng = np.random.default_rng(2)
    w = (W + 0.05 * rng.standard_normal(W.shape)).astype(np.float32)
    cfg = qat.QATConfig(n=n, k=2, L=L)
    loss, grad = qat.step(dev(w), dev(W), dev(X), dev(c), cfg, T)
    torch.cuda.synchronize()
    ref_loss, ref_g, _ = oqat.loss_and_grad(w, W, X, c, n, 2, L, T)
    assert_rel(float(loss), ref_loss, RTOL_FWD, "loss")
    assert_normwise(grad.cpu().numpy(), ref_g, RTOL_GRAD, "dloss/dw")


def test_annealed_run_matches_oracle():
    n, R, C, N, L = 8, 4, 1024, 512, 256
    steps, lr, t0, t_end = 6, 2.5e-4, 0.3, 0.05
    log_case(f"qat loop n={n} R={R} C={C} steps={steps}")
    W, X, _, c = synth.qat_layer(R, C, N, n, seed=4)
    cfg = qat.QATConfig(n=n, k=2, L=L, t0=t0, t_end=t_end, steps=steps, lr=lr)
    res = qat.train(dev(W), dev(X), dev(c), cfg, log_every=1)
    w_ref, g_max_ref, losses_ref = oqat.train(W, X, c, n, 2, L, t0, t_end, steps, lr)
    for i, rec in enumerate(res.history):
        assert rec["T"] == pytest.approx(oqat.temperature(t0, t_end, steps, i), rel=1e-12)
    assert_rel([r["soft_loss"] for r in res.history], losses_ref, RTOL_FWD, "loss curve")
    drift = res.w.cpu().numpy().astype(np.float64) - W
    assert_normwise(drift, w_ref.astype(np.float64) - W, RTOL_GRAD, "w - W")
    assert res.g_max == pytest.approx(g_max_ref, rel=RTOL_GRAD)


def test_drift_budget_escape_and_stay():
    """Budget far above r_Voronoi: the hard code leaves the PTQ code and the held-out output
    error drops; budget far below: the code stays (nearly) the PTQ code. Drift never exceeds
    eta * N * g_max."""
    rows, cols, N, n = 256, 1024, 2048, 8
    out = {}
    for lr in (1e-4, 1e-9):
        log_case(f"qat drift budget lr={lr}")
        cfg = qat.QATConfig(n=n, k=2, L=256, t0=0.3, t_end=0.01, steps=40, lr=lr)
        r = qat.run(rows, cols, N, cfg, seed=0)
        assert r["drift_inf"] <= r["drift_budget"] * (1 + 1e-6) + cfg.steps * 2.0 ** -22
        out[lr] = r
    big, small = out[1e-4], out[1e-9]
    assert big["budget_exceeds_r_voronoi"] and not small["budget_exceeds_r_voronoi"]
    assert big["chains_with_new_code"] > 0.5
    assert big["qat_loss_heldout"] < 0.95 * big["ptq_loss_heldout"]
    assert small["chains_with_new_code"] <= 0.01
    assert small["qat_loss_heldout"] == pytest.approx(small["ptq_loss_heldout"], rel=1e-3)


def test_hard_code_of_trained_weights_round_trips():
    """The driver's output is exported as the hard code and read back bit-exactly."""
    n, R, C, L = 8, 8, 512, 256
    log_case("qat export round trip")
    W, X, _, c = synth.qat_layer(R, C, 256, n, seed=5)
    cfg = qat.QATConfig(n=n, k=2, L=L, steps=3)
    res = qat.train(dev(W), dev(X), dev(c), cfg)
    states, w_hard = qat.hard(res.w, dev(c), cfg)
    code = bcjr.bcjr_pack_code(states, n, 2)
    st2, wh2 = bcjr.bcjr_unpack_code(code, n, 2, L, codebook=dev(c))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(st2.cpu().numpy(), states.cpu().numpy())
    np.testing.assert_array_equal(wh2.cpu().numpy().reshape(R, C), w_hard.cpu().numpy())
    ref = oracle.viterbi(n, 2, c, res.w.cpu().numpy().reshape(-1, L))
    np.testing.assert_array_equal(states.cpu().numpy(), ref["states"])


def test_segmented_step_matches_oracle():
    """One step with whole rows as chains through the parallel-in-L soft quantiser."""
    n, R, C, N, T = 8, 2, 3000, 256, 0.2
    log_case(f"qat segmented step n={n} R={R} C={C} (one chain per row)")
    W, X, _, c = synth.qat_layer(R, C, N, n, seed=6)
    rng = np.random.default_rng(3)
    w = (W + 0.05 * rng.standard_normal(W.shape)).astype(np.float32)
    cfg = qat.QATConfig(n=n, k=2, L=C, segmented=True)
    loss, grad = qat.step(dev(w), dev(W), dev(X), dev(c), cfg, T)
    torch.cuda.synchronize()
    ref_loss, ref_g, _ = oqat.loss_and_grad(w, W, X, c, n, 2, C, T)
    assert_rel(float(loss), ref_loss, RTOL_FWD, "loss")
    assert_normwise(grad.cpu().numpy(), ref_g, RTOL_GRAD, "dloss/dw")
