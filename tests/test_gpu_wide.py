"""Chains of 1024 lanes (S >= 2^15, one 16-wave block per chain): k_sparse_fwd_wide and
k_sparse_bwd_wide against the oracle element by element, with more chains than workspace slots
(so that slots accumulate the codebook gradient over several chains), full and checkpointed
histories, ragged segments, an upstream log Z gradient, and fp64 messages at low T."""
import numpy as np
import pytest
import torch

import oracle
from bcjr_soft_decoding_amd import bcjr, synth
from tests.gpu_helpers import (RTOL_FWD, RTOL_GRAD, assert_normwise, assert_refused, assert_rel, dev,
                               log_case)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bcjr.lib()


def _run(n, c, w, g, h, T, ckpt):
    k = 2
    B, L = w.shape
    cd, wd = dev(c), dev(w)
    wf = bcjr.workspace(n, k, B, L, bcjr.FWD_CKPT if ckpt else bcjr.FWD)
    wb = bcjr.workspace(n, k, B, L, bcjr.BWD_CKPT if ckpt else bcjr.BWD)
    w_hat, log_z, saved = bcjr.bcjr_forward(cd, wd, n, k, T, ws=wf)
    gw, gc = bcjr.bcjr_backward(cd, wd, n, k, T, saved, dev(g), dev(h), ws=wb)
    torch.cuda.synchronize()
    return {"w_hat": w_hat.cpu().numpy(), "log_z": log_z.cpu().numpy(), "grad_w": gw.cpu().numpy(),
            "grad_codebook": gc.cpu().numpy()}


# (n, B, L, T, histories): B above the 256 resident blocks of a 256-CU device
CASES = [
    (16, 300, 24, 0.3, ("full", "ckpt")),
    (16, 270, 7, 0.05, ("full", "ckpt")),   # ragged checkpoint segments (3, 3, 1)
    (15, 280, 20, 0.2, ("full",)),           # 2 blocks per lane
    (15, 280, 20, 0.02, ("full", "ckpt")),   # fp64 messages
    (14, 300, 16, 0.02, ("full",)),          # fp64 messages, 1 block per lane
    (16, 3, 1, 0.3, ("full", "ckpt")),       # L = 1: no recursion step at all
    (16, 3, 2, 0.3, ("full", "ckpt")),       # L = 2: one step each way
    (15, 2, 1, 0.02, ("full", "ckpt")),      # L = 1 with fp64 messages
]


@pytest.mark.parametrize("n,B,L,T,hists", CASES)
def test_wide_chains_match_oracle(n, B, L, T, hists):
    c = synth.normal(7100 + n, (1 << n,))
    w = synth.normal(7200 + n + L, (B, L))
    g = synth.normal(7300 + n + L, (B, L))
    h = synth.normal(7400 + n, (B,))
    ref = oracle.sparse_forward(n, 2, c, w, T)
    rb = oracle.sparse_backward(n, 2, c, w, T, g, h)
    for hist in hists:
        log_case(f"wide n={n} B={B} L={L} T={T} history={hist}")
        got = _run(n, c, w, g, h, T, hist == "ckpt")
        assert_normwise(got["w_hat"], ref["w_hat"], RTOL_FWD, f"{hist} w_hat")
        assert_rel(got["log_z"], ref["log_z"], RTOL_FWD, f"{hist} log_z")
        assert_normwise(got["grad_w"], rb["grad_w"], RTOL_GRAD, f"{hist} grad_w")
        assert_normwise(got["grad_codebook"], rb["grad_codebook"], RTOL_GRAD, f"{hist} grad_c")


@pytest.mark.parametrize("n,B,L,T", [(14, 256, 16, 0.02), (16, 260, 9, 0.3)])
def test_wide_bitwise_deterministic(n, B, L, T):
    """Repeated runs (one with a NaN-poisoned workspace) agree bitwise. The fp64-message chains
    mix double and float chain reductions; the fp32 ones read their accumulator rows back."""
    c = dev(synth.normal(7100 + n, (1 << n,)))
    w = dev(synth.normal(7200 + n + L, (B, L)))
    g = dev(synth.normal(7300 + n + L, (B, L)))
    h = dev(synth.normal(7400 + n, (B,)))
    log_case(f"wide determinism n={n} B={B} L={L} T={T}")
    outs = []
    for rep in range(3):
        wf = bcjr.workspace(n, 2, B, L, bcjr.FWD)
        wb = bcjr.workspace(n, 2, B, L, bcjr.BWD)
        wf.view(torch.uint8).fill_(0xFF if rep == 1 else 0)
        wb.view(torch.uint8).fill_(0xFF if rep == 1 else 0)
        w_hat, log_z, saved = bcjr.bcjr_forward(c, w, n, 2, T, ws=wf)
        gw, gc = bcjr.bcjr_backward(c, w, n, 2, T, saved, g, h, ws=wb)
        torch.cuda.synchronize()
        outs.append([x.cpu().numpy().copy() for x in (w_hat, log_z, gw, gc)])
    for other in outs[1:]:
        for a, b in zip(outs[0], other):
            assert np.all(np.isfinite(b))
            np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("T", [0.0299, 0.02, 0.01, 0.004, 0.001])
def test_2_16_states_below_the_floor_refused(T):
    """The 2^16-state trellis has no fp64-message kernels (their two message buffers would not
    fit LDS); with fp32 messages and the fp64 emission randomized sweeps put rare gradients at
    4e-3 at T = 0.02 and 5.5e-3 at 0.01: forward and backward refuse temperatures below 0.03 with
    BCJR_E_UNSUPPORTED, enqueue nothing and leave their outputs untouched."""
    n, B, L = 16, 5, 24
    log_case(f"n=16 refused T={T}")
    c = synth.normal(7500, (1 << n,))
    w = synth.normal(7501, (B, L))
    g = synth.normal(7502, (B, L))
    assert_refused(n, 2, c, w, T, g)


@pytest.mark.parametrize("seed,B,L", [(7500, 5, 24), (7600, 6, 40)])
@pytest.mark.parametrize("T", [0.045, 0.035, 0.03])
def test_2_16_states_below_threshold_fp64_emission(T, seed, B, L):
    """Below T = 0.05 the 2^16-state kernels keep fp32 messages and form the emission in fp64
    (w - c exactly, its square and its sum with the message in fp64). Against the oracle, both
    histories, on the input whose gradient erred by 0.51 at T = 0.002 with the fp32 emission
    (a near-tie between paths; seed 7500) and on a second one."""
    n = 16
    c = synth.normal(seed, (1 << n,))
    w = synth.normal(seed + 1, (B, L))
    g = synth.normal(seed + 2, (B, L))
    h = synth.normal(seed + 3, (B,))
    ref = oracle.sparse_forward(n, 2, c, w, T)
    rb = oracle.sparse_backward(n, 2, c, w, T, g, h)
    for hist in ("full", "ckpt"):
        log_case(f"n=16 T={T} seed={seed} history={hist}")
        got = _run(n, c, w, g, h, T, hist == "ckpt")
        assert_normwise(got["w_hat"], ref["w_hat"], RTOL_FWD, f"{hist} w_hat")
        assert_rel(got["log_z"], ref["log_z"], RTOL_FWD, f"{hist} log_z")
        assert_normwise(got["grad_w"], rb["grad_w"], RTOL_GRAD, f"{hist} grad_w")
        assert_normwise(got["grad_codebook"], rb["grad_codebook"], RTOL_GRAD, f"{hist} grad_c")


def test_2_16_states_at_the_threshold_match_oracle():
    """T = 0.05 exactly, the lowest temperature of the fp32 emission at 2^16 states, and T = 0.03
    (the fp64 emission at the floor), against the oracle on the input that erred by 0.51 at T = 0.002 with the
    fp32 emission."""
    for T in (0.05, 0.03):
        _threshold_case(T)


def _threshold_case(T):
    n, B, L = 16, 5, 24
    c = synth.normal(7500, (1 << n,))
    w = synth.normal(7501, (B, L))
    g = synth.normal(7502, (B, L))
    h = synth.normal(7503, (B,))
    ref = oracle.sparse_forward(n, 2, c, w, T)
    rb = oracle.sparse_backward(n, 2, c, w, T, g, h)
    for hist in ("full", "ckpt"):
        log_case(f"n=16 T={T} history={hist}")
        got = _run(n, c, w, g, h, T, hist == "ckpt")
        assert_normwise(got["w_hat"], ref["w_hat"], RTOL_FWD, f"{hist} w_hat")
        assert_rel(got["log_z"], ref["log_z"], RTOL_FWD, f"{hist} log_z")
        assert_normwise(got["grad_w"], rb["grad_w"], RTOL_GRAD, f"{hist} grad_w")
        assert_normwise(got["grad_codebook"], rb["grad_codebook"], RTOL_GRAD, f"{hist} grad_c")
