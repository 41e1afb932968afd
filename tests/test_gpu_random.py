"""Seeded random shapes against the oracle: bitshift trellises n = 4..16 with random B, L, T,
history layout and upstream log Z gradient (plus Viterbi bit-exactness), and the segmented and
dense paths with random lengths, segment lengths and sizes. The cases are drawn once, at import,
from fixed seeds, so every run checks the same ones. log Z is compared normwise like the other
outputs: its fp32 error scales with the size of the summed terms, so a chain whose log Z happens
to lie near zero would fail a purely relative test. Below each state size's temperature floor
(0.002 for n <= 12, 0.015 for n = 13..15, 0.03 for n = 16) the library refuses the call
(BCJR_E_UNSUPPORTED): such draws check the refusal."""
import numpy as np
import pytest
import torch

import oracle
from bcjr_soft_decoding_amd import bcjr
from tests.gpu_helpers import RTOL_FWD, RTOL_GRAD, assert_normwise, assert_refused, dev, log_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bcjr.lib()


def _sparse_cases(seed, count):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        n = int(rng.integers(4, 17))
        L = int(rng.integers(1, 300))
        B = int(rng.integers(1, int(max(1, min(400, 3e7 // (L * (1 << n)) + 1))) + 1))
        T = float(rng.choice([0.004, 0.02, 0.08, 0.3, 1.0, 4.0]))
        ckpt = bool(rng.integers(0, 2))
        data_seed = int(rng.integers(0, 1 << 30))
        with_h = bool(rng.integers(0, 2))
        out.append((n, B, L, T, ckpt, with_h, data_seed))
    return out


def _other_cases(seed, count):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        data_seed = int(rng.integers(0, 1 << 30))
        if i % 2 == 0:
            n = int(rng.integers(4, 11))
            L = int(rng.integers(16, 3000))
            B = int(rng.integers(1, max(2, min(8, int(2e7 // (L * (1 << n))) + 1))))
            T = float(rng.choice([0.006, 0.02, 0.1, 0.5, 2.0]))
            seg = int(rng.choice([0, 0, int(rng.integers(16, max(17, L // 2 + 1)))]))
            out.append(("scan", n, B, L, T, seg, bool(rng.integers(0, 2)), data_seed))
        else:
            S = int(rng.choice([32, 64, 128, 256]))
            B = int(rng.integers(1, 40))
            L = int(rng.integers(1, 120))
            T = float(rng.choice([0.1, 0.2, 1.0, 3.0]))
            out.append(("dense", S, B, L, T, 0, bool(rng.integers(0, 2)), data_seed))
    return out


SPARSE = _sparse_cases(3, 80)
OTHER = _other_cases(5, 50)


@pytest.mark.parametrize("n,B,L,T,ckpt,with_h,data_seed", SPARSE)
def test_random_bitshift_shapes(n, B, L, T, ckpt, with_h, data_seed):
    log_case(f"random n={n} B={B} L={L} T={T} ckpt={ckpt} h={with_h} seed={data_seed}")
    r = np.random.default_rng(data_seed)
    c = r.standard_normal(1 << n).astype(np.float32)
    w = (r.standard_normal((B, L)) * r.choice([0.3, 1.0, 2.0])).astype(np.float32)
    g = r.standard_normal((B, L)).astype(np.float32)
    h = r.standard_normal(B).astype(np.float32) if with_h else None
    if T < (0.002 if n <= 12 else 0.015 if n <= 15 else 0.03):
        assert_refused(n, 2, c, w, T, g)
        return
    ref = oracle.sparse_forward(n, 2, c, w, T)
    rb = oracle.sparse_backward(n, 2, c, w, T, g, h)
    cd, wd = dev(c), dev(w)
    wf = bcjr.workspace(n, 2, B, L, bcjr.FWD_CKPT if ckpt else bcjr.FWD)
    wb = bcjr.workspace(n, 2, B, L, bcjr.BWD_CKPT if ckpt else bcjr.BWD)
    w_hat, log_z, saved = bcjr.bcjr_forward(cd, wd, n, 2, T, ws=wf)
    gw, gc = bcjr.bcjr_backward(cd, wd, n, 2, T, saved, dev(g), None if h is None else dev(h), ws=wb)
    states, _ = bcjr.viterbi_decode(cd, wd, n, 2)
    torch.cuda.synchronize()
    assert_normwise(w_hat.cpu().numpy(), ref["w_hat"], RTOL_FWD, "w_hat")
    assert_normwise(log_z.cpu().numpy(), ref["log_z"], RTOL_FWD, "log_z")
    assert_normwise(gw.cpu().numpy(), rb["grad_w"], RTOL_GRAD, "grad_w")
    assert_normwise(gc.cpu().numpy(), rb["grad_codebook"], RTOL_GRAD, "grad_c")
    np.testing.assert_array_equal(states.cpu().numpy(), oracle.viterbi(n, 2, c, w)["states"])


@pytest.mark.parametrize("path,size,B,L,T,seg,with_h,data_seed", OTHER)
def test_random_segmented_and_dense_shapes(path, size, B, L, T, seg, with_h, data_seed):
    log_case(f"random {path} size={size} B={B} L={L} T={T} seg={seg} h={with_h} seed={data_seed}")
    r = np.random.default_rng(data_seed)
    if path == "scan":
        n = size
        c = r.standard_normal(1 << n).astype(np.float32)
        w = (r.standard_normal((B, L)) * r.choice([0.5, 1.0, 2.0])).astype(np.float32)
        g = r.standard_normal((B, L)).astype(np.float32)
        h = r.standard_normal(B).astype(np.float32) if with_h else None
        wh, lz = bcjr.bcjr_forward_scan(dev(c), dev(w), n, 2, T, seg)
        gw, gc = bcjr.bcjr_backward_scan(dev(c), dev(w), n, 2, T, wh, dev(g),
                                         None if h is None else dev(h), seg)
        torch.cuda.synchronize()
        ref = oracle.sparse_forward(n, 2, c, w, T)
        rb = oracle.sparse_backward(n, 2, c, w, T, g, h)
        grads = [(gw, rb["grad_w"], "grad_w"), (gc, rb["grad_codebook"], "grad_c")]
    else:
        S = size
        theta = r.standard_normal((S, S)).astype(np.float32)
        c = r.standard_normal(S).astype(np.float32)
        w = r.standard_normal((B, L)).astype(np.float32)
        g = r.standard_normal((B, L)).astype(np.float32)
        h = r.standard_normal(B).astype(np.float32) if with_h else None
        wh, lz, saved = bcjr.bcjr_dense_forward(dev(theta), dev(c), dev(w), T)
        gw, gc, gt = bcjr.bcjr_dense_backward(dev(theta), dev(c), dev(w), T, saved, dev(g),
                                              None if h is None else dev(h))
        torch.cuda.synchronize()
        ref = oracle.dense_forward(theta, c, w, T)
        rb = oracle.dense_backward(theta, c, w, T, g, h)
        grads = [(gw, rb["grad_w"], "grad_w"), (gc, rb["grad_codebook"], "grad_c"),
                 (gt, rb["grad_theta"], "grad_theta")]
    assert_normwise(wh.cpu().numpy(), ref["w_hat"], RTOL_FWD, "w_hat")
    assert_normwise(lz.cpu().numpy(), ref["log_z"], RTOL_FWD, "log_z")
    for got, want, what in grads:
        assert_normwise(got.cpu().numpy(), want, RTOL_GRAD, what)
