"""Conventions of the C ABI that hold for every trellis kernel, beyond agreement with the oracle:
- chains are independent: a NaN in one chain's weights reaches that chain's outputs and leaves
  every other chain's outputs bitwise unchanged, including chains that share a wave or a
  workspace slot with it (the codebook gradient, a sum over chains, is not compared);
- calls made at once from several host threads, each on its own stream, give the serial
  results bitwise;
- with no chains the codebook gradient (a sum over none) is written as zeros."""
import threading

import numpy as np
import pytest
import torch

from bcjr_soft_decoding_amd import bcjr, synth
from tests.gpu_helpers import dev, log_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bcjr.lib()


def _inputs(n, B, L, seed):
    rng = np.random.default_rng(seed)
    c = rng.standard_normal(1 << n).astype(np.float32)
    w = rng.standard_normal((B, L)).astype(np.float32)
    g = rng.standard_normal((B, L)).astype(np.float32)
    h = rng.standard_normal(B).astype(np.float32)
    return c, w, g, h


def _sparse(n, c, w, g, h, T, ckpt=False):
    k = 2
    B, L = w.shape
    cd, wd = dev(c), dev(w)
    wf = bcjr.workspace(n, k, B, L, bcjr.FWD_CKPT if ckpt else bcjr.FWD)
    wb = bcjr.workspace(n, k, B, L, bcjr.BWD_CKPT if ckpt else bcjr.BWD)
    w_hat, log_z, saved = bcjr.bcjr_forward(cd, wd, n, k, T, ws=wf)
    gw, gc = bcjr.bcjr_backward(cd, wd, n, k, T, saved, dev(g), dev(h), ws=wb)
    states, w_hard = bcjr.viterbi_decode(cd, wd, n, k)
    torch.cuda.synchronize()
    return {"w_hat": w_hat, "log_z": log_z, "grad_w": gw, "states": states, "w_hard": w_hard,
            "grad_codebook": gc}


def _check_isolated(clean, poisoned, j, what):
    for key, a in clean.items():
        if key == "grad_codebook":  # a sum over chains
            continue
        a = a.cpu().numpy()
        b = poisoned[key].cpu().numpy()
        others = np.arange(a.shape[0]) != j
        assert np.array_equal(a[others].view(np.uint8), b[others].view(np.uint8)), \
            f"{what}: {key} of another chain changed"
    assert np.isnan(poisoned["log_z"][j].item()), f"{what}: the NaN did not reach log Z"


# (n, B, L, T, checkpointed history): chains that share a wave (S = 16, 256), one or two waves
# per chain (S = 4096), 1024-lane chains with fp32 and fp64 messages
CASES = [
    (4, 70, 33, 0.3, False),
    (8, 90, 40, 0.1, False),
    (8, 90, 40, 0.1, True),
    (12, 20, 30, 0.1, False),
    (14, 5, 12, 0.02, False),
    (16, 5, 10, 0.3, False),
]


@pytest.mark.parametrize("n,B,L,T,ckpt", CASES)
def test_nan_stays_in_its_chain(n, B, L, T, ckpt):
    log_case(f"NaN isolation n={n} B={B} L={L} T={T} ckpt={ckpt}")
    c, w, g, h = _inputs(n, B, L, 100 + n)
    clean = _sparse(n, c, w, g, h, T, ckpt)
    j = B // 2 + 1
    w2 = w.copy()
    w2[j, L // 2] = np.nan
    poisoned = _sparse(n, c, w2, g, h, T, ckpt)
    _check_isolated(clean, poisoned, j, f"n={n}")
    assert np.all(np.isnan(poisoned["w_hat"][j].cpu().numpy())), "NaN did not reach w_hat"


# NaN or Inf in the inputs propagates (nothing is checked or reported): a non-finite weight
# makes its chain's w_hat, log_z and grad_w NaN and, through the sum over chains, the codebook
# gradient; a non-finite codebook entry or theta entry reaches every chain.
@pytest.mark.parametrize("n,B,L,T", [(8, 20, 30, 0.3), (12, 6, 20, 0.1), (10, 6, 20, 0.005),
                                     (16, 3, 8, 0.3)])
@pytest.mark.parametrize("bad", [float("nan"), float("inf"), -float("inf")])
def test_non_finite_weight_propagates(n, B, L, T, bad):
    log_case(f"non-finite weight {bad} n={n} B={B} L={L} T={T}")
    c, w, g, h = _inputs(n, B, L, 300 + n)
    j = B // 2
    w[j, L // 3] = bad
    out = _sparse(n, c, w, g, h, T)
    for key in ("w_hat", "grad_w"):
        assert np.all(np.isnan(out[key][j].cpu().numpy())), f"{key} of the chain is not all NaN"
    assert np.isnan(out["log_z"][j].item())
    assert np.all(np.isnan(out["grad_codebook"].cpu().numpy())), "grad_codebook is not all NaN"


@pytest.mark.parametrize("n", [8, 16])
def test_non_finite_codebook_entry_reaches_every_chain(n):
    log_case(f"NaN codebook entry n={n}")
    B, L, T = 4, 12, 0.3
    c, w, g, h = _inputs(n, B, L, 400 + n)
    c[(1 << n) // 3] = np.nan
    out = _sparse(n, c, w, g, h, T)
    for key in ("w_hat", "log_z", "grad_w", "grad_codebook"):
        assert np.all(np.isnan(out[key].cpu().numpy())), f"{key} is not all NaN"


def test_non_finite_dense_inputs_propagate():
    S, B, L, T = 64, 6, 16, 0.3
    rng = np.random.default_rng(19)
    theta = rng.standard_normal((S, S)).astype(np.float32)
    c = rng.standard_normal(S).astype(np.float32)
    w = rng.standard_normal((B, L)).astype(np.float32)
    g = rng.standard_normal((B, L)).astype(np.float32)

    def run(th, ww):
        wh, lz, sv = bcjr.bcjr_dense_forward(dev(th), dev(c), dev(ww), T)
        gw, gc, gt = bcjr.bcjr_dense_backward(dev(th), dev(c), dev(ww), T, sv, dev(g))
        torch.cuda.synchronize()
        return {k: v.cpu().numpy() for k, v in
                dict(w_hat=wh, log_z=lz, grad_w=gw, grad_codebook=gc, grad_theta=gt).items()}

    log_case("dense: NaN weight")
    w2 = w.copy()
    w2[2, 7] = np.nan
    out = run(theta, w2)
    for key in ("w_hat", "grad_w"):
        assert np.all(np.isnan(out[key][2])), key
    assert np.isnan(out["log_z"][2])
    assert np.all(np.isnan(out["grad_codebook"])) and np.all(np.isnan(out["grad_theta"]))
    log_case("dense: NaN theta entry")
    th2 = theta.copy()
    th2[5, 9] = np.nan
    out = run(th2, w)
    for key, v in out.items():
        assert np.all(np.isnan(v)), key


def test_nan_stays_in_its_chain_segmented_and_dense():
    n, B, L, T = 8, 40, 96, 0.1
    log_case(f"NaN isolation, segmented n={n} B={B} L={L}")
    c, w, g, _ = _inputs(n, B, L, 7)
    j = 13
    w2 = w.copy()
    w2[j, 5] = np.nan
    outs = []
    for ww in (w, w2):
        wh, lz = bcjr.bcjr_forward_scan(dev(c), dev(ww), n, 2, T, seg_len=16)
        gw, _ = bcjr.bcjr_backward_scan(dev(c), dev(ww), n, 2, T, wh, dev(g), seg_len=16)
        torch.cuda.synchronize()
        outs.append({"w_hat": wh, "log_z": lz, "grad_w": gw})
    _check_isolated(outs[0], outs[1], j, "segmented")

    S, B, L, T = 64, 30, 20, 0.2
    log_case(f"NaN isolation, dense S={S} B={B} L={L}")
    rng = np.random.default_rng(9)
    theta = rng.standard_normal((S, S)).astype(np.float32)
    c = rng.standard_normal(S).astype(np.float32)
    w = rng.standard_normal((B, L)).astype(np.float32)
    g = rng.standard_normal((B, L)).astype(np.float32)
    w2 = w.copy()
    w2[j, 3] = np.nan
    outs = []
    for ww in (w, w2):
        wh, lz, saved = bcjr.bcjr_dense_forward(dev(theta), dev(c), dev(ww), T)
        gw, _, _ = bcjr.bcjr_dense_backward(dev(theta), dev(c), dev(ww), T, saved, dev(g))
        torch.cuda.synchronize()
        outs.append({"w_hat": wh, "log_z": lz, "grad_w": gw})
    _check_isolated(outs[0], outs[1], j, "dense")


def test_threads_on_their_own_streams_match_serial():
    """Two host threads, each issuing forward, backward and Viterbi calls on its own stream
    (default priority) four times over, while the other does the same."""
    jobs = [(12, 300, 64, 0.1, 1), (8, 3000, 128, 0.3, 2)]
    inputs = [_inputs(n, B, L, seed) for n, B, L, _, seed in jobs]
    log_case("threads: serial reference")
    ref = [_sparse(n, *inp, T) for (n, _, _, T, _), inp in zip(jobs, inputs)]
    results = [[] for _ in jobs]
    errors = []

    def work(i):
        try:
            n, _, _, T, _ = jobs[i]
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(4):
                    out = _sparse_on_stream(n, *inputs[i], T)
                    results[i].append(out)
            s.synchronize()
        except Exception as e:  # reported by the main thread
            errors.append(e)

    log_case("threads: two concurrent workers")
    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(jobs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    for i, runs in enumerate(results):
        assert len(runs) == 4
        for out in runs:
            for key, a in ref[i].items():
                assert np.array_equal(a.cpu().numpy().view(np.uint8),
                                      out[key].cpu().numpy().view(np.uint8)), (i, key)


def _sparse_on_stream(n, c, w, g, h, T):
    """As _sparse, synchronising only the current stream (the other worker keeps running)."""
    k = 2
    B, L = w.shape
    cd, wd = dev(c), dev(w)
    w_hat, log_z, saved = bcjr.bcjr_forward(cd, wd, n, k, T)
    gw, gc = bcjr.bcjr_backward(cd, wd, n, k, T, saved, dev(g), dev(h))
    states, w_hard = bcjr.viterbi_decode(cd, wd, n, k)
    torch.cuda.current_stream().synchronize()
    return {"w_hat": w_hat, "log_z": log_z, "grad_w": gw, "states": states, "w_hard": w_hard,
            "grad_codebook": gc}


@pytest.mark.parametrize("n,T,ckpt", [(8, 0.5, False), (8, 0.5, True), (15, 0.02, False),
                                      (16, 0.3, False), (16, 0.3, True)])
def test_zero_chains_overwrite_the_codebook_gradient(n, T, ckpt):
    """B = 0: the codebook gradient (a sum over no chains) is written as zeros over a
    NaN-filled buffer, and the other outputs are empty."""
    log_case(f"B=0 n={n} T={T} ckpt={ckpt}")
    k, L = 2, 9
    c = dev(synth.normal(40 + n, (1 << n,)))
    w = torch.empty((0, L), dtype=torch.float32, device="cuda")
    wf = bcjr.workspace(n, k, 0, L, bcjr.FWD_CKPT if ckpt else bcjr.FWD)
    wb = bcjr.workspace(n, k, 0, L, bcjr.BWD_CKPT if ckpt else bcjr.BWD)
    w_hat, log_z, saved = bcjr.bcjr_forward(c, w, n, k, T, ws=wf)
    gc = torch.full((1 << n,), float("nan"), dtype=torch.float32, device="cuda")
    gw, gc2 = bcjr.bcjr_backward(c, w, n, k, T, saved, torch.empty_like(w), grad_codebook=gc, ws=wb)
    states, w_hard = bcjr.viterbi_decode(c, w, n, k)
    torch.cuda.synchronize()
    assert w_hat.numel() == 0 and log_z.numel() == 0 and gw.numel() == 0 and states.numel() == 0
    assert gc2.data_ptr() == gc.data_ptr()
    assert torch.count_nonzero(gc).item() == 0 and not torch.isnan(gc).any().item()
