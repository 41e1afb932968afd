"""The oracle's pins must catch plausible mistakes (CPU only).

Each case plants one mistake in a private copy of the oracle's C source (a dropped term, a
wrong sign, an off-by-one index, a transposed operand), builds it, and checks that the
brute-force pins then fail. Nothing here touches the GPU or the HIP library.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

from bcjr_soft_decoding_amd import synth
from tests import bruteforce as bf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "bcjr_oracle.c")

MUTATIONS = {
    "beta_drops_future_emission": ("b->ell[(t + 1) * S + sp] + b->beta[(t + 1) * S + sp]",
                                   "b->beta[(t + 1) * S + sp]"),
    "pred_wrong_shift": ("(sp >> v->k) | (a << (v->n - v->k))", "(sp >> v->k) | (a << (v->k))"),
    "emission_sign": ("b->ell[t * S + s] = -(d * d) / T;", "b->ell[t * S + s] = -(d * d) * T;"),
    "fwd_uses_current_g": ("(fwd[(t - 1) * S + s] + (double)gq[t - 1] * (double)c[s])",
                           "(fwd[(t - 1) * S + s] + (double)gq[t] * (double)c[s])"),
    "bwd_transposed_codeword": ("(bwd[(t + 1) * S + sp] + (double)gq[t + 1] * (double)c[sp])",
                                "(bwd[(t + 1) * S + sp] + (double)gq[t + 1] * (double)c[s])"),
    "mu_dropped": ("+ bwd[t * S + s] - mu);", "+ bwd[t * S + s]);"),
    "grad_c_sign": ("(2.0 / T) * (wt - (double)c[s]) * (D + hq * gm)",
                    "(2.0 / T) * ((double)c[s] - wt) * (D + hq * gm)"),
    "grad_w_h_term_dropped": ("(2.0 / T) * acc - (2.0 * hq / T) * (wt - what[t])", "(2.0 / T) * acc"),
}


def _build(name, old, new, tmp_path):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / f"{name}.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-shared",
                           "-fPIC", "-o", str(so), str(path), "-lm"])
    lib = ctypes.CDLL(str(so))
    P, I, Lg, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_long, ctypes.c_double
    lib.oracle_sparse_forward.argtypes = [I, I, P, P, Lg, Lg, D, P, P, P, P, P]
    lib.oracle_sparse_backward.argtypes = [I, I, P, P, Lg, Lg, D, P, P, P, P]
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _pins_pass(lib):
    n, k, L, T = 5, 2, 6, 0.3
    c = synth.normal(901, (32,))
    w = synth.normal(902, (2, L))
    g = synth.normal(903, (2, L))
    h = np.array([0.5, -0.8], np.float32)
    what = np.empty((2, L)); logz = np.empty(2)
    lib.oracle_sparse_forward(n, k, _p(c), _p(w), 2, L, T, _p(what), _p(logz), None, None, None)
    gw = np.empty((2, L)); gc = np.empty(32)
    lib.oracle_sparse_backward(n, k, _p(c), _p(w), 2, L, T, _p(g), _p(h), _p(gw), _p(gc))
    paths = bf.bitshift_paths(n, k, L)
    gc_ref = np.zeros(32)
    ok = True
    for b in range(2):
        ex = bf.exact_stats(paths, c, w[b], T, 32, g=g[b], h=float(h[b]))
        ok &= np.allclose(logz[b], ex["log_z"], rtol=1e-9)
        ok &= np.allclose(what[b], ex["w_hat"], rtol=1e-8, atol=1e-10)
        ok &= np.allclose(gw[b], ex["grad_w"], rtol=1e-7, atol=1e-9)
        gc_ref += ex["grad_c"]
    ok &= np.allclose(gc, gc_ref, rtol=1e-7, atol=1e-9)
    return bool(ok)


def test_unmutated_oracle_passes(tmp_path):
    src = open(SRC).read()
    lib = _build("clean", src[:40], src[:40], tmp_path)
    assert _pins_pass(lib)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    lib = _build(name, old, new, tmp_path)
    assert not _pins_pass(lib), f"planted mistake '{name}' was not caught by the pins"
