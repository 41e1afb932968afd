"""ctypes front end of the plain C oracle (``bcjr_oracle.c``) -- test infrastructure only.

Every function takes the fp32 inputs exactly as the GPU library receives them and returns
float64 results (the Viterbi decoder returns the fp32 path it defines). See the C file's
header for the method, its source passages and the readings taken where the pages are silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bcjr_oracle.c")
# BCJR_SANITIZE=1 (the CPU sanitizer run, tests/run_sanitizers.py) selects the build with
# AddressSanitizer and UndefinedBehaviorSanitizer.
_SANITIZE = os.environ.get("BCJR_SANITIZE") == "1"
_LIB_PATH = os.path.join(_HERE, "liboracle_san.so" if _SANITIZE else "liboracle.so")
_lib = None

_CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-shared", "-fPIC"]
# The sanitized build uses clang, whose sanitizer runtime the HIP library's sanitized build
# (hipcc, i.e. clang) shares: one process cannot hold two sanitizer runtimes.
_CLANG_DIR = "/opt/rocm/llvm"
_SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def build(force: bool = True, sanitize: bool | None = None) -> str:
    """Compile the oracle with gcc into ``oracle/liboracle.so`` (with ``sanitize``, with clang
    and the address and undefined-behaviour sanitizers into ``oracle/liboracle_san.so``)."""
    sanitize = _SANITIZE if sanitize is None else sanitize
    path = os.path.join(_HERE, "liboracle_san.so" if sanitize else "liboracle.so")
    if force or not os.path.exists(path):
        tmp = path + ".tmp"
        if sanitize:
            lib = os.path.join(_CLANG_DIR, "lib")
            subprocess.check_call([os.path.join(_CLANG_DIR, "bin", "clang"), *_CFLAGS, *_SAN_FLAGS,
                                   "-o", tmp, _SRC, "-lm", f"-L{lib}", f"-Wl,-rpath,{lib}"])
        else:
            subprocess.check_call(["gcc", *_CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, path)
    return path


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I, Lg, D = ctypes.c_int, ctypes.c_long, ctypes.c_double
    lib.oracle_sparse_forward.argtypes = [I, I, P, P, Lg, Lg, D, P, P, P, P, P]
    lib.oracle_sparse_backward.argtypes = [I, I, P, P, Lg, Lg, D, P, P, P, P]
    lib.oracle_dense_forward.argtypes = [I, P, P, P, Lg, Lg, D, P, P, P]
    lib.oracle_dense_backward.argtypes = [I, P, P, P, Lg, Lg, D, P, P, P, P, P]
    lib.oracle_viterbi_f32.argtypes = [I, I, P, P, Lg, Lg, P, P, P]
    lib.oracle_viterbi_f64.argtypes = [I, I, P, P, Lg, Lg, P, P, P]
    lib.oracle_set_threads.argtypes = [I]
    lib.oracle_code_words.argtypes = [I, I, Lg]
    lib.oracle_code_words.restype = Lg
    lib.oracle_pack_states.argtypes = [I, I, P, Lg, Lg, P, P]
    lib.oracle_unpack_code.argtypes = [I, I, P, P, Lg, Lg, P, P]
    for name in ("oracle_sparse_forward", "oracle_sparse_backward", "oracle_dense_forward",
                 "oracle_dense_backward", "oracle_viterbi_f32", "oracle_viterbi_f64",
                 "oracle_set_threads", "oracle_pack_states", "oracle_unpack_code"):
        getattr(lib, name).restype = I
    _lib = lib
    return lib


def _f32(x):
    return np.ascontiguousarray(x, dtype=np.float32)


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with code {rc}")


def set_threads(n: int = 0) -> int:
    """Set the OpenMP thread count (0 keeps it) and return the count in effect."""
    return int(_load().oracle_set_threads(int(n)))


def sparse_forward(n, k, codebook, w, T, want_gamma=False, want_alpha_beta=False):
    """Bitshift trellis forward-backward. Returns a dict with ``w_hat`` [B,L], ``log_z`` [B]
    and, on request, ``gamma``/``alpha``/``beta`` [B,L,S] (natural-log units)."""
    lib = _load()
    c, w = _f32(codebook), _f32(w)
    B, L = w.shape
    S = 1 << n
    assert c.shape == (S,)
    what = np.empty((B, L), np.float64)
    logz = np.empty((B,), np.float64)
    gamma = np.empty((B, L, S), np.float64) if want_gamma else None
    alpha = np.empty((B, L, S), np.float64) if want_alpha_beta else None
    beta = np.empty((B, L, S), np.float64) if want_alpha_beta else None
    _check(lib.oracle_sparse_forward(n, k, _p(c), _p(w), B, L, float(T), _p(what), _p(logz),
                                     _p(gamma), _p(alpha), _p(beta)), "sparse_forward")
    out = {"w_hat": what, "log_z": logz}
    if want_gamma:
        out["gamma"] = gamma
    if want_alpha_beta:
        out["alpha"], out["beta"] = alpha, beta
    return out


def sparse_backward(n, k, codebook, w, T, g, h=None):
    """Gradient of sum(g * w_hat) + sum(h * log_z) w.r.t. w [B,L] and codebook [S]."""
    lib = _load()
    c, w, g = _f32(codebook), _f32(w), _f32(g)
    B, L = w.shape
    S = 1 << n
    assert c.shape == (S,) and g.shape == (B, L)
    hh = None if h is None else _f32(h)
    gw = np.empty((B, L), np.float64)
    gc = np.empty((S,), np.float64)
    _check(lib.oracle_sparse_backward(n, k, _p(c), _p(w), B, L, float(T), _p(g), _p(hh), _p(gw),
                                      _p(gc)), "sparse_backward")
    return {"grad_w": gw, "grad_codebook": gc}


def dense_forward(theta, codebook, w, T, want_gamma=False):
    lib = _load()
    th, c, w = _f32(theta), _f32(codebook), _f32(w)
    S = c.shape[0]
    B, L = w.shape
    assert th.shape == (S, S)
    what = np.empty((B, L), np.float64)
    logz = np.empty((B,), np.float64)
    gamma = np.empty((B, L, S), np.float64) if want_gamma else None
    _check(lib.oracle_dense_forward(S, _p(th), _p(c), _p(w), B, L, float(T), _p(what), _p(logz),
                                    _p(gamma)), "dense_forward")
    out = {"w_hat": what, "log_z": logz}
    if want_gamma:
        out["gamma"] = gamma
    return out


def dense_backward(theta, codebook, w, T, g, h=None):
    lib = _load()
    th, c, w, g = _f32(theta), _f32(codebook), _f32(w), _f32(g)
    S = c.shape[0]
    B, L = w.shape
    hh = None if h is None else _f32(h)
    gw = np.empty((B, L), np.float64)
    gc = np.empty((S,), np.float64)
    gt = np.empty((S, S), np.float64)
    _check(lib.oracle_dense_backward(S, _p(th), _p(c), _p(w), B, L, float(T), _p(g), _p(hh),
                                     _p(gw), _p(gc), _p(gt)), "dense_backward")
    return {"grad_w": gw, "grad_codebook": gc, "grad_theta": gt}


def viterbi(n, k, codebook, w, precision="f32"):
    """Hard decode. Returns ``states`` int32 [B,L], ``w_hard`` fp32 [B,L], ``energy`` [B]."""
    lib = _load()
    c, w = _f32(codebook), _f32(w)
    B, L = w.shape
    states = np.empty((B, L), np.int32)
    w_hard = np.empty((B, L), np.float32)
    energy = np.empty((B,), np.float64)
    fn = lib.oracle_viterbi_f32 if precision == "f32" else lib.oracle_viterbi_f64
    _check(fn(n, k, _p(c), _p(w), B, L, _p(states), _p(w_hard), _p(energy)), "viterbi")
    return {"states": states, "w_hard": w_hard, "energy": energy}


def code_words(n: int, k: int, L: int) -> int:
    return int(_load().oracle_code_words(n, k, L))


def pack_states(n, k, states):
    """Hard code of every chain: uint32 [B, words]; also the number of non-successor steps."""
    lib = _load()
    st = np.ascontiguousarray(states, dtype=np.int32)
    B, L = st.shape
    code = np.zeros((B, code_words(n, k, L)), np.uint32)
    bad = ctypes.c_long(0)
    _check(lib.oracle_pack_states(n, k, _p(st), B, L, _p(code), ctypes.byref(bad)), "pack_states")
    return code, int(bad.value)


def unpack_code(n, k, codebook, code, L):
    """States int32 [B, L] and w_hard = c(states) fp32 [B, L] from the hard code."""
    lib = _load()
    c = _f32(codebook)
    cd = np.ascontiguousarray(code, dtype=np.uint32)
    B = cd.shape[0]
    states = np.empty((B, L), np.int32)
    w_hard = np.empty((B, L), np.float32)
    _check(lib.oracle_unpack_code(n, k, _p(c), _p(cd), B, L, _p(states), _p(w_hard)), "unpack_code")
    return states, w_hard
