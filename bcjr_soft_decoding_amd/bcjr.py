"""Thin ctypes binding of ``libbcjr.so`` (C ABI in ``include/bcjr.h``).

The functions carry the C names. They only marshal arguments: torch supplies device memory
and the current stream, the library does every step of the computation in HIP kernels.
If the library is missing the import of any function raises; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# BCJR_LIB may point at another build of the same library (e.g. a tuning variant).
LIB_PATH = os.environ.get("BCJR_LIB", os.path.join(_PKG, "_lib", "libbcjr.so"))

BCJR_OK, BCJR_E_ARG, BCJR_E_SHAPE, BCJR_E_WORKSPACE, BCJR_E_DEVICE, BCJR_E_UNSUPPORTED = range(6)
FWD, BWD, VIT, FWD_CKPT, BWD_CKPT = 0, 1, 2, 3, 4

EXPORTED = (
    "bcjr_supported", "bcjr_saved_bytes", "bcjr_workspace_bytes", "bcjr_forward",
    "bcjr_backward", "viterbi_decode", "bcjr_dense_supported", "bcjr_dense_saved_bytes",
    "bcjr_dense_workspace_bytes", "bcjr_dense_forward", "bcjr_dense_backward",
    "bcjr_code_words", "bcjr_pack_code", "bcjr_unpack_code", "bcjr_status_string",
    "bcjr_scan_segment_length", "bcjr_scan_workspace_bytes", "bcjr_forward_scan",
    "bcjr_scan_backward_workspace_bytes", "bcjr_backward_scan",
)


class BcjrError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: status {status} ({status_text(status)})")
        self.status = status


class Trellis(ctypes.Structure):
    _fields_ = [
        ("state_bits", ctypes.c_int32),
        ("bits_per_step", ctypes.c_int32),
        ("weights_per_step", ctypes.c_int32),
        ("codebook", ctypes.c_void_p),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load the HIP library (raises FileNotFoundError if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise FileNotFoundError(
            f"{LIB_PATH} is missing: build it with `python -m bcjr_soft_decoding_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I64, I32, F, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    TP = ctypes.POINTER(Trellis)
    L.bcjr_supported.argtypes = [TP]
    L.bcjr_supported.restype = ctypes.c_int
    L.bcjr_saved_bytes.argtypes = [TP, I64, I64]
    L.bcjr_saved_bytes.restype = SZ
    L.bcjr_workspace_bytes.argtypes = [TP, I64, I64, ctypes.c_int]
    L.bcjr_workspace_bytes.restype = SZ
    L.bcjr_forward.argtypes = [TP, P, I64, I64, F, P, P, P, P, SZ, P]
    L.bcjr_forward.restype = ctypes.c_int
    L.bcjr_backward.argtypes = [TP, P, I64, I64, F, P, P, P, P, P, P, SZ, P]
    L.bcjr_backward.restype = ctypes.c_int
    L.viterbi_decode.argtypes = [TP, P, I64, I64, P, P, P, SZ, P]
    L.viterbi_decode.restype = ctypes.c_int
    L.bcjr_dense_supported.argtypes = [I32]
    L.bcjr_dense_supported.restype = ctypes.c_int
    L.bcjr_dense_saved_bytes.argtypes = [I32, I64, I64]
    L.bcjr_dense_saved_bytes.restype = SZ
    L.bcjr_dense_workspace_bytes.argtypes = [I32, I64, I64, ctypes.c_int]
    L.bcjr_dense_workspace_bytes.restype = SZ
    L.bcjr_dense_forward.argtypes = [I32, P, P, P, I64, I64, F, P, P, P, P, SZ, P]
    L.bcjr_dense_forward.restype = ctypes.c_int
    L.bcjr_dense_backward.argtypes = [I32, P, P, P, I64, I64, F, P, P, P, P, P, P, P, SZ, P]
    L.bcjr_dense_backward.restype = ctypes.c_int
    L.bcjr_code_words.argtypes = [TP, I64]
    L.bcjr_code_words.restype = I64
    L.bcjr_pack_code.argtypes = [TP, P, I64, I64, P, P]
    L.bcjr_pack_code.restype = ctypes.c_int
    L.bcjr_unpack_code.argtypes = [TP, P, I64, I64, P, P, P]
    L.bcjr_unpack_code.restype = ctypes.c_int
    L.bcjr_scan_segment_length.argtypes = [TP, I64, I64, I64]
    L.bcjr_scan_segment_length.restype = I64
    L.bcjr_scan_workspace_bytes.argtypes = [TP, I64, I64, I64]
    L.bcjr_scan_workspace_bytes.restype = SZ
    L.bcjr_forward_scan.argtypes = [TP, P, I64, I64, F, I64, P, P, P, SZ, P]
    L.bcjr_forward_scan.restype = ctypes.c_int
    L.bcjr_scan_backward_workspace_bytes.argtypes = [TP, I64, I64, I64]
    L.bcjr_scan_backward_workspace_bytes.restype = SZ
    L.bcjr_backward_scan.argtypes = [TP, P, I64, I64, F, I64, P, P, P, P, P, P, SZ, P]
    L.bcjr_backward_scan.restype = ctypes.c_int
    L.bcjr_status_string.argtypes = [ctypes.c_int]
    L.bcjr_status_string.restype = ctypes.c_char_p
    _lib = L
    return L


def status_text(status: int) -> str:
    return lib().bcjr_status_string(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def trellis(n: int, k: int, codebook=None, v: int = 1) -> Trellis:
    return Trellis(int(n), int(k), int(v), None if codebook is None else codebook.data_ptr())


def _check(st: int, what: str):
    if st != BCJR_OK:
        raise BcjrError(st, what)


def _f32(t, name):
    if not (t.dtype == torch.float32 and t.is_cuda and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous float32 CUDA tensor")
    return t


def bcjr_supported(n: int, k: int, v: int = 1) -> bool:
    tr = trellis(n, k, None, v)
    return bool(lib().bcjr_supported(ctypes.byref(tr)))


def bcjr_saved_bytes(n: int, k: int, B: int, L: int) -> int:
    tr = trellis(n, k)
    return int(lib().bcjr_saved_bytes(ctypes.byref(tr), B, L))


def bcjr_workspace_bytes(n: int, k: int, B: int, L: int, which: int) -> int:
    tr = trellis(n, k)
    return int(lib().bcjr_workspace_bytes(ctypes.byref(tr), B, L, which))


def workspace(n, k, B, L, which, device="cuda"):
    """Allocate a device workspace of the queried size (uint8 tensor)."""
    nb = bcjr_workspace_bytes(n, k, B, L, which)
    return torch.empty(max(nb, 1), dtype=torch.uint8, device=device)


def bcjr_forward(codebook, w, n, k, T, w_hat=None, log_z=None, saved=None, ws=None):
    """Soft codeword w_hat [B,L] and log Z [B]; returns (w_hat, log_z, saved)."""
    _f32(codebook, "codebook"); _f32(w, "w")
    B, L = w.shape
    dev = w.device
    w_hat = torch.empty_like(w) if w_hat is None else w_hat
    log_z = torch.empty(B, dtype=torch.float32, device=dev) if log_z is None else log_z
    if saved is None:
        saved = torch.empty(max(bcjr_saved_bytes(n, k, B, L), 1), dtype=torch.uint8, device=dev)
    if ws is None:
        ws = workspace(n, k, B, L, FWD, dev)
    tr = trellis(n, k, codebook)
    st = lib().bcjr_forward(ctypes.byref(tr), _ptr(w), B, L, float(T), _ptr(w_hat), _ptr(log_z),
                            _ptr(saved), _ptr(ws), ws.numel(), _stream())
    _check(st, "bcjr_forward")
    return w_hat, log_z, saved


def bcjr_scan_segment_length(n: int, k: int, B: int, L: int, seg_len: int = 0) -> int:
    tr = trellis(n, k)
    return int(lib().bcjr_scan_segment_length(ctypes.byref(tr), B, L, seg_len))


def bcjr_scan_workspace_bytes(n: int, k: int, B: int, L: int, seg_len: int = 0) -> int:
    tr = trellis(n, k)
    return int(lib().bcjr_scan_workspace_bytes(ctypes.byref(tr), B, L, seg_len))


def bcjr_forward_scan(codebook, w, n, k, T, seg_len=0, w_hat=None, log_z=None, ws=None):
    """Segmented (parallel-in-L) forward for few, long chains; returns (w_hat, log_z)."""
    _f32(codebook, "codebook"); _f32(w, "w")
    B, L = w.shape
    dev = w.device
    w_hat = torch.empty_like(w) if w_hat is None else w_hat
    log_z = torch.empty(B, dtype=torch.float32, device=dev) if log_z is None else log_z
    if ws is None:
        nb = bcjr_scan_workspace_bytes(n, k, B, L, seg_len)
        ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    tr = trellis(n, k, codebook)
    st = lib().bcjr_forward_scan(ctypes.byref(tr), _ptr(w), B, L, float(T), int(seg_len),
                                 _ptr(w_hat), _ptr(log_z), _ptr(ws), ws.numel(), _stream())
    _check(st, "bcjr_forward_scan")
    return w_hat, log_z


def bcjr_scan_backward_workspace_bytes(n: int, k: int, B: int, L: int, seg_len: int = 0) -> int:
    tr = trellis(n, k)
    return int(lib().bcjr_scan_backward_workspace_bytes(ctypes.byref(tr), B, L, seg_len))


def bcjr_backward_scan(codebook, w, n, k, T, w_hat, grad_w_hat, grad_log_z=None, seg_len=0,
                       grad_w=None, grad_codebook=None, ws=None):
    """Segmented (parallel-in-L) backward; returns (grad_w, grad_codebook)."""
    _f32(codebook, "codebook"); _f32(w, "w"); _f32(w_hat, "w_hat"); _f32(grad_w_hat, "grad_w_hat")
    B, L = w.shape
    dev = w.device
    grad_w = torch.empty_like(w) if grad_w is None else grad_w
    grad_codebook = torch.empty_like(codebook) if grad_codebook is None else grad_codebook
    if ws is None:
        nb = bcjr_scan_backward_workspace_bytes(n, k, B, L, seg_len)
        ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    tr = trellis(n, k, codebook)
    st = lib().bcjr_backward_scan(ctypes.byref(tr), _ptr(w), B, L, float(T), int(seg_len),
                                  _ptr(w_hat), _ptr(grad_w_hat), _ptr(grad_log_z), _ptr(grad_w),
                                  _ptr(grad_codebook), _ptr(ws), ws.numel(), _stream())
    _check(st, "bcjr_backward_scan")
    return grad_w, grad_codebook


def bcjr_backward(codebook, w, n, k, T, saved, grad_w_hat, grad_log_z=None, grad_w=None,
                  grad_codebook=None, ws=None):
    """Gradient of sum(g * w_hat) + sum(h * log_z); returns (grad_w, grad_codebook)."""
    _f32(codebook, "codebook"); _f32(w, "w"); _f32(grad_w_hat, "grad_w_hat")
    if grad_log_z is not None:
        _f32(grad_log_z, "grad_log_z")
    B, L = w.shape
    dev = w.device
    grad_w = torch.empty_like(w) if grad_w is None else grad_w
    grad_codebook = torch.empty_like(codebook) if grad_codebook is None else grad_codebook
    if ws is None:
        ws = workspace(n, k, B, L, BWD, dev)
    tr = trellis(n, k, codebook)
    st = lib().bcjr_backward(ctypes.byref(tr), _ptr(w), B, L, float(T), _ptr(saved),
                             _ptr(grad_w_hat), _ptr(grad_log_z), _ptr(grad_w),
                             _ptr(grad_codebook), _ptr(ws), ws.numel(), _stream())
    _check(st, "bcjr_backward")
    return grad_w, grad_codebook


def viterbi_decode(codebook, w, n, k, states=None, w_hard=None, want_w_hard=True, ws=None):
    """Hard decode (the T -> 0 limit); returns (states int32 [B,L], w_hard [B,L] or None)."""
    _f32(codebook, "codebook"); _f32(w, "w")
    B, L = w.shape
    dev = w.device
    states = torch.empty((B, L), dtype=torch.int32, device=dev) if states is None else states
    if want_w_hard and w_hard is None:
        w_hard = torch.empty_like(w)
    if ws is None:
        ws = workspace(n, k, B, L, VIT, dev)
    tr = trellis(n, k, codebook)
    st = lib().viterbi_decode(ctypes.byref(tr), _ptr(w), B, L, _ptr(states), _ptr(w_hard),
                              _ptr(ws), ws.numel(), _stream())
    _check(st, "viterbi_decode")
    return states, w_hard


# ---- dense (fully connected) trellis ---------------------------------------------------------

def bcjr_dense_supported(S: int) -> bool:
    return bool(lib().bcjr_dense_supported(int(S)))


def bcjr_dense_saved_bytes(S: int, B: int, L: int) -> int:
    return int(lib().bcjr_dense_saved_bytes(int(S), B, L))


def bcjr_dense_workspace_bytes(S: int, B: int, L: int, which: int) -> int:
    return int(lib().bcjr_dense_workspace_bytes(int(S), B, L, which))


def dense_workspace(S, B, L, which, device="cuda"):
    """Allocate a device workspace of the queried size (uint8 tensor)."""
    nb = bcjr_dense_workspace_bytes(S, B, L, which)
    return torch.empty(max(nb, 1), dtype=torch.uint8, device=device)


def bcjr_dense_forward(theta, codebook, w, T, w_hat=None, log_z=None, saved=None, ws=None):
    """Dense trellis: soft codeword w_hat [B,L] and log Z [B]; returns (w_hat, log_z, saved)."""
    _f32(theta, "theta"); _f32(codebook, "codebook"); _f32(w, "w")
    S = codebook.numel()
    B, L = w.shape
    dev = w.device
    w_hat = torch.empty_like(w) if w_hat is None else w_hat
    log_z = torch.empty(B, dtype=torch.float32, device=dev) if log_z is None else log_z
    if saved is None:
        saved = torch.empty(max(bcjr_dense_saved_bytes(S, B, L), 1), dtype=torch.uint8, device=dev)
    if ws is None:
        ws = dense_workspace(S, B, L, FWD, dev)
    st = lib().bcjr_dense_forward(S, _ptr(theta), _ptr(codebook), _ptr(w), B, L, float(T),
                                  _ptr(w_hat), _ptr(log_z), _ptr(saved), _ptr(ws), ws.numel(),
                                  _stream())
    _check(st, "bcjr_dense_forward")
    return w_hat, log_z, saved


def bcjr_dense_backward(theta, codebook, w, T, saved, grad_w_hat, grad_log_z=None, grad_w=None,
                        grad_codebook=None, grad_theta=None, ws=None):
    """Dense trellis gradient of sum(g * w_hat) + sum(h * log_z); returns
    (grad_w, grad_codebook, grad_theta)."""
    _f32(theta, "theta"); _f32(codebook, "codebook"); _f32(w, "w"); _f32(grad_w_hat, "grad_w_hat")
    if grad_log_z is not None:
        _f32(grad_log_z, "grad_log_z")
    S = codebook.numel()
    B, L = w.shape
    dev = w.device
    grad_w = torch.empty_like(w) if grad_w is None else grad_w
    grad_codebook = torch.empty_like(codebook) if grad_codebook is None else grad_codebook
    grad_theta = torch.empty_like(theta) if grad_theta is None else grad_theta
    if ws is None:
        ws = dense_workspace(S, B, L, BWD, dev)
    st = lib().bcjr_dense_backward(S, _ptr(theta), _ptr(codebook), _ptr(w), B, L, float(T),
                                   _ptr(saved), _ptr(grad_w_hat), _ptr(grad_log_z), _ptr(grad_w),
                                   _ptr(grad_codebook), _ptr(grad_theta), _ptr(ws), ws.numel(),
                                   _stream())
    _check(st, "bcjr_dense_backward")
    return grad_w, grad_codebook, grad_theta


# ---- hard-code export (bitshift trellis) --------------------------------------------------------

def bcjr_code_words(n: int, k: int, L: int) -> int:
    tr = trellis(n, k)
    return int(lib().bcjr_code_words(ctypes.byref(tr), L))


def bcjr_pack_code(states, n, k, code=None):
    """Pack int32 state paths [B,L] into uint32 codes [B, words] (n bits of s_0, then k bits per
    step, most significant first)."""
    if not (states.dtype == torch.int32 and states.is_cuda and states.is_contiguous()):
        raise ValueError("states must be a contiguous int32 CUDA tensor")
    B, L = states.shape
    if code is None:
        code = torch.empty((B, max(bcjr_code_words(n, k, L), 1)), dtype=torch.uint32,
                           device=states.device)
    tr = trellis(n, k)
    st = lib().bcjr_pack_code(ctypes.byref(tr), _ptr(states), B, L, _ptr(code), _stream())
    _check(st, "bcjr_pack_code")
    return code


def bcjr_unpack_code(code, n, k, L, codebook=None, states=None, w_hard=None):
    """States int32 [B,L] (and w_hard = c(states) if a codebook is given) from uint32 codes."""
    if not (code.dtype == torch.uint32 and code.is_cuda and code.is_contiguous()):
        raise ValueError("code must be a contiguous uint32 CUDA tensor")
    B = code.shape[0]
    dev = code.device
    states = torch.empty((B, L), dtype=torch.int32, device=dev) if states is None else states
    if codebook is not None:
        _f32(codebook, "codebook")
        if w_hard is None:
            w_hard = torch.empty((B, L), dtype=torch.float32, device=dev)
    tr = trellis(n, k, codebook)
    st = lib().bcjr_unpack_code(ctypes.byref(tr), _ptr(code), B, L, _ptr(states), _ptr(w_hard),
                                _stream())
    _check(st, "bcjr_unpack_code")
    return states, w_hard
