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
LIB_PATH = os.path.join(_PKG, "_lib", "libbcjr.so")

BCJR_OK, BCJR_E_ARG, BCJR_E_SHAPE, BCJR_E_WORKSPACE, BCJR_E_DEVICE, BCJR_E_UNSUPPORTED = range(6)
FWD, BWD, VIT, FWD_CKPT, BWD_CKPT = 0, 1, 2, 3, 4

EXPORTED = (
    "bcjr_supported", "bcjr_saved_bytes", "bcjr_workspace_bytes", "bcjr_forward",
    "bcjr_backward", "viterbi_decode", "bcjr_dense_supported", "bcjr_dense_saved_bytes",
    "bcjr_dense_workspace_bytes", "bcjr_dense_forward", "bcjr_dense_backward",
    "bcjr_code_words", "bcjr_pack_code", "bcjr_unpack_code", "bcjr_status_string",
    "bcjr_scan_segment_length", "bcjr_scan_workspace_bytes", "bcjr_forward_scan",
    "bcjr_scan_backward_workspace_bytes", "bcjr_backward_scan", "bcjr_forward_noalloc",
)
# Size of the fixed device array bcjr_forward_noalloc takes its workspace from.
NOALLOC_SCRATCH_BYTES = 256 << 20


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
    L.bcjr_forward_noalloc.argtypes = [TP, P, I64, I64, F, P, P, P, P]
    L.bcjr_forward_noalloc.restype = ctypes.c_int
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


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def trellis(n: int, k: int, codebook=None, v: int = 1) -> Trellis:
    return Trellis(int(n), int(k), int(v), None if codebook is None else codebook.data_ptr())


def _check(st: int, what: str):
    if st != BCJR_OK:
        raise BcjrError(st, what)


# ---- argument checks -----------------------------------------------------------------------
# The C ABI receives raw pointers and cannot see a tensor's extent, so every tensor is checked
# here against the sizes the call implies before anything is passed down: a short codebook or
# output would otherwise be read or written past its end on the device. Shapes and dtypes are
# checked first, then that every tensor is a CUDA tensor on one device; nothing is allocated
# or launched before both pass.

F32, I32, U32 = torch.float32, torch.int32, torch.uint32


def _spec(t, name, dtype, shape):
    """t (None = not given) must be a contiguous tensor of this dtype and exact shape."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(int(s) for s in shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(int(s) for s in shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _spec_bytes(t, name, need, align=16):
    """A byte buffer of any dtype (None = not given) holding at least `need` bytes; returns its
    size in bytes."""
    if t is None:
        return 0
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    have = t.numel() * t.element_size()
    if have < need:
        raise ValueError(f"{name} holds {have} bytes, the call needs {need}")
    if t.data_ptr() % align:
        raise ValueError(f"{name} must be {align}-byte aligned")
    return have


def _chains2(t, name, dtype=F32):
    """The [B, L] array that fixes a call's shape; returns (B, L)."""
    _spec(t, name, dtype, None)
    if t.dim() != 2:
        raise ValueError(f"{name} must have shape [B, L], got {tuple(t.shape)}")
    return int(t.shape[0]), int(t.shape[1])


def _device(*tensors):
    """Every given tensor must be a CUDA tensor, all on one device; returns that device."""
    dev = None
    for t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"expected CUDA tensors, got one on {t.device}")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"tensors on {dev} and {t.device}: a call runs on one device")
    return dev


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
    B, L = _chains2(w, "w")
    S = 1 << int(n)
    _spec(codebook, "codebook", F32, (S,))
    _spec(w_hat, "w_hat", F32, (B, L))
    _spec(log_z, "log_z", F32, (B,))
    need_saved = bcjr_saved_bytes(n, k, B, L)
    _spec_bytes(saved, "saved", need_saved)
    _spec_bytes(ws, "ws", 0)
    dev = _device(w, codebook, w_hat, log_z, saved, ws)
    w_hat = torch.empty_like(w) if w_hat is None else w_hat
    log_z = torch.empty(B, dtype=F32, device=dev) if log_z is None else log_z
    if saved is None:
        saved = torch.empty(max(need_saved, 1), dtype=torch.uint8, device=dev)
    if ws is None:
        ws = workspace(n, k, B, L, FWD, dev)
    tr = trellis(n, k, codebook)
    with torch.cuda.device(dev):
        st = lib().bcjr_forward(ctypes.byref(tr), _ptr(w), B, L, float(T), _ptr(w_hat),
                                _ptr(log_z), _ptr(saved), _ptr(ws), _spec_bytes(ws, "ws", 0),
                                _stream(dev))
    _check(st, "bcjr_forward")
    return w_hat, log_z, saved


def bcjr_forward_noalloc(codebook, w, n, k, T, w_hat, log_z, saved):
    """bcjr_forward with the library's fixed scratch array as workspace: the C entry point makes
    no device allocation, so every output (w_hat [B,L], log_z [B], saved) is the caller's.
    Returns (w_hat, log_z, saved)."""
    B, L = _chains2(w, "w")
    _spec(codebook, "codebook", F32, (1 << int(n),))
    for t, name in ((w_hat, "w_hat"), (log_z, "log_z"), (saved, "saved")):
        if t is None:
            raise ValueError(f"{name}: bcjr_forward_noalloc writes into caller-owned outputs")
    _spec(w_hat, "w_hat", F32, (B, L))
    _spec(log_z, "log_z", F32, (B,))
    _spec_bytes(saved, "saved", bcjr_saved_bytes(n, k, B, L))
    dev = _device(w, codebook, w_hat, log_z, saved)
    tr = trellis(n, k, codebook)
    with torch.cuda.device(dev):
        st = lib().bcjr_forward_noalloc(ctypes.byref(tr), _ptr(w), B, L, float(T), _ptr(w_hat),
                                        _ptr(log_z), _ptr(saved), _stream(dev))
    _check(st, "bcjr_forward_noalloc")
    return w_hat, log_z, saved


def bcjr_scan_segment_length(n: int, k: int, B: int, L: int, seg_len: int = 0) -> int:
    tr = trellis(n, k)
    return int(lib().bcjr_scan_segment_length(ctypes.byref(tr), B, L, seg_len))


def bcjr_scan_workspace_bytes(n: int, k: int, B: int, L: int, seg_len: int = 0) -> int:
    tr = trellis(n, k)
    return int(lib().bcjr_scan_workspace_bytes(ctypes.byref(tr), B, L, seg_len))


def bcjr_forward_scan(codebook, w, n, k, T, seg_len=0, w_hat=None, log_z=None, ws=None):
    """Segmented (parallel-in-L) forward for few, long chains; returns (w_hat, log_z)."""
    B, L = _chains2(w, "w")
    _spec(codebook, "codebook", F32, (1 << int(n),))
    _spec(w_hat, "w_hat", F32, (B, L))
    _spec(log_z, "log_z", F32, (B,))
    _spec_bytes(ws, "ws", 0)
    dev = _device(w, codebook, w_hat, log_z, ws)
    w_hat = torch.empty_like(w) if w_hat is None else w_hat
    log_z = torch.empty(B, dtype=F32, device=dev) if log_z is None else log_z
    if ws is None:
        nb = bcjr_scan_workspace_bytes(n, k, B, L, seg_len)
        ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    tr = trellis(n, k, codebook)
    with torch.cuda.device(dev):
        st = lib().bcjr_forward_scan(ctypes.byref(tr), _ptr(w), B, L, float(T), int(seg_len),
                                     _ptr(w_hat), _ptr(log_z), _ptr(ws), _spec_bytes(ws, "ws", 0),
                                     _stream(dev))
    _check(st, "bcjr_forward_scan")
    return w_hat, log_z


def bcjr_scan_backward_workspace_bytes(n: int, k: int, B: int, L: int, seg_len: int = 0) -> int:
    tr = trellis(n, k)
    return int(lib().bcjr_scan_backward_workspace_bytes(ctypes.byref(tr), B, L, seg_len))


def bcjr_backward_scan(codebook, w, n, k, T, w_hat, grad_w_hat, grad_log_z=None, seg_len=0,
                       grad_w=None, grad_codebook=None, ws=None):
    """Segmented (parallel-in-L) backward; returns (grad_w, grad_codebook)."""
    B, L = _chains2(w, "w")
    S = 1 << int(n)
    _spec(codebook, "codebook", F32, (S,))
    _spec(w_hat, "w_hat", F32, (B, L))
    _spec(grad_w_hat, "grad_w_hat", F32, (B, L))
    _spec(grad_log_z, "grad_log_z", F32, (B,))
    _spec(grad_w, "grad_w", F32, (B, L))
    _spec(grad_codebook, "grad_codebook", F32, (S,))
    _spec_bytes(ws, "ws", 0)
    dev = _device(w, codebook, w_hat, grad_w_hat, grad_log_z, grad_w, grad_codebook, ws)
    grad_w = torch.empty_like(w) if grad_w is None else grad_w
    grad_codebook = torch.empty_like(codebook) if grad_codebook is None else grad_codebook
    if ws is None:
        nb = bcjr_scan_backward_workspace_bytes(n, k, B, L, seg_len)
        ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    tr = trellis(n, k, codebook)
    with torch.cuda.device(dev):
        st = lib().bcjr_backward_scan(ctypes.byref(tr), _ptr(w), B, L, float(T), int(seg_len),
                                      _ptr(w_hat), _ptr(grad_w_hat), _ptr(grad_log_z),
                                      _ptr(grad_w), _ptr(grad_codebook), _ptr(ws),
                                      _spec_bytes(ws, "ws", 0), _stream(dev))
    _check(st, "bcjr_backward_scan")
    return grad_w, grad_codebook


def bcjr_backward(codebook, w, n, k, T, saved, grad_w_hat, grad_log_z=None, grad_w=None,
                  grad_codebook=None, ws=None):
    """Gradient of sum(g * w_hat) + sum(h * log_z); returns (grad_w, grad_codebook)."""
    B, L = _chains2(w, "w")
    S = 1 << int(n)
    _spec(codebook, "codebook", F32, (S,))
    if saved is None:
        raise ValueError("saved (the forward's context) is required")
    _spec_bytes(saved, "saved", bcjr_saved_bytes(n, k, B, L))
    _spec(grad_w_hat, "grad_w_hat", F32, (B, L))
    _spec(grad_log_z, "grad_log_z", F32, (B,))
    _spec(grad_w, "grad_w", F32, (B, L))
    _spec(grad_codebook, "grad_codebook", F32, (S,))
    _spec_bytes(ws, "ws", 0)
    dev = _device(w, codebook, saved, grad_w_hat, grad_log_z, grad_w, grad_codebook, ws)
    grad_w = torch.empty_like(w) if grad_w is None else grad_w
    grad_codebook = torch.empty_like(codebook) if grad_codebook is None else grad_codebook
    if ws is None:
        ws = workspace(n, k, B, L, BWD, dev)
    tr = trellis(n, k, codebook)
    with torch.cuda.device(dev):
        st = lib().bcjr_backward(ctypes.byref(tr), _ptr(w), B, L, float(T), _ptr(saved),
                                 _ptr(grad_w_hat), _ptr(grad_log_z), _ptr(grad_w),
                                 _ptr(grad_codebook), _ptr(ws), _spec_bytes(ws, "ws", 0),
                                 _stream(dev))
    _check(st, "bcjr_backward")
    return grad_w, grad_codebook


def viterbi_decode(codebook, w, n, k, states=None, w_hard=None, want_w_hard=True, ws=None):
    """Hard decode (the T -> 0 limit); returns (states int32 [B,L], w_hard [B,L] or None)."""
    B, L = _chains2(w, "w")
    _spec(codebook, "codebook", F32, (1 << int(n),))
    _spec(states, "states", I32, (B, L))
    _spec(w_hard, "w_hard", F32, (B, L))
    _spec_bytes(ws, "ws", 0)
    dev = _device(w, codebook, states, w_hard, ws)
    states = torch.empty((B, L), dtype=I32, device=dev) if states is None else states
    if w_hard is None and want_w_hard:
        w_hard = torch.empty_like(w)
    if ws is None:
        ws = workspace(n, k, B, L, VIT, dev)
    tr = trellis(n, k, codebook)
    with torch.cuda.device(dev):
        st = lib().viterbi_decode(ctypes.byref(tr), _ptr(w), B, L, _ptr(states), _ptr(w_hard),
                                  _ptr(ws), _spec_bytes(ws, "ws", 0), _stream(dev))
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


def _dense_shape(theta, codebook, w):
    """(S, B, L) of a dense call: the codebook is [S], theta [S, S], w [B, L]."""
    B, L = _chains2(w, "w")
    _spec(codebook, "codebook", F32, None)
    if codebook.dim() != 1:
        raise ValueError(f"codebook must have shape [S], got {tuple(codebook.shape)}")
    S = int(codebook.numel())
    _spec(theta, "theta", F32, (S, S))
    return S, B, L


def bcjr_dense_forward(theta, codebook, w, T, w_hat=None, log_z=None, saved=None, ws=None):
    """Dense trellis: soft codeword w_hat [B,L] and log Z [B]; returns (w_hat, log_z, saved)."""
    S, B, L = _dense_shape(theta, codebook, w)
    _spec(w_hat, "w_hat", F32, (B, L))
    _spec(log_z, "log_z", F32, (B,))
    need_saved = bcjr_dense_saved_bytes(S, B, L)
    _spec_bytes(saved, "saved", need_saved)
    _spec_bytes(ws, "ws", 0)
    dev = _device(w, codebook, theta, w_hat, log_z, saved, ws)
    w_hat = torch.empty_like(w) if w_hat is None else w_hat
    log_z = torch.empty(B, dtype=F32, device=dev) if log_z is None else log_z
    if saved is None:
        saved = torch.empty(max(need_saved, 1), dtype=torch.uint8, device=dev)
    if ws is None:
        ws = dense_workspace(S, B, L, FWD, dev)
    with torch.cuda.device(dev):
        st = lib().bcjr_dense_forward(S, _ptr(theta), _ptr(codebook), _ptr(w), B, L, float(T),
                                      _ptr(w_hat), _ptr(log_z), _ptr(saved), _ptr(ws),
                                      _spec_bytes(ws, "ws", 0), _stream(dev))
    _check(st, "bcjr_dense_forward")
    return w_hat, log_z, saved


def bcjr_dense_backward(theta, codebook, w, T, saved, grad_w_hat, grad_log_z=None, grad_w=None,
                        grad_codebook=None, grad_theta=None, ws=None):
    """Dense trellis gradient of sum(g * w_hat) + sum(h * log_z); returns
    (grad_w, grad_codebook, grad_theta)."""
    S, B, L = _dense_shape(theta, codebook, w)
    if saved is None:
        raise ValueError("saved (the forward's context) is required")
    _spec_bytes(saved, "saved", bcjr_dense_saved_bytes(S, B, L))
    _spec(grad_w_hat, "grad_w_hat", F32, (B, L))
    _spec(grad_log_z, "grad_log_z", F32, (B,))
    _spec(grad_w, "grad_w", F32, (B, L))
    _spec(grad_codebook, "grad_codebook", F32, (S,))
    _spec(grad_theta, "grad_theta", F32, (S, S))
    _spec_bytes(ws, "ws", 0)
    dev = _device(w, codebook, theta, saved, grad_w_hat, grad_log_z, grad_w, grad_codebook,
                  grad_theta, ws)
    grad_w = torch.empty_like(w) if grad_w is None else grad_w
    grad_codebook = torch.empty_like(codebook) if grad_codebook is None else grad_codebook
    grad_theta = torch.empty_like(theta) if grad_theta is None else grad_theta
    if ws is None:
        ws = dense_workspace(S, B, L, BWD, dev)
    with torch.cuda.device(dev):
        st = lib().bcjr_dense_backward(S, _ptr(theta), _ptr(codebook), _ptr(w), B, L, float(T),
                                       _ptr(saved), _ptr(grad_w_hat), _ptr(grad_log_z),
                                       _ptr(grad_w), _ptr(grad_codebook), _ptr(grad_theta),
                                       _ptr(ws), _spec_bytes(ws, "ws", 0), _stream(dev))
    _check(st, "bcjr_dense_backward")
    return grad_w, grad_codebook, grad_theta


# ---- hard-code export (bitshift trellis) --------------------------------------------------------

def bcjr_code_words(n: int, k: int, L: int) -> int:
    tr = trellis(n, k)
    return int(lib().bcjr_code_words(ctypes.byref(tr), L))


def bcjr_pack_code(states, n, k, code=None):
    """Pack int32 state paths [B,L] into uint32 codes [B, words] (n bits of s_0, then k bits per
    step, most significant first)."""
    B, L = _chains2(states, "states", I32)
    words = bcjr_code_words(n, k, L)
    _spec(code, "code", U32, (B, words))
    dev = _device(states, code)
    if code is None:
        code = torch.empty((B, max(words, 1)), dtype=U32, device=dev)
    tr = trellis(n, k)
    with torch.cuda.device(dev):
        st = lib().bcjr_pack_code(ctypes.byref(tr), _ptr(states), B, L, _ptr(code), _stream(dev))
    _check(st, "bcjr_pack_code")
    return code


def bcjr_unpack_code(code, n, k, L, codebook=None, states=None, w_hard=None):
    """States int32 [B,L] (and w_hard = c(states) if a codebook is given) from uint32 codes."""
    B, nw = _chains2(code, "code", U32)
    words = bcjr_code_words(n, k, L)
    if nw != words:
        raise ValueError(f"code has {nw} words per chain; n={n}, k={k}, L={L} need {words}")
    _spec(codebook, "codebook", F32, (1 << int(n),))
    _spec(states, "states", I32, (B, L))
    _spec(w_hard, "w_hard", F32, (B, L))
    if w_hard is not None and codebook is None:
        raise ValueError("w_hard needs the codebook")
    dev = _device(code, codebook, states, w_hard)
    states = torch.empty((B, L), dtype=I32, device=dev) if states is None else states
    if codebook is not None and w_hard is None:
        w_hard = torch.empty((B, L), dtype=F32, device=dev)
    tr = trellis(n, k, codebook)
    with torch.cuda.device(dev):
        st = lib().bcjr_unpack_code(ctypes.byref(tr), _ptr(code), B, L, _ptr(states),
                                    _ptr(w_hard), _stream(dev))
    _check(st, "bcjr_unpack_code")
    return states, w_hard
