"""BCJR soft trellis decoding on MI355X (gfx950).

The work is done by hand-written HIP kernels behind the C ABI declared in ``include/bcjr.h``
(``libbcjr.so``); ``bcjr_soft_decoding_amd.bcjr`` is the thin ctypes binding over it and
``bcjr_soft_decoding_amd.autograd`` wraps it as a differentiable soft quantiser and
``bcjr_soft_decoding_amd.qat`` drives annealed quantisation-aware training of a layer with it.
The library is loaded on first use, and a missing library is an error, never a fallback.
"""

__all__ = ["autograd", "bcjr", "qat", "synth"]
