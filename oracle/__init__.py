"""Plain CPU oracle for BCJR-QAT soft trellis decoding -- test infrastructure only.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may import this
package. It shares no code with the HIP library in ``bcjr_soft_decoding_amd``.
"""
from .oracle import (  # noqa: F401
    build,
    code_words,
    dense_backward,
    dense_forward,
    pack_states,
    set_threads,
    sparse_backward,
    sparse_forward,
    unpack_code,
    viterbi,
)
