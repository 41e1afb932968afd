"""bcjr_forward_noalloc (the forward whose workspace is the library's fixed device array) against
bcjr_forward with a workspace of its own: the same kernels, so w_hat, log_z and the saved
context agree bitwise. Two calls in a row, the second on a smaller input (the array keeps the
first call's contents), one through the checkpointed history and one through the full history;
shapes beyond the array are refused before anything is enqueued."""
import numpy as np
import pytest
import torch

from bcjr_soft_decoding_amd import bcjr
from tests.gpu_helpers import log_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bcjr.lib()


def _inputs(n, B, L, seed):
    rng = np.random.default_rng(seed)
    c = torch.from_numpy(rng.standard_normal(1 << n).astype(np.float32)).cuda()
    w = torch.from_numpy(rng.standard_normal((B, L)).astype(np.float32)).cuda()
    return c, w


def _outputs(n, B, L, fill):
    wh = torch.full((B, L), fill, dtype=torch.float32, device="cuda")
    lz = torch.full((B,), fill, dtype=torch.float32, device="cuda")
    sv = torch.full((bcjr.bcjr_saved_bytes(n, 2, B, L),), 0x5A, dtype=torch.uint8, device="cuda")
    return wh, lz, sv


def _compare(n, B, L, T, seed):
    c, w = _inputs(n, B, L, seed)
    full = bcjr.bcjr_workspace_bytes(n, 2, B, L, 0)
    ckpt = bcjr.bcjr_workspace_bytes(n, 2, B, L, 3)
    path = "full" if full <= bcjr.NOALLOC_SCRATCH_BYTES else "checkpointed"
    log_case(f"noalloc n={n} B={B} L={L} T={T} seed={seed} history={path} "
             f"(full {full >> 20} MiB, checkpointed {ckpt >> 20} MiB)")
    wh1, lz1, sv1 = _outputs(n, B, L, float("nan"))
    bcjr.bcjr_forward_noalloc(c, w, n, 2, T, wh1, lz1, sv1)
    # the reference: the ordinary entry point with its own workspace of the same layout
    ws = torch.empty(full if path == "full" else ckpt, dtype=torch.uint8, device="cuda")
    wh0, lz0, sv0 = _outputs(n, B, L, 0.0)
    bcjr.bcjr_forward(c, w, n, 2, T, wh0, lz0, sv0, ws)
    torch.cuda.synchronize()
    assert torch.isfinite(wh1).all() and torch.isfinite(lz1).all()
    assert torch.equal(wh1, wh0), "w_hat differs from bcjr_forward"
    assert torch.equal(lz1, lz0), "log_z differs from bcjr_forward"
    assert torch.equal(sv1, sv0), "saved context differs from bcjr_forward"
    return path


def test_two_calls_in_a_row_second_smaller():
    # S = 4096, 600 chains of 256 steps: the full history (1.2 GiB) does not fit the array, the
    # checkpointed one (151 MiB) does
    assert _compare(12, 600, 256, 0.1, seed=11) == "checkpointed"
    # then a smaller input over the array the first call left behind: the full history
    assert _compare(8, 37, 100, 0.3, seed=12) == "full"


def test_fp64_messages_and_ragged_chains():
    # below T = 0.05 the forward carries fp64 messages; an odd chain count leaves a ragged unit
    assert _compare(8, 29, 65, 0.005, seed=13) == "full"
    assert _compare(10, 3, 7, 0.05, seed=14) == "full"


def test_no_chains_and_refused_sizes():
    n, L = 12, 256
    c, w0 = _inputs(n, 0, L, 15)
    wh, lz, sv = _outputs(n, 0, L, 0.0)
    bcjr.bcjr_forward_noalloc(c, w0, n, 2, 0.1, wh, lz, sv)  # B = 0: nothing to do
    # the smallest chain count whose checkpointed history exceeds the array
    B = 1
    while bcjr.bcjr_workspace_bytes(n, 2, B, L, 3) <= bcjr.NOALLOC_SCRATCH_BYTES:
        B *= 2
    log_case(f"noalloc refusal n={n} B={B} L={L}")
    c, w = _inputs(n, B, L, 16)
    wh, lz, sv = _outputs(n, B, L, 7.0)
    with pytest.raises(bcjr.BcjrError) as e:
        bcjr.bcjr_forward_noalloc(c, w, n, 2, 0.1, wh, lz, sv)
    assert e.value.status == bcjr.BCJR_E_WORKSPACE
    torch.cuda.synchronize()
    assert bool((wh == 7.0).all()) and bool((lz == 7.0).all()), "a refused call wrote outputs"
