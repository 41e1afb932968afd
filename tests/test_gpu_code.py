"""GPU parity of the hard-code export: pack and unpack kernels against the oracle, bit-exact."""
import numpy as np
import pytest
import torch

import oracle
from bcjr_soft_decoding_amd import bcjr, synth
from tests.gpu_helpers import dev, log_case
from tests.test_oracle_code import random_paths

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bcjr.lib()


@pytest.mark.parametrize("n,k", [(4, 1), (4, 2), (5, 3), (8, 2), (12, 3), (16, 1), (16, 2), (16, 16)])
@pytest.mark.parametrize("B,L", [(1, 1), (3, 2), (7, 33), (65, 256)])
def test_pack_unpack_bit_exact(n, k, B, L):
    log_case(f"code n={n} k={k} B={B} L={L}")
    st = random_paths(n, k, B, L, 7 * n + 3 * k + L)
    c = synth.normal(600 + n, (1 << n,))
    ref_code, _ = oracle.pack_states(n, k, st)
    code = bcjr.bcjr_pack_code(dev(st), n, k)
    states, w_hard = bcjr.bcjr_unpack_code(code, n, k, L, dev(c))
    torch.cuda.synchronize()
    got = code.cpu().numpy().view(np.uint32)
    np.testing.assert_array_equal(got, ref_code)
    np.testing.assert_array_equal(states.cpu().numpy(), st)
    np.testing.assert_array_equal(w_hard.cpu().numpy(), c[st])


def test_viterbi_export_round_trip_workload2():
    """Workload 2 (S=256, 4096 x 256): decode at T -> 0, pack, unpack; the codes equal the oracle's
    packing of the oracle's decode and the unpacked w_hard equals the decoder's."""
    n, k = 8, 2
    c, w = synth.codebook(2), synth.weights(2)
    log_case("viterbi export wl2 4096x256")
    cd = dev(c)
    st, wh = bcjr.viterbi_decode(cd, dev(w), n, k)
    code = bcjr.bcjr_pack_code(st, n, k)
    st2, wh2 = bcjr.bcjr_unpack_code(code, n, k, w.shape[1], cd)
    torch.cuda.synchronize()
    rv = oracle.viterbi(n, k, c, w)
    ref_code, bad = oracle.pack_states(n, k, rv["states"])
    assert bad == 0
    np.testing.assert_array_equal(code.cpu().numpy().view(np.uint32), ref_code)
    np.testing.assert_array_equal(st2.cpu().numpy(), rv["states"])
    np.testing.assert_array_equal(wh2.cpu().numpy(), wh.cpu().numpy())
    assert code.shape == (4096, (8 + 2 * 255 + 31) // 32)


def test_unpack_without_codebook():
    n, k, L = 10, 2, 50
    st = random_paths(n, k, 4, L, 5)
    code = bcjr.bcjr_pack_code(dev(st), n, k)
    states, w_hard = bcjr.bcjr_unpack_code(code, n, k, L)
    torch.cuda.synchronize()
    assert w_hard is None
    np.testing.assert_array_equal(states.cpu().numpy(), st)
