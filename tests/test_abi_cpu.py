"""The C ABI library on the CPU: it loads, exports every declared symbol, answers size queries
and rejects bad arguments before touching the device (no compute call is made here)."""
import ctypes
import os
import re

import pytest

from bcjr_soft_decoding_amd import bcjr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = []
    for fn in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^[A-Za-z_][\w\s\*]*?\b(\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bcjr.LIB_PATH):
        pytest.fail(f"{bcjr.LIB_PATH} not built (run __graft_entry__.build())")
    return bcjr.lib()


def test_exports_every_declared_symbol(lib):
    declared = _declared_functions()
    assert set(bcjr.EXPORTED) <= set(declared)
    for name in declared:
        assert hasattr(lib, name), f"{name} declared in include/ but not exported"


def test_status_strings(lib):
    for s in range(6):
        assert len(bcjr.status_text(s)) > 0
    assert bcjr.status_text(0) == "ok"


def test_supported_shapes(lib):
    for n in range(4, 17):
        assert bcjr.bcjr_supported(n, 2)
    assert not bcjr.bcjr_supported(3, 2)   # n < 2k: no kernel built
    assert not bcjr.bcjr_supported(17, 2)  # n out of range
    assert not bcjr.bcjr_supported(8, 2, v=2)


def test_size_queries(lib):
    # forward workspace grows with L and B, backward needs more than forward
    a = bcjr.bcjr_workspace_bytes(12, 2, 1000, 64, bcjr.FWD)
    b = bcjr.bcjr_workspace_bytes(12, 2, 1000, 128, bcjr.FWD)
    c = bcjr.bcjr_workspace_bytes(12, 2, 1000, 64, bcjr.BWD)
    assert 0 < a < b and c > a
    assert bcjr.bcjr_workspace_bytes(12, 2, 1000, 64, 7) == 0
    assert bcjr.bcjr_workspace_bytes(12, 2, -1, 64, 0) == 0
    assert bcjr.bcjr_workspace_bytes(12, 2, 0, 64, 0) == 0
    assert bcjr.bcjr_saved_bytes(8, 2, 4096, 256) >= 4096 * 4
    assert bcjr.bcjr_saved_bytes(8, 9, 4096, 256) == 0
    # slots are capped, so the workspace stops growing with B once every slot is busy
    big1 = bcjr.bcjr_workspace_bytes(12, 2, 1 << 20, 256, bcjr.FWD)
    big2 = bcjr.bcjr_workspace_bytes(12, 2, 1 << 21, 256, bcjr.FWD)
    assert big1 == big2


def _fwd(lib, n=8, k=2, v=1, cb=0x1000, w=0x2000, B=4, L=8, T=0.5, wh=0x3000, lz=0x4000,
         sv=0x5000, ws=0x6000, wsb=1 << 40):
    tr = bcjr.Trellis(n, k, v, cb)
    P = ctypes.c_void_p
    return lib.bcjr_forward(ctypes.byref(tr), P(w), B, L, T, P(wh), P(lz), P(sv), P(ws), wsb, None)


def test_forward_rejects_bad_arguments_without_device(lib):
    assert lib.bcjr_forward(None, None, 1, 1, 1.0, None, None, None, None, 0, None) == bcjr.BCJR_E_ARG
    assert _fwd(lib, n=0) == bcjr.BCJR_E_SHAPE
    assert _fwd(lib, n=17) == bcjr.BCJR_E_SHAPE
    assert _fwd(lib, k=0) == bcjr.BCJR_E_SHAPE
    assert _fwd(lib, k=9) == bcjr.BCJR_E_SHAPE
    assert _fwd(lib, B=-1) == bcjr.BCJR_E_SHAPE
    assert _fwd(lib, L=0) == bcjr.BCJR_E_SHAPE
    assert _fwd(lib, v=2) == bcjr.BCJR_E_UNSUPPORTED
    assert _fwd(lib, n=5, k=3) == bcjr.BCJR_E_UNSUPPORTED
    assert _fwd(lib, T=0.0) == bcjr.BCJR_E_ARG
    assert _fwd(lib, T=-1.0) == bcjr.BCJR_E_ARG
    assert _fwd(lib, T=float("nan")) == bcjr.BCJR_E_ARG
    assert _fwd(lib, T=float("inf")) == bcjr.BCJR_E_ARG
    assert _fwd(lib, cb=0) == bcjr.BCJR_E_ARG
    assert _fwd(lib, w=0) == bcjr.BCJR_E_ARG
    assert _fwd(lib, wh=0) == bcjr.BCJR_E_ARG
    assert _fwd(lib, sv=0) == bcjr.BCJR_E_ARG
    assert _fwd(lib, ws=0) == bcjr.BCJR_E_WORKSPACE
    need = bcjr.bcjr_workspace_bytes(8, 2, 4, 8, bcjr.FWD_CKPT)  # the smaller, checkpointed layout
    assert _fwd(lib, wsb=need - 1) == bcjr.BCJR_E_WORKSPACE
    assert _fwd(lib, ws=0x6008) == bcjr.BCJR_E_WORKSPACE  # 16-byte alignment
    assert _fwd(lib, sv=0x5008) == bcjr.BCJR_E_ARG  # the context holds doubles: 16-byte aligned
    # B = 0 is valid and enqueues nothing (null outputs allowed)
    assert _fwd(lib, B=0, w=0, wh=0, lz=0, sv=0, ws=0, wsb=0) == bcjr.BCJR_OK
    # B * L beyond 2^40 (64-bit offsets and workspace sizes stay exact below it)
    assert _fwd(lib, B=1 << 21, L=1 << 20) == bcjr.BCJR_E_SHAPE
    assert _fwd(lib, B=1, L=(1 << 40) + 1) == bcjr.BCJR_E_SHAPE


def test_temperatures_below_each_floor_are_refused(lib):
    """Each state size meets the tolerances down to its floor (0.002 for n <= 12, 0.015 for
    n = 13..15, 0.03 for n = 16, where no fp64-message kernels fit LDS); below it forward and
    backward refuse before any device call, at and above it validation passes (the call then
    needs a device: not made here, so only the status of a refused workspace is observed)."""
    P = ctypes.c_void_p
    for n, floor in ((16, 0.03), (15, 0.015), (13, 0.015), (12, 0.002), (4, 0.002)):
        for T in (floor * 0.999, floor / 2, 1e-4):
            assert _fwd(lib, n=n, T=T) == bcjr.BCJR_E_UNSUPPORTED
            assert _fwd(lib, n=n, T=T, B=0, w=0, wh=0, lz=0, sv=0, ws=0, wsb=0) == bcjr.BCJR_E_UNSUPPORTED
            tr = bcjr.Trellis(n, 2, 1, 0x1000)
            st = lib.bcjr_backward(ctypes.byref(tr), P(0x2000), 4, 8, T, P(0x3000), P(0x4000), None,
                                   P(0x5000), P(0x6000), P(0x7000), 1 << 40, None)
            assert st == bcjr.BCJR_E_UNSUPPORTED
        for T in (floor, floor * 1.5, 0.1):
            assert _fwd(lib, n=n, T=T, wsb=0) == bcjr.BCJR_E_WORKSPACE


def test_temperatures_below_the_fp64_floor_are_refused(lib):
    """The fp64-message kernels meet the tolerances down to T = 0.002 (their fp32 exponentials and
    expectations put rare gradients at 2e-3 by T = 0.0005); below it every soft entry point of the
    bitshift trellis, whole-chain and segmented, refuses before any device call."""
    P = ctypes.c_void_p
    for n in (4, 8, 12, 15):
        for T in (0.0019, 0.001, 1e-5):
            assert _fwd(lib, n=n, T=T) == bcjr.BCJR_E_UNSUPPORTED
            assert _fwd(lib, n=n, T=T, B=0, w=0, wh=0, lz=0, sv=0, ws=0, wsb=0) == bcjr.BCJR_E_UNSUPPORTED
            tr = bcjr.Trellis(n, 2, 1, 0x1000)
            st = lib.bcjr_backward(ctypes.byref(tr), P(0x2000), 4, 8, T, P(0x3000), P(0x4000), None,
                                   P(0x5000), P(0x6000), P(0x7000), 1 << 40, None)
            assert st == bcjr.BCJR_E_UNSUPPORTED
        if n <= 12:
            tr = bcjr.Trellis(n, 2, 1, 0x1000)
            for T, want in ((0.001, bcjr.BCJR_E_UNSUPPORTED), (0.002, bcjr.BCJR_E_WORKSPACE)):
                st = lib.bcjr_forward_scan(ctypes.byref(tr), P(0x2000), 1, 4096, T, 0, P(0x3000),
                                           P(0x4000), P(0x5000), 0, None)
                assert st == want, (n, T, st)
                st = lib.bcjr_backward_scan(ctypes.byref(tr), P(0x2000), 1, 4096, T, 0, P(0x3000),
                                            P(0x4000), None, P(0x5000), P(0x6000), P(0x7000), 0, None)
                assert st == want, (n, T, st)


def test_backward_and_viterbi_reject_bad_arguments_without_device(lib):
    P = ctypes.c_void_p
    tr = bcjr.Trellis(8, 2, 1, 0x1000)
    ok = dict(w=P(0x2000), sv=P(0x3000), g=P(0x4000), gw=P(0x5000), gc=P(0x6000), ws=P(0x7000))

    def bwd(T=0.5, B=4, L=8, wsb=1 << 40, **kw):
        a = dict(ok, **kw)
        return lib.bcjr_backward(ctypes.byref(tr), a["w"], B, L, T, a["sv"], a["g"], None, a["gw"],
                                 a["gc"], a["ws"], wsb, None)

    assert bwd(T=0.0) == bcjr.BCJR_E_ARG
    assert bwd(gc=P(0)) == bcjr.BCJR_E_ARG
    assert bwd(sv=P(0)) == bcjr.BCJR_E_ARG
    assert bwd(g=P(0)) == bcjr.BCJR_E_ARG
    assert bwd(wsb=0) == bcjr.BCJR_E_WORKSPACE
    assert bwd(wsb=bcjr.bcjr_workspace_bytes(8, 2, 4, 8, bcjr.BWD_CKPT) - 1) == bcjr.BCJR_E_WORKSPACE
    assert bwd(L=0) == bcjr.BCJR_E_SHAPE

    def vit(B=4, L=8, wsb=1 << 40, st=P(0x8000), ws=P(0x7000)):
        return lib.viterbi_decode(ctypes.byref(tr), P(0x2000), B, L, st, None, ws, wsb, None)

    assert vit(st=P(0)) == bcjr.BCJR_E_ARG
    assert vit(wsb=1) == bcjr.BCJR_E_WORKSPACE
    assert vit(B=-2) == bcjr.BCJR_E_SHAPE
    assert vit(B=0, st=P(0), ws=P(0), wsb=0) == bcjr.BCJR_OK


def test_dense_size_queries(lib):
    for S in (32, 64, 128, 256):
        assert bcjr.bcjr_dense_supported(S)
    for S in (0, 16, 48, 512):
        assert not bcjr.bcjr_dense_supported(S)
    S, B, L = 256, 1024, 1024
    sv = bcjr.bcjr_dense_saved_bytes(S, B, L)
    # two [B, L, S] fp32 message histories dominate the context
    assert 2 * B * L * S * 4 + 16 * B * L <= sv < 2 * B * L * S * 4 + 16 * B * L + 4096 + 8 * B
    f = bcjr.bcjr_dense_workspace_bytes(S, B, L, 0)
    b = bcjr.bcjr_dense_workspace_bytes(S, B, L, 1)
    assert 0 < f < b and b >= 3 * B * L * S * 4
    assert bcjr.bcjr_dense_workspace_bytes(S, B, L, 2) == 0
    assert bcjr.bcjr_dense_workspace_bytes(48, B, L, 0) == 0
    assert bcjr.bcjr_dense_workspace_bytes(S, 0, L, 1) == 0
    assert bcjr.bcjr_dense_saved_bytes(S, -1, L) == 0
    assert bcjr.bcjr_dense_saved_bytes(S, B, 0) == 0


def test_dense_rejects_bad_arguments_without_device(lib):
    P = ctypes.c_void_p
    ok = dict(th=P(0x1000), cb=P(0x1100), w=P(0x2000), wh=P(0x3000), lz=P(0x4000), sv=P(0x5000),
              ws=P(0x6000), g=P(0x7000), gw=P(0x8000), gc=P(0x9000), gt=P(0xA000))

    def fwd(S=64, B=4, L=8, T=0.5, wsb=1 << 40, **kw):
        a = dict(ok, **kw)
        return lib.bcjr_dense_forward(S, a["th"], a["cb"], a["w"], B, L, T, a["wh"], a["lz"],
                                      a["sv"], a["ws"], wsb, None)

    def bwd(S=64, B=4, L=8, T=0.5, wsb=1 << 40, **kw):
        a = dict(ok, **kw)
        return lib.bcjr_dense_backward(S, a["th"], a["cb"], a["w"], B, L, T, a["sv"], a["g"], None,
                                       a["gw"], a["gc"], a["gt"], a["ws"], wsb, None)

    assert fwd(S=0) == bcjr.BCJR_E_SHAPE
    assert fwd(B=-1) == bcjr.BCJR_E_SHAPE
    assert fwd(L=0) == bcjr.BCJR_E_SHAPE
    assert fwd(B=1 << 40, L=1 << 30) == bcjr.BCJR_E_SHAPE
    assert fwd(S=48) == bcjr.BCJR_E_UNSUPPORTED
    assert fwd(T=0.0) == bcjr.BCJR_E_ARG
    assert fwd(T=float("nan")) == bcjr.BCJR_E_ARG
    assert fwd(th=P(0)) == bcjr.BCJR_E_ARG
    assert fwd(cb=P(0)) == bcjr.BCJR_E_ARG
    assert fwd(sv=P(0x5004)) == bcjr.BCJR_E_ARG  # context must be 16-byte aligned
    assert fwd(ws=P(0)) == bcjr.BCJR_E_WORKSPACE
    assert fwd(ws=P(0x6008)) == bcjr.BCJR_E_WORKSPACE
    need = bcjr.bcjr_dense_workspace_bytes(64, 4, 8, 0)
    assert fwd(wsb=need - 1) == bcjr.BCJR_E_WORKSPACE
    assert fwd(B=0, th=P(0), w=P(0), wh=P(0), lz=P(0), sv=P(0), ws=P(0), wsb=0) == bcjr.BCJR_OK

    assert bwd(T=-1.0) == bcjr.BCJR_E_ARG
    assert bwd(gt=P(0)) == bcjr.BCJR_E_ARG
    assert bwd(gc=P(0)) == bcjr.BCJR_E_ARG
    assert bwd(g=P(0)) == bcjr.BCJR_E_ARG
    assert bwd(S=100) == bcjr.BCJR_E_UNSUPPORTED
    # the linear-domain dense path is refused below T = 0.1 (its states underflow there)
    for T in (0.0999, 0.05, 0.01):
        assert fwd(T=T) == bcjr.BCJR_E_UNSUPPORTED
        assert bwd(T=T) == bcjr.BCJR_E_UNSUPPORTED
        assert fwd(T=T, B=0, th=P(0), w=P(0), wh=P(0), lz=P(0), sv=P(0), ws=P(0), wsb=0) == \
            bcjr.BCJR_E_UNSUPPORTED
    assert fwd(T=0.1, wsb=0) == bcjr.BCJR_E_WORKSPACE  # accepted from 0.1 on
    need = bcjr.bcjr_dense_workspace_bytes(64, 4, 8, 1)
    assert bwd(wsb=need - 1) == bcjr.BCJR_E_WORKSPACE


def test_autograd_wrapper_refuses_cpu_tensors():
    import torch
    from bcjr_soft_decoding_amd import autograd
    w = torch.zeros((2, 8), dtype=torch.float32)
    c = torch.zeros(16, dtype=torch.float32)
    with pytest.raises(ValueError):
        autograd.soft_quantize(w, c, 4, 2, 0.5)
    with pytest.raises(ValueError):
        autograd.dense_soft_quantize(w, torch.zeros(32), torch.zeros((32, 32)), 0.5)


def test_checkpointed_workspace_sizes(lib):
    # checkpoints every C = ceil(sqrt(L)) steps plus one C-step replay buffer per slot
    for n, L in [(12, 256), (16, 256), (8, 1000), (16, 4096)]:
        for full, ck in [(bcjr.FWD, bcjr.FWD_CKPT), (bcjr.BWD, bcjr.BWD_CKPT)]:
            f = bcjr.bcjr_workspace_bytes(n, 2, 4096, L, full)
            c = bcjr.bcjr_workspace_bytes(n, 2, 4096, L, ck)
            assert 0 < c < f
    # at S = 65536, L = 4096 the full forward history is 128x the checkpointed one's history
    f = bcjr.bcjr_workspace_bytes(16, 2, 16384, 4096, bcjr.FWD)
    c = bcjr.bcjr_workspace_bytes(16, 2, 16384, 4096, bcjr.FWD_CKPT)
    assert f > 200 * 2**30 and c < 16 * 2**30
    assert bcjr.bcjr_workspace_bytes(8, 2, 16, 16, 5) == 0
    assert bcjr.bcjr_workspace_bytes(8, 2, 0, 16, bcjr.BWD_CKPT) == 0


def test_code_export_queries_and_validation(lib):
    import oracle
    for n, k, L in [(4, 2, 1), (8, 2, 256), (16, 2, 256), (12, 3, 100), (16, 1, 4096)]:
        assert bcjr.bcjr_code_words(n, k, L) == oracle.code_words(n, k, L)
    assert bcjr.bcjr_code_words(17, 2, 10) == 0
    assert bcjr.bcjr_code_words(8, 2, 0) == 0
    P = ctypes.c_void_p
    tr = bcjr.Trellis(8, 2, 1, 0)
    assert lib.bcjr_pack_code(ctypes.byref(tr), None, 4, 8, P(0x1000), None) == bcjr.BCJR_E_ARG
    assert lib.bcjr_pack_code(ctypes.byref(tr), P(0x1000), -1, 8, P(0x1000), None) == bcjr.BCJR_E_SHAPE
    assert lib.bcjr_pack_code(ctypes.byref(tr), None, 0, 8, None, None) == bcjr.BCJR_OK
    # w_hard needs the codebook
    assert lib.bcjr_unpack_code(ctypes.byref(tr), P(0x1000), 4, 8, P(0x2000), P(0x3000), None) == bcjr.BCJR_E_ARG
    tr2 = bcjr.Trellis(8, 2, 2, 0x4000)
    assert lib.bcjr_unpack_code(ctypes.byref(tr2), P(0x1000), 4, 8, P(0x2000), None, None) == bcjr.BCJR_E_UNSUPPORTED


def test_qat_driver_validates_before_any_gpu_call():
    import torch
    from bcjr_soft_decoding_amd import qat
    W = torch.zeros(2, 512)
    with pytest.raises(TypeError):
        qat.train(W, torch.zeros(4, 512), torch.zeros(256), qat.QATConfig(n=8, steps=1))
    with pytest.raises(ValueError):
        qat.train(W, torch.zeros(4, 512), torch.zeros(256), qat.QATConfig(n=8, L=300))
    with pytest.raises(ValueError):
        qat.QATConfig(t0=0.0).check()
    with pytest.raises(ValueError):
        qat.QATConfig(n=3, k=2).check()
    cfg = qat.QATConfig(t0=0.3, t_end=0.01, steps=5)
    assert qat.temperature(cfg, 0) == pytest.approx(0.3) and qat.temperature(cfg, 4) == pytest.approx(0.01)


def test_scan_size_queries_and_plan(lib):
    # default segment length ~ sqrt(L), longer for wider transfer matrices and (where the
    # boundary scan is a tree over the segments, M <= 64) for more chains, at least 16 steps
    d20 = bcjr.bcjr_scan_segment_length(8, 2, 1, 1 << 20)
    d16 = bcjr.bcjr_scan_segment_length(8, 2, 1, 1 << 16)
    assert 128 <= d20 <= 512 and 32 <= d16 <= 128 and d16 < d20
    assert bcjr.bcjr_scan_segment_length(8, 2, 16, 1 << 16) >= 2 * d16
    assert bcjr.bcjr_scan_segment_length(12, 2, 1, 1 << 16) > 2 * d16
    assert bcjr.bcjr_scan_segment_length(4, 2, 1, 20) == 16
    assert bcjr.bcjr_scan_segment_length(8, 2, 4, 5000, 300) == 300    # explicit length kept
    assert bcjr.bcjr_scan_segment_length(8, 2, 4, 5000, -1) == 0       # invalid
    assert bcjr.bcjr_scan_segment_length(13, 2, 4, 5000) == 0          # not built for S > 4096
    # workspace: transfer matrices B * P * M^2 doubles dominate; a single segment needs none
    M, B, L, seg = 64, 2, 4096, 256
    ws = bcjr.bcjr_scan_workspace_bytes(8, 2, B, L, seg)
    assert ws >= B * (L // seg) * M * M * 8
    one = bcjr.bcjr_scan_workspace_bytes(8, 2, B, L, L)
    assert 0 < one < B * M * M * 8 + bcjr.bcjr_workspace_bytes(8, 2, B, L, bcjr.FWD) + 65536
    # a ragged tail adds one segment
    assert bcjr.bcjr_scan_workspace_bytes(8, 2, B, L + 1, seg) > ws
    assert bcjr.bcjr_scan_workspace_bytes(8, 2, 0, L, seg) == 0


def test_scan_rejects_bad_arguments_without_device(lib):
    P = ctypes.c_void_p

    def scan(n=8, k=2, cb=0x1000, w=0x2000, B=2, L=64, T=0.5, seg=16, wh=0x3000, lz=0x4000,
             ws=0x6000, wsb=1 << 40):
        tr = bcjr.Trellis(n, k, 1, cb)
        return lib.bcjr_forward_scan(ctypes.byref(tr), P(w), B, L, T, seg, P(wh), P(lz), P(ws),
                                     wsb, None)

    assert lib.bcjr_forward_scan(None, None, 1, 1, 1.0, 0, None, None, None, 0, None) == bcjr.BCJR_E_ARG
    assert scan(seg=-1) == bcjr.BCJR_E_ARG
    assert scan(T=0.0) == bcjr.BCJR_E_ARG
    assert scan(T=float("nan")) == bcjr.BCJR_E_ARG
    assert scan(cb=0) == bcjr.BCJR_E_ARG
    assert scan(w=0) == bcjr.BCJR_E_ARG
    assert scan(wh=0) == bcjr.BCJR_E_ARG
    assert scan(lz=0) == bcjr.BCJR_E_ARG
    assert scan(n=13) == bcjr.BCJR_E_UNSUPPORTED
    assert scan(n=0) == bcjr.BCJR_E_SHAPE
    assert scan(L=0) == bcjr.BCJR_E_SHAPE
    assert scan(B=-1) == bcjr.BCJR_E_SHAPE
    need = bcjr.bcjr_scan_workspace_bytes(8, 2, 2, 64, 16)
    assert scan(wsb=need - 1) == bcjr.BCJR_E_WORKSPACE
    assert scan(ws=0x6008) == bcjr.BCJR_E_WORKSPACE
    assert scan(B=0, w=0, wh=0, lz=0, ws=0, wsb=0) == bcjr.BCJR_OK


def test_scan_backward_rejects_bad_arguments_without_device(lib):
    P = ctypes.c_void_p

    def bscan(n=8, cb=0x1000, w=0x2000, B=2, L=64, T=0.5, seg=16, wh=0x3000, g=0x4000, gw=0x5000,
              gc=0x7000, ws=0x6000, wsb=1 << 40):
        tr = bcjr.Trellis(n, 2, 1, cb)
        return lib.bcjr_backward_scan(ctypes.byref(tr), P(w), B, L, T, seg, P(wh), P(g), None,
                                      P(gw), P(gc), P(ws), wsb, None)

    assert bscan(seg=-1) == bcjr.BCJR_E_ARG
    assert bscan(T=0.0) == bcjr.BCJR_E_ARG
    assert bscan(gc=0) == bcjr.BCJR_E_ARG
    assert bscan(wh=0) == bcjr.BCJR_E_ARG
    assert bscan(g=0) == bcjr.BCJR_E_ARG
    assert bscan(gw=0) == bcjr.BCJR_E_ARG
    assert bscan(n=13) == bcjr.BCJR_E_UNSUPPORTED
    need = bcjr.bcjr_scan_backward_workspace_bytes(8, 2, 2, 64, 16)
    assert need > bcjr.bcjr_scan_workspace_bytes(8, 2, 2, 64, 16)   # moment rows and partials
    assert bscan(wsb=need - 1) == bcjr.BCJR_E_WORKSPACE
    assert bscan(ws=0x6008) == bcjr.BCJR_E_WORKSPACE
    assert bcjr.bcjr_scan_backward_workspace_bytes(8, 2, 0, 64, 16) == 0


def test_noalloc_forward_refuses_oversized_shapes_without_device(lib):
    # the checkpointed history of 2^20 chains of S = 4096 exceeds the fixed array; the refusal
    # comes before any device call (there is no device here)
    tr = bcjr.trellis(12, 2, None)
    P = ctypes.c_void_p
    B, L = 1 << 20, 256
    assert bcjr.bcjr_workspace_bytes(12, 2, B, L, 3) > bcjr.NOALLOC_SCRATCH_BYTES
    st = lib.bcjr_forward_noalloc(ctypes.byref(tr), P(0x2000), B, L, 0.1, P(0x3000), P(0x4000),
                                  P(0x5000), None)
    assert st == bcjr.BCJR_E_WORKSPACE
    header = open(os.path.join(ROOT, "include", "bcjr.h")).read()
    assert re.search(r"#define BCJR_NOALLOC_SCRATCH_BYTES \(\(size_t\)256 << 20\)", header)
    assert bcjr.NOALLOC_SCRATCH_BYTES == 256 << 20
