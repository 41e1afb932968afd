"""Throughput benchmark of the BCJR soft-decoding hot path on one MI355X.

One step = bcjr_forward + bcjr_backward (soft codeword, log Z, gradient to w and the codebook)
over the whole workload, inputs resident in HBM, workspaces preallocated. The default
workload is the Llama-3.2-1B MLP up-projection shape: a 2048 x 8192 Gaussian matrix at unit
RMS cut into 65536 chains of 256 weights, 2^12-state bitshift trellis with 2 bits per step,
T = 0.1 (synthetic data; see bcjr_soft_decoding_amd/synth.py).

    python bench.py [--steps K] [--warmup W] [--workload 3] [--no-cpu-baseline]

Prints ONE JSON line. `value` is trellis state-steps per second (B * L * S per step) from the
median of the per-step HIP event times. The `roofline` object prices one forward + backward step
against the ALU peak with the frozen operation model in OPMODEL.md, crediting only the method's
own work (the backward's recomputation of the forward's recursions is overhead); per-kernel
fields sit beside it. `cpu_baseline` times the plain CPU oracle on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "BCJR fwd+bwd trellis state-steps/sec (1 MI355X) + % of HBM/compute roofline"

# ---------------------------------------------------------------------------------------------
# Operation model of the bitshift forward-backward, frozen in OPMODEL.md (read from its JSON
# block): slots per trellis state-step of each phase, and whether the phase is the method's own
# work or the backward's recomputation of the forward's recursions. `roofline.frac` credits only
# the method's work (30.25 slots per forward + backward state-step) against the whole step's
# median time; the per-kernel fields give each kernel's model slots against its own time.
# Peak: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz = 39.32 T VALU slots/s; a transcendental takes 2.
# ---------------------------------------------------------------------------------------------
OPMODEL_PATH = os.path.join(ROOT, "OPMODEL.md")


def load_opmodel(path: str = OPMODEL_PATH) -> dict:
    import re
    text = open(path).read()
    m = re.search(r"```json\n(.*?)```", text, re.S)
    if m is None:
        raise RuntimeError(f"{path} has no JSON block")
    return json.loads(m.group(1))


OPMODEL = load_opmodel()
TRANS_SLOTS = float(OPMODEL["trans_slots"])
PEAK_TOPS = float(OPMODEL["peak_slots_per_s"]) / 1e12


def _slots(pred) -> float:
    return sum(v["valu"] + TRANS_SLOTS * v["trans"] for v in OPMODEL["phases"].values() if pred(v))


def op_slots(kernel: str) -> float:
    """Model slots per state-step the kernel is built to issue ("fwd" or "bwd"), recompute incl."""
    return _slots(lambda v: v["kernel"] == kernel)


def method_slots() -> float:
    """Slots per state-step of the method's own work over one forward + backward."""
    return _slots(lambda v: v["credit"] == "method")


def phase_slots(name: str) -> float:
    v = OPMODEL["phases"][name]
    return v["valu"] + TRANS_SLOTS * v["trans"]


# HBM traffic of the profiled kernels, read from the committed rocprofv3 summaries; reported only
# while the kernel sources still hash to the value recorded there.
TRAFFIC_PROFILES = {
    "fwd": os.path.join(ROOT, "profiles", "k_sparse_fwd_llama32-1b-mlp-up-s4096_pmc.md"),
    "bwd": os.path.join(ROOT, "profiles", "k_sparse_bwd_llama32-1b-mlp-up-s4096_pmc.md"),
}
KERNEL_SOURCES = ["bcjr_soft_decoding_amd/csrc/sparse_kernels.hip", "bcjr_soft_decoding_amd/csrc/sparse_device.h",
                  "bcjr_soft_decoding_amd/csrc/geom.h", "bcjr_soft_decoding_amd/csrc/internal.h"]


def kernel_names(n: int, k: int):
    """Names of the forward and backward kernels that run for (n, k) with fp32 messages: chains
    whose S / K^2 blocks need more than 1024 lanes at the kernel's states per lane (64 forward,
    32 backward) use the wide kernels."""
    ng = (1 << n) >> (2 * k)

    def wide(target):
        g = max(min(max(target >> (2 * k), 1), ng), ng // 1024)
        return ng // g >= 1024
    return ("k_sparse_fwd_wide" if wide(64) else "k_sparse_fwd",
            "k_sparse_bwd_wide" if wide(32) else "k_sparse_bwd")


def median_ms(pairs):
    import numpy as np
    return float(np.median([a.elapsed_time(b) for a, b in pairs]))


def kernel_source_hash() -> str:
    """sha256 of the profiled kernels' sources and of the compiler options they are built with
    (include paths, which name the checkout's location, left out)."""
    import hashlib
    from bcjr_soft_decoding_amd import build
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    opts = [build.ARCH, [f for f in build.FLAGS if not f.startswith("-I")],
            build.EXTRA_FLAGS.get("sparse_kernels.hip", []), build.ILP_FLAGS]
    h.update(repr(opts).encode())
    return h.hexdigest()


def profiled_traffic(workload_name: str):
    """HBM bytes of one forward + backward (both kernels' launches) from the committed counter
    summaries, or None if there is none for this workload or the kernels changed since."""
    total = 0.0
    for path in TRAFFIC_PROFILES.values():
        if not os.path.exists(path) or workload_name not in path:
            return None
        fields = {}
        for line in open(path):
            if ":" in line and line.strip().startswith("- "):
                k, v = line.strip()[2:].split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
        if fields.get("source_sha256") != kernel_source_hash():
            return None
        try:
            total += float(fields["traffic_bytes_per_launch"])
        except (KeyError, ValueError):
            return None
    return total


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--temp", type=float, default=None)
    ap.add_argument("--history", choices=["full", "ckpt"], default=None,
                    help="bitshift message histories: every step, or checkpoints + segment replay "
                         "(default: checkpoints every 16 steps for the S = 65536 workload, as that "
                         "configuration is specified; every step otherwise)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=1536,
                    help="chains timed on the CPU oracle (at most CPU_SAMPLE_STATE_STEPS state-steps)")
    ap.add_argument("--cpu-sample-dense", type=int, default=64,
                    help="chains of the dense workload timed on the CPU oracle")
    ap.add_argument("--viterbi", action="store_true",
                    help="time the Viterbi decoder (the T -> 0 limit) on the workload instead")
    ap.add_argument("--export", action="store_true",
                    help="time the hard-code export (pack / unpack of Viterbi paths) instead")
    ap.add_argument("--seg-len", type=int, default=0,
                    help="segment length of the segmented forward (workload 6); 0 = default")
    ap.add_argument("--cpu-scan-steps", type=int, default=1 << 17,
                    help="chain steps timed on the CPU oracle for workload 6")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (HBM counter calibration)")
    return ap.parse_args()


def copy_calibration():
    import torch
    n = 1 << 28  # 2^28 floats = 1 GiB
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": 4 * n, "copy_calibration_bytes_written": 4 * n}))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# The oracle's sample is capped at this many state-steps (about 15 s of fp64 work on 16 host
# threads), so that large trellises (S = 65536) do not hold the run for minutes.
CPU_SAMPLE_STATE_STEPS = 1536 * 256 * 4096


def cpu_sample_chains(args, wl):
    return max(1, min(args.cpu_sample, wl.B, CPU_SAMPLE_STATE_STEPS // (wl.L * wl.S)))


def cpu_baseline(wl, c, w, g, T, sample):
    import oracle
    cores = oracle.set_threads(0)
    ws = w[:sample]
    gs = g[:sample]
    t0 = time.perf_counter()
    oracle.sparse_forward(wl.n, wl.k, c, ws, T)
    oracle.sparse_backward(wl.n, wl.k, c, ws, T, gs)
    dt = time.perf_counter() - t0
    # the same work on one thread, on a sixteenth of the sample
    s1 = max(1, sample // 16)
    oracle.set_threads(1)
    t1 = time.perf_counter()
    oracle.sparse_forward(wl.n, wl.k, c, w[:s1], T)
    oracle.sparse_backward(wl.n, wl.k, c, w[:s1], T, g[:s1])
    d1 = time.perf_counter() - t1
    oracle.set_threads(cores)
    return {
        "value": sample * wl.L * wl.S / dt,
        "unit": "state-steps/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"first {sample} of {wl.B} chains (L={wl.L}, S={wl.S}), fp64 oracle forward + "
                  f"backward, {dt:.1f} s on {cores} OpenMP threads",
        "value_1thread": s1 * wl.L * wl.S / d1,
        "cpu_model": cpu_model(),
    }


# ---------------------------------------------------------------------------------------------
# Dense trellis (fully connected, S x S transition matrix): algorithmic matrix-core work per
# state-step, counted from the recursions (a multiply-add is 2 flops):
#   forward call : alpha sweep S MACs + beta sweep S MACs                       -> 4 S flops
#   backward call: Psi sweep S MACs + Phi sweep S MACs + theta gradient 2 S MACs -> 8 S flops
#                  (the theta gradient runs over the L-1 transitions of a chain)
# Peak: dense fp32 MFMA, 157.3 TFLOP/s on MI355X.
# ---------------------------------------------------------------------------------------------
PEAK_FP32_MFMA = 157.3


def dense_flops(B, L, S):
    fwd = 2.0 * (2 * S) * B * L * S
    bwd = 2.0 * (2 * S) * B * L * S + 2.0 * (2 * S) * B * (L - 1) * S
    return fwd, bwd


def cpu_baseline_dense(wl, th, c, w, g, T, sample):
    import oracle
    cores = oracle.set_threads(0)
    t0 = time.perf_counter()
    oracle.dense_forward(th, c, w[:sample], T)
    oracle.dense_backward(th, c, w[:sample], T, g[:sample])
    dt = time.perf_counter() - t0
    return {
        "value": sample * wl.L * wl.S / dt,
        "unit": "state-steps/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"first {sample} of {wl.B} chains (L={wl.L}, S={wl.S} dense), fp64 oracle "
                  f"forward + backward incl. theta gradient, {dt:.1f} s on {cores} OpenMP threads",
        "cpu_model": cpu_model(),
    }


def bench_dense(args, wl):
    import numpy as np
    import torch

    from bcjr_soft_decoding_amd import bcjr, synth
    T = args.temp if args.temp is not None else wl.temps[0]
    B, L, S = wl.B, wl.L, wl.S
    i = wl.index
    th_np, c_np, w_np, g_np = synth.theta(i), synth.codebook(i), synth.weights(i), synth.upstream_grad(i)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    th, c, w, g = (torch.from_numpy(a).to(dev) for a in (th_np, c_np, w_np, g_np))
    w_hat = torch.empty_like(w)
    log_z = torch.empty(B, dtype=torch.float32, device=dev)
    saved = torch.empty(bcjr.bcjr_dense_saved_bytes(S, B, L), dtype=torch.uint8, device=dev)
    grad_w = torch.empty_like(w)
    grad_c = torch.empty_like(c)
    grad_th = torch.empty_like(th)
    wsf = bcjr.dense_workspace(S, B, L, bcjr.FWD, dev)
    wsb = bcjr.dense_workspace(S, B, L, bcjr.BWD, dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        bcjr.bcjr_dense_forward(th, c, w, T, w_hat, log_z, saved, wsf)
        if ev is not None:
            ev[1].record()
        bcjr.bcjr_dense_backward(th, c, w, T, saved, g, None, grad_w, grad_c, grad_th, wsb)
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    step_ms = median_ms([(e[0], e[2]) for e in evs])
    fwd_ms = median_ms([(e[0], e[1]) for e in evs])
    bwd_ms = median_ms([(e[1], e[2]) for e in evs])
    assert torch.isfinite(w_hat).all() and torch.isfinite(grad_th).all()
    ff, fb = dense_flops(B, L, S)
    achieved = fb / (bwd_ms * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": B * L * S / (step_ms * 1e-3),
        "unit": "state-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "L": L, "S": S, "T": T, "trellis": "dense",
                   "parallelism": "single-gpu"},
        "timing": "median of per-step HIP event times (forward + backward) over the timed steps",
        "wall_ms_per_step": elapsed * 1e3 / args.steps,
        "kernels_ms": {"forward": fwd_ms, "backward": bwd_ms},
        # trellis edges per second: every state follows every state, S per state-step
        "edges_per_s": B * L * S / (step_ms * 1e-3) * S,
        "roofline": {
            "bound": "mfma",
            "kernel": "bcjr_dense_backward (k_dense_sweep Psi + Phi, k_dense_theta_gemm)",
            "achieved": achieved,
            "peak": PEAK_FP32_MFMA,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_FP32_MFMA,
            "flops_per_launch": fb,
            "forward_frac": ff / (fwd_ms * 1e-3) / 1e12 / PEAK_FP32_MFMA,
            "traffic": None,
        },
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_dense(wl, th_np, c_np, w_np, g_np, T,
                                                 min(args.cpu_sample_dense, B))
    print(json.dumps(out))


# Hard-code export: pack reads the int32 state path and writes k bits per step; unpack reads the
# code (each word serves 32/k states through the caches) and writes the int32 states and the fp32
# hard codeword. Algorithmic HBM bytes per chain-step: pack 4 + k/8, unpack k/8 + 8.
PEAK_HBM = 8.0e12


def bench_export(args, wl):
    import numpy as np
    import torch

    from bcjr_soft_decoding_amd import bcjr, synth
    n, k, B, L = wl.n, wl.k, wl.B, wl.L
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    c = torch.from_numpy(synth.codebook(wl.index)).to(dev)
    w = torch.from_numpy(synth.weights(wl.index)).to(dev)
    states, _ = bcjr.viterbi_decode(c, w, n, k, want_w_hard=False)
    code = bcjr.bcjr_pack_code(states, n, k)
    st2 = torch.empty_like(states)
    wh2 = torch.empty_like(w)
    for _ in range(args.warmup):
        bcjr.bcjr_pack_code(states, n, k, code)
        bcjr.bcjr_unpack_code(code, n, k, L, c, st2, wh2)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e in ev:
        e[0].record()
        bcjr.bcjr_pack_code(states, n, k, code)
        e[1].record()
        bcjr.bcjr_unpack_code(code, n, k, L, c, st2, wh2)
        e[2].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    assert torch.equal(st2, states)
    step_ms = median_ms([(e[0], e[2]) for e in ev])
    pack_ms = median_ms([(e[0], e[1]) for e in ev])
    unpack_ms = median_ms([(e[1], e[2]) for e in ev])
    steps = B * L
    pack_b, unpack_b = steps * (4 + k / 8), steps * (k / 8 + 8)
    ach = unpack_b / (unpack_ms * 1e-3)
    print(json.dumps({
        "metric": "hard-code export chain-steps/sec (pack + unpack, 1 MI355X)",
        "value": steps / (step_ms * 1e-3), "unit": "chain-steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": step_ms,
        "wall_ms_per_step": elapsed * 1e3 / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u32",
        "data": "synthetic",
        "config": {"workload": wl.name + "-viterbi-export", "B": B, "L": L, "S": wl.S, "k": k,
                   "code_words_per_chain": int(code.shape[1]), "parallelism": "single-gpu"},
        "kernels_ms": {"pack": pack_ms, "unpack": unpack_ms},
        "roofline": {"bound": "hbm", "kernel": "k_unpack_code", "achieved": ach / 1e9,
                     "peak": PEAK_HBM / 1e9, "unit": "GB/s", "frac": ach / PEAK_HBM,
                     "pack_frac": pack_b / (pack_ms * 1e-3) / PEAK_HBM, "traffic": None},
    }))


# Segmented forward-backward of long chains (parallel in L). Algorithmic ALU work per call:
#   forward : phase 1 runs the alpha recursion from S/K one-hot starts per segment (alpha side:
#             4.5 VALU + 1.25 trans = 7.0 slots per state-step over L * S * S/K state-steps),
#             phase 3 the full forward over L * S state-steps (16.5 slots);
#   backward: phase 1 runs the alpha + Phi recursion from the one-hot starts (7.25 VALU + 1.5
#             trans = 10.25 slots over L * S * S/K), phase 3 the full backward (29.25 slots).
# The boundary scans between them do O(segments * (S/K)^2) work, counted as 0.
SCAN_FWD_ROW_SLOTS = phase_slots("fwd_alpha")
SCAN_BWD_ROW_SLOTS = phase_slots("bwd_alpha") + phase_slots("bwd_phi")


def cpu_baseline_scan(wl, c, w, g, T, steps):
    import oracle
    cores = oracle.set_threads(0)
    t0 = time.perf_counter()
    oracle.sparse_forward(wl.n, wl.k, c, w[:, :steps], T)
    oracle.sparse_backward(wl.n, wl.k, c, w[:, :steps], T, g[:, :steps])
    dt = time.perf_counter() - t0
    return {
        "value": wl.B * steps * wl.S / dt,
        "unit": "state-steps/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"first {steps} of {wl.L} steps of the chain (S={wl.S}), fp64 oracle forward + "
                  f"backward (sequential in L; one chain runs on one thread), {dt:.1f} s",
        "cpu_model": cpu_model(),
    }


def bench_scan(args, wl):
    import numpy as np
    import torch

    from bcjr_soft_decoding_amd import bcjr, synth
    T = args.temp if args.temp is not None else wl.temps[0]
    n, k, B, L, S = wl.n, wl.k, wl.B, wl.L, wl.S
    M = S >> k
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    c_np, w_np, g_np = synth.codebook(wl.index), synth.weights(wl.index), synth.upstream_grad(wl.index)
    c, w, g = (torch.from_numpy(a).to(dev) for a in (c_np, w_np, g_np))
    seg = bcjr.bcjr_scan_segment_length(n, k, B, L, args.seg_len)
    wsf = torch.empty(bcjr.bcjr_scan_workspace_bytes(n, k, B, L, seg), dtype=torch.uint8, device=dev)
    wsb = torch.empty(bcjr.bcjr_scan_backward_workspace_bytes(n, k, B, L, seg), dtype=torch.uint8,
                      device=dev)
    w_hat = torch.empty_like(w)
    log_z = torch.empty(B, dtype=torch.float32, device=dev)
    grad_w = torch.empty_like(w)
    grad_c = torch.empty_like(c)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        bcjr.bcjr_forward_scan(c, w, n, k, T, seg, w_hat, log_z, wsf)
        if ev is not None:
            ev[1].record()
        bcjr.bcjr_backward_scan(c, w, n, k, T, w_hat, g, None, seg, grad_w, grad_c, wsb)
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e in ev:
        step(e)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    step_ms = median_ms([(e[0], e[2]) for e in ev])
    fwd_ms = median_ms([(e[0], e[1]) for e in ev])
    bwd_ms = median_ms([(e[1], e[2]) for e in ev])
    assert torch.isfinite(w_hat).all() and torch.isfinite(grad_w).all() and torch.isfinite(grad_c).all()
    # the sequential entry points on the same chain, for reference (one untimed warm-up each)
    wh2, lz2, saved = bcjr.bcjr_forward(c, w, n, k, T)
    gw2, gc2 = bcjr.bcjr_backward(c, w, n, k, T, saved, g)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    bcjr.bcjr_forward(c, w, n, k, T, wh2, lz2, saved)
    bcjr.bcjr_backward(c, w, n, k, T, saved, g, None, gw2, gc2)
    torch.cuda.synchronize()
    seq_ms = (time.perf_counter() - t1) * 1e3
    diff_w = float((w_hat - wh2).abs().max() / wh2.abs().max())
    diff_g = float((grad_w - gw2).abs().max() / gw2.abs().max())
    fslots = SCAN_FWD_ROW_SLOTS * L * S * M * B + op_slots("fwd") * L * S * B
    bslots = SCAN_BWD_ROW_SLOTS * L * S * M * B + op_slots("bwd") * L * S * B
    ach_b = bslots / (bwd_ms * 1e-3) / 1e12
    out = {
        "metric": "segmented BCJR fwd+bwd (parallel in L) trellis state-steps/sec (1 MI355X)",
        "value": B * L * S / (step_ms * 1e-3),
        "unit": "state-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "wall_ms_per_step": elapsed * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "L": L, "S": S, "k": k, "T": T,
                   "segment_length": seg, "segments": -(-L // seg),
                   "workspace_bytes": int(wsf.numel() + wsb.numel()), "parallelism": "single-gpu"},
        "kernels_ms": {"forward": fwd_ms, "backward": bwd_ms},
        "edges_per_s": B * L * S / (step_ms * 1e-3) * (1 << k),
        "sequential_fwd_bwd_ms": seq_ms,
        "speedup_vs_sequential": seq_ms / step_ms,
        "max_rel_diff_vs_sequential": {"w_hat": diff_w, "grad_w": diff_g},
        "roofline": {
            "bound": "alu",
            "kernel": "bcjr_backward_scan (k_sparse_bwd transfer/moment rows + k_scan_bounds + "
                      "k_sparse_bwd segments + k_reduce_slots)",
            "achieved": ach_b,
            "peak": PEAK_TOPS,
            "unit": "Tops/s",
            "frac": ach_b / PEAK_TOPS,
            "slots_per_launch": bslots,
            "accounting": "model slots per launch (OPMODEL.md phases, recompute included)",
            "forward_frac": fslots / (fwd_ms * 1e-3) / 1e12 / PEAK_TOPS,
            "traffic": None,
        },
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_scan(wl, c_np, w_np, g_np, T, min(args.cpu_scan_steps, L))
    print(json.dumps(out))


# Viterbi: per state-step (K = 4) a candidate costs sub + mul + add, and 3 of the K candidates a
# compare and two selects (value, index) for the first strict minimum: 5.25 VALU; backpointers
# 1 byte per butterfly = 0.25 B of HBM writes per state-step. ALU-bound (21 ops/B > ~5).
VIT_SLOTS = 5.25


def bench_viterbi(args, wl):
    import numpy as np
    import torch

    from bcjr_soft_decoding_amd import bcjr, synth
    n, k, B, L, S = wl.n, wl.k, wl.B, wl.L, wl.S
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    c_np, w_np = synth.codebook(wl.index), synth.weights(wl.index)
    c, w = torch.from_numpy(c_np).to(dev), torch.from_numpy(w_np).to(dev)
    states = torch.empty((B, L), dtype=torch.int32, device=dev)
    w_hard = torch.empty_like(w)
    ws = bcjr.workspace(n, k, B, L, bcjr.VIT, dev)
    for _ in range(args.warmup):
        bcjr.viterbi_decode(c, w, n, k, states, w_hard, ws=ws)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e in ev:
        e[0].record()
        bcjr.viterbi_decode(c, w, n, k, states, w_hard, ws=ws)
        e[1].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = median_ms([(e[0], e[1]) for e in ev])
    achieved = VIT_SLOTS * B * L * S / (ms * 1e-3) / 1e12
    out = {
        "metric": "Viterbi decode trellis state-steps/sec (1 MI355X)",
        "value": B * L * S / (ms * 1e-3), "unit": "state-steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "wall_ms_per_step": elapsed * 1e3 / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name + "-viterbi", "B": B, "L": L, "S": S, "k": k,
                   "workspace_bytes": int(ws.numel()), "parallelism": "single-gpu"},
        "kernels_ms": {"viterbi": ms},
        "roofline": {"bound": "alu", "kernel": "k_viterbi", "achieved": achieved, "peak": PEAK_TOPS,
                     "unit": "Tops/s", "frac": achieved / PEAK_TOPS,
                     "ops_per_state_step": VIT_SLOTS, "traffic": None},
    }
    if not args.no_cpu_baseline:
        import oracle
        cores = oracle.set_threads(0)
        sample = cpu_sample_chains(args, wl)
        t1 = time.perf_counter()
        ref = oracle.viterbi(n, k, c_np, w_np[:sample])
        dt = time.perf_counter() - t1
        assert np.array_equal(ref["states"], states[:sample].cpu().numpy()), "Viterbi paths differ"
        out["cpu_baseline"] = {
            "value": sample * L * S / dt, "unit": "state-steps/s", "cores": cores,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"first {sample} of {B} chains (L={L}, S={S}), fp32 oracle Viterbi "
                      f"(paths checked equal to the GPU's), {dt:.1f} s on {cores} OpenMP threads"}
    print(json.dumps(out))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (--gpus {args.gpus} requested); the "
              "multi-GPU sharding of the chains is a design note, not a built path.",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import numpy as np
    import torch

    from bcjr_soft_decoding_amd import bcjr, synth

    wl = synth.WORKLOADS[args.workload]
    if args.export:
        if wl.dense:
            raise SystemExit("the hard-code export is defined for the bitshift trellis")
        return bench_export(args, wl)
    if args.viterbi:
        if wl.dense:
            raise SystemExit("the Viterbi decoder is defined for the bitshift trellis")
        return bench_viterbi(args, wl)
    if wl.dense:
        return bench_dense(args, wl)
    if wl.index == 6:
        return bench_scan(args, wl)
    T = args.temp if args.temp is not None else wl.temps[0]
    n, k, B, L, S = wl.n, wl.k, wl.B, wl.L, wl.S
    c_np, w_np, g_np = synth.codebook(args.workload), synth.weights(args.workload), synth.upstream_grad(args.workload)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    c = torch.from_numpy(c_np).to(dev)
    w = torch.from_numpy(w_np).to(dev)
    g = torch.from_numpy(g_np).to(dev)
    w_hat = torch.empty_like(w)
    log_z = torch.empty(B, dtype=torch.float32, device=dev)
    saved = torch.empty(bcjr.bcjr_saved_bytes(n, k, B, L), dtype=torch.uint8, device=dev)
    grad_w = torch.empty_like(w)
    grad_c = torch.empty_like(c)
    if args.history is None:
        args.history = "ckpt" if args.workload == 4 else "full"
    ck = args.history == "ckpt"
    wsf = bcjr.workspace(n, k, B, L, bcjr.FWD_CKPT if ck else bcjr.FWD, dev)
    wsb = bcjr.workspace(n, k, B, L, bcjr.BWD_CKPT if ck else bcjr.BWD, dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        bcjr.bcjr_forward(c, w, n, k, T, w_hat, log_z, saved, wsf)
        if ev is not None:
            ev[1].record()
        bcjr.bcjr_backward(c, w, n, k, T, saved, g, None, grad_w, grad_c, wsb)
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # per-step HIP event times on the stream the kernels run on; medians over the timed steps
    step_ms = median_ms([(e[0], e[2]) for e in evs])
    fwd_ms = median_ms([(e[0], e[1]) for e in evs])
    bwd_ms = median_ms([(e[1], e[2]) for e in evs])
    assert torch.isfinite(w_hat).all() and torch.isfinite(grad_w).all() and torch.isfinite(grad_c).all()

    state_steps = B * L * S
    value = state_steps / (step_ms * 1e-3)
    fwd_name, bwd_name = kernel_names(n, k)
    method = method_slots()
    achieved = method * state_steps / (step_ms * 1e-3) / 1e12

    def kernel_fields(kind, ms):
        model = op_slots(kind)
        return {"median_ms": ms, "model_slots_per_state_step": model,
                "model_frac": model * state_steps / (ms * 1e-3) / 1e12 / PEAK_TOPS}

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "state-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "L": L, "S": S, "k": k, "T": T,
                   "history": args.history, "workspace_bytes": int(wsf.numel() + wsb.numel()),
                   "parallelism": "single-gpu"},
        "timing": "median of per-step HIP event times (forward + backward) over the timed steps",
        "wall_ms_per_step": elapsed * 1e3 / args.steps,
        "kernels_ms": {"forward": fwd_ms, "backward": bwd_ms},
        # trellis edges per second: K per state-step
        "edges_per_s": value * (1 << k),
        "roofline": {
            "bound": "alu",
            "kernel": f"{fwd_name} + {bwd_name} (+ k_reduce_slots): one forward + backward step",
            "achieved": achieved,
            "peak": PEAK_TOPS,
            "unit": "Tops/s",
            "frac": achieved / PEAK_TOPS,
            "ops_per_state_step": method,
            "accounting": "the method's slots per forward + backward state-step (OPMODEL.md); the "
                          "backward's recomputation of the forward's recursions is not credited",
            "per_kernel": {fwd_name: kernel_fields("fwd", fwd_ms),
                           bwd_name: kernel_fields("bwd", bwd_ms)},
            "traffic": profiled_traffic(wl.name) if not ck else None,
        },
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, c_np, w_np, g_np, T, cpu_sample_chains(args, wl))
    print(json.dumps(out))


if __name__ == "__main__":
    main()
