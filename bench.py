"""Benchmark of the selective-scan hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mamba2p8b]

A step is one forward selective scan (ssm_selective_scan_fwd: load, step size,
discretization, scan, readout, skip, gate, store) over the whole batch of the
Mamba-2.8B-shaped layer (batch 4, dim 5120, N 16, L 8192, bf16 io, fp32
arithmetic and state).  Inputs are generated once, uploaded, and resident in
HBM before timing starts.  The one-token decode step (ssm_state_update) is
timed separately on the decode workload and reported under "decode", and the
backward pass (ssm_selective_scan_bwd) on the same workload under "backward",
the causal conv1d in front of the scan (forward and backward) under
"conv1d", the Mamba-2 scan (scalar A per head, on MFMA) under "ssd", the
forward scan on the long-context workload under "long_context", the
forward under each discretization rule under "rules" and the time-invariant
path under "lti".

Prints one JSON line: the metric (scan elements B*D*L*N per second), the
roofline of the scan kernel (live HIP-event timing; HBM traffic from the
committed rocprofv3 counter summary when it matches the current kernel
source), the HBM view the metric asks for, and the fp64 oracle timed on host
cores as a baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402

HBM_PEAK_GBPS = 8000.0
# VALU issue capacity: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz lane-slots/s.
VALU_PEAK_TSLOTS = 256 * 4 * 16 * 2.4e9 / 1e12
# Minimal VALU lane-slots per scan element: Delta*A (1), exp (2: half rate on
# gfx950), (Delta u)*B (1), state fma (1), readout fma (1).
SLOTS_PER_ELEMENT = 6
KERNEL_SRC = os.path.join(ROOT, "selective_state_space_43_amd", "csrc", "selscan.hip")
PMC_SUMMARY = os.path.join(ROOT, "profiles", "scan_fwd_mamba2p8b_pmc.md")
VALU_SUMMARY = os.path.join(ROOT, "profiles", "scan_fwd_mamba2p8b_valu.md")


SCAN_SOURCE_END = b"// ---------------------------------------------------------------- backward"


def kernel_source_hash() -> str:
    """Hash of the forward scan's source: selscan.hip up to the backward
    section (the helpers and both forward kernels); later kernels do not change
    the scan's traffic."""
    with open(KERNEL_SRC, "rb") as f:
        src = f.read()
    end = src.find(SCAN_SOURCE_END)
    return hashlib.sha256(src[:end] if end >= 0 else src).hexdigest()[:16]


def committed_traffic():
    """HBM bytes per scan launch from the committed counter summary, or None if
    the summary is missing or was taken on a different kernel source."""
    try:
        text = open(PMC_SUMMARY).read()
    except OSError:
        return None
    m_src = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_tr = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m_src and m_tr) or m_src.group(1) != kernel_source_hash():
        return None
    return float(m_tr.group(1))


def committed_valu_busy():
    """VALU busy fraction of the scan kernel from the committed counter
    summary, or None if it is missing or was taken on a different source."""
    try:
        text = open(VALU_SUMMARY).read()
    except OSError:
        return None
    m_src = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_b = re.search(r"VALU busy:.*=\s*([0-9.]+)", text)
    if not (m_src and m_b) or m_src.group(1) != kernel_source_hash():
        return None
    return float(m_b.group(1))


def to_dev(a, dev):
    import torch
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def host_threads() -> int:
    """Threads for the oracle baseline: the host cores this process may run
    on, at most 16 (the share of the host that comes with one GPU of an
    eight-GPU node; more would take cores that belong to other GPUs' work)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def settle(fn, torch, warmup, min_ms=250.0):
    """Untimed calls before a timed region: `warmup` of them, and more until
    the GPU has run this work for `min_ms` (clocks ramp up under sustained
    load; a short burst after an idle gap is timed at lower clocks)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < min_ms:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()


# Infinity Cache (MALL) of the MI355X: 256 MB.  A workload whose bytes fit in
# it would be timed from the cache on repeated launches, so such workloads get
# a read of FLUSH_BYTES from a scratch buffer between timed launches (a read,
# not a write: it leaves no dirty lines whose write-back the timed launch
# would pay for).
MALL_BYTES = 256 * 2**20
FLUSH_BYTES = 512 * 2**20


def make_flush(torch, dev):
    """A function that evicts the Infinity Cache by reading FLUSH_BYTES."""
    buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    out = torch.empty((), dtype=torch.float32, device=dev)
    return lambda: torch.sum(buf, dim=0, out=out)


def bench_scan(ssm, torch, w, x, dev, steps, warmup):
    """The forward scan: `warmup` untimed launches plus at least 250 ms of
    sustained work (clocks settle), then `steps` launches each bracketed by
    HIP events on the library's stream.  Returns per-step and per-launch
    statistics (ms)."""
    u, dl, A, B, C = (to_dev(x[k], dev) for k in ("u", "delta", "A", "B", "C"))
    D, z, bias = to_dev(x["D"], dev), to_dev(x["z"], dev), to_dev(x["delta_bias"], dev)
    y = torch.empty_like(u)
    fs = torch.empty((w.batch, w.dim, w.dstate), dtype=torch.float32, device=dev)

    def step():
        ssm.ssm_selective_scan_fwd(u, dl, A, B, C, D=D, z=z, delta_bias=bias,
                                   delta_softplus=True, y=y, final_state=fs)

    flush = make_flush(torch, dev) if w.io_bytes < MALL_BYTES else None
    settle(step, torch, warmup)
    stream = torch.cuda.current_stream(dev)  # the library launches on this stream
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for a, b in ev:
        if flush is not None:
            flush()  # evicts the inputs from the Infinity Cache (untimed)
        a.record(stream)
        step()
        b.record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    per_launch = np.array([a.elapsed_time(b) for a, b in ev])
    total_ms = t_start.elapsed_time(t_end)
    # with flushes in the region, a step is the launch alone
    ms_step = float(per_launch.mean()) if flush is not None else total_ms / steps
    return dict(ms_step=ms_step, mean=float(per_launch.mean()),
                median=float(np.median(per_launch)), min=float(per_launch.min()),
                max=float(per_launch.max()), wall=wall, flushed=flush is not None)


def bench_rules(ssm, torch, w, x, dev, steps):
    """The forward scan on the same inputs under each discretization rule
    (delta*B, exact ZOH, Euler, bilinear): milliseconds per call."""
    u, dl, A, B, C = (to_dev(x[k], dev) for k in ("u", "delta", "A", "B", "C"))
    D, z, bias = to_dev(x["D"], dev), to_dev(x["z"], dev), to_dev(x["delta_bias"], dev)
    y = torch.empty_like(u)
    fs = torch.empty((w.batch, w.dim, w.dstate), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    res = {"workload": f"{w.name} forward, same inputs, per discretization rule"}
    for rule in ("delta", "zoh", "euler", "bilinear"):
        def step():
            ssm.ssm_selective_scan_fwd(u, dl, A, B, C, D=D, z=z, delta_bias=bias,
                                       delta_softplus=True, bbar=rule, y=y, final_state=fs)
        settle(step, torch, 2)
        a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(steps):
            step()
        e.record(stream)
        torch.cuda.synchronize()
        res[rule + "_ms"] = round(a.elapsed_time(e) / steps, 4)
    res["steps"] = steps
    return res


def bench_decode(ssm, torch, dev, steps, warmup):
    """Decode steps captured once in a HIP graph (as a serving loop would run
    them) and replayed, so the time is the GPU's, not the Python launcher's."""
    w = wl.WORKLOADS["decode"]
    A, D, bias = wl.params(w)
    state = to_dev(wl.decode_state(w), dev)
    pool = []
    for i in range(4):  # a few distinct token batches, resident in HBM, used in turn
        s = wl.decode_step(w, i)
        pool.append({k: to_dev(v, dev) for k, v in s.items()})
    Ad, Dd, bd = to_dev(A, dev), to_dev(D, dev), to_dev(bias, dev)
    y = torch.empty((w.batch, w.dim), dtype=torch.bfloat16, device=dev)

    def step(i):
        p = pool[i % len(pool)]
        ssm.ssm_state_update(state, p["u"], p["delta"], Ad, p["B"], p["C"], D=Dd, z=p["z"],
                             delta_bias=bd, delta_softplus=True, y=y)

    ctr = iter(range(1 << 30))
    settle(lambda: step(next(ctr)), torch, warmup)
    per_graph = 50
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(per_graph):
            step(i)
    torch.cuda.synchronize()
    settle(g.replay, torch, 1)
    reps = max(1, steps // per_graph)
    stream = torch.cuda.current_stream(dev)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    n_steps = reps * per_graph
    us = a.elapsed_time(b) * 1e3 / n_steps
    state_bytes = 2 * w.batch * w.dim * w.dstate * 4  # read + write in place
    io_bytes = w.batch * w.dim * 2 * 4 + 2 * w.batch * w.dstate * 2  # u, delta, z, y; B, C
    # The 84 MB state stays in the 256 MB Infinity Cache from one replayed step
    # to the next, as it would in a decode loop.  For the HBM rate, single
    # steps are also timed with a 512 MB read in between (state and inputs
    # evicted); the read also covers the launch of the step that follows it.
    flush = make_flush(torch, dev)
    cold = []
    for i in range(20):
        flush()
        ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ea.record(stream)
        step(i)
        eb.record(stream)
        cold.append((ea, eb))
    torch.cuda.synchronize()
    us_cold = float(np.mean([ea.elapsed_time(eb) for ea, eb in cold])) * 1e3
    gbps = (state_bytes + io_bytes) / (us_cold * 1e-6) / 1e9
    return {
        "workload": f"decode: batch {w.batch}, dim {w.dim}, N {w.dstate}, one bf16 token, "
                    "fp32 state in place",
        "us_per_step": round(us, 3),
        "tokens_per_s": round(w.batch / (us * 1e-6), 1),
        "elements_per_s": float("%.4g" % (w.batch * w.dim * w.dstate / (us * 1e-6))),
        "timing": "HIP graph of 50 steps, replayed (state resident in the Infinity Cache "
                  "between steps)",
        "us_per_step_cold": round(us_cold, 3),
        "hbm_bytes_per_step": state_bytes + io_bytes,
        "hbm_gbps": round(gbps, 1),
        "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "hbm_timing": "single steps after a 512 MB read that evicts the state (mean of 20)",
        "steps": n_steps,
    }


def bench_bwd(ssm, torch, w, x, dev, steps, warmup):
    """The backward pass (ssm_selective_scan_bwd: checkpointed forward, adjoint
    carries, gradients) on the same inputs with a seeded upstream gradient.
    Every gradient is produced; the workspace is allocated once outside the
    timed region.  Timed standalone (the backward recomputes its checkpoints),
    as a training step (a forward that writes checkpoints followed by a
    backward that takes them), and as that backward alone."""
    g = wl.grad_inputs(w)
    u, dl, A, B, C = (to_dev(x[k], dev) for k in ("u", "delta", "A", "B", "C"))
    D, z, bias = to_dev(x["D"], dev), to_dev(x["z"], dev), to_dev(x["delta_bias"], dev)
    dy = to_dev(g["dy"], dev)
    ws = torch.empty(ssm.ssm_selective_scan_bwd_workspace_size(w.batch, w.dim, w.dstate,
                                                               w.seqlen),
                     dtype=torch.uint8, device=dev)

    ck = torch.empty(ssm.ssm_checkpoint_shape(w.batch, w.dim, w.dstate, w.seqlen),
                     dtype=torch.float32, device=dev)
    y = torch.empty_like(u)

    def step():
        return ssm.ssm_selective_scan_bwd(u, dl, A, B, C, dy, D=D, z=z, delta_bias=bias,
                                          delta_softplus=True, workspace=ws, want_dh0=True)

    def train_step():
        ssm.ssm_selective_scan_fwd(u, dl, A, B, C, D=D, z=z, delta_bias=bias, delta_softplus=True,
                                   y=y, want_final_state=False, checkpoints=ck)
        return ssm.ssm_selective_scan_bwd(u, dl, A, B, C, dy, D=D, z=z, delta_bias=bias,
                                          delta_softplus=True, workspace=ws, want_dh0=True,
                                          checkpoints=ck)

    stream = torch.cuda.current_stream(dev)

    def timed(fn):
        settle(fn, torch, warmup)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(steps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    def bwd_from_checkpoints():
        return ssm.ssm_selective_scan_bwd(u, dl, A, B, C, dy, D=D, z=z, delta_bias=bias,
                                          delta_softplus=True, workspace=ws, want_dh0=True,
                                          checkpoints=ck)

    ms = timed(step)
    ms_train = timed(train_step)
    ms_ckpt = timed(bwd_from_checkpoints)  # ck holds the forward's checkpoints by now
    es = 2 if w.dtype == "bf16" else 4
    seq = w.batch * w.dim * w.seqlen * es
    bc = w.batch * w.dstate * w.seqlen * es
    n_seq_in = 4 if w.gate else 3      # u, delta, dy (, z)
    n_seq_out = 3 if w.gate else 2     # du, ddelta (, dz)
    algo = (n_seq_in + n_seq_out) * seq + 4 * bc  # B, C read; dB, dC written
    gbps = algo / (ms * 1e-3) / 1e9
    return {
        "workload": f"{w.name} backward: every gradient (du, ddelta, dz, dA, dB, dC, dD, "
                    "ddelta_bias, dh0)",
        "ms_per_call": round(ms, 4),
        "elements_per_s": float("%.4g" % (w.elements / (ms * 1e-3))),
        "algorithmic_bytes": algo,
        "hbm_gbps": round(gbps, 1),
        "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "train_step_ms": round(ms_train, 4),
        "train_step": "forward writing checkpoints, then the backward taking them",
        "ms_from_checkpoints": round(ms_ckpt, 4),
        "from_checkpoints": "the backward alone, given the forward's checkpoints (no checkpoint pass)",
        "steps": steps,
    }


def bench_conv(ssm, torch, w, dev, steps, warmup):
    """The causal conv1d + silu in front of the scan (width 4, bias) at the
    workload's [batch, dim, L] shape: forward and backward, HBM-bound."""
    c = wl.conv_inputs(w, width=4)
    x, wt, b, dout = (to_dev(c[k], dev) for k in ("x", "weight", "bias", "dout"))
    out = torch.empty_like(x)
    stream = torch.cuda.current_stream(dev)

    def timed(fn):
        settle(fn, torch, warmup)
        a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(steps):
            fn()
        e.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(e) / steps

    ms_f = timed(lambda: ssm.ssm_causal_conv1d_fwd(x, wt, b, out=out))
    ms_b = timed(lambda: ssm.ssm_causal_conv1d_bwd(x, wt, dout, b))
    seq = x.numel() * x.element_size()
    res = {"workload": f"{w.name} conv1d: x [{w.batch}, {w.dim}, {w.seqlen}] {w.dtype}, width 4, "
                       "bias, silu"}
    for name, ms, nbytes in (("fwd", ms_f, 2 * seq), ("bwd", ms_b, 3 * seq)):
        gbps = nbytes / (ms * 1e-3) / 1e9
        res[name] = {"ms": round(ms, 4), "algorithmic_bytes": nbytes, "hbm_gbps": round(gbps, 1),
                     "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4)}
    return res


def bench_long(ssm, torch, dev, steps, warmup):
    """The forward scan on the long-context workload (batch 1, dim 2048, N 16,
    L 524288, bf16, no gate): 64 lanes per channel, 1024-step chunks."""
    w = wl.WORKLOADS["long_context"]
    x = wl.scan_inputs(w)
    u, dl, A, B, C = (to_dev(x[k], dev) for k in ("u", "delta", "A", "B", "C"))
    D = to_dev(x["D"], dev)
    del x
    y = torch.empty_like(u)
    fs = torch.empty((w.batch, w.dim, w.dstate), dtype=torch.float32, device=dev)

    def step():
        ssm.ssm_selective_scan_fwd(u, dl, A, B, C, D=D, delta_softplus=True, y=y, final_state=fs)

    settle(step, torch, warmup)
    stream = torch.cuda.current_stream(dev)
    a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        step()
    e.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(e) / steps
    gbps = w.io_bytes / (ms * 1e-3) / 1e9
    slots = SLOTS_PER_ELEMENT * w.elements / (ms * 1e-3) / 1e12
    return {"workload": f"{w.name}: batch {w.batch}, dim {w.dim}, N {w.dstate}, L {w.seqlen}, "
                        "bf16, no gate",
            "ms_per_call": round(ms, 4),
            "elements_per_s": float("%.4g" % (w.elements / (ms * 1e-3))),
            "algorithmic_bytes": w.io_bytes, "hbm_gbps": round(gbps, 1),
            "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
            "alu_frac": round(slots / VALU_PEAK_TSLOTS, 4), "steps": steps}


def bench_lti(ssm, torch, dev, steps, warmup):
    """The time-invariant path on the mamba130m shape (batch 8, dim 1536,
    N 16, L 2048, bf16 u and y): the kernel K from ssm_lti_kernel, then
    y = K * u + D u by the direct causal sum and by FFT."""
    w = wl.WORKLOADS["mamba130m"]
    A, D, _ = wl.params(w)
    r = np.random.default_rng(w.seed)
    Bv, Cv = r.standard_normal(w.dstate).astype(np.float32), r.standard_normal(w.dstate).astype(np.float32)
    step = r.uniform(0.01, 0.2, w.dim).astype(np.float32)
    u = torch.randn((w.batch, w.dim, w.seqlen), generator=torch.Generator().manual_seed(w.seed)
                    ).to(torch.bfloat16).to(dev)
    Ad, Bd, Cd, sd, Dd = (to_dev(v, dev) for v in (A, Bv, Cv, step, D))
    K = ssm.ssm_lti_kernel(Ad, Bd, Cd, sd, w.seqlen)
    y = torch.empty_like(u)
    stream = torch.cuda.current_stream(dev)

    def timed(fn):
        settle(fn, torch, warmup)
        a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(steps):
            fn()
        e.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(e) / steps

    ms_k = timed(lambda: ssm.ssm_lti_kernel(Ad, Bd, Cd, sd, w.seqlen, K=K))
    ms_d = timed(lambda: ssm.ssm_lti_conv(K, u, D=Dd, y=y))
    ms_f = timed(lambda: ssm.ssm_lti_conv(K, u, D=Dd, y=y, method="fft"))
    # longer sequences at the same batch and dim: L 8192 (M 16384, one
    # in-LDS transform per signal) and L 65536 (M 131072 = 256 x 512, the
    # four-step transforms through the workspace)
    Ll = 4 * w.seqlen
    Kl = ssm.ssm_lti_kernel(Ad, Bd, Cd, sd, Ll)
    ul = torch.randn((w.batch, w.dim, Ll), generator=torch.Generator().manual_seed(w.seed + 1)
                     ).to(torch.bfloat16).to(dev)
    yl = torch.empty_like(ul)
    wsl = torch.empty(ssm.ssm_lti_conv_fft_workspace_size(w.dim, Ll), dtype=torch.uint8, device=dev)
    ms_fl = timed(lambda: ssm.ssm_lti_conv(Kl, ul, D=Dd, y=yl, method="fft", workspace=wsl))
    del Kl, ul, yl, wsl
    Lx = 32 * w.seqlen
    Kx = ssm.ssm_lti_kernel(Ad, Bd, Cd, sd, Lx)
    ux = torch.randn((w.batch, w.dim, Lx), device=dev,  # drawn on the GPU: 805 M values
                     generator=torch.Generator(device=dev).manual_seed(w.seed + 2)).to(torch.bfloat16)
    yx = torch.empty_like(ux)
    wsx = torch.empty(ssm.ssm_lti_conv_fft_workspace_size(w.dim, Lx), dtype=torch.uint8, device=dev)
    ms_fx = timed(lambda: ssm.ssm_lti_conv(Kx, ux, D=Dd, y=yx, method="fft", workspace=wsx))
    del Kx, ux, yx, wsx
    return {"workload": f"LTI path: batch {w.batch}, dim {w.dim}, N {w.dstate}, L {w.seqlen}, "
                        "bf16 u and y",
            "kernel_ms": round(ms_k, 4), "conv_direct_ms": round(ms_d, 4),
            "conv_fft_ms": round(ms_f, 4), "conv_fft_long_L": Ll,
            "conv_fft_long_ms": round(ms_fl, 4), "conv_fft_longer_L": Lx,
            "conv_fft_longer_ms": round(ms_fx, 4), "steps": steps}


MFMA_BF16_PEAK_TFLOPS = 2500.0


def bench_ssd(ssm, torch, dev, steps, warmup):
    """The Mamba-2 scan (scalar A per head, chunks of 64 on MFMA) on the
    Mamba-2 2.7B layer shape."""
    w = wl.SSD_WORKLOADS["mamba2_2p7b"]
    x = wl.ssd_inputs(w)
    t = {k: to_dev(v, dev) for k, v in x.items() if v is not None}
    y = torch.empty_like(t["x"])
    fs = torch.empty((w.batch, w.nheads, w.headdim, w.dstate), dtype=torch.float32, device=dev)
    ws = torch.empty(ssm.ssm_ssd_workspace_size(w.batch, w.seqlen, w.ngroups, w.dstate),
                     dtype=torch.uint8, device=dev)

    def step():
        ssm.ssm_ssd_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], w.nheads, w.ngroups, D=t["D"],
                        z=t["z"], dt_bias=t["dt_bias"], dt_softplus=True, y=y, final_state=fs,
                        workspace=ws)

    settle(step, torch, warmup)
    stream = torch.cuda.current_stream(dev)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        step()
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    T = 64
    chunks = -(-w.seqlen // T)
    # algorithmic FLOPs of the chunked form: per (sequence, head, chunk) M X, C S^T and the
    # state update; per (sequence, group, chunk) C B^T
    flops = (w.batch * w.nheads * chunks * (2 * T * T * w.headdim + 4 * T * w.dstate * w.headdim)
             + w.batch * w.ngroups * chunks * 2 * T * T * w.dstate)
    gbps = w.io_bytes / (ms * 1e-3) / 1e9
    tflops = flops / (ms * 1e-3) / 1e12
    return {
        "workload": f"{w.name}: batch {w.batch}, L {w.seqlen}, {w.nheads} heads x {w.headdim}, "
                    f"N {w.dstate}, {w.ngroups} group, bf16, gate",
        "ms_per_call": round(ms, 4),
        "elements_per_s": float("%.4g" % (w.elements / (ms * 1e-3))),
        "algorithmic_bytes": w.io_bytes,
        "hbm_gbps": round(gbps, 1),
        "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "algorithmic_tflops": round(tflops, 2),
        "mfma_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "steps": steps,
    }


def cpu_baseline(w, x, seconds_target=12.0):
    """The fp64 oracle on host cores over whole channels of the same inputs:
    as many channels (full length each) as fit the time target."""
    import oracle
    n_thr = host_threads()
    total = w.batch * w.dim
    probe = np.arange(0, total, max(1, total // (4 * n_thr)))[: 4 * n_thr]
    t0 = time.perf_counter()
    oracle.selective_scan(x["u"], x["delta"], x["A"], x["B"], x["C"], D=x["D"], z=x["z"],
                          delta_bias=x["delta_bias"], delta_softplus=True, channels=probe,
                          want_y=False, n_threads=n_thr)
    per_ch = (time.perf_counter() - t0) / len(probe)
    n_ch = int(min(total, max(len(probe), seconds_target / max(per_ch, 1e-9))))
    chans = np.linspace(0, total - 1, n_ch).astype(np.int64)
    t0 = time.perf_counter()
    oracle.selective_scan(x["u"], x["delta"], x["A"], x["B"], x["C"], D=x["D"], z=x["z"],
                          delta_bias=x["delta_bias"], delta_softplus=True, channels=chans,
                          want_y=False, n_threads=n_thr)
    dt = time.perf_counter() - t0
    el = n_ch * w.seqlen * w.dstate
    return {"value": float("%.4g" % (el / dt)), "unit": "elements/s", "cores": n_thr,
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"{n_ch} of {total} channels (b, d), full length {w.seqlen}, all "
                      f"{w.dstate} states, same {w.dtype} inputs; fp64 sequential recurrence"}


def main(argv=None):
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=300)
    p.add_argument("--workload", default="mamba2p8b",
                   choices=[k for k in wl.WORKLOADS if k != "decode"])
    p.add_argument("--decode-steps", type=int, default=200)
    p.add_argument("--no-decode", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-backward", action="store_true")
    p.add_argument("--no-conv", action="store_true")
    p.add_argument("--no-ssd", action="store_true")
    p.add_argument("--no-lti", action="store_true")
    p.add_argument("--no-long", action="store_true")
    p.add_argument("--no-rules", action="store_true")
    p.add_argument("--backward-steps", type=int, default=5)
    p.add_argument("--copy-check", type=int, default=0, metavar="BYTES",
                   help="also run torch's plain copy of BYTES three times (counter calibration "
                        "under rocprofv3)")
    args = p.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the scan shards by batch and channel with no "
              "communication, and this build runs on a single MI355X; use --gpus 1.",
              file=sys.stderr)
        return 2

    import torch
    import selective_state_space_43_amd as ssm
    ssm.lib()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")

    w = wl.WORKLOADS[args.workload]
    t0 = time.perf_counter()
    x = wl.scan_inputs(w)
    print(f"[bench] inputs for {w.name} generated in {time.perf_counter() - t0:.1f}s",
          file=sys.stderr, flush=True)
    st = bench_scan(ssm, torch, w, x, dev, args.steps, args.warmup)
    ms_step, ms_kernel = st["ms_step"], st["mean"]
    print(f"[bench] scan: {ms_step:.4f} ms/step, kernel mean {ms_kernel:.4f} ms, median "
          f"{st['median']:.4f}, min {st['min']:.4f}, max {st['max']:.4f}", file=sys.stderr,
          flush=True)
    el = w.elements
    value = el / (ms_step * 1e-3)
    hbm_gbps = w.io_bytes / (ms_kernel * 1e-3) / 1e9
    achieved_tslots = SLOTS_PER_ELEMENT * el / (ms_kernel * 1e-3) / 1e12
    # the committed counter summary is taken on the 2.8B workload
    traffic = committed_traffic() if w.name == "mamba2p8b" else None

    out = {
        "metric": "selective-scan elements/sec (B*D*L*N)",
        "value": float("%.5g" % value),
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",  # arithmetic; u, delta, B, C, z and y are stored as config.io_dtype
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: Mamba-2.8B-shaped selective scan" if w.name == "mamba2p8b"
            else w.name,
            "batch": w.batch, "dim": w.dim, "dstate": w.dstate, "seqlen": w.seqlen,
            "io_dtype": w.dtype, "gate": w.gate, "delta_softplus": True,
            "delta_bias": w.bias, "bbar": "delta*B", "parallelism": "single GPU",
        },
        "roofline": {
            "kernel": "scan_fwd_pipe_kernel",
            "bound": "hbm",
            "achieved": round(hbm_gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(hbm_gbps / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": w.io_bytes,
            "kernel_ms_mean": round(ms_kernel, 4),
            "kernel_ms_median": round(st["median"], 4),
            "kernel_ms_min": round(st["min"], 4),
            "launches": args.steps,
            "cache_flushed_between_launches": st["flushed"],
        },
        # the scan issues far more VALU work per byte than HBM can feed at
        # 8 TB/s: the same kernel time against the VALU issue rate, with a
        # minimum of 6 lane-slots per element (delta*A, exp (half rate),
        # (delta u)*B, state fma, readout fma)
        "alu_view": {
            "achieved": round(achieved_tslots, 3),
            "peak": round(VALU_PEAK_TSLOTS, 3),
            "unit": "T VALU lane-slots/s (6 slots per element)",
            "frac": round(achieved_tslots / VALU_PEAK_TSLOTS, 4),
            "valu_busy": committed_valu_busy() if w.name == "mamba2p8b" else None,
        },
    }
    if args.copy_check:
        src = torch.empty(args.copy_check // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_check_bytes"] = args.copy_check
        del src, dst
    if not args.no_decode:
        out["decode"] = bench_decode(ssm, torch, dev, args.decode_steps, 10)
        print(f"[bench] decode: {out['decode']['us_per_step']} us/step (state cached), "
              f"{out['decode']['us_per_step_cold']} us/step from HBM", file=sys.stderr, flush=True)
    if not args.no_backward and w.dstate <= 64:
        out["backward"] = bench_bwd(ssm, torch, w, x, dev, args.backward_steps, 1)
        print(f"[bench] backward: {out['backward']['ms_per_call']} ms/call", file=sys.stderr,
              flush=True)
    if not args.no_conv:
        out["conv1d"] = bench_conv(ssm, torch, w, dev, 50, 2)
        print(f"[bench] conv1d: fwd {out['conv1d']['fwd']['ms']} ms, bwd "
              f"{out['conv1d']['bwd']['ms']} ms", file=sys.stderr, flush=True)
    if not args.no_ssd:
        out["ssd"] = bench_ssd(ssm, torch, dev, 30, 2)
        print(f"[bench] ssd: {out['ssd']['ms_per_call']} ms/call", file=sys.stderr, flush=True)
    if not args.no_rules:
        out["rules"] = bench_rules(ssm, torch, w, x, dev, 20)
        print(f"[bench] rules: " + ", ".join(f"{k} {v}" for k, v in out["rules"].items()
                                              if k.endswith("_ms")), file=sys.stderr, flush=True)
    if not args.no_long:
        out["long_context"] = bench_long(ssm, torch, dev, 10, 1)
        print(f"[bench] long_context: {out['long_context']['ms_per_call']} ms/call",
              file=sys.stderr, flush=True)
    if not args.no_lti:
        out["lti"] = bench_lti(ssm, torch, dev, 5, 1)
        print(f"[bench] lti: kernel {out['lti']['kernel_ms']} ms, conv direct "
              f"{out['lti']['conv_direct_ms']} ms, fft {out['lti']['conv_fft_ms']} ms, fft at L "
              f"{out['lti']['conv_fft_long_L']} {out['lti']['conv_fft_long_ms']} ms, fft at L "
              f"{out['lti']['conv_fft_longer_L']} {out['lti']['conv_fft_longer_ms']} ms",
              file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, x)
        print(f"[bench] cpu baseline: {out['cpu_baseline']['seconds']}s", file=sys.stderr,
              flush=True)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
