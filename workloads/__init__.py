"""Seeded synthetic inputs for the selective-scan workloads.

This module only draws random numbers and rounds them to the storage dtype; it
holds none of the scan's arithmetic and imports neither the HIP library nor the
oracle, so both sides can consume the same bits.

Rows of a tensor are drawn in blocks of about 2^19 values, each block from its
own PCG64 stream keyed by ``SeedSequence(seed, spawn_key=(tensor_id, block))``,
so any block can be regenerated alone and blocks are drawn in parallel threads
(numpy releases the GIL while filling).  Values are drawn in float32 and, for bf16 workloads,
rounded to bf16 with round-to-nearest-even; both the GPU and the oracle read
those exact bits.

Workloads (shapes, dtypes and distributions of the Mamba-style scans):

  tiny_fp32     batch 1, dim 16, N 4, L 256, fp32; u~N(0,1); raw delta~N(-2,0.5)
                with softplus, no bias; A[d,n] = -(n+1); B,C~N(0,1); D~N(0,1);
                no gate.
  mamba130m     batch 8, dim 1536, N 16, L 2048, bf16 u/delta/B/C/z; fp32
                A, D, bias; u,z~N(0,1); raw delta~N(0,1); delta_bias =
                log(expm1(U[1e-3, 1e-1])); A = -exp(log(1..16)); B,C~N(0,1);
                D~N(0,1); silu(z) gate.
  mamba2p8b     as mamba130m at batch 4, dim 5120, N 16, L 8192.
  long_context  batch 1, dim 2048, N 16, L 524288, bf16; u~N(0,1); raw
                delta~N(-4,1) with softplus, no bias; A = -exp(U[ln 0.5, ln 16])
                iid per (d, n); B,C~N(0,1); D~N(0,1); no gate.
  decode        batch 256, dim 5120, N 16, one token per step, 1000 steps;
                fp32 state ~N(0, 0.1); per step fresh bf16 u, raw delta, z ~N(0,1)
                [256, 5120] and B, C ~N(0,1) [256, 16]; bias, A, D as mamba130m.

N(mu, sigma) names the standard deviation as the second parameter.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

# tensor ids used in the per-row stream keys
T_U, T_DELTA, T_Z, T_B, T_C, T_A, T_D, T_BIAS, T_STATE, T_DY, T_DFINAL = range(11)
T_CX, T_CW, T_CB, T_CSTATE, T_CDOUT = range(11, 16)
T_SX, T_SDT, T_SB, T_SC, T_SZ, T_SA, T_SD, T_SBIAS, T_SH0 = range(16, 25)


@dataclass(frozen=True)
class Workload:
    name: str
    index: int            # position in the list of measured configurations (1-based)
    batch: int
    dim: int
    dstate: int
    seqlen: int           # tokens per sequence (1 for decode)
    dtype: str            # "f32" or "bf16": dtype of u, delta, B, C, z, y
    gate: bool            # silu(z) gate present
    delta_mean: float
    delta_std: float
    bias: bool            # delta_bias = log(expm1(U[1e-3, 1e-1]))
    a_init: str           # "s4d_real": A = -(n+1);  "loguniform": A = -exp(U[ln .5, ln 16])
    steps: int = 0        # decode steps (decode workload only)

    @property
    def seed(self) -> int:
        return 4300 + self.index

    @property
    def elements(self) -> int:
        """Scan elements per pass, batch * dim * L * N."""
        return self.batch * self.dim * self.seqlen * self.dstate

    @property
    def io_bytes(self) -> int:
        """Bytes of u, delta, (z), B, C read once plus y written once."""
        s = 2 if self.dtype == "bf16" else 4
        seq = self.batch * self.dim * self.seqlen
        return s * (seq * (2 + int(self.gate)) + 2 * self.batch * self.dstate * self.seqlen + seq)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_fp32", 1, 1, 16, 4, 256, "f32", False, -2.0, 0.5, False, "s4d_real"),
        Workload("mamba130m", 2, 8, 1536, 16, 2048, "bf16", True, 0.0, 1.0, True, "s4d_real"),
        Workload("mamba2p8b", 3, 4, 5120, 16, 8192, "bf16", True, 0.0, 1.0, True, "s4d_real"),
        Workload("long_context", 4, 1, 2048, 16, 524288, "bf16", False, -4.0, 1.0, False,
                 "loguniform"),
        Workload("decode", 5, 256, 5120, 16, 1, "bf16", True, 0.0, 1.0, True, "s4d_real",
                 steps=1000),
    ]
}


def threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def rng(seed: int, tensor_id: int, row: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(tensor_id, row))))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return to_bf16_bits(x) if dtype == "bf16" else x.astype(np.float32, copy=False)


def rows_per_stream(n: int, per_stream: int = 1 << 19) -> int:
    """Rows of length n drawn from one stream (about per_stream values)."""
    return max(1, per_stream // max(1, n))


def _normal_rows(seed, tid, key0, out, mean, std, dtype, per_stream=1 << 19):
    """Fill out[rows, n] with stored N(mean, std) draws.  Rows are grouped in
    blocks of rows_per_stream(n, per_stream); block k is drawn from stream
    (tid, key0 + k).  Blocks are spread over worker threads (numpy releases
    the GIL while it fills large arrays)."""
    rows, n = out.shape
    rb = rows_per_stream(n, per_stream)
    nblk = -(-rows // rb)

    def one(k):
        lo, hi = k * rb, min(rows, (k + 1) * rb)
        x = rng(seed, tid, key0 + k).standard_normal((hi - lo) * n, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        if mean != 0.0:
            x += np.float32(mean)
        out[lo:hi] = _store(x, dtype).reshape(hi - lo, n)

    with ThreadPoolExecutor(threads()) as ex:
        list(ex.map(one, range(nblk)))
    return out


def seq_tensor(w: Workload, tid: int, mean: float, std: float, seed=None):
    """A [batch, dim, L] (tid in u/delta/z) or [batch, N, L] (tid in B/C) tensor."""
    seed = w.seed if seed is None else seed
    inner = w.dim if tid in (T_U, T_DELTA, T_Z, T_DY) else w.dstate
    rows = w.batch * inner
    np_dtype = np.uint16 if w.dtype == "bf16" else np.float32
    out = np.empty((rows, w.seqlen), dtype=np_dtype)
    _normal_rows(seed, tid, 0, out, mean, std, w.dtype)
    return out.reshape(w.batch, inner, w.seqlen)


def params(w: Workload, seed=None):
    """A [dim, N], D [dim], delta_bias [dim] or None, all float32."""
    seed = w.seed if seed is None else seed
    if w.a_init == "s4d_real":
        # A = -exp(log(1..N)), repeated over channels; in fp64 then rounded to fp32
        a_row = (-np.exp(np.log(np.arange(1, w.dstate + 1, dtype=np.float64)))).astype(np.float32)
        A = np.tile(a_row, (w.dim, 1))
    else:
        lo, hi = np.log(0.5), np.log(16.0)
        A = np.empty((w.dim, w.dstate), dtype=np.float32)
        for d in range(w.dim):
            A[d] = (-np.exp(rng(seed, T_A, d).uniform(lo, hi, w.dstate))).astype(np.float32)
    D = rng(seed, T_D, 0).standard_normal(w.dim, dtype=np.float32)
    bias = None
    if w.bias:
        # inverse softplus of U[1e-3, 1e-1]: the initial step sizes of a Mamba layer
        dt0 = rng(seed, T_BIAS, 0).uniform(1e-3, 1e-1, w.dim)
        bias = np.log(np.expm1(dt0)).astype(np.float32)
    return np.ascontiguousarray(A), D, bias


def scan_inputs(w: Workload, seed=None):
    """All inputs of one forward scan as numpy arrays (bf16 as uint16 bits)."""
    A, D, bias = params(w, seed)
    return dict(
        u=seq_tensor(w, T_U, 0.0, 1.0, seed),
        delta=seq_tensor(w, T_DELTA, w.delta_mean, w.delta_std, seed),
        z=seq_tensor(w, T_Z, 0.0, 1.0, seed) if w.gate else None,
        B=seq_tensor(w, T_B, 0.0, 1.0, seed),
        C=seq_tensor(w, T_C, 0.0, 1.0, seed),
        A=A, D=D, delta_bias=bias, delta_softplus=True)


def grad_inputs(w: Workload, seed=None):
    """Upstream gradients for the backward pass: dy [batch, dim, L] ~N(0,1) in
    the workload's storage dtype and dfinal [batch, dim, N] ~N(0,1) float32."""
    seed = w.seed if seed is None else seed
    dfinal = np.empty((w.batch * w.dim, w.dstate), dtype=np.float32)
    _normal_rows(seed, T_DFINAL, 0, dfinal, 0.0, 1.0, "f32")
    return dict(dy=seq_tensor(w, T_DY, 0.0, 1.0, seed),
                dfinal=dfinal.reshape(w.batch, w.dim, w.dstate))


def conv_inputs(w: Workload, width=4, seed=None):
    """Inputs of the causal conv1d in front of the scan, at the workload's
    [batch, dim, L] shape: x ~ N(0,1) and dout ~ N(0,1) in the storage dtype;
    weight ~ U(-1/sqrt(W), 1/sqrt(W)) and bias ~ U(-1/sqrt(W), 1/sqrt(W))
    float32 (the default init of a depthwise Conv1d, fan-in W); state_in
    [batch, dim, W-1] ~ N(0,1) float32."""
    seed = w.seed if seed is None else seed
    rows = w.batch * w.dim
    np_dtype = np.uint16 if w.dtype == "bf16" else np.float32
    x = np.empty((rows, w.seqlen), dtype=np_dtype)
    _normal_rows(seed, T_CX, 0, x, 0.0, 1.0, w.dtype)
    dout = np.empty((rows, w.seqlen), dtype=np_dtype)
    _normal_rows(seed, T_CDOUT, 0, dout, 0.0, 1.0, w.dtype)
    bound = 1.0 / np.sqrt(width)
    weight = rng(seed, T_CW, 0).uniform(-bound, bound, (w.dim, width)).astype(np.float32)
    bias = rng(seed, T_CB, 0).uniform(-bound, bound, w.dim).astype(np.float32)
    state = np.empty((rows, max(width - 1, 1)), dtype=np.float32)
    _normal_rows(seed, T_CSTATE, 0, state, 0.0, 1.0, "f32")
    return dict(x=x.reshape(w.batch, w.dim, w.seqlen), weight=weight, bias=bias,
                state_in=state[:, :width - 1].reshape(w.batch, w.dim, width - 1).copy(),
                dout=dout.reshape(w.batch, w.dim, w.seqlen))


@dataclass(frozen=True)
class SsdWorkload:
    """A Mamba-2 layer's scan: x, z [batch, nheads * headdim, L], dt [batch,
    nheads, L], B, C [batch, ngroups * dstate, L], all bf16."""
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    ngroups: int
    dstate: int
    gate: bool = True
    seed: int = 4400

    @property
    def elements(self) -> int:
        return self.batch * self.seqlen * self.nheads * self.headdim * self.dstate

    @property
    def io_bytes(self) -> int:
        seq = self.batch * self.nheads * self.headdim * self.seqlen * 2
        return ((3 if self.gate else 2) * seq + self.batch * self.nheads * self.seqlen * 2
                + 2 * self.batch * self.ngroups * self.dstate * self.seqlen * 2)


# Mamba-2 2.7B-shaped layer (d_inner 5120 = 80 heads x 64, N 128, one group)
SSD_WORKLOADS = {
    "mamba2_2p7b": SsdWorkload("mamba2_2p7b", 4, 8192, 80, 64, 1, 128),
}


def ssd_inputs(w: SsdWorkload, seed=None, with_h0=False):
    """x, z, B, C ~ N(0,1) and raw dt ~ N(0,1) in bf16; A = -U[1, 16] per head
    (A = -exp(log U[1, 16])), D ~ N(0,1), dt_bias = log(expm1(U[1e-3, 1e-1]))
    (a step of 0.001..0.1 at zero raw input), all float32; h0 [batch, nheads,
    headdim, dstate] ~ N(0, 0.1) float32 when asked for."""
    seed = w.seed if seed is None else seed
    hp = w.nheads * w.headdim

    def seq(tid, rows):
        out = np.empty((w.batch * rows, w.seqlen), dtype=np.uint16)
        _normal_rows(seed, tid, 0, out, 0.0, 1.0, "bf16")
        return out.reshape(w.batch, rows, w.seqlen)

    A = -rng(seed, T_SA, 0).uniform(1.0, 16.0, w.nheads).astype(np.float32)
    D = rng(seed, T_SD, 0).standard_normal(w.nheads).astype(np.float32)
    step = rng(seed, T_SBIAS, 0).uniform(1e-3, 1e-1, w.nheads)
    bias = np.log(np.expm1(step)).astype(np.float32)
    x = dict(x=seq(T_SX, hp), dt=seq(T_SDT, w.nheads), B=seq(T_SB, w.ngroups * w.dstate),
             C=seq(T_SC, w.ngroups * w.dstate), z=seq(T_SZ, hp) if w.gate else None,
             A=A, D=D, dt_bias=bias, h0=None)
    if with_h0:
        h0 = np.empty((w.batch * w.nheads, w.headdim * w.dstate), dtype=np.float32)
        _normal_rows(seed, T_SH0, 0, h0, 0.0, 0.1, "f32")
        x["h0"] = h0.reshape(w.batch, w.nheads, w.headdim, w.dstate)
    return x


def decode_state(w: Workload, seed=None) -> np.ndarray:
    """Initial fp32 decode state [batch, dim, N] ~ N(0, 0.1), one stream per
    sequence b."""
    seed = w.seed if seed is None else seed
    out = np.empty((w.batch, w.dim * w.dstate), dtype=np.float32)
    _normal_rows(seed, T_STATE, 0, out, 0.0, 0.1, "f32")
    return out.reshape(w.batch, w.dim, w.dstate)


def decode_step(w: Workload, step: int, seed=None):
    """Fresh per-step inputs: u, delta, z [batch, dim]; B, C [batch, N].

    Each tensor is drawn in blocks of about 2^16 values, one stream per
    (tensor, step, block), so a step's inputs are generated in parallel."""
    seed = w.seed if seed is None else seed
    np_dtype = np.uint16 if w.dtype == "bf16" else np.float32

    def t(tid, inner, mean, std):
        out = np.empty((w.batch, inner), dtype=np_dtype)
        _normal_rows(seed, tid, (step + 1) << 32, out, mean, std, w.dtype, per_stream=1 << 16)
        return out

    return dict(u=t(T_U, w.dim, 0.0, 1.0),
                delta=t(T_DELTA, w.dim, w.delta_mean, w.delta_std),
                z=t(T_Z, w.dim, 0.0, 1.0) if w.gate else None,
                B=t(T_B, w.dstate, 0.0, 1.0),
                C=t(T_C, w.dstate, 0.0, 1.0))


def custom(batch, dim, dstate, seqlen, dtype="bf16", gate=True, bias=True,
           delta_mean=0.0, delta_std=1.0, a_init="s4d_real", seed=1234, name="custom"):
    """A workload of any shape with the Mamba-layer distributions (for parity
    sweeps over tiles and ragged tails)."""
    w = Workload(name, 0, batch, dim, dstate, seqlen, dtype, gate, delta_mean, delta_std,
                 bias, a_init)
    return w, scan_inputs(w, seed)
