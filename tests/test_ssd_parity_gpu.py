"""Parity of the Mamba-2 scan (ssm_ssd_fwd, through the C ABI) against the
fp64 oracle on the same seeded bf16 inputs.  Bound, elementwise for y and the
final state: |gpu - oracle| <= 2e-2 (1 + |oracle|) (bf16 inputs; the MFMA
operands are bf16, accumulation and the state float32)."""
import numpy as np
import pytest

import oracle
import workloads as wl
from helpers import TOL, norm_err, to_dev, to_np

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ssm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_43_amd as m
    m.lib()
    return m


@pytest.fixture(scope="module")
def dev(ssm):
    return torch.device("cuda:0")


def run_gpu(ssm, dev, w, x, softplus=True):
    return ssm.ssm_ssd_fwd(to_dev(x["x"], dev), to_dev(x["dt"], dev), to_dev(x["A"], dev),
                           to_dev(x["B"], dev), to_dev(x["C"], dev), w.nheads, w.ngroups,
                           D=to_dev(x["D"], dev), z=to_dev(x["z"], dev),
                           dt_bias=to_dev(x["dt_bias"], dev), dt_softplus=softplus,
                           h0=to_dev(x["h0"], dev))


def run_oracle(w, x, softplus=True):
    return oracle.ssd(x["x"], x["dt"], x["A"], x["B"], x["C"], w.nheads, w.ngroups, D=x["D"],
                      z=x["z"], dt_bias=x["dt_bias"], dt_softplus=softplus, h0=x["h0"])


CASES = [  # batch, L, nheads, ngroups, dstate, gate, softplus, h0
    (1, 64, 2, 1, 32, False, True, False),
    (2, 300, 4, 2, 128, True, True, True),
    (1, 1000, 3, 1, 64, True, True, False),
    (1, 129, 2, 1, 256, False, True, True),
    (2, 517, 8, 4, 128, True, False, False),
    (1, 7, 2, 1, 128, True, True, True),
    (3, 4096, 2, 1, 128, True, True, False),
    (1, 2048, 2, 1, 256, True, True, True),    # N 256 over 32 chunks
    (2, 3001, 4, 2, 64, False, True, True),    # ragged, unaligned rows, two groups
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_ssd_shapes(ssm, dev, case):
    batch, L, H, G, N, gate, softplus, h0 = case
    w = wl.SsdWorkload("case", batch, L, H, 64, G, N, gate, seed=4500 + L)
    x = wl.ssd_inputs(w, with_h0=h0)
    if not softplus:  # raw steps used as they are: keep them mostly positive
        x["dt_bias"] = np.full(H, 3.0, dtype=np.float32)
    y, fs = run_gpu(ssm, dev, w, x, softplus)
    torch.cuda.synchronize()
    yr, fr = run_oracle(w, x, softplus)
    ey = norm_err(to_np(y), yr)
    es = norm_err(to_np(fs), fr)
    print(f"{case}: y {ey:.2e} state {es:.2e}", flush=True)
    assert ey <= TOL["bf16"] and es <= TOL["bf16"], (ey, es)


def test_ssd_resume_from_final_state(ssm, dev):
    """Two calls with the state carried equal one call (within the bound)."""
    w = wl.SsdWorkload("resume", 1, 640, 4, 64, 1, 128, True, seed=4600)
    x = wl.ssd_inputs(w)
    y, fs = run_gpu(ssm, dev, w, x)
    cut = 256
    def part(a, s):
        return None if a is None else np.ascontiguousarray(a[..., s])
    w1 = wl.SsdWorkload("a", 1, cut, 4, 64, 1, 128, True)
    w2 = wl.SsdWorkload("b", 1, 640 - cut, 4, 64, 1, 128, True)
    x1 = dict(x, **{k: part(x[k], slice(0, cut)) for k in ("x", "dt", "B", "C", "z")})
    x2 = dict(x, **{k: part(x[k], slice(cut, None)) for k in ("x", "dt", "B", "C", "z")})
    y1, f1 = run_gpu(ssm, dev, w1, x1)
    x2["h0"] = to_np(f1).astype(np.float32)
    y2, f2 = run_gpu(ssm, dev, w2, x2)
    torch.cuda.synchronize()
    yr, fr = run_oracle(w, x)
    assert norm_err(to_np(torch.cat([y1, y2], dim=-1)), yr) <= TOL["bf16"]
    assert norm_err(to_np(f2), fr) <= TOL["bf16"]


def test_ssd_repeatable(ssm, dev):
    w = wl.SsdWorkload("rep", 2, 300, 4, 64, 2, 64, True, seed=4700)
    x = wl.ssd_inputs(w, with_h0=True)
    a, fa = run_gpu(ssm, dev, w, x)
    b, fb = run_gpu(ssm, dev, w, x)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(fa, fb)


def test_ssd_mamba2_2p7b_full(ssm, dev):
    """The Mamba-2 2.7B layer shape at full size (batch 4, L 8192, 80 heads of
    64, N 128, one group): every head of every sequence against the oracle,
    which runs over blocks of 16 heads."""
    w = wl.SSD_WORKLOADS["mamba2_2p7b"]
    x = wl.ssd_inputs(w)
    y, fs = run_gpu(ssm, dev, w, x)
    torch.cuda.synchronize()
    ey = es = 0.0
    for h0 in range(0, w.nheads, 16):
        heads = np.arange(h0, min(w.nheads, h0 + 16))
        rows = (heads[:, None] * 64 + np.arange(64)[None, :]).reshape(-1)
        ws = wl.SsdWorkload("sub", w.batch, w.seqlen, len(heads), 64, 1, w.dstate, True)
        xs = dict(x=np.ascontiguousarray(x["x"][:, rows]), z=np.ascontiguousarray(x["z"][:, rows]),
                  dt=np.ascontiguousarray(x["dt"][:, heads]), B=x["B"], C=x["C"],
                  A=x["A"][heads], D=x["D"][heads], dt_bias=x["dt_bias"][heads], h0=None)
        yr, fr = run_oracle(ws, xs)
        ey = max(ey, norm_err(to_np(y[:, rows[0]:rows[-1] + 1]), yr))
        es = max(es, norm_err(to_np(fs[:, heads[0]:heads[-1] + 1]), fr))
        del yr
    print(f"mamba2_2p7b all {w.nheads} heads: y {ey:.2e} state {es:.2e}", flush=True)
    assert ey <= TOL["bf16"] and es <= TOL["bf16"]
