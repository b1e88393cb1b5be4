"""Seeded sweep of shapes and options against the fp64 oracle: the forward
scan under every discretization rule and the backward under both exponential
rules, over random (batch, dim, N, L) with and without gate, bias, softplus
and an initial state.  Bounds as in the other parity tests: elementwise
|gpu - oracle| <= tol (1 + |oracle|), tol 1e-4 for float32 inputs and 2e-2
for bf16 (sums over steps or channels in the backward element by element
against the sum of the absolute values of their terms, 1e-4 (1 + sum |term|))."""
import numpy as np
import pytest

import oracle
import workloads as wl
from helpers import TOL, norm_err, scan_gpu, scan_oracle, to_dev, to_np
from test_bwd_parity_gpu import _case as bwd_case

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


def _fwd_cases(n, seed):
    r = np.random.default_rng(seed)
    out = []
    for i in range(n):
        out.append(dict(
            batch=int(r.integers(1, 4)), dim=int(r.integers(1, 41)), N=int(r.integers(1, 65)),
            L=int(r.choice([1, 2, 7, 64, 255, 256, 257, 300, 511, 700])),
            dt=str(r.choice(["f32", "bf16"])), rule=str(r.choice(["delta", "zoh", "euler", "bilinear"])),
            gate=bool(r.integers(0, 2)), bias=bool(r.integers(0, 2)), h0=bool(r.integers(0, 2)),
            seed=int(9000 + i)))
    return out


FWD = _fwd_cases(24, 2026)


@pytest.mark.parametrize("c", FWD, ids=lambda c: "b{batch}_d{dim}_n{N}_l{L}_{dt}_{rule}".format(**c))
def test_forward_sweep(ssm, dev, c):
    kw = dict(delta_mean=-4.0, delta_std=0.5) if c["rule"] == "euler" else {}
    w, x = wl.custom(c["batch"], c["dim"], c["N"], c["L"], dtype=c["dt"], gate=c["gate"],
                     bias=c["bias"], seed=c["seed"], **kw)
    h0 = None
    if c["h0"]:
        h0 = np.random.default_rng(c["seed"]).normal(0.0, 0.5, (c["batch"], c["dim"], c["N"]))
        h0 = h0.astype(np.float32)
    y, fs = scan_gpu(ssm, x, dev, bbar=c["rule"], h0=to_dev(h0, dev))
    torch.cuda.synchronize()
    yr, fr = scan_oracle(oracle, x, bbar=c["rule"],
                         h0=None if h0 is None else h0.reshape(-1, c["N"]).astype(np.float64))
    ey = norm_err(to_np(y).reshape(yr.shape), yr)
    es = norm_err(to_np(fs).reshape(fr.shape), fr)
    print(f"{c}: y {ey:.2e} state {es:.2e}", flush=True)
    assert ey <= TOL[c["dt"]] and es <= TOL[c["dt"]], (ey, es)


def _bwd_cases(n, seed):
    r = np.random.default_rng(seed)
    return [dict(batch=int(r.integers(1, 3)), dim=int(r.integers(1, 33)),
                 N=int(r.choice([1, 3, 8, 16, 17, 24, 33, 64])),
                 L=int(r.choice([1, 5, 128, 129, 250, 384, 500])),
                 dt=str(r.choice(["f32", "bf16"])), rule=str(r.choice(["delta", "zoh"])),
                 gate=bool(r.integers(0, 2)), bias=bool(r.integers(0, 2)), seed=int(9500 + i))
            for i in range(n)]


BWD = _bwd_cases(14, 2027)


@pytest.mark.parametrize("c", BWD, ids=lambda c: "b{batch}_d{dim}_n{N}_l{L}_{dt}_{rule}".format(**c))
def test_backward_sweep(ssm, dev, c):
    w, x = wl.custom(c["batch"], c["dim"], c["N"], c["L"], dtype=c["dt"], gate=c["gate"],
                     bias=c["bias"], seed=c["seed"])
    bwd_case(ssm, dev, w, x, bbar=c["rule"], label=str(c))
