"""Pins for the oracle's backward pass: every gradient against central finite
differences of the (pinned) forward oracle, in float64, on tiny inputs."""
import numpy as np
import pytest

import oracle


def _case(seed, gate=True, bias=True, softplus=True, h0=True):
    r = np.random.default_rng(seed)
    Bt, Dm, N, L = 2, 2, 3, 6
    x = dict(
        u=r.standard_normal((Bt, Dm, L)),
        delta=r.normal(-0.5, 0.8, (Bt, Dm, L)) if softplus else r.uniform(0.05, 0.9, (Bt, Dm, L)),
        A=-r.uniform(0.2, 2.5, (Dm, N)),
        B=r.standard_normal((Bt, N, L)),
        C=r.standard_normal((Bt, N, L)),
        D=r.standard_normal(Dm),
        z=r.standard_normal((Bt, Dm, L)) if gate else None,
        delta_bias=r.normal(0, 0.3, Dm) if bias else None,
        h0=r.normal(0, 0.5, (Bt * Dm, N)) if h0 else None,
    )
    dy = r.standard_normal((Bt, Dm, L))
    dfinal = r.standard_normal((Bt * Dm, N))
    return x, dy, dfinal, softplus


def _loss(x, dy, dfinal, softplus, bbar):
    y, fs = oracle.selective_scan(x["u"], x["delta"], x["A"], x["B"], x["C"], D=x["D"], z=x["z"],
                                  delta_bias=x["delta_bias"], delta_softplus=softplus, bbar=bbar,
                                  h0=x["h0"], n_threads=1)
    return float(np.sum(dy.reshape(y.shape) * y) + np.sum(dfinal * fs))


def _fd(x, key, dy, dfinal, softplus, bbar, eps=1e-6):
    base = x[key]
    g = np.zeros_like(base)
    it = np.nditer(base, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        h = eps * max(1.0, abs(base[idx]))
        xp = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in x.items()}
        xm = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in x.items()}
        xp[key][idx] += h
        xm[key][idx] -= h
        g[idx] = (_loss(xp, dy, dfinal, softplus, bbar) - _loss(xm, dy, dfinal, softplus, bbar)) / (2 * h)
    return g


@pytest.mark.parametrize("bbar,gate,bias,softplus", [
    ("delta", True, True, True),
    ("zoh", True, True, True),
    ("delta", False, False, False),
    ("zoh", False, True, True),
])
def test_backward_matches_finite_differences(bbar, gate, bias, softplus):
    x, dy, dfinal, sp = _case(3 + gate + 2 * bias, gate=gate, bias=bias, softplus=softplus)
    g = oracle.selective_scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, D=x["D"],
                                  z=x["z"], delta_bias=x["delta_bias"], delta_softplus=sp,
                                  bbar=bbar, h0=x["h0"], dfinal=dfinal, n_threads=2)
    checks = [("u", "du"), ("delta", "ddelta"), ("A", "dA"), ("B", "dB"), ("C", "dC"),
              ("D", "dD"), ("h0", "dh0")]
    if gate:
        checks.append(("z", "dz"))
    if bias:
        checks.append(("delta_bias", "ddelta_bias"))
    for key, gk in checks:
        fd = _fd(x, key, dy, dfinal, sp, bbar)
        got = g[gk].reshape(fd.shape)
        err = np.max(np.abs(got - fd) / (1 + np.abs(fd)))
        assert err < 1e-7, (key, err)


def test_backward_channel_selection_and_zero_gradients():
    x, dy, dfinal, sp = _case(9)
    full = oracle.selective_scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, D=x["D"],
                                     z=x["z"], delta_bias=x["delta_bias"], delta_softplus=sp,
                                     h0=x["h0"], dfinal=dfinal)
    sel = [3, 1]
    part = oracle.selective_scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, D=x["D"],
                                     z=x["z"], delta_bias=x["delta_bias"], delta_softplus=sp,
                                     h0=x["h0"][sel], dfinal=dfinal[sel], channels=sel)
    for k in ("du", "ddelta", "dz", "dh0"):
        assert np.allclose(part[k], full[k][sel], rtol=1e-13, atol=1e-14)
    # zero upstream gradient gives zero everywhere
    z0 = oracle.selective_scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], np.zeros_like(dy),
                                   D=x["D"], z=x["z"], delta_bias=x["delta_bias"],
                                   delta_softplus=sp, h0=x["h0"])
    for k, v in z0.items():
        if v is not None:
            assert np.all(v == 0), k


def test_backward_float32_parameters_marshalled_like_float64():
    """A, D and delta_bias stored as float32 (as the workloads hold them) give
    the same gradients as their exact float64 copies: the float64 buffers the
    wrapper makes must stay alive through the C call."""
    r = np.random.default_rng(21)
    Bt, Dm, N, L = 1, 16, 16, 128
    u = r.standard_normal((Bt, Dm, L)).astype(np.float32)
    delta = r.standard_normal((Bt, Dm, L)).astype(np.float32)
    B = r.standard_normal((Bt, N, L)).astype(np.float32)
    C = r.standard_normal((Bt, N, L)).astype(np.float32)
    A = -np.tile(np.arange(1, N + 1, dtype=np.float32), (Dm, 1))
    D = r.standard_normal(Dm).astype(np.float32)
    bias = r.normal(-1, 0.5, Dm).astype(np.float32)
    dy = r.standard_normal((Bt, Dm, L))
    dfinal = r.standard_normal((Bt * Dm, N))
    for bbar in ("delta", "zoh"):
        g32 = oracle.selective_scan_bwd(u, delta, A, B, C, dy, D=D, delta_bias=bias,
                                        delta_softplus=True, bbar=bbar, dfinal=dfinal,
                                        n_threads=1)
        g64 = oracle.selective_scan_bwd(u, delta, A.astype(np.float64), B, C, dy,
                                        D=D.astype(np.float64),
                                        delta_bias=bias.astype(np.float64),
                                        delta_softplus=True, bbar=bbar, dfinal=dfinal,
                                        n_threads=1)
        for k, v in g64.items():
            if v is not None:
                assert np.array_equal(g32[k], v), (bbar, k)


SUMS = ("dA", "dB", "dC", "dD", "ddelta_bias")


def _nonneg_case(seed, sign=1.0):
    """Inputs for which every term of every summed gradient has the sign of
    `sign`: u, B, C >= 0, a positive A (so exp(delta A) > 0, the exact-ZOH
    coefficient and both of its derivatives are positive), no gate, zero
    initial state (so every state is >= 0) and upstream gradients of one
    sign (so every adjoint has that sign)."""
    r = np.random.default_rng(seed)
    Bt, Dm, N, L = 2, 3, 4, 7
    x = dict(u=r.uniform(0.1, 1.0, (Bt, Dm, L)), delta=r.normal(-0.5, 0.5, (Bt, Dm, L)),
             A=r.uniform(0.1, 0.6, (Dm, N)), B=r.uniform(0.1, 1.0, (Bt, N, L)),
             C=r.uniform(0.1, 1.0, (Bt, N, L)), D=r.uniform(0.1, 1.0, Dm),
             delta_bias=r.normal(0, 0.3, Dm))
    dy = sign * r.uniform(0.1, 1.0, (Bt, Dm, L))
    dfinal = sign * r.uniform(0.1, 1.0, (Bt * Dm, N))
    return x, dy, dfinal


@pytest.mark.parametrize("bbar", ["delta", "zoh"])
@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_abs_sums_equal_the_sums_when_terms_share_a_sign(bbar, sign):
    """The sums of |term| that bound the rounding of the summed gradients:
    where every term has one sign they equal the (finite-difference pinned)
    gradient itself, or its negation, so each holds exactly the terms of its
    sum, each once."""
    x, dy, dfinal = _nonneg_case(31, sign)
    g = oracle.selective_scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, D=x["D"],
                                  delta_bias=x["delta_bias"], delta_softplus=True, bbar=bbar,
                                  dfinal=dfinal, want_abs=True, n_threads=2)
    for k in SUMS:
        assert np.all(g[k] * sign > 0), k
        assert np.allclose(g[k + "_abs"], sign * g[k], rtol=1e-14, atol=0), k


@pytest.mark.parametrize("bbar", ["delta", "zoh"])
def test_abs_sums_bound_the_sums(bbar):
    """With terms of both signs (the usual case) each sum of |term| is at
    least |gradient| and, somewhere, strictly more."""
    x, dy, dfinal, sp = _case(5)
    g = oracle.selective_scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, D=x["D"],
                                  z=x["z"], delta_bias=x["delta_bias"], delta_softplus=sp,
                                  bbar=bbar, h0=x["h0"], dfinal=dfinal, want_abs=True,
                                  n_threads=1)
    # one thread each: the per-thread partial sums merge in a fixed order
    plain = oracle.selective_scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, D=x["D"],
                                      z=x["z"], delta_bias=x["delta_bias"], delta_softplus=sp,
                                      bbar=bbar, h0=x["h0"], dfinal=dfinal, n_threads=1)
    for k in SUMS:
        assert np.array_equal(g[k], plain[k]), k  # asking for them changes nothing else
        assert np.all(g[k + "_abs"] >= np.abs(g[k]) * (1 - 1e-14)), k
        assert np.any(g[k + "_abs"] > np.abs(g[k]) * (1 + 1e-6)), k
    assert "dA_abs" not in plain
