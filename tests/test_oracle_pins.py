"""Pins for the fp64 oracle: values the pages print, closed forms, invariants
and brute force on tiny inputs.  None of these re-types the oracle's loop; each
checks it against something else the pages or the mathematics fix.

CPU only (no GPU marker).
"""
import math

import numpy as np
import pytest

import oracle
import workloads as wl


def scalar_scan(A, B, C, delta, u, *, D=0.0, bbar="zoh", softplus=False, bias=None,
                z=None, h0=None):
    """Run the oracle on a single channel with N = len(A) states (fp32 inputs)."""
    A = np.atleast_1d(np.asarray(A, dtype=np.float32))
    N = A.size
    L = len(u)
    Bm = np.broadcast_to(np.asarray(B, dtype=np.float32).reshape(N, -1), (N, L)).copy()
    Cm = np.broadcast_to(np.asarray(C, dtype=np.float32).reshape(N, -1), (N, L)).copy()
    dl = np.broadcast_to(np.asarray(delta, dtype=np.float32), (L,)).copy()
    args = dict(D=np.array([D], np.float32), bbar=bbar, delta_softplus=softplus,
                delta_bias=None if bias is None else np.array([bias], np.float32))
    if z is not None:
        args["z"] = np.asarray(z, np.float32).reshape(1, 1, L)
    if h0 is not None:
        args["h0"] = np.asarray(h0, np.float64).reshape(1, N)
    y, fs = oracle.selective_scan(np.asarray(u, np.float32).reshape(1, 1, L), dl.reshape(1, 1, L),
                                  A.reshape(1, N), Bm.reshape(1, N, L), Cm.reshape(1, N, L), **args)
    return y[0], fs[0]


# ---------------------------------------------------------------- printed values

def test_zoh_worked_example(golden):
    g = golden("zoh_scalar_decay.txt")
    y, fs = scalar_scan(g["A"], g["B"], g["C"], g["delta"][0], g["u"])
    assert np.allclose(y, g["y"], atol=g["tol"][0], rtol=0)
    assert abs(fs[0] - g["y"][-1]) <= g["tol"][0]
    # abar and bbar read back through the recurrence: one step from state 1 with
    # u = 0 gives abar; one step from 0 with u = 1 gives bbar.
    ya, _ = scalar_scan(g["A"], g["B"], g["C"], g["delta"][0], [0.0], h0=[1.0])
    yb, _ = scalar_scan(g["A"], g["B"], g["C"], g["delta"][0], [1.0])
    assert abs(ya[0] - g["abar"][0]) <= g["tol"][0]
    assert abs(yb[0] - g["bbar"][0]) <= g["tol"][0]


def test_zoh_step_size_independence(golden):
    g = golden("zoh_step_independence.txt")
    y, _ = scalar_scan(g["A"], g["B"], g["C"], g["delta"][0], g["u"])
    assert np.allclose(y, g["y"], atol=g["tol"][0], rtol=0)
    ya, _ = scalar_scan(g["A"], g["B"], g["C"], g["delta"][0], [0.0], h0=[1.0])
    assert abs(ya[0] - g["abar"][0]) <= g["tol"][0]
    # same continuous trajectory as the step-0.5 run sampled at t = 1 and t = 2
    y_half, _ = scalar_scan(g["A"], g["B"], g["C"], 0.5, [1, 1, 0, 0])
    assert np.allclose(y, y_half[1::2], atol=1e-12, rtol=0)


def test_zoh_active_recall_answer(golden):
    g = golden("zoh_answer1.txt")
    yb, _ = scalar_scan(g["A"], g["B"], [1.0], g["delta"][0], [1.0])
    assert abs(yb[0] - g["bbar"][0]) <= g["tol"][0]
    assert abs(yb[0] - (1 - math.exp(-0.5)) / 2) < 1e-15
    ya, _ = scalar_scan(g["A"], g["B"], [1.0], g["delta"][0], [0.0], h0=[1.0])
    assert abs(ya[0] - g["abar"][0]) <= g["tol"][0]


def test_selection_example(golden):
    g = golden("selection_example.txt")
    w = g["weight"][0]
    for x, dt_page, abar_page in g["row"]:
        # Delta-times-B input rule with B = C = 1, u = 1, D = 0 and a zero state
        # reads out y = delta itself.
        y, _ = scalar_scan(g["A"], [1.0], [1.0], w * x, [1.0], bbar="delta", softplus=True)
        assert abs(y[0] - dt_page) <= g["tol"][0]
        ya, _ = scalar_scan(g["A"], [1.0], [1.0], w * x, [0.0], bbar="delta", softplus=True,
                            h0=[1.0])
        assert abs(ya[0] - abar_page) <= g["tol"][0]
        # closed form for A = -1: exp(-softplus(s)) = 1 / (1 + e^s)
        assert abs(ya[0] - 1.0 / (1.0 + math.exp(np.float32(w * x)))) < 1e-15


def test_scalar_impulse_response(golden):
    g = golden("scalar_impulse.txt")
    a, b, c = g["a"][0], g["b"][0], g["c"][0]
    # delta = 1, A = ln a makes abar = a; the delta*B rule makes bbar = b.
    L = 24
    u = np.zeros(L, np.float32)
    u[0] = 1
    y, _ = scalar_scan([np.float32(math.log(a))], [b], [c], 1.0, u, bbar="delta")
    a32 = math.exp(float(np.float32(math.log(a))))
    expect = float(np.float32(c)) * float(np.float32(b)) * a32 ** np.arange(L)
    assert np.allclose(y, expect, rtol=1e-13, atol=0)
    assert abs(-1.0 / math.log(a) - g["tau"][0]) < g["tau_tol"][0]


# ---------------------------------------------------------------- closed forms

def test_delta_b_rule_hand_derived():
    # P1's system under the delta*B input rule: h_1 = 0.5, then
    # h_t = e^{-0.5} h_{t-1} + 0.5 u_t.
    y, _ = scalar_scan([-1.0], [1.0], [1.0], 0.5, [1, 1, 0, 0], bbar="delta")
    e = math.exp(-0.5)
    expect = [0.5, 0.5 * e + 0.5, (0.5 * e + 0.5) * e, (0.5 * e + 0.5) * e * e]
    assert np.allclose(y, expect, rtol=1e-15, atol=0)
    assert np.allclose(y, [0.5, 0.80327, 0.48721, 0.29550], atol=1e-5)


def test_zoh_matches_ode_closed_form():
    """Exact ZOH with a time-varying step, piecewise-constant input and
    input matrix: the state at the end of each step equals the integral of
    the continuous ODE h' = A h + B(t) u(t)."""
    r = np.random.default_rng(7)
    N, L = 4, 40
    A = -np.exp(r.uniform(np.log(0.3), np.log(5.0), N)).astype(np.float32)
    dt = r.uniform(0.01, 1.2, L).astype(np.float32)
    u = r.standard_normal(L).astype(np.float32)
    B = r.standard_normal((N, L)).astype(np.float32)
    C = r.standard_normal((N, L)).astype(np.float32)
    y, fs = scalar_scan(A, B, C, dt, u, bbar="zoh")
    A64, dt64 = A.astype(np.float64), dt.astype(np.float64)
    T = np.cumsum(dt64)
    Tprev = T - dt64
    h_ode = np.zeros((L, N))
    for t in range(L):
        s = np.arange(t + 1)
        for n in range(N):
            a = A64[n]
            # integral of e^{a (T_t - tau)} over (T_{s-1}, T_s]
            w = (np.exp(a * (T[t] - Tprev[s])) - np.exp(a * (T[t] - T[s]))) / a
            h_ode[t, n] = np.sum(w * B[n, s] * u[s])
    y_ode = np.sum(C.T.astype(np.float64) * h_ode, axis=1)
    assert np.allclose(y, y_ode, rtol=1e-11, atol=1e-13)
    assert np.allclose(fs, h_ode[-1], rtol=1e-11, atol=1e-13)


# ---------------------------------------------------------------- brute force

def _silu(z):
    return z / (1 + math.exp(-z))


def _softplus(x):
    return math.log(1 + math.exp(x)) if x < 30 else x


@pytest.mark.parametrize("bbar", ["delta", "zoh"])
def test_bruteforce_unrolled_sum(bbar):
    """y_t = [sum_{s<=t} sum_n C_{t,n} (prod_{r=s+1..t} abar_{r,n}) bbar_{s,n} u_s
    + D u_t] * silu(z_t), with the products formed explicitly (two batches,
    three channels, N = 3, L = 7, softplus with a per-channel bias)."""
    r = np.random.default_rng(11)
    Bt, Dm, N, L = 2, 3, 3, 7
    u = r.standard_normal((Bt, Dm, L)).astype(np.float32)
    raw = r.normal(-0.5, 1.0, (Bt, Dm, L)).astype(np.float32)
    z = r.standard_normal((Bt, Dm, L)).astype(np.float32)
    A = -r.uniform(0.2, 3.0, (Dm, N)).astype(np.float32)
    Bm = r.standard_normal((Bt, N, L)).astype(np.float32)
    Cm = r.standard_normal((Bt, N, L)).astype(np.float32)
    Dv = r.standard_normal(Dm).astype(np.float32)
    bias = r.normal(0, 0.5, Dm).astype(np.float32)
    y, fs = oracle.selective_scan(u, raw, A, Bm, Cm, D=Dv, z=z, delta_bias=bias,
                                  delta_softplus=True, bbar=bbar)
    y = y.reshape(Bt, Dm, L)
    fs = fs.reshape(Bt, Dm, N)
    for b in range(Bt):
        for d in range(Dm):
            dt = [_softplus(float(raw[b, d, t]) + float(bias[d])) for t in range(L)]
            for t in range(L):
                tot = 0.0
                for s in range(t + 1):
                    for n in range(N):
                        a = float(A[d, n])
                        prod = 1.0
                        for rr in range(s + 1, t + 1):
                            prod *= math.exp(dt[rr] * a)
                        coef = dt[s] if bbar == "delta" else (math.exp(dt[s] * a) - 1) / a
                        tot += float(Cm[b, n, t]) * prod * coef * float(Bm[b, n, s]) * float(u[b, d, s])
                expect = (tot + float(Dv[d]) * float(u[b, d, t])) * _silu(float(z[b, d, t]))
                assert abs(y[b, d, t] - expect) <= 1e-12 * (1 + abs(expect))
            # final state: the same sum without C, at t = L-1
            for n in range(N):
                a = float(A[d, n])
                tot = 0.0
                for s in range(L):
                    coef = dt[s] if bbar == "delta" else (math.exp(dt[s] * a) - 1) / a
                    tot += math.exp(a * sum(dt[s + 1:])) * coef * float(Bm[b, n, s]) * float(u[b, d, s])
                assert abs(fs[b, d, n] - tot) <= 1e-12 * (1 + abs(tot))


def test_bf16_widening_exact():
    # bf16 bit patterns: 1.0, 2.0, 0.33203125, -3.0
    u = np.array([[[0x3F80]]], np.uint16)
    dl = np.array([[[0x4000]]], np.uint16)
    Bm = np.array([[[0x3EAA]]], np.uint16)
    Cm = np.array([[[0xC040]]], np.uint16)
    y, fs = oracle.selective_scan(u, dl, np.zeros((1, 1), np.float32), Bm, Cm, bbar="delta")
    assert y[0, 0] == -3.0 * 2.0 * 0.33203125
    assert fs[0, 0] == 2.0 * 0.33203125


# ---------------------------------------------------------------- LTI invariants

def _lti_case(r, N, L, D, bbar):
    A = -r.uniform(0.05, 2.0, (D, N)).astype(np.float32)
    dt = r.uniform(0.05, 0.8, D).astype(np.float32)
    Bv = r.standard_normal(N).astype(np.float32)
    Cv = r.standard_normal(N).astype(np.float32)
    Dv = r.standard_normal(D).astype(np.float32)
    u = r.standard_normal((1, D, L)).astype(np.float32)
    delta = np.repeat(dt[None, :, None], L, axis=2).astype(np.float32)
    Bm = np.repeat(Bv[None, :, None], L, axis=2)
    Cm = np.repeat(Cv[None, :, None], L, axis=2)
    y, _ = oracle.selective_scan(u, delta, A, Bm, Cm, D=Dv, bbar=bbar)
    K = oracle.lti_kernel(A, Bv, Cv, dt, L, bbar=bbar)
    return A, dt, Bv, Cv, Dv, u, y, K


@pytest.mark.parametrize("bbar", ["delta", "zoh"])
def test_recurrence_equals_causal_convolution(bbar):
    r = np.random.default_rng(3)
    D, L = 3, 300
    A, dt, Bv, Cv, Dv, u, y, K = _lti_case(r, 4, L, D, bbar)
    for d in range(D):
        yc = oracle.causal_conv(K[d], u[0, d], float(Dv[d]))
        assert np.allclose(y[d], yc, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("bbar", ["delta", "zoh"])
def test_impulse_response_is_kernel(bbar):
    r = np.random.default_rng(5)
    N, L = 5, 64
    A = -r.uniform(0.05, 2.0, (1, N)).astype(np.float32)
    dt = np.float32(0.3)
    Bv = r.standard_normal(N).astype(np.float32)
    Cv = r.standard_normal(N).astype(np.float32)
    y, _ = scalar_scan(A[0], Bv, Cv, dt, np.eye(1, L, 0, dtype=np.float32)[0], bbar=bbar)
    K = oracle.lti_kernel(A, Bv, Cv, np.array([dt]), L, bbar=bbar)
    assert np.allclose(y, K[0], rtol=1e-12, atol=1e-14)
    Kp = oracle.lti_kernel(A, Bv, Cv, np.array([dt]), L, bbar=bbar, method="powers")
    assert np.allclose(K, Kp, rtol=1e-12, atol=1e-14)


def test_shift_invariance_only_without_selection():
    r = np.random.default_rng(9)
    N, L, t0 = 4, 80, 17
    A = -r.uniform(0.05, 1.0, N).astype(np.float32)
    Bv = r.standard_normal(N).astype(np.float32)
    Cv = r.standard_normal(N).astype(np.float32)
    e0 = np.zeros(L, np.float32)
    e0[0] = 1
    et = np.zeros(L, np.float32)
    et[t0] = 1
    y0, _ = scalar_scan(A, Bv, Cv, 0.4, e0, bbar="delta")
    yt, _ = scalar_scan(A, Bv, Cv, 0.4, et, bbar="delta")
    assert np.allclose(yt[t0:], y0[:L - t0], rtol=1e-13, atol=1e-15)
    assert np.all(yt[:t0] == 0)
    # with a time-varying step the translated copy no longer holds
    dts = r.uniform(0.05, 1.0, L).astype(np.float32)
    y0v, _ = scalar_scan(A, Bv, Cv, dts, e0, bbar="delta")
    ytv, _ = scalar_scan(A, Bv, Cv, dts, et, bbar="delta")
    assert not np.allclose(ytv[t0:], y0v[:L - t0], rtol=1e-3, atol=1e-6)


# ---------------------------------------------------------------- scan structure

def combine(p, q):
    """(a1, b1) then (a2, b2) is the single step (a1 a2, a2 b1 + b2)."""
    return (p[0] * q[0], q[0] * p[1] + q[1])


def test_combine_is_associative_with_identity():
    r = np.random.default_rng(1)
    for _ in range(200):
        p, q, s = [(r.uniform(0, 1), r.standard_normal()) for _ in range(3)]
        lhs = combine(combine(p, q), s)
        rhs = combine(p, combine(q, s))
        assert abs(lhs[0] - rhs[0]) <= 1e-15 and abs(lhs[1] - rhs[1]) <= 1e-14
        assert combine((1.0, 0.0), p) == p and combine(p, (1.0, 0.0)) == p


def test_chunk_aggregates_compose_to_full_scan():
    """Per-chunk aggregates (prod abar, state from zero), combined in order
    with the operator, give the full scan's final state: the decomposition a
    parallel scan relies on."""
    w, x = wl.custom(1, 2, 4, 97, dtype="f32", gate=False, seed=21)
    kw = dict(D=x["D"], delta_bias=x["delta_bias"], delta_softplus=True)
    _, fs_full = oracle.selective_scan(x["u"], x["delta"], x["A"], x["B"], x["C"], **kw)
    cuts = [0, 13, 40, 41, 97]
    agg = [(np.ones((2, 4)), np.zeros((2, 4)))]
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        sl = slice(lo, hi)
        _, h_loc = oracle.selective_scan(x["u"][..., sl], x["delta"][..., sl], x["A"],
                                         x["B"][..., sl], x["C"][..., sl], **kw)
        raw = x["delta"][0, :, sl].astype(np.float64) + x["delta_bias"][:, None]
        dsum = np.sum(np.logaddexp(0, raw), axis=1)
        a_prod = np.exp(dsum[:, None] * x["A"].astype(np.float64))
        agg.append(combine(agg[-1], (a_prod, h_loc)))
    assert np.allclose(agg[-1][1], fs_full, rtol=1e-11, atol=1e-13)


def test_chunked_resume_and_decode_equal_full_scan():
    w, x = wl.custom(2, 3, 4, 50, dtype="bf16", gate=True, seed=5)
    kw = dict(D=x["D"], delta_bias=x["delta_bias"], delta_softplus=True)
    y, fs = oracle.selective_scan(x["u"], x["delta"], x["A"], x["B"], x["C"], z=x["z"], **kw)
    y1, f1 = oracle.selective_scan(x["u"][..., :23], x["delta"][..., :23], x["A"],
                                   x["B"][..., :23], x["C"][..., :23], z=x["z"][..., :23], **kw)
    y2, f2 = oracle.selective_scan(x["u"][..., 23:], x["delta"][..., 23:], x["A"],
                                   x["B"][..., 23:], x["C"][..., 23:], z=x["z"][..., 23:],
                                   h0=f1, **kw)
    assert np.array_equal(np.concatenate([y1, y2], axis=1), y)
    assert np.array_equal(f2, fs)
    state = np.zeros((6, 4))
    for t in range(50):
        yt = oracle.state_update(state, x["u"][..., t], x["delta"][..., t], x["A"],
                                 x["B"][..., t], x["C"][..., t], z=x["z"][..., t], **kw)
        assert np.array_equal(yt, y[:, t])
    assert np.array_equal(state, fs)


def test_channel_selection_matches_full_run():
    w, x = wl.custom(2, 5, 4, 33, dtype="bf16", gate=True, seed=8)
    kw = dict(D=x["D"], z=x["z"], delta_bias=x["delta_bias"], delta_softplus=True)
    y, fs = oracle.selective_scan(x["u"], x["delta"], x["A"], x["B"], x["C"], **kw)
    sel = [7, 0, 9, 3]
    ys, fss = oracle.selective_scan(x["u"], x["delta"], x["A"], x["B"], x["C"],
                                    channels=sel, **kw)
    assert np.array_equal(ys, y[sel]) and np.array_equal(fss, fs[sel])


# ---------------------------------------------------------------- limits and wiring

def test_selection_limits():
    # tiny step (softplus(-30) ~ 9e-14): the state is frozen, y = C.h0 + D u
    N, L = 3, 10
    A = np.array([-1.0, -2.0, -4.0], np.float32)
    Bm = np.ones((N, L), np.float32)
    Cm = np.tile(np.array([[0.5], [-1.0], [2.0]], np.float32), (1, L))
    h0 = np.array([1.0, 2.0, -3.0])
    u = np.linspace(-1, 1, L).astype(np.float32)
    y, fs = scalar_scan(A, Bm, Cm, -30.0, u, D=0.7, softplus=True, h0=h0, bbar="zoh")
    # the drift is bounded by |A| * delta * L * |h| ~ 1e-11
    assert np.allclose(fs, h0, rtol=0, atol=5e-11)
    assert np.allclose(y, 0.5 * 1 - 1.0 * 2 + 2.0 * -3 + np.float32(0.7) * u, atol=5e-11)
    # huge step under exact ZOH: the state is replaced by -B u / A
    y, fs = scalar_scan(A, Bm, Cm, 60.0, np.full(L, 0.25, np.float32), bbar="zoh", h0=h0)
    assert np.allclose(fs, -0.25 / A.astype(np.float64), rtol=1e-12)


def test_skip_and_gate_wiring():
    r = np.random.default_rng(2)
    N, L = 2, 9
    u = r.standard_normal(L).astype(np.float32)
    z = r.standard_normal(L).astype(np.float32)
    A = np.array([-1.0, -0.5], np.float32)
    Bm = r.standard_normal((N, L)).astype(np.float32)
    # C = 0: only the gated skip remains
    y, _ = scalar_scan(A, Bm, np.zeros((N, L)), 0.3, u, D=1.5, z=z)
    expect = [1.5 * float(u[t]) * _silu(float(z[t])) for t in range(L)]
    assert np.allclose(y, expect, rtol=1e-14, atol=0)
    # z = 0 closes the gate; u = 0 with a zero state gives zero
    y, _ = scalar_scan(A, Bm, np.ones((N, L)), 0.3, u, D=1.5, z=np.zeros(L))
    assert np.all(y == 0)
    y, _ = scalar_scan(A, Bm, np.ones((N, L)), 0.3, np.zeros(L), D=1.5)
    assert np.all(y == 0)
    # softplus(0) = ln 2 and silu(1) = 1 / (1 + e^-1)
    y, _ = scalar_scan([-1.0], [1.0], [1.0], 0.0, [1.0], bbar="delta", softplus=True)
    assert abs(y[0] - math.log(2)) < 1e-15
    y, _ = scalar_scan([-1.0], [1.0], [0.0], 0.1, [1.0], D=1.0, z=[1.0])
    assert abs(y[0] - 1 / (1 + math.exp(-1))) < 1e-15


# ---------------------------------------------------------------- generators

def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.0, 0.33203125, 3.0e38], np.float32)
    bits = wl.to_bf16_bits(x)
    assert list(bits) == [0x3F80, 0x3F80, 0x3F82, 0xC000, 0x3EAA, 0x7F62]
    assert np.array_equal(wl.bf16_bits_to_f32(bits)[:5], np.array(
        [1.0, 1.0, 1.015625, -2.0, 0.33203125], np.float32))


def test_generators_are_seeded_and_row_addressable():
    w, x1 = wl.custom(2, 3, 4, 40, seed=99)
    _, x2 = wl.custom(2, 3, 4, 40, seed=99)
    for k in ("u", "delta", "z", "B", "C", "A", "D", "delta_bias"):
        assert np.array_equal(x1[k], x2[k])
    # a stream block can be regenerated alone (here all six rows share block 0)
    assert wl.rows_per_stream(40) >= 6
    blk = wl.to_bf16_bits(wl.rng(99, wl.T_U, 0).standard_normal(6 * 40, dtype=np.float32))
    assert np.array_equal(blk.reshape(6, 40), x1["u"].reshape(6, 40))
    A, D, bias = wl.params(wl.WORKLOADS["mamba130m"])
    assert np.array_equal(A[17], -np.arange(1, 17, dtype=np.float32))
    dt0 = np.log1p(np.exp(bias.astype(np.float64)))
    assert dt0.min() >= 1e-3 * (1 - 1e-6) and dt0.max() <= 1e-1 * (1 + 1e-6)
