"""Pins for the oracle's Mamba-2 scan (a scalar A per head; "State-space
models", section "The parallel scan"; "Structured State Space Models and
Mamba ...", section "State Space Duality and Mamba-2").

- special case of the pinned diagonal scan: every head channel is a channel
  of the diagonal scan with A[d, n] = A_h for all n, the head's step and its
  group's B and C;
- the masked-attention form the pages print, Y = (L o (C B^T)) (dt x) with
  the 1-semiseparable decay L[t, s] = exp(A sum_{s<r<=t} dt_r) for s <= t,
  computed with numpy matmuls;
- brute force for the initial-state term: y_t gains C_t . (prod_{r<=t} a_r) h0;
- a sequence split in two with the state carried equals one pass bit for bit."""
import numpy as np
import pytest

import oracle


def _case(seed, batch=2, H=4, P=3, G=2, N=5, L=17, h0=False):
    r = np.random.default_rng(seed)
    x = r.standard_normal((batch, H * P, L))
    dt = r.normal(-1.0, 0.7, (batch, H, L))
    A = -r.uniform(0.3, 4.0, H)
    B = r.standard_normal((batch, G * N, L))
    C = r.standard_normal((batch, G * N, L))
    D = r.standard_normal(H)
    z = r.standard_normal((batch, H * P, L))
    bias = r.normal(0.0, 0.5, H)
    s0 = r.normal(0.0, 0.5, (batch, H, P, N)) if h0 else None
    return dict(x=x, dt=dt, A=A, B=B, C=C, D=D, z=z, dt_bias=bias, h0=s0, H=H, G=G, P=P, N=N)


@pytest.mark.parametrize("gate,h0,softplus", [(True, True, True), (False, False, True),
                                              (True, False, False)])
def test_ssd_is_the_diagonal_scan_with_a_scalar_a_per_head(gate, h0, softplus):
    c = _case(1 + gate + 2 * h0, h0=h0)
    H, G, P, N = c["H"], c["G"], c["P"], c["N"]
    dt = c["dt"] if softplus else np.abs(c["dt"]) + 0.05
    y, fs = oracle.ssd(c["x"], dt, c["A"], c["B"], c["C"], H, G, D=c["D"],
                       z=c["z"] if gate else None, dt_bias=c["dt_bias"], dt_softplus=softplus,
                       h0=c["h0"])
    batch, _, L = c["x"].shape
    hpg = H // G
    for g in range(G):
        heads = range(g * hpg, (g + 1) * hpg)
        rows = [h * P + p for h in heads for p in range(P)]
        u = c["x"][:, rows, :]
        delta = np.repeat(dt[:, g * hpg:(g + 1) * hpg, :], P, axis=1)
        A1 = np.repeat(np.repeat(c["A"][g * hpg:(g + 1) * hpg], P)[:, None], N, axis=1)
        D1 = np.repeat(c["D"][g * hpg:(g + 1) * hpg], P)
        b1 = np.repeat(c["dt_bias"][g * hpg:(g + 1) * hpg], P)
        Bg = c["B"][:, g * N:(g + 1) * N, :].copy()
        Cg = c["C"][:, g * N:(g + 1) * N, :].copy()
        h01 = None if c["h0"] is None else c["h0"][:, g * hpg:(g + 1) * hpg].reshape(-1, N)
        yr, fr = oracle.selective_scan(np.ascontiguousarray(u), np.ascontiguousarray(delta), A1,
                                       Bg, Cg, D=D1, z=np.ascontiguousarray(c["z"][:, rows, :])
                                       if gate else None, delta_bias=b1,
                                       delta_softplus=softplus, bbar="delta", h0=h01)
        assert np.allclose(y[:, rows, :].reshape(yr.shape), yr, rtol=1e-12, atol=1e-12)
        assert np.allclose(fs[:, g * hpg:(g + 1) * hpg].reshape(fr.shape), fr, rtol=1e-12,
                           atol=1e-12)


def _softplus(v):
    return np.maximum(v, 0) + np.log1p(np.exp(-np.abs(v)))


def test_ssd_equals_masked_attention_form():
    c = _case(7, batch=1, H=2, P=4, G=1, N=6, L=23, h0=True)
    H, P, N = c["H"], c["P"], c["N"]
    y, _ = oracle.ssd(c["x"], c["dt"], c["A"], c["B"], c["C"], H, 1, dt_bias=c["dt_bias"],
                      h0=c["h0"])
    L = c["x"].shape[2]
    Cm = c["C"][0].T  # [L, N]
    Bm = c["B"][0].T
    for h in range(H):
        dt = _softplus(c["dt"][0, h] + c["dt_bias"][h])
        cum = np.cumsum(dt * c["A"][h])
        Ldec = np.tril(np.exp(cum[:, None] - cum[None, :]))   # L[t, s], s <= t
        M = Ldec * (Cm @ Bm.T) * dt[None, :]
        X = c["x"][0, h * P:(h + 1) * P, :].T                  # [L, P]
        Y = M @ X
        # initial state, brute force: C_t . (prod_{r<=t} a_r) h0
        Y += np.exp(cum)[:, None] * (Cm @ c["h0"][0, h].T)
        assert np.allclose(y[0, h * P:(h + 1) * P, :].T, Y, rtol=1e-11, atol=1e-11)


def test_ssd_split_equals_one_pass():
    c = _case(9, L=30, h0=True)
    kw = dict(D=c["D"], z=c["z"], dt_bias=c["dt_bias"])
    y, fs = oracle.ssd(c["x"], c["dt"], c["A"], c["B"], c["C"], c["H"], c["G"], h0=c["h0"], **kw)
    cut = 13
    part = lambda a, s: np.ascontiguousarray(a[..., s])  # noqa: E731
    y1, f1 = oracle.ssd(part(c["x"], slice(0, cut)), part(c["dt"], slice(0, cut)), c["A"],
                        part(c["B"], slice(0, cut)), part(c["C"], slice(0, cut)), c["H"], c["G"],
                        h0=c["h0"], D=c["D"], z=part(c["z"], slice(0, cut)), dt_bias=c["dt_bias"])
    y2, f2 = oracle.ssd(part(c["x"], slice(cut, None)), part(c["dt"], slice(cut, None)), c["A"],
                        part(c["B"], slice(cut, None)), part(c["C"], slice(cut, None)), c["H"],
                        c["G"], h0=f1, D=c["D"], z=part(c["z"], slice(cut, None)),
                        dt_bias=c["dt_bias"])
    assert np.array_equal(np.concatenate([y1, y2], axis=-1), y)
    assert np.array_equal(f2, fs)


def test_ssd_bf16_bits_widen_exactly():
    c = _case(11, batch=1, H=2, P=2, G=1, N=3, L=9)
    def bits(a):
        return (a.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    def back(b):
        return (b.astype(np.uint32) << 16).view(np.float32)
    xb, dtb, Bb, Cb = bits(c["x"]), bits(c["dt"]), bits(c["B"]), bits(c["C"])
    y1, _ = oracle.ssd(xb, dtb, c["A"], Bb, Cb, 2, 1)
    y2, _ = oracle.ssd(back(xb), back(dtb), c["A"], back(Bb), back(Cb), 2, 1)
    assert np.array_equal(y1, y2)
