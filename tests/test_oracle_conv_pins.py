"""Pins for the oracle's depthwise causal convolution (+ silu), the step in
front of the scan in the Mamba block ("State-space models", section "Mamba:
selection": a depthwise causal convolution of width 4 and a silu).

- library routine: torch's conv1d in float64 on the CPU, grouped per channel,
  padded by W-1 on the left and cut to L outputs (the page's own F.conv1d
  convention, "State-space models", section "Implementation");
- closed forms: the identity tap gives silu(x + bias); a tap on the oldest
  input delays the sequence by W-1 steps (causality);
- invariants: a sequence split in two with the state carried equals one pass
  bit for bit, and L one-token steps reproduce it; bf16 inputs are widened
  exactly;
- backward: every gradient against central finite differences."""
import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")


def _silu(v):
    return v / (1.0 + np.exp(-v))


def _case(seed, batch=2, dim=3, L=11, W=4):
    r = np.random.default_rng(seed)
    return (r.standard_normal((batch, dim, L)), r.standard_normal((dim, W)),
            r.standard_normal(dim), r.standard_normal((batch, dim, W - 1)))


@pytest.mark.parametrize("W", [1, 2, 3, 4])
@pytest.mark.parametrize("silu", [True, False])
def test_conv1d_matches_torch(W, silu):
    x, w, b, s = _case(W + 10 * silu, W=W)
    out, st = oracle.conv1d(x, w, bias=b, silu=silu)
    ref = torch.nn.functional.conv1d(torch.from_numpy(x), torch.from_numpy(w)[:, None, :],
                                     torch.from_numpy(b), padding=W - 1,
                                     groups=x.shape[1])[..., :x.shape[2]].numpy()
    if silu:
        ref = _silu(ref)
    assert np.allclose(out, ref, rtol=1e-13, atol=1e-13)
    # with a given state: the same as convolving the state followed by x
    out2, _ = oracle.conv1d(x, w, bias=b, state_in=s[..., :W - 1], silu=silu)
    xs = np.concatenate([s[..., :W - 1], x], axis=-1)
    ref2 = torch.nn.functional.conv1d(torch.from_numpy(xs), torch.from_numpy(w)[:, None, :],
                                      torch.from_numpy(b), groups=x.shape[1]).numpy()
    if silu:
        ref2 = _silu(ref2)
    assert np.allclose(out2, ref2, rtol=1e-13, atol=1e-13)


def test_identity_and_delay_taps():
    x, _, b, _ = _case(3)
    W = 4
    ident = np.zeros((3, W))
    ident[:, W - 1] = 1.0
    out, _ = oracle.conv1d(x, ident, bias=b)
    assert np.allclose(out, _silu(x + b[None, :, None]), rtol=1e-14, atol=1e-15)
    delay = np.zeros((3, W))
    delay[:, 0] = 1.0
    out, _ = oracle.conv1d(x, delay, bias=None, silu=False)
    assert np.all(out[..., :W - 1] == 0.0)
    assert np.array_equal(out[..., W - 1:], x[..., :-(W - 1)])


def test_state_out_is_last_inputs():
    x, w, b, s = _case(4)
    _, st = oracle.conv1d(x, w, bias=b, state_in=s)
    assert np.array_equal(st, x[..., -3:])
    # shorter than the window: the state keeps part of state_in
    _, st2 = oracle.conv1d(x[..., :2].copy(), w, bias=b, state_in=s)
    assert np.array_equal(st2, np.concatenate([s[..., 2:], x[..., :2]], axis=-1))


def test_split_and_token_steps_reproduce_one_pass():
    x, w, b, s = _case(5, L=13)
    full, st_full = oracle.conv1d(x, w, bias=b, state_in=s)
    a, st_a = oracle.conv1d(x[..., :6].copy(), w, bias=b, state_in=s)
    c, st_c = oracle.conv1d(x[..., 6:].copy(), w, bias=b, state_in=st_a)
    assert np.array_equal(np.concatenate([a, c], axis=-1), full)
    assert np.array_equal(st_c, st_full)
    st = s
    for t in range(x.shape[2]):
        o, st = oracle.conv1d(x[..., t:t + 1].copy(), w, bias=b, state_in=st)
        assert np.array_equal(o[..., 0], full[..., t])
    assert np.array_equal(st, st_full)


def test_bf16_bits_widen_exactly():
    r = np.random.default_rng(6)
    vals = r.standard_normal((1, 2, 9)).astype(np.float32)
    bits = (vals.view(np.uint32) >> 16).astype(np.uint16)
    exact = (bits.astype(np.uint32) << 16).view(np.float32)
    w = r.standard_normal((2, 4))
    o_bits, _ = oracle.conv1d(bits, w)
    o_f32, _ = oracle.conv1d(exact, w)
    assert np.array_equal(o_bits, o_f32)


def _loss(x, w, b, s, dout, silu):
    out, _ = oracle.conv1d(x, w, bias=b, state_in=s, silu=silu)
    return float(np.sum(out * dout))


@pytest.mark.parametrize("silu,W", [(True, 4), (False, 4), (True, 2)])
def test_conv1d_backward_matches_finite_differences(silu, W):
    x, w, b, s = _case(7 + W, L=9, W=W)
    dout = np.random.default_rng(8).standard_normal(x.shape)
    g = oracle.conv1d_bwd(x, w, dout, bias=b, state_in=s, silu=silu)
    args = dict(x=x, w=w, b=b, s=s)
    for key, gk in (("x", "dx"), ("w", "dw"), ("b", "dbias"), ("s", "dstate_in")):
        base = args[key]
        fd = np.zeros_like(base)
        it = np.nditer(base, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            h = 1e-6 * max(1.0, abs(base[idx]))
            ap = {k: v.copy() for k, v in args.items()}
            am = {k: v.copy() for k, v in args.items()}
            ap[key][idx] += h
            am[key][idx] -= h
            fd[idx] = (_loss(ap["x"], ap["w"], ap["b"], ap["s"], dout, silu)
                       - _loss(am["x"], am["w"], am["b"], am["s"], dout, silu)) / (2 * h)
        err = np.max(np.abs(g[gk].reshape(fd.shape) - fd) / (1 + np.abs(fd)))
        assert err < 1e-7, (key, err)


@pytest.mark.parametrize("silu", [True, False])
def test_conv1d_abs_sums(silu):
    """The sums of |term| of dweight and dbias: equal to the gradients where
    every term is positive (x, w, bias > 0 keep silu' > 0; dout > 0), at least
    |gradient| and somewhere more with mixed signs."""
    r = np.random.default_rng(17)
    x, w = r.uniform(0.1, 1, (2, 3, 9)), r.uniform(0.1, 1, (3, 4))
    b, dout = r.uniform(0.1, 1, 3), r.uniform(0.1, 1, (2, 3, 9))
    g = oracle.conv1d_bwd(x, w, dout, bias=b, silu=silu, want_abs=True)
    assert np.all(g["dw"] > 0) and np.all(g["dbias"] > 0)
    assert np.allclose(g["dw_abs"], g["dw"], rtol=1e-14, atol=0)
    assert np.allclose(g["dbias_abs"], g["dbias"], rtol=1e-14, atol=0)
    xm, wm, bm, s = _case(23)
    dm = r.standard_normal(xm.shape)
    g = oracle.conv1d_bwd(xm, wm, dm, bias=bm, state_in=s, silu=silu, want_abs=True)
    for k in ("dw", "dbias"):
        assert np.all(g[k + "_abs"] >= np.abs(g[k]) * (1 - 1e-14))
        assert np.any(g[k + "_abs"] > np.abs(g[k]) * (1 + 1e-6))
