"""The autograd functions of the binding against the fp64 oracle's
gradients: selective_scan_fn (forward with checkpoints, backward through
ssm_selective_scan_bwd) for the loss sum(dy y) + sum(dfinal final_state),
and causal_conv1d_fn (backward through ssm_causal_conv1d_bwd) for
sum(dout out), with the bounds of the backward parity tests."""
import numpy as np
import pytest

import oracle
import workloads as wl
from helpers import TOL, TOL_SUM, norm_err, sum_err, to_dev, to_np
from test_bwd_parity_gpu import compare, run_oracle

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


@pytest.mark.parametrize("dt,bbar,N", [("f32", "delta", 16), ("bf16", "delta", 16),
                                        ("f32", "zoh", 24), ("bf16", "zoh", 8)])
def test_selective_scan_fn_gradients(ssm, dev, dt, bbar, N):
    w, x = wl.custom(2, 20, N, 300, dtype=dt, gate=True, bias=True, seed=6100 + N)
    g = wl.grad_inputs(w)
    h0 = wl.decode_state(w)
    leaf = {k: to_dev(x[k], dev).requires_grad_() for k in ("u", "delta", "A", "B", "C", "D", "z",
                                                         "delta_bias")}
    h0d = to_dev(h0, dev).requires_grad_()
    y, fs = ssm.selective_scan_fn(leaf["u"], leaf["delta"], leaf["A"], leaf["B"], leaf["C"],
                                  D=leaf["D"], z=leaf["z"], delta_bias=leaf["delta_bias"],
                                  delta_softplus=True, h0=h0d, bbar=bbar)
    dy, dfinal = to_dev(g["dy"], dev), to_dev(g["dfinal"], dev)
    loss = (y.float() * dy.float()).sum() + (fs * dfinal).sum()
    loss.backward()
    torch.cuda.synchronize()
    got = dict(du=leaf["u"].grad, ddelta=leaf["delta"].grad, dz=leaf["z"].grad, dh0=h0d.grad,
               dA=leaf["A"].grad, dB=leaf["B"].grad, dC=leaf["C"].grad, dD=leaf["D"].grad,
               ddelta_bias=leaf["delta_bias"].grad)
    ref = run_oracle(x, g, bbar, h0, g["dfinal"])
    compare(w, got, ref, f"selective_scan_fn {dt} {bbar} N {N}")
    # and the forward values are the plain forward's
    y0, f0 = ssm.ssm_selective_scan_fwd(*(leaf[k].detach() for k in ("u", "delta", "A", "B", "C")),
                                        D=leaf["D"].detach(), z=leaf["z"].detach(),
                                        delta_bias=leaf["delta_bias"].detach(),
                                        delta_softplus=True, h0=h0d.detach(), bbar=bbar)
    assert torch.equal(y0, y.detach()) and torch.equal(f0, fs.detach())


def test_selective_scan_fn_unsupported_rule_raises_in_backward(ssm, dev):
    w, x = wl.custom(1, 8, 4, 64, dtype="f32", seed=6200)
    u = to_dev(x["u"], dev).requires_grad_()
    y, _ = ssm.selective_scan_fn(u, to_dev(x["delta"], dev), to_dev(x["A"], dev),
                                 to_dev(x["B"], dev), to_dev(x["C"], dev), delta_softplus=True,
                                 bbar="bilinear")
    with pytest.raises(ssm.SelscanError, match="SSM_E_UNSUPPORTED"):
        y.sum().backward()


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_causal_conv1d_fn_gradients(ssm, dev, dt):
    w = wl.Workload("conv", 0, 2, 24, 16, 300, dt, False, 0.0, 1.0, False, "s4d_real")
    c = wl.conv_inputs(w, width=4, seed=6300)
    x = to_dev(c["x"], dev).requires_grad_()
    wt = to_dev(c["weight"], dev).requires_grad_()
    b = to_dev(c["bias"], dev).requires_grad_()
    st = to_dev(c["state_in"], dev).requires_grad_()
    out = ssm.causal_conv1d_fn(x, wt, b, st, silu=True)
    dout = to_dev(c["dout"], dev)
    (out.float() * dout.float()).sum().backward()
    torch.cuda.synchronize()
    f64 = (lambda a: wl.bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16
           else a.astype(np.float64))
    ref = oracle.conv1d_bwd(c["x"], c["weight"], f64(c["dout"]), bias=c["bias"],
                            state_in=c["state_in"], silu=True, want_abs=True)
    tol = TOL[dt]
    assert norm_err(to_np(x.grad), ref["dx"]) <= tol
    assert norm_err(to_np(st.grad), ref["dstate_in"]) <= tol
    assert sum_err(to_np(wt.grad), ref["dw"], ref["dw_abs"]) <= TOL_SUM
    assert sum_err(to_np(b.grad), ref["dbias"], ref["dbias_abs"]) <= TOL_SUM
