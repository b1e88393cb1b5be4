"""Parity of the backward pass (through the C ABI) against the fp64 oracle's
adjoint recurrence on the same seeded inputs and upstream gradients.

Bounds: per-step gradients (du, ddelta, dz) and dh0 elementwise,
|gpu - oracle| <= tol * (1 + |oracle|), as for y.  Gradients that are sums
over many steps or channels (dA, dB, dC, dD, ddelta_bias) are accumulated in
float32 in an order that depends on scheduling; each element is bounded by
the sum of the absolute values of its own terms, which the oracle returns:
|gpu - oracle| <= 1e-4 * (1 + sum |term|) for both io dtypes, plus 2^-8 |oracle|
for dB and dC when they are stored in bf16 (their final rounding).
tol = 1e-4 for float32 inputs, 2e-2 for bf16 inputs."""
import numpy as np
import pytest

import oracle
import workloads as wl
from helpers import Q_OUT, TOL, TOL_SUM, norm_err, sum_err, to_dev, to_np

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

PER_STEP = ("du", "ddelta", "dz", "dh0")
REDUCED = ("dA", "dB", "dC", "dD", "ddelta_bias")


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


def _as_f64(a):
    return wl.bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def run_gpu(ssm, dev, x, g, bbar, h0, dfinal):
    return ssm.ssm_selective_scan_bwd(
        to_dev(x["u"], dev), to_dev(x["delta"], dev), to_dev(x["A"], dev), to_dev(x["B"], dev),
        to_dev(x["C"], dev), to_dev(g["dy"], dev), D=to_dev(x["D"], dev),
        z=to_dev(x.get("z"), dev), delta_bias=to_dev(x.get("delta_bias"), dev),
        delta_softplus=x.get("delta_softplus", True), h0=to_dev(h0, dev),
        dfinal_state=to_dev(dfinal, dev), bbar=bbar, want_dh0=True)


def run_oracle(x, g, bbar, h0, dfinal, channels=None):
    return oracle.selective_scan_bwd(
        x["u"], x["delta"], x["A"], x["B"], x["C"], _as_f64(g["dy"]), D=x["D"], z=x.get("z"),
        delta_bias=x.get("delta_bias"), delta_softplus=x.get("delta_softplus", True), bbar=bbar,
        h0=h0, dfinal=dfinal, channels=channels, want_abs=True)


def compare(w, got, ref, label, channels=None, reduced=REDUCED):
    """Largest error of every gradient; asserts the bounds."""
    tol = TOL[w.dtype]
    errs = {}
    rows = None if channels is None else torch.as_tensor(channels, device=got["du"].device)
    for k in PER_STEP:
        if ref.get(k) is None or got.get(k) is None:
            continue
        gk = got[k].reshape(w.batch * w.dim, -1)
        if rows is not None:
            gk = gk[rows]
        r = ref[k].reshape(gk.shape[0], -1)
        # row blocks: the full-size tensors are large
        errs[k] = max(norm_err(to_np(gk[i:i + 2048]), r[i:i + 2048])
                      for i in range(0, gk.shape[0], 2048))
    for k in reduced:
        if ref.get(k) is None or got.get(k) is None:
            continue
        # dB and dC are stored in the io dtype, the other sums in float32
        q = Q_OUT[w.dtype] if k in ("dB", "dC") else 0.0
        errs[k] = sum_err(to_np(got[k]).reshape(ref[k].shape), ref[k], ref[k + "_abs"], q)
    print(f"{label}: " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if not v <= (TOL_SUM if k in reduced else tol)}
    assert not bad, bad
    return errs


def _case(ssm, dev, w, x, bbar="delta", with_h0=True, with_dfinal=True, label=""):
    g = wl.grad_inputs(w)
    h0 = wl.decode_state(w) if with_h0 else None
    dfinal = g["dfinal"] if with_dfinal else None
    got = run_gpu(ssm, dev, x, g, bbar, h0, dfinal)
    torch.cuda.synchronize()
    ref = run_oracle(x, g, bbar, h0, dfinal)
    return compare(w, got, ref, label or w.name)


def test_bwd_tiny_fp32(ssm, dev):
    w = wl.WORKLOADS["tiny_fp32"]
    _case(ssm, dev, w, wl.scan_inputs(w))


# (batch, dim, dstate, L, dtype, gate, bias, bbar): several chunks of 128
# steps with ragged tails, dim not a multiple of 16, N below 16, odd L (the
# unvectorised loads), both discretization rules
BWD_CASES = [
    (2, 40, 16, 300, "f32", True, True, "delta"),
    (1, 24, 16, 333, "f32", True, False, "zoh"),
    (2, 17, 5, 129, "f32", False, True, "delta"),
    (1, 16, 16, 128, "f32", False, False, "zoh"),
    (1, 8, 1, 77, "f32", True, True, "delta"),
    (2, 48, 16, 1000, "bf16", True, True, "delta"),
    (1, 33, 16, 517, "bf16", True, True, "zoh"),
    (3, 16, 8, 260, "bf16", False, False, "delta"),
    # more than 16 states: tiles of 16, one launch each, the last ragged
    (2, 40, 32, 300, "f32", True, True, "delta"),
    (1, 24, 40, 333, "f32", True, False, "zoh"),
    (2, 20, 64, 260, "bf16", True, True, "delta"),
    (1, 17, 48, 129, "bf16", False, True, "zoh"),
    (1, 8, 17, 77, "f32", True, True, "delta"),
    # 8192 channels and more with 16 states and bf16 rows: the time-pipelined
    # checkpoint and carry passes (a ragged last chunk of 64 steps and block of
    # 128, odd L: the element-wise loads, dim not a multiple of 16)
    (1, 8200, 16, 77, "bf16", True, True, "delta"),
    (2, 4104, 16, 200, "bf16", False, False, "zoh"),
    (1, 8192, 16, 384, "bf16", True, False, "delta"),
    (3, 2740, 16, 203, "bf16", True, True, "zoh"),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "x".join(map(str, c)))
def test_bwd_shapes(ssm, dev, case):
    batch, dim, N, L, dt, gate, bias, bbar = case
    w, x = wl.custom(batch, dim, N, L, dtype=dt, gate=gate, bias=bias, seed=5100 + L)
    _case(ssm, dev, w, x, bbar=bbar, label=f"{case}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_bwd_exact_zoh_degenerate_a(ssm, dev, dt):
    """The exact-ZOH gradients where the coefficient and its derivative in A
    are delicate: A = 0, |delta A| far below 1/32 and around it."""
    w, x = wl.custom(1, 24, 16, 333, dtype=dt, seed=5900)
    A = x["A"].copy()
    A[:, 0], A[:, 1], A[:, 2], A[:, 3], A[:, 4] = 0.0, -1e-4, -0.3, -0.6, -1e-6
    x["A"] = A
    _case(ssm, dev, w, x, bbar="zoh", label=f"zoh, degenerate A, {dt}")


def test_bwd_no_h0_no_dfinal(ssm, dev):
    w, x = wl.custom(2, 32, 16, 400, dtype="f32", seed=5200)
    _case(ssm, dev, w, x, with_h0=False, with_dfinal=False, label="no h0 / dfinal")


@pytest.mark.parametrize("shape", [(1, 32, 16, 300, "f32"), (1, 8200, 16, 200, "bf16")],
                         ids=["f32", "bf16_pipelined"])
def test_bwd_no_softplus(ssm, dev, shape):
    # raw steps used as they are: keep them positive (the bf16 shape takes the
    # time-pipelined checkpoint and carry passes)
    b, d, n, L, dt = shape
    w, x = wl.custom(b, d, n, L, dtype=dt, bias=False, delta_mean=0.3, delta_std=0.05,
                     seed=5300)
    x["delta_softplus"] = False
    _case(ssm, dev, w, x, label=f"no softplus {dt}")


def test_bwd_optional_outputs_absent(ssm, dev):
    """dD, ddelta_bias and dh0 may be left out; the rest is unchanged."""
    w, x = wl.custom(1, 32, 16, 256, dtype="f32", seed=5400)
    g = wl.grad_inputs(w)
    full = run_gpu(ssm, dev, x, g, "delta", None, g["dfinal"])
    part = ssm.ssm_selective_scan_bwd(
        to_dev(x["u"], dev), to_dev(x["delta"], dev), to_dev(x["A"], dev), to_dev(x["B"], dev),
        to_dev(x["C"], dev), to_dev(g["dy"], dev), z=to_dev(x["z"], dev),
        delta_bias=None, delta_softplus=True, dfinal_state=to_dev(g["dfinal"], dev))
    torch.cuda.synchronize()
    assert part["dD"] is None and part["ddelta_bias"] is None and part["dh0"] is None
    ref = run_oracle(dict(x, D=None, delta_bias=None), g, "delta", None, g["dfinal"])
    compare(w, part, ref, "no D / bias")
    assert full["dD"] is not None


def test_bwd_workspace_reuse(ssm, dev):
    """A caller-owned workspace reused by two calls of different sizes; the
    contents left by the first call do not leak into the second."""
    w1, x1 = wl.custom(2, 48, 16, 700, dtype="bf16", seed=5500)
    w2, x2 = wl.custom(1, 32, 16, 300, dtype="bf16", seed=5501)
    need = ssm.ssm_selective_scan_bwd_workspace_size(2, 48, 16, 700)
    assert need >= ssm.ssm_selective_scan_bwd_workspace_size(1, 32, 16, 300)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    for w, x in ((w1, x1), (w2, x2)):
        g = wl.grad_inputs(w)
        got = ssm.ssm_selective_scan_bwd(
            to_dev(x["u"], dev), to_dev(x["delta"], dev), to_dev(x["A"], dev),
            to_dev(x["B"], dev), to_dev(x["C"], dev), to_dev(g["dy"], dev),
            D=to_dev(x["D"], dev), z=to_dev(x["z"], dev),
            delta_bias=to_dev(x["delta_bias"], dev), delta_softplus=True,
            dfinal_state=to_dev(g["dfinal"], dev), workspace=ws, want_dh0=True)
        torch.cuda.synchronize()
        ref = run_oracle(x, g, "delta", None, g["dfinal"])
        compare(w, got, ref, f"workspace reuse {w.batch}x{w.dim}x{w.seqlen}")


def test_bwd_rejects_large_dstate(ssm, dev):
    w, x = wl.custom(1, 16, 65, 64, dtype="f32", seed=5600)
    g = wl.grad_inputs(w)
    with pytest.raises(ssm.SelscanError, match="SSM_E_UNSUPPORTED"):
        run_gpu(ssm, dev, x, g, "delta", None, None)


def test_bwd_mamba130m_full(ssm, dev):
    """The full mamba130m shape: every gradient, every channel."""
    w = wl.WORKLOADS["mamba130m"]
    x = wl.scan_inputs(w)
    g = wl.grad_inputs(w)
    got = run_gpu(ssm, dev, x, g, "delta", None, None)
    torch.cuda.synchronize()
    ref = run_oracle(x, g, "delta", None, None)
    compare(w, got, ref, w.name)


def test_bwd_mamba2p8b_full(ssm, dev):
    """The mamba2p8b shape at full size: every gradient of every channel,
    including dB and dC, the sums over all 5120 channels of a sequence."""
    w = wl.WORKLOADS["mamba2p8b"]
    x = wl.scan_inputs(w)
    g = wl.grad_inputs(w)
    got = run_gpu(ssm, dev, x, g, "delta", None, g["dfinal"])
    torch.cuda.synchronize()
    print("mamba2p8b backward: GPU done, running the oracle", flush=True)
    ref = run_oracle(x, g, "delta", None, g["dfinal"])
    compare(w, got, ref, w.name + " full")


# (batch, dim, dstate, L, dtype, gate, bias, bbar): the three lane layouts of
# the forward (16384 channels and more: 16 lanes per channel; fewer: 32 or 64)
CKPT_CASES = [
    (2, 40, 16, 300, "bf16", True, True, "delta"),
    (1, 24, 16, 333, "f32", True, False, "zoh"),
    (2, 8192, 16, 256, "bf16", True, True, "delta"),
    (1, 8192, 8, 640, "f32", False, True, "zoh"),
    (1, 24, 48, 300, "f32", True, True, "delta"),
]


@pytest.mark.parametrize("case", CKPT_CASES, ids=lambda c: "x".join(map(str, c)))
def test_bwd_with_forward_checkpoints(ssm, dev, case):
    """A forward that writes checkpoints leaves y and the final state bit for
    bit as they are without; its checkpoints are the oracle's states at every
    128-step block start; the backward that takes them meets the bounds."""
    batch, dim, N, L, dt, gate, bias, bbar = case
    w, x = wl.custom(batch, dim, N, L, dtype=dt, gate=gate, bias=bias, seed=5800 + L)
    g = wl.grad_inputs(w)
    h0 = wl.decode_state(w)
    t = {k: to_dev(x.get(k), dev) for k in ("u", "delta", "A", "B", "C", "D", "z", "delta_bias")}
    h0d = to_dev(h0, dev)
    kw = dict(D=t["D"], z=t["z"], delta_bias=t["delta_bias"], delta_softplus=True, h0=h0d,
              bbar=bbar)
    ck = torch.full(ssm.ssm_checkpoint_shape(batch, dim, N, L), float("nan"),
                    dtype=torch.float32, device=dev)
    y0, f0 = ssm.ssm_selective_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], **kw)
    y1, f1 = ssm.ssm_selective_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], **kw,
                                        checkpoints=ck)
    got = ssm.ssm_selective_scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"],
                                     to_dev(g["dy"], dev), D=t["D"], z=t["z"],
                                     delta_bias=t["delta_bias"], delta_softplus=True, h0=h0d,
                                     dfinal_state=to_dev(g["dfinal"], dev), bbar=bbar,
                                     want_dh0=True, checkpoints=ck)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(f0, f1)
    # the checkpoints: h0, then the oracle's state after every whole block
    cks = to_np(ck)
    assert np.array_equal(cks[:, :, 0, :], h0)
    rows = np.random.default_rng(L).choice(batch * dim, min(batch * dim, 48), replace=False)
    for blk in range(1, cks.shape[2]):
        cut = 128 * blk
        part = {k: np.ascontiguousarray(x[k][..., :cut]) for k in ("u", "delta", "B", "C")}
        _, fr = oracle.selective_scan(part["u"], part["delta"], x["A"], part["B"], part["C"],
                                      D=x["D"], delta_bias=x.get("delta_bias"),
                                      delta_softplus=True, bbar=bbar,
                                      h0=h0.reshape(batch * dim, N)[rows], want_y=False,
                                      channels=rows)
        err = norm_err(cks[:, :, blk, :].reshape(batch * dim, N)[rows], fr)
        assert err <= TOL[dt], (blk, err)
    ref = run_oracle(x, g, bbar, h0, g["dfinal"])
    compare(w, got, ref, f"{case} with forward checkpoints")
