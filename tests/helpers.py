"""Shared test helpers: numpy <-> torch transfer and the parity measures."""
import numpy as np

# Parity bounds, elementwise: |got - ref| <= tol * (1 + |ref|), tol by the
# io dtype (2e-2 covers the bf16 rounding of outputs stored in bf16).
TOL = {"f32": 1e-4, "bf16": 2e-2}
# Gradients that are sums of terms (dA, dB, dC, dD, ddelta_bias; conv dweight,
# dbias) are accumulated in float32 from terms formed in float32 from the same
# input bits as the oracle's: for every io dtype, |got - ref| <= TOL_SUM *
# (1 + sum |term|) + q |ref|, where q covers the final rounding of an output
# stored in bf16 (dB, dC of a bf16 scan; round to nearest: 2^-9, with margin
# 2^-8) and is 0 for float32 outputs.
TOL_SUM = 1e-4
Q_OUT = {"f32": 0.0, "bf16": 2.0 ** -8}


def to_dev(a, dev):
    import torch
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def to_np(t):
    """torch tensor (any float dtype) -> float64 numpy."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def norm_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if got.size == 0:
        return 0.0
    if not np.all(np.isfinite(got)):
        return float("inf")
    return float(np.max(np.abs(got - ref) / (1.0 + np.abs(ref))))


def sum_err(got, ref, ref_abs, q=0.0):
    """Largest error of a summed gradient, element by element, against the
    sum of the absolute values of the element's terms (the oracle's
    ``*_abs`` outputs): max (|got - ref| - q |ref|)+ / (1 + abs_sum), with q
    the relative rounding of the output's storage type.  The rounding of a
    float32 accumulation of those terms, in any order, scales with that sum,
    not with |ref|, which can be small by cancellation."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    ref_abs = np.asarray(ref_abs, dtype=np.float64)
    assert got.shape == ref.shape == ref_abs.shape, (got.shape, ref.shape, ref_abs.shape)
    if got.size == 0:
        return 0.0
    if not np.all(np.isfinite(got)):
        return float("inf")
    return float(np.max(np.maximum(np.abs(got - ref) - q * np.abs(ref), 0.0) / (1.0 + ref_abs)))


def scan_gpu(ssm, x, dev, bbar="delta", h0=None, final_state=None, want_final_state=True):
    """Run the library's forward scan on the numpy inputs of a workload."""
    return ssm.ssm_selective_scan_fwd(
        to_dev(x["u"], dev), to_dev(x["delta"], dev), to_dev(x["A"], dev), to_dev(x["B"], dev),
        to_dev(x["C"], dev), D=to_dev(x["D"], dev), z=to_dev(x.get("z"), dev),
        delta_bias=to_dev(x.get("delta_bias"), dev),
        delta_softplus=x.get("delta_softplus", True), h0=h0, bbar=bbar,
        final_state=final_state, want_final_state=want_final_state)


def scan_oracle(oracle, x, bbar="delta", h0=None, channels=None, want_y=True):
    return oracle.selective_scan(x["u"], x["delta"], x["A"], x["B"], x["C"], D=x["D"],
                                 z=x.get("z"), delta_bias=x.get("delta_bias"),
                                 delta_softplus=x.get("delta_softplus", True), bbar=bbar,
                                 h0=h0, channels=channels, want_y=want_y)
