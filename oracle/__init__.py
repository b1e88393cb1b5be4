"""Double-precision CPU oracle for the selective state-space scan.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this package.  It shares
no code with the HIP library: the arithmetic lives in ``ssm_oracle.c`` (plain C,
fp64, sequential in time), and this module only marshals numpy arrays.

Inputs are numpy arrays.  Sequence tensors (u, delta, z: [batch, dim, L];
B, C: [batch, dstate, L]) are either ``float32`` or ``uint16`` holding bf16
bit patterns, or ``float64`` (used by the finite-difference pins); the C code
widens them itself.  Per-channel parameters (A, D,
delta_bias, h0) are widened to float64 here with ``astype`` (exact for float32).

Each function cites the page passage it follows in ``ssm_oracle.c``.
The backward functions can also return, for every gradient that is a sum
(dA, dB, dC, dD, ddelta_bias; conv dw, dbias), the sum of the absolute values
of its terms: the parity tests bound each such element by tol * (1 + that sum).
Parity status: every function here is pinned by ``tests/test_oracle_pins.py`` (forward,
decode, LTI), ``tests/test_oracle_bwd_pins.py`` (backward, by finite differences) and
``tests/test_oracle_conv_pins.py`` (causal conv1d: torch's conv1d, closed forms, finite
differences) and ``tests/test_oracle_ssd_pins.py`` (Mamba-2 scan: the diagonal scan with a
per-head A, the masked-attention form, brute force).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssm_oracle.c")
_SO = os.path.join(_HERE, "libssm_oracle.so")
_SO_SANITIZED = os.path.join(_HERE, "libssm_oracle_san.so")
# A prebuilt oracle library to load instead (the sanitizer test points this at
# the AddressSanitizer / UndefinedBehaviorSanitizer build); not built here.
_SO_OVERRIDE = os.environ.get("SSM_ORACLE_LIB")
_LIB = None

BBAR_MODES = {"delta": 0, "delta_b": 0, "zoh": 1, "zoh_exact": 1, "euler": 2, "bilinear": 3}


def build(force: bool = False) -> str:
    """Compile ssm_oracle.c into libssm_oracle.so with gcc (plain C, no GPU)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared",
             "-o", tmp, _SRC, "-lm", "-lpthread"])
        os.replace(tmp, _SO)
    return _SO


def build_sanitized() -> str:
    """The same source built with AddressSanitizer and UndefinedBehaviorSanitizer
    (host code only; run the pins against it with the sanitizer runtimes
    preloaded and SSM_ORACLE_LIB pointing at the returned path)."""
    tmp = _SO_SANITIZED + ".tmp%d" % os.getpid()
    subprocess.check_call(
        ["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
         "-fno-omit-frame-pointer", "-o", tmp, _SRC, "-lm", "-lpthread"])
    os.replace(tmp, _SO_SANITIZED)
    return _SO_SANITIZED


def _lib():
    global _LIB
    if _LIB is None:
        if _SO_OVERRIDE:
            lib = ctypes.CDLL(_SO_OVERRIDE)
        else:
            build()
            lib = ctypes.CDLL(_SO)
        i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        lib.ssm_oracle_selective_scan.argtypes = [
            i32, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, vp,
            i64, i64, i64, i64, vp, i64, vp, vp, i32]
        lib.ssm_oracle_state_update.argtypes = [
            i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32,
            i64, i64, i64, vp, i64, vp, i32]
        lib.ssm_oracle_lti_kernel.argtypes = [
            vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, i32, vp]
        lib.ssm_oracle_causal_conv.argtypes = [vp, vp, ctypes.c_double, i64, vp]
        lib.ssm_oracle_selective_scan_bwd.argtypes = [
            i32, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, vp, vp, vp,
            i64, i64, i64, i64, vp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp,
            vp, vp, vp, vp, vp, i32]
        lib.ssm_oracle_ssd.argtypes = [i32, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp,
                                       i64, i64, i64, i64, i64, i64, vp, vp, i32]
        lib.ssm_oracle_conv1d.argtypes = [i32, vp, vp, vp, vp, i64, i64, i64, i64, i32, vp, vp]
        lib.ssm_oracle_conv1d_bwd.argtypes = [i32, vp, vp, vp, vp, vp, i64, i64, i64, i64, i32,
                                              vp, vp, vp, vp, vp, vp]
        for f in (lib.ssm_oracle_selective_scan, lib.ssm_oracle_state_update,
                  lib.ssm_oracle_lti_kernel, lib.ssm_oracle_causal_conv,
                  lib.ssm_oracle_selective_scan_bwd, lib.ssm_oracle_conv1d, lib.ssm_oracle_ssd,
                  lib.ssm_oracle_conv1d_bwd):
            f.restype = i32
        _LIB = lib
    return _LIB


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _seq(x, name):
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, 0
    if x.dtype == np.uint16:
        return x, 1
    if x.dtype == np.float64:
        return x, 2
    raise TypeError(f"{name}: expected float32, float64 or uint16 (bf16 bits), got {x.dtype}")


def _f64(x):
    return None if x is None else np.ascontiguousarray(x, dtype=np.float64)


def _ptr(x):
    return None if x is None else x.ctypes.data


def selective_scan(u, delta, A, B, C, D=None, z=None, delta_bias=None,
                   delta_softplus=False, bbar="delta", h0=None, channels=None,
                   want_y=True, n_threads=None):
    """Sequential fp64 selective scan.

    Returns ``(y, final_state)`` with y float64 ``[n_sel, L]`` (or None) and
    final_state float64 ``[n_sel, dstate]``, where the rows follow ``channels``
    (flat ``b*dim + d``; None = every channel in order).  ``h0`` is
    ``[n_sel, dstate]`` aligned with the same selection.
    """
    u, dt = _seq(u, "u")
    delta, dt2 = _seq(delta, "delta")
    B, dt3 = _seq(B, "B")
    C, dt4 = _seq(C, "C")
    if len({dt, dt2, dt3, dt4}) != 1:
        raise TypeError("u, delta, B, C must share one dtype")
    if z is not None:
        z, dt5 = _seq(z, "z")
        if dt5 != dt:
            raise TypeError("z must share the io dtype")
    batch, dim, L = u.shape
    N = A.shape[1]
    assert delta.shape == u.shape and B.shape == (batch, N, L) and C.shape == (batch, N, L)
    assert A.shape == (dim, N)
    if z is not None:
        assert z.shape == u.shape
    A64, D64, bias64 = _f64(A), _f64(D), _f64(delta_bias)
    if channels is None:
        sel = None
        n_sel = batch * dim
    else:
        sel = np.ascontiguousarray(channels, dtype=np.int64)
        n_sel = sel.size
    h064 = None
    if h0 is not None:
        h064 = np.ascontiguousarray(h0, dtype=np.float64).reshape(n_sel, N)
    y = np.empty((n_sel, L), dtype=np.float64) if want_y else None
    fs = np.empty((n_sel, N), dtype=np.float64)
    rc = _lib().ssm_oracle_selective_scan(
        dt, _ptr(u), _ptr(delta), _ptr(B), _ptr(C), _ptr(z), _ptr(A64), _ptr(D64),
        _ptr(bias64), int(bool(delta_softplus)), BBAR_MODES[bbar], _ptr(h064),
        batch, dim, N, L, _ptr(sel), n_sel, _ptr(y), _ptr(fs),
        int(n_threads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"ssm_oracle_selective_scan failed ({rc})")
    return y, fs


def state_update(state, u, delta, A, B, C, D=None, z=None, delta_bias=None,
                 delta_softplus=False, bbar="delta", channels=None, n_threads=None):
    """One decode step.  ``state`` is float64 ``[n_sel, dstate]`` and is updated
    in place; u, delta, z are ``[batch, dim]``; B, C ``[batch, dstate]``.
    Returns y float64 ``[n_sel]``."""
    if not (isinstance(state, np.ndarray) and state.dtype == np.float64
            and state.flags.c_contiguous):
        raise TypeError("state must be a C-contiguous float64 array")
    u, dt = _seq(u, "u")
    delta, _ = _seq(delta, "delta")
    B, _ = _seq(B, "B")
    C, _ = _seq(C, "C")
    if z is not None:
        z, _ = _seq(z, "z")
    batch, dim = u.shape
    N = A.shape[1]
    sel = None if channels is None else np.ascontiguousarray(channels, dtype=np.int64)
    n_sel = batch * dim if sel is None else sel.size
    assert state.shape == (n_sel, N)
    A64, D64, bias64 = _f64(A), _f64(D), _f64(delta_bias)
    y = np.empty(n_sel, dtype=np.float64)
    rc = _lib().ssm_oracle_state_update(
        dt, _ptr(state), _ptr(u), _ptr(delta), _ptr(B), _ptr(C), _ptr(z), _ptr(A64),
        _ptr(D64), _ptr(bias64), int(bool(delta_softplus)), BBAR_MODES[bbar],
        batch, dim, N, _ptr(sel), n_sel, _ptr(y), int(n_threads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"ssm_oracle_state_update failed ({rc})")
    return y


def lti_kernel(A, Bv, Cv, delta, L, bbar="delta", method="direct"):
    """K[d, k] = sum_n C[d,n] Abar[d,n]^k Bbar[d,n] in fp64.  Bv/Cv may be
    ``[dstate]`` (shared by every channel) or ``[dim, dstate]``."""
    A64 = _f64(A)
    dim, N = A64.shape
    Bv64, Cv64, d64 = _f64(Bv), _f64(Cv), _f64(delta)
    bs = 0 if Bv64.ndim == 1 else N
    cs = 0 if Cv64.ndim == 1 else N
    K = np.empty((dim, L), dtype=np.float64)
    rc = _lib().ssm_oracle_lti_kernel(
        _ptr(A64), _ptr(Bv64), _ptr(Cv64), _ptr(d64), dim, N, L, bs, cs,
        BBAR_MODES[bbar], {"direct": 0, "powers": 1}[method], _ptr(K))
    if rc != 0:
        raise RuntimeError("ssm_oracle_lti_kernel failed")
    return K


def causal_conv(K, u, D=0.0):
    """y[t] = sum_{k<=t} K[k] u[t-k] + D u[t], direct O(L^2) sum in fp64."""
    K64, u64 = _f64(K), _f64(u)
    L = u64.size
    assert K64.size >= L
    y = np.empty(L, dtype=np.float64)
    rc = _lib().ssm_oracle_causal_conv(_ptr(K64), _ptr(u64), float(D), L, _ptr(y))
    if rc != 0:
        raise RuntimeError("ssm_oracle_causal_conv failed")
    return y


def selective_scan_bwd(u, delta, A, B, C, dy, D=None, z=None, delta_bias=None,
                       delta_softplus=False, bbar="delta", h0=None, dfinal=None, channels=None,
                       want_abs=False, n_threads=None):
    """Gradients of the fp64 selective scan for the loss sum(dy * y) +
    sum(dfinal * final_state).  Returns a dict of float64 arrays: per selected
    channel du, ddelta (raw step), dz (if z), dh0 ([n_sel, dstate]); summed over
    the selected channels dA [dim, dstate], dB, dC [batch, dstate, L], dD,
    ddelta_bias [dim].  With ``want_abs`` also dA_abs, dB_abs, dC_abs, dD_abs,
    ddelta_bias_abs: per element the sum of the absolute values of the terms
    that the corresponding sum adds (the scale of its rounding error)."""
    u, dt = _seq(u, "u")
    delta, _ = _seq(delta, "delta")
    B, _ = _seq(B, "B")
    C, _ = _seq(C, "C")
    if z is not None:
        z, _ = _seq(z, "z")
    batch, dim, L = u.shape
    N = A.shape[1]
    sel = None if channels is None else np.ascontiguousarray(channels, dtype=np.int64)
    n_sel = batch * dim if sel is None else sel.size
    dy64 = np.ascontiguousarray(dy, dtype=np.float64)
    assert dy64.shape == (batch, dim, L)
    h064 = None if h0 is None else np.ascontiguousarray(h0, dtype=np.float64).reshape(n_sel, N)
    df64 = None if dfinal is None else np.ascontiguousarray(dfinal, dtype=np.float64).reshape(n_sel, N)
    # held in locals: the C call reads them through raw addresses
    A64, D64, bias64 = _f64(A), _f64(D), _f64(delta_bias)
    out = dict(du=np.empty((n_sel, L)), ddelta=np.empty((n_sel, L)),
               dz=np.empty((n_sel, L)) if z is not None else None,
               dh0=np.empty((n_sel, N)),
               dA=np.empty((dim, N)), dB=np.empty((batch, N, L)), dC=np.empty((batch, N, L)),
               dD=np.empty(dim), ddelta_bias=np.empty(dim))
    ab = dict(dA_abs=np.empty((dim, N)), dB_abs=np.empty((batch, N, L)),
              dC_abs=np.empty((batch, N, L)), dD_abs=np.empty(dim),
              ddelta_bias_abs=np.empty(dim)) if want_abs else {}
    rc = _lib().ssm_oracle_selective_scan_bwd(
        dt, _ptr(u), _ptr(delta), _ptr(B), _ptr(C), _ptr(z), _ptr(A64), _ptr(D64),
        _ptr(bias64), int(bool(delta_softplus)), BBAR_MODES[bbar], _ptr(h064),
        _ptr(dy64), _ptr(df64), batch, dim, N, L, _ptr(sel), n_sel,
        _ptr(out["du"]), _ptr(out["ddelta"]), _ptr(out["dA"]), _ptr(out["dB"]), _ptr(out["dC"]),
        _ptr(out["dD"]), _ptr(out["dz"]), _ptr(out["ddelta_bias"]), _ptr(out["dh0"]),
        _ptr(ab.get("dA_abs")), _ptr(ab.get("dB_abs")), _ptr(ab.get("dC_abs")),
        _ptr(ab.get("dD_abs")), _ptr(ab.get("ddelta_bias_abs")),
        int(n_threads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"ssm_oracle_selective_scan_bwd failed ({rc})")
    out.update(ab)
    return out


def conv1d(x, w, bias=None, state_in=None, silu=True):
    """Depthwise causal convolution (width W = w.shape[1]) with optional silu.
    x: [batch, dim, L] float32 / bf16 bits / float64; w: [dim, W]; bias: [dim];
    state_in: [batch, dim, W-1] (the inputs before t = 0, oldest first) or None.
    Returns (out float64 [batch, dim, L], state_out float64 [batch, dim, W-1])."""
    x, dt = _seq(x, "x")
    batch, dim, L = x.shape
    w64 = _f64(w)
    W = w64.shape[1]
    b64, s64 = _f64(bias), _f64(state_in)
    out = np.empty((batch, dim, L), dtype=np.float64)
    st = np.empty((batch, dim, W - 1), dtype=np.float64)
    rc = _lib().ssm_oracle_conv1d(dt, _ptr(x), _ptr(w64), _ptr(b64), _ptr(s64), batch, dim, L,
                                  W, int(bool(silu)), _ptr(out), _ptr(st) if W > 1 else None)
    if rc != 0:
        raise RuntimeError(f"ssm_oracle_conv1d failed ({rc})")
    return out, st


def conv1d_bwd(x, w, dout, bias=None, state_in=None, silu=True, want_abs=False):
    """Gradients of conv1d for the loss sum(dout * out): dict of float64 dx
    [batch, dim, L], dw [dim, W], dbias [dim], dstate_in [batch, dim, W-1];
    with ``want_abs`` also dw_abs and dbias_abs, the sums of the absolute
    values of the terms of dw and dbias."""
    x, dt = _seq(x, "x")
    batch, dim, L = x.shape
    w64 = _f64(w)
    W = w64.shape[1]
    b64, s64 = _f64(bias), _f64(state_in)
    d64 = np.ascontiguousarray(dout, dtype=np.float64)
    assert d64.shape == (batch, dim, L)
    g = dict(dx=np.empty((batch, dim, L)), dw=np.empty((dim, W)), dbias=np.empty(dim),
             dstate_in=np.empty((batch, dim, W - 1)))
    if want_abs:
        g["dw_abs"], g["dbias_abs"] = np.empty((dim, W)), np.empty(dim)
    rc = _lib().ssm_oracle_conv1d_bwd(dt, _ptr(x), _ptr(w64), _ptr(b64), _ptr(s64), _ptr(d64),
                                      batch, dim, L, W, int(bool(silu)), _ptr(g["dx"]),
                                      _ptr(g["dw"]), _ptr(g["dbias"]),
                                      _ptr(g["dstate_in"]) if W > 1 else None,
                                      _ptr(g.get("dw_abs")), _ptr(g.get("dbias_abs")))
    if rc != 0:
        raise RuntimeError(f"ssm_oracle_conv1d_bwd failed ({rc})")
    return g


def ssd(x, dt, A, B, C, nheads, ngroups, D=None, z=None, dt_bias=None, dt_softplus=True, h0=None,
        n_threads=None):
    """Mamba-2 scan (scalar A per head) in fp64.  x, z: [batch, nheads*headdim, L];
    dt: [batch, nheads, L]; B, C: [batch, ngroups*dstate, L] (float32, bf16 bits
    or float64, one dtype); A, D, dt_bias: [nheads]; h0: [batch, nheads, headdim,
    dstate].  Returns (y float64 [batch, nheads*headdim, L], final_state float64
    [batch, nheads, headdim, dstate])."""
    x, dtc = _seq(x, "x")
    dt, _ = _seq(dt, "dt")
    B, _ = _seq(B, "B")
    C, _ = _seq(C, "C")
    if z is not None:
        z, _ = _seq(z, "z")
    batch, HP, L = x.shape
    P = HP // nheads
    N = B.shape[1] // ngroups
    A64, D64, b64, h064 = _f64(A), _f64(D), _f64(dt_bias), _f64(h0)
    y = np.empty((batch, HP, L), dtype=np.float64)
    fs = np.empty((batch, nheads, P, N), dtype=np.float64)
    rc = _lib().ssm_oracle_ssd(dtc, _ptr(x), _ptr(dt), _ptr(B), _ptr(C), _ptr(z), _ptr(A64),
                               _ptr(D64), _ptr(b64), int(bool(dt_softplus)), _ptr(h064), batch, L,
                               nheads, P, ngroups, N, _ptr(y), _ptr(fs),
                               int(n_threads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"ssm_oracle_ssd failed ({rc})")
    return y, fs
