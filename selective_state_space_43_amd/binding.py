"""torch tensors -> C ABI calls.  Checks dtype, device, shape and contiguity,
allocates outputs with torch when the caller did not pass them, and enqueues
the library call on torch's current stream of the tensors' device."""
from __future__ import annotations

import torch

from ._lib import SSM_DTYPE_BF16, SSM_DTYPE_F32, check, lib

_IO = {torch.bfloat16: SSM_DTYPE_BF16, torch.float32: SSM_DTYPE_F32}
_BBAR = {"delta": 0, "delta_b": 0, "zoh": 1, "zoh_exact": 1, "euler": 2, "bilinear": 3}


def _dev(t, name, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _io(t, name, dtype, shape, device):
    _dev(t, name, device)
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _f32(t, name, shape, device):
    if t is None:
        return None
    return _io(t, name, torch.float32, shape, device)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


CKPT_STEPS = 128  # steps between the forward's checkpoints


def ssm_checkpoint_shape(batch, dim, dstate, seqlen):
    """Shape of the forward's checkpoints: the state entering every 128-step
    block."""
    return (batch, dim, (seqlen + CKPT_STEPS - 1) // CKPT_STEPS, dstate)


def ssm_selective_scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None,
                           delta_softplus=False, h0=None, bbar="delta", y=None,
                           final_state=None, want_final_state=True, checkpoints=None):
    """Forward selective scan; returns (y, final_state or None).  With
    `checkpoints` (a float32 tensor of ssm_checkpoint_shape) it also writes the
    states the backward can take instead of recomputing them."""
    _dev(u, "u", None)
    dev = u.device
    if u.dim() != 3:
        raise ValueError("u must be [batch, dim, L]")
    if u.dtype not in _IO:
        raise TypeError(f"u has dtype {u.dtype}; expected bfloat16 or float32")
    batch, dim, L = u.shape
    if A.dim() != 2:
        raise ValueError("A must be [dim, dstate]")
    N = A.shape[1]
    io = u.dtype
    _io(delta, "delta", io, (batch, dim, L), dev)
    _io(A, "A", torch.float32, (dim, N), dev)
    _io(B, "B", io, (batch, N, L), dev)
    _io(C, "C", io, (batch, N, L), dev)
    _f32(D, "D", (dim,), dev)
    if z is not None:
        _io(z, "z", io, (batch, dim, L), dev)
    _f32(delta_bias, "delta_bias", (dim,), dev)
    _f32(h0, "h0", (batch, dim, N), dev)
    if y is None:
        y = torch.empty((batch, dim, L), dtype=io, device=dev)
    else:
        _io(y, "y", io, (batch, dim, L), dev)
    if final_state is None and want_final_state:
        final_state = torch.empty((batch, dim, N), dtype=torch.float32, device=dev)
    elif final_state is not None:
        _f32(final_state, "final_state", (batch, dim, N), dev)
    _f32(checkpoints, "checkpoints", ssm_checkpoint_shape(batch, dim, N, L), dev)
    with torch.cuda.device(dev):
        st = lib().ssm_selective_scan_fwd(
            _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
            int(bool(delta_softplus)), _ptr(h0), _ptr(y), _ptr(final_state), _ptr(checkpoints),
            batch, dim, N, L, _IO[io], _BBAR[bbar], _stream(dev))
    check(st, "ssm_selective_scan_fwd")
    return y, final_state


def ssm_state_update(state, u, delta, A, B, C, D=None, z=None, delta_bias=None,
                     delta_softplus=False, bbar="delta", y=None):
    """One decode step; updates `state` in place and returns y [batch, dim]."""
    _dev(state, "state", None)
    dev = state.device
    if state.dim() != 3 or state.dtype != torch.float32:
        raise ValueError("state must be float32 [batch, dim, dstate]")
    batch, dim, N = state.shape
    if u.dtype not in _IO:
        raise TypeError(f"u has dtype {u.dtype}; expected bfloat16 or float32")
    io = u.dtype
    _io(u, "u", io, (batch, dim), dev)
    _io(delta, "delta", io, (batch, dim), dev)
    _io(A, "A", torch.float32, (dim, N), dev)
    _io(B, "B", io, (batch, N), dev)
    _io(C, "C", io, (batch, N), dev)
    _f32(D, "D", (dim,), dev)
    if z is not None:
        _io(z, "z", io, (batch, dim), dev)
    _f32(delta_bias, "delta_bias", (dim,), dev)
    if y is None:
        y = torch.empty((batch, dim), dtype=io, device=dev)
    else:
        _io(y, "y", io, (batch, dim), dev)
    with torch.cuda.device(dev):
        st = lib().ssm_state_update(
            _ptr(state), _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
            _ptr(delta_bias), int(bool(delta_softplus)), _ptr(y), batch, dim, N, _IO[io],
            _BBAR[bbar], _stream(dev))
    check(st, "ssm_state_update")
    return y


def ssm_lti_kernel(A, Bv, Cv, delta, L, bbar="delta", K=None):
    """K[d, k] = sum_n C Abar^k Bbar for k < L.  Bv/Cv are [dstate] (shared by
    every channel) or [dim, dstate]."""
    _dev(A, "A", None)
    dev = A.device
    dim, N = A.shape
    _io(A, "A", torch.float32, (dim, N), dev)
    bs = 0 if Bv.dim() == 1 else N
    cs = 0 if Cv.dim() == 1 else N
    _io(Bv, "Bv", torch.float32, (N,) if bs == 0 else (dim, N), dev)
    _io(Cv, "Cv", torch.float32, (N,) if cs == 0 else (dim, N), dev)
    _io(delta, "delta", torch.float32, (dim,), dev)
    if K is None:
        K = torch.empty((dim, L), dtype=torch.float32, device=dev)
    else:
        _io(K, "K", torch.float32, (dim, L), dev)
    with torch.cuda.device(dev):
        st = lib().ssm_lti_kernel(_ptr(A), _ptr(Bv), _ptr(Cv), _ptr(delta), _ptr(K), dim, N, L,
                                  bs, cs, _BBAR[bbar], _stream(dev))
    check(st, "ssm_lti_kernel")
    return K


def ssm_lti_conv_fft_workspace_size(dim, seqlen):
    """Bytes of workspace the FFT convolution needs (0 up to seqlen 4096)."""
    n = lib().ssm_lti_conv_fft_workspace_size(dim, seqlen)
    if n < 0:
        raise ValueError("extents out of range")
    return int(n)


def ssm_lti_conv(K, u, D=None, y=None, method="direct", workspace=None):
    """y = K * u + D u per channel (causal): K [dim, L] float32, u [batch, dim, L].
    method "direct" (the causal sum, any L) or "fft" (L up to 2^20; past 4096
    through a workspace of ssm_lti_conv_fft_workspace_size bytes, allocated
    here unless given)."""
    if method not in ("direct", "fft"):
        raise ValueError(f"method {method!r}: expected 'direct' or 'fft'")
    _dev(u, "u", None)
    dev = u.device
    if u.dim() != 3 or u.dtype not in _IO:
        raise TypeError("u must be [batch, dim, L] bfloat16 or float32")
    batch, dim, L = u.shape
    _io(K, "K", torch.float32, (dim, L), dev)
    _f32(D, "D", (dim,), dev)
    if y is None:
        y = torch.empty_like(u)
    else:
        _io(y, "y", u.dtype, (batch, dim, L), dev)
    with torch.cuda.device(dev):
        if method == "fft":
            need = int(lib().ssm_lti_conv_fft_workspace_size(dim, L))  # -1: the call reports why
            if workspace is None and need > 0:
                workspace = torch.empty(need, dtype=torch.uint8, device=dev)
            nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
            st = lib().ssm_lti_conv_fft(_ptr(K), _ptr(u), _ptr(D), _ptr(y), _ptr(workspace), nbytes,
                                        batch, dim, L, _IO[u.dtype], _stream(dev))
        else:
            st = lib().ssm_lti_conv(_ptr(K), _ptr(u), _ptr(D), _ptr(y), batch, dim, L,
                                    _IO[u.dtype], _stream(dev))
    check(st, "ssm_lti_conv_fft" if method == "fft" else "ssm_lti_conv")
    return y


def ssm_selective_scan_bwd_workspace_size(batch, dim, dstate, seqlen):
    n = lib().ssm_selective_scan_bwd_workspace_size(batch, dim, dstate, seqlen)
    if n < 0:
        raise ValueError("extents out of range")
    return int(n)


def ssm_selective_scan_bwd(u, delta, A, B, C, dy, D=None, z=None, delta_bias=None,
                           delta_softplus=False, h0=None, dfinal_state=None, bbar="delta",
                           workspace=None, want_dh0=None, checkpoints=None):
    """Gradients of sum(dy * y) + sum(dfinal_state * final_state).  Returns a
    dict with du, ddelta (raw step), dA, dB, dC, and dD / dz / ddelta_bias /
    dh0 when D / z / delta_bias / h0 (or want_dh0) are given.  `checkpoints`
    from the forward on the same inputs saves recomputing them."""
    _dev(u, "u", None)
    dev = u.device
    if u.dim() != 3 or u.dtype not in _IO:
        raise TypeError("u must be [batch, dim, L] bfloat16 or float32")
    batch, dim, L = u.shape
    N = A.shape[1]
    io = u.dtype
    for t, n, shp in ((delta, "delta", (batch, dim, L)), (dy, "dy", (batch, dim, L)),
                      (B, "B", (batch, N, L)), (C, "C", (batch, N, L))):
        _io(t, n, io, shp, dev)
    _io(A, "A", torch.float32, (dim, N), dev)
    _f32(D, "D", (dim,), dev)
    if z is not None:
        _io(z, "z", io, (batch, dim, L), dev)
    _f32(delta_bias, "delta_bias", (dim,), dev)
    _f32(h0, "h0", (batch, dim, N), dev)
    _f32(dfinal_state, "dfinal_state", (batch, dim, N), dev)
    _f32(checkpoints, "checkpoints", ssm_checkpoint_shape(batch, dim, N, L), dev)
    need = ssm_selective_scan_bwd_workspace_size(batch, dim, N, L)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace needs {need} bytes")
    g = dict(du=torch.empty_like(u), ddelta=torch.empty_like(u),
             dA=torch.empty((dim, N), dtype=torch.float32, device=dev),
             dB=torch.empty_like(B), dC=torch.empty_like(C),
             dD=torch.empty(dim, dtype=torch.float32, device=dev) if D is not None else None,
             dz=torch.empty_like(u) if z is not None else None,
             ddelta_bias=(torch.empty(dim, dtype=torch.float32, device=dev)
                          if delta_bias is not None else None),
             dh0=(torch.empty((batch, dim, N), dtype=torch.float32, device=dev)
                  if (h0 is not None or want_dh0) else None))
    with torch.cuda.device(dev):
        st = lib().ssm_selective_scan_bwd(
            _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
            int(bool(delta_softplus)), _ptr(h0), _ptr(dy), _ptr(dfinal_state),
            _ptr(checkpoints), _ptr(g["du"]),
            _ptr(g["ddelta"]), _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g["dD"]),
            _ptr(g["dz"]), _ptr(g["ddelta_bias"]), _ptr(g["dh0"]), _ptr(workspace),
            workspace.numel() * workspace.element_size(), batch, dim, N, L, _IO[io],
            _BBAR[bbar], _stream(dev))
    check(st, "ssm_selective_scan_bwd")
    return g



class _SelectiveScanFn(torch.autograd.Function):
    """The scan as an autograd function: the forward writes the checkpoints
    that the backward then takes instead of recomputing them."""

    @staticmethod
    def forward(ctx, u, delta, A, B, C, D, z, delta_bias, h0, delta_softplus, bbar):
        batch, dim, L = u.shape
        ck = torch.empty(ssm_checkpoint_shape(batch, dim, A.shape[1], L), dtype=torch.float32,
                         device=u.device)
        y, final_state = ssm_selective_scan_fwd(u, delta, A, B, C, D=D, z=z, delta_bias=delta_bias,
                                                delta_softplus=delta_softplus, h0=h0, bbar=bbar,
                                                checkpoints=ck)
        ctx.save_for_backward(u, delta, A, B, C, D, z, delta_bias, h0, ck)
        ctx.delta_softplus, ctx.bbar = delta_softplus, bbar
        return y, final_state

    @staticmethod
    def backward(ctx, dy, dfinal):
        u, delta, A, B, C, D, z, delta_bias, h0, ck = ctx.saved_tensors
        dy = torch.zeros_like(u) if dy is None else dy.contiguous()
        g = ssm_selective_scan_bwd(u, delta, A, B, C, dy, D=D, z=z, delta_bias=delta_bias,
                                   delta_softplus=ctx.delta_softplus, h0=h0,
                                   dfinal_state=None if dfinal is None else dfinal.contiguous(),
                                   bbar=ctx.bbar, checkpoints=ck)
        return (g["du"], g["ddelta"], g["dA"], g["dB"], g["dC"], g["dD"], g["dz"],
                g["ddelta_bias"], g["dh0"], None, None)


def selective_scan_fn(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False,
                      h0=None, bbar="delta"):
    """(y, final_state) of ssm_selective_scan_fwd, differentiable in every
    tensor argument through ssm_selective_scan_bwd (rules "delta" and "zoh";
    the backward raises for the others)."""
    return _SelectiveScanFn.apply(u, delta, A, B, C, D, z, delta_bias, h0, delta_softplus, bbar)

def _conv_params(x, weight, bias, dev):
    if x.dim() != 3 or x.dtype not in _IO:
        raise TypeError("x must be [batch, dim, L] bfloat16 or float32")
    batch, dim, L = x.shape
    if weight.dim() != 2 or weight.shape[0] != dim:
        raise ValueError("weight must be [dim, width]")
    W = weight.shape[1]
    _io(weight, "weight", torch.float32, (dim, W), dev)
    _f32(bias, "bias", (dim,), dev)
    return batch, dim, L, W


def ssm_causal_conv1d_fwd(x, weight, bias=None, state_in=None, silu=True, out=None,
                          state_out=None, want_state_out=False):
    """Depthwise causal conv1d (+ silu); returns (out, state_out or None)."""
    _dev(x, "x", None)
    dev = x.device
    batch, dim, L, W = _conv_params(x, weight, bias, dev)
    _f32(state_in, "state_in", (batch, dim, W - 1), dev)
    if out is None:
        out = torch.empty_like(x)
    else:
        _io(out, "out", x.dtype, (batch, dim, L), dev)
    if state_out is None and want_state_out:
        state_out = torch.empty((batch, dim, W - 1), dtype=torch.float32, device=dev)
    elif state_out is not None:
        _f32(state_out, "state_out", (batch, dim, W - 1), dev)
    with torch.cuda.device(dev):
        st = lib().ssm_causal_conv1d_fwd(_ptr(x), _ptr(weight), _ptr(bias), _ptr(state_in),
                                         _ptr(out), _ptr(state_out), batch, dim, L, W,
                                         int(bool(silu)), _IO[x.dtype], _stream(dev))
    check(st, "ssm_causal_conv1d_fwd")
    return out, state_out


def ssm_causal_conv1d_update(x, conv_state, weight, bias=None, silu=True, out=None):
    """One token: x [batch, dim]; conv_state [batch, dim, W-1] updated in place."""
    _dev(x, "x", None)
    dev = x.device
    if x.dim() != 2 or x.dtype not in _IO:
        raise TypeError("x must be [batch, dim] bfloat16 or float32")
    batch, dim = x.shape
    W = weight.shape[1]
    _io(weight, "weight", torch.float32, (dim, W), dev)
    _f32(bias, "bias", (dim,), dev)
    _f32(conv_state, "conv_state", (batch, dim, W - 1), dev)
    if out is None:
        out = torch.empty_like(x)
    else:
        _io(out, "out", x.dtype, (batch, dim), dev)
    with torch.cuda.device(dev):
        st = lib().ssm_causal_conv1d_update(_ptr(x), _ptr(conv_state), _ptr(weight), _ptr(bias),
                                            _ptr(out), batch, dim, W, int(bool(silu)),
                                            _IO[x.dtype], _stream(dev))
    check(st, "ssm_causal_conv1d_update")
    return out


def ssm_causal_conv1d_bwd(x, weight, dout, bias=None, state_in=None, silu=True,
                          want_dstate_in=False):
    """Gradients of ssm_causal_conv1d_fwd: dict dx, dweight, dbias (if bias),
    dstate_in (if state_in or want_dstate_in)."""
    _dev(x, "x", None)
    dev = x.device
    batch, dim, L, W = _conv_params(x, weight, bias, dev)
    _io(dout, "dout", x.dtype, (batch, dim, L), dev)
    _f32(state_in, "state_in", (batch, dim, W - 1), dev)
    g = dict(dx=torch.empty_like(x),
             dweight=torch.empty((dim, W), dtype=torch.float32, device=dev),
             dbias=torch.empty(dim, dtype=torch.float32, device=dev) if bias is not None else None,
             dstate_in=(torch.empty((batch, dim, W - 1), dtype=torch.float32, device=dev)
                        if (state_in is not None or want_dstate_in) else None))
    with torch.cuda.device(dev):
        st = lib().ssm_causal_conv1d_bwd(_ptr(x), _ptr(weight), _ptr(bias), _ptr(state_in),
                                         _ptr(dout), _ptr(g["dx"]), _ptr(g["dweight"]),
                                         _ptr(g["dbias"]), _ptr(g["dstate_in"]), batch, dim, L,
                                         W, int(bool(silu)), _IO[x.dtype], _stream(dev))
    check(st, "ssm_causal_conv1d_bwd")
    return g



class _CausalConv1dFn(torch.autograd.Function):
    """The depthwise causal conv1d (+ silu) as an autograd function."""

    @staticmethod
    def forward(ctx, x, weight, bias, state_in, silu):
        out, _ = ssm_causal_conv1d_fwd(x, weight, bias=bias, state_in=state_in, silu=silu)
        ctx.save_for_backward(x, weight, bias, state_in)
        ctx.silu = silu
        return out

    @staticmethod
    def backward(ctx, dout):
        x, weight, bias, state_in = ctx.saved_tensors
        g = ssm_causal_conv1d_bwd(x, weight, dout.contiguous(), bias=bias, state_in=state_in,
                                  silu=ctx.silu)
        return g["dx"], g["dweight"], g["dbias"], g["dstate_in"], None


def causal_conv1d_fn(x, weight, bias=None, state_in=None, silu=True):
    """ssm_causal_conv1d_fwd's output, differentiable in x, weight, bias and
    state_in through ssm_causal_conv1d_bwd."""
    return _CausalConv1dFn.apply(x, weight, bias, state_in, silu)

def ssm_ssd_workspace_size(batch, seqlen, ngroups, dstate):
    n = lib().ssm_ssd_workspace_size(batch, seqlen, ngroups, dstate)
    if n < 0:
        raise ValueError("extents out of range")
    return int(n)


def ssm_ssd_fwd(x, dt, A, B, C, nheads, ngroups, D=None, z=None, dt_bias=None,
                dt_softplus=True, h0=None, y=None, final_state=None, want_final_state=True,
                workspace=None):
    """Mamba-2 scan (scalar A per head); returns (y, final_state or None)."""
    _dev(x, "x", None)
    dev = x.device
    if x.dim() != 3 or x.dtype != torch.bfloat16:
        raise TypeError("x must be [batch, nheads * headdim, L] bfloat16")
    batch, hp, L = x.shape
    if hp % nheads:
        raise ValueError("x's channel count is not a multiple of nheads")
    P = hp // nheads
    if B.dim() != 3 or B.shape[1] % ngroups:
        raise ValueError("B must be [batch, ngroups * dstate, L]")
    N = B.shape[1] // ngroups
    _io(dt, "dt", torch.bfloat16, (batch, nheads, L), dev)
    _io(B, "B", torch.bfloat16, (batch, ngroups * N, L), dev)
    _io(C, "C", torch.bfloat16, (batch, ngroups * N, L), dev)
    _io(A, "A", torch.float32, (nheads,), dev)
    _f32(D, "D", (nheads,), dev)
    _f32(dt_bias, "dt_bias", (nheads,), dev)
    if z is not None:
        _io(z, "z", torch.bfloat16, (batch, hp, L), dev)
    _f32(h0, "h0", (batch, nheads, P, N), dev)
    if y is None:
        y = torch.empty_like(x)
    else:
        _io(y, "y", torch.bfloat16, (batch, hp, L), dev)
    if final_state is None and want_final_state:
        final_state = torch.empty((batch, nheads, P, N), dtype=torch.float32, device=dev)
    elif final_state is not None:
        _f32(final_state, "final_state", (batch, nheads, P, N), dev)
    need = ssm_ssd_workspace_size(batch, L, ngroups, N)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        st = lib().ssm_ssd_fwd(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                               _ptr(dt_bias), int(bool(dt_softplus)), _ptr(h0), _ptr(y),
                               _ptr(final_state), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), batch, L, nheads, P,
                               ngroups, N, SSM_DTYPE_BF16, _stream(dev))
    check(st, "ssm_ssd_fwd")
    return y, final_state


def ssm_ssd_scratch_bytes():
    """Size of the library's static scratch for ssm_ssd_fwd_noalloc."""
    return int(lib().ssm_ssd_scratch_bytes())


def ssm_ssd_fwd_noalloc(x, dt, A, B, C, nheads, ngroups, y, D=None, z=None, dt_bias=None,
                        dt_softplus=True, h0=None, final_state=None):
    """ssm_ssd_fwd with its workspace in the library's static scratch: nothing
    is allocated, here or in the library (y and final_state are the
    caller's).  Calls on one GPU share the scratch and must not overlap."""
    _dev(x, "x", None)
    dev = x.device
    if x.dim() != 3 or x.dtype != torch.bfloat16:
        raise TypeError("x must be [batch, nheads * headdim, L] bfloat16")
    batch, hp, L = x.shape
    if hp % nheads:
        raise ValueError("x's channel count is not a multiple of nheads")
    P = hp // nheads
    if B.dim() != 3 or B.shape[1] % ngroups:
        raise ValueError("B must be [batch, ngroups * dstate, L]")
    N = B.shape[1] // ngroups
    _io(dt, "dt", torch.bfloat16, (batch, nheads, L), dev)
    _io(B, "B", torch.bfloat16, (batch, ngroups * N, L), dev)
    _io(C, "C", torch.bfloat16, (batch, ngroups * N, L), dev)
    _io(A, "A", torch.float32, (nheads,), dev)
    _f32(D, "D", (nheads,), dev)
    _f32(dt_bias, "dt_bias", (nheads,), dev)
    if z is not None:
        _io(z, "z", torch.bfloat16, (batch, hp, L), dev)
    _f32(h0, "h0", (batch, nheads, P, N), dev)
    _io(y, "y", torch.bfloat16, (batch, hp, L), dev)
    _f32(final_state, "final_state", (batch, nheads, P, N), dev)
    with torch.cuda.device(dev):
        st = lib().ssm_ssd_fwd_noalloc(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                       _ptr(z), _ptr(dt_bias), int(bool(dt_softplus)), _ptr(h0),
                                       _ptr(y), _ptr(final_state), batch, L, nheads, P, ngroups,
                                       N, SSM_DTYPE_BF16, _stream(dev))
    check(st, "ssm_ssd_fwd_noalloc")
    return y, final_state
