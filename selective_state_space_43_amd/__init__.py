"""Thin Python binding over libselscan's C ABI (include/selscan.h).

Argument marshalling only: every step of the scan runs in the HIP kernels of
``libselscan.so``.  PyTorch supplies device memory and the current stream.
There is no CPU fallback: if the library is missing the first call raises.

Entry points carry the C names:

  ssm_selective_scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None,
                         delta_softplus=False, h0=None, bbar="delta",
                         y=None, final_state=None, want_final_state=True,
                         checkpoints=None)
      -> (y, final_state)
  ssm_checkpoint_shape(batch, dim, dstate, seqlen) -> shape of `checkpoints`
  ssm_state_update(state, u, delta, A, B, C, D=None, z=None, delta_bias=None,
                   delta_softplus=False, bbar="delta", y=None) -> y
  ssm_lti_kernel(A, Bv, Cv, delta, L, bbar="delta", K=None) -> K
  ssm_lti_conv(K, u, D=None, y=None, method="direct") -> y  (y = K * u + D u, causal;
                                                              method "direct" or "fft")
  ssm_selective_scan_bwd(u, delta, A, B, C, dy, D=None, z=None, delta_bias=None,
                         delta_softplus=False, h0=None, dfinal_state=None,
                         bbar="delta", workspace=None, checkpoints=None)
      -> dict of gradients
  ssm_causal_conv1d_fwd(x, weight, bias=None, state_in=None, silu=True,
                        out=None, state_out=None, want_state_out=False)
      -> (out, state_out)
  ssm_causal_conv1d_update(x, conv_state, weight, bias=None, silu=True) -> out
  ssm_causal_conv1d_bwd(x, weight, dout, bias=None, state_in=None, silu=True)
      -> dict of gradients
  ssm_ssd_fwd(x, dt, A, B, C, nheads, ngroups, D=None, z=None, dt_bias=None,
              dt_softplus=True, h0=None) -> (y, final_state)      (Mamba-2 scan)
  ssm_ssd_fwd_noalloc(x, dt, A, B, C, nheads, ngroups, y, ...) -> (y, final_state)
      the same with the workspace in the library's static scratch: allocates
      nothing (for callers that cannot allocate; ssm_ssd_scratch_bytes())
  selective_scan_fn(u, delta, A, B, C, D=None, z=None, delta_bias=None,
                    delta_softplus=False, h0=None, bbar="delta")
      -> (y, final_state), differentiable (torch.autograd): the forward's
         checkpoints feed ssm_selective_scan_bwd
  causal_conv1d_fn(x, weight, bias=None, state_in=None, silu=True) -> out,
      differentiable through ssm_causal_conv1d_bwd

Layouts: u, delta, z, y [batch, dim, L]; B, C [batch, dstate, L]; A
[dim, dstate]; D, delta_bias [dim]; h0 / final_state / state
[batch, dim, dstate].  Sequence tensors are torch.bfloat16 or torch.float32
(one dtype for all of them); everything else is float32.
"""
from __future__ import annotations

from ._lib import (SSM_BBAR_DELTA_B, SSM_BBAR_ZOH_EXACT, SSM_DTYPE_BF16, SSM_DTYPE_F32,
                   SelscanError, library_path, lib, ssm_abi_version, ssm_last_error,
                   ssm_status_str)
from .binding import (ssm_causal_conv1d_bwd, ssm_causal_conv1d_fwd, ssm_causal_conv1d_update,
                      ssm_checkpoint_shape, ssm_lti_conv, ssm_lti_conv_fft_workspace_size,
                      ssm_lti_kernel,
                      ssm_selective_scan_bwd, ssm_ssd_fwd, ssm_ssd_fwd_noalloc,
                      ssm_ssd_scratch_bytes, ssm_ssd_workspace_size,
                      ssm_selective_scan_bwd_workspace_size, ssm_selective_scan_fwd,
                      ssm_state_update, selective_scan_fn, causal_conv1d_fn)

__all__ = [
    "ssm_selective_scan_fwd", "ssm_state_update", "ssm_lti_kernel", "ssm_lti_conv",
    "ssm_lti_conv_fft_workspace_size",
    "ssm_selective_scan_bwd", "ssm_checkpoint_shape", "selective_scan_fn", "causal_conv1d_fn",
    "ssm_selective_scan_bwd_workspace_size", "ssm_causal_conv1d_fwd", "ssm_causal_conv1d_update",
    "ssm_causal_conv1d_bwd", "ssm_ssd_fwd", "ssm_ssd_workspace_size", "ssm_ssd_fwd_noalloc",
    "ssm_ssd_scratch_bytes", "ssm_status_str",
    "ssm_last_error", "ssm_abi_version", "SelscanError", "library_path", "lib",
    "SSM_DTYPE_F32", "SSM_DTYPE_BF16", "SSM_BBAR_DELTA_B", "SSM_BBAR_ZOH_EXACT",
]
