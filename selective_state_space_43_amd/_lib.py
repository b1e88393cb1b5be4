"""Loads libselscan.so and declares the C signatures of include/selscan.h."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libselscan.so")

ABI_VERSION = 3  # the SSM_ABI_VERSION these signatures follow
SSM_DTYPE_F32, SSM_DTYPE_BF16 = 0, 1
SSM_BBAR_DELTA_B, SSM_BBAR_ZOH_EXACT, SSM_DISC_EULER, SSM_DISC_BILINEAR = 0, 1, 2, 3
STATUS_NAMES = {0: "SSM_OK", 1: "SSM_E_NULL", 2: "SSM_E_SHAPE", 3: "SSM_E_DTYPE",
                4: "SSM_E_ALIGN", 5: "SSM_E_ALIAS", 6: "SSM_E_UNSUPPORTED", 7: "SSM_E_HIP"}

_LIB = None


class SelscanError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {detail}")


def library_path() -> str:
    return _SO


def lib() -> ctypes.CDLL:
    """The loaded library.  Raises if it has not been built: there is no
    fallback implementation."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(_SO):
            raise ImportError(
                f"libselscan.so not found at {_SO}; build it first "
                "(python -c 'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(_SO)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        L.ssm_selective_scan_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp,
                                             vp, i64, i64, i64, i64, i32, i32, vp]
        L.ssm_state_update.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp,
                                       i64, i64, i64, i32, i32, vp]
        L.ssm_lti_kernel.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, vp]
        L.ssm_selective_scan_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp,
                                             vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64,
                                             i64, i64, i64, i64, i32, i32, vp]
        L.ssm_selective_scan_bwd_workspace_size.argtypes = [i64, i64, i64, i64]
        L.ssm_selective_scan_bwd_workspace_size.restype = i64
        L.ssm_causal_conv1d_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i32,
                                            i32, vp]
        L.ssm_causal_conv1d_update.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, vp]
        L.ssm_causal_conv1d_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64,
                                            i64, i32, i32, vp]
        L.ssm_ssd_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, i64,
                                  i64, i64, i64, i64, i64, i64, i32, vp]
        L.ssm_lti_conv.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, vp]
        L.ssm_lti_conv_fft.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, vp]
        L.ssm_lti_conv_fft_workspace_size.argtypes = [i64, i64]
        L.ssm_lti_conv_fft_workspace_size.restype = i64
        L.ssm_ssd_workspace_size.argtypes = [i64, i64, i64, i64]
        L.ssm_ssd_workspace_size.restype = i64
        L.ssm_ssd_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp,
                                          i64, i64, i64, i64, i64, i64, i32, vp]
        L.ssm_ssd_fwd_noalloc.restype = i32
        L.ssm_ssd_scratch_bytes.argtypes = []
        L.ssm_ssd_scratch_bytes.restype = i64
        for f in (L.ssm_selective_scan_fwd, L.ssm_state_update, L.ssm_lti_kernel,
                  L.ssm_selective_scan_bwd, L.ssm_causal_conv1d_fwd, L.ssm_causal_conv1d_update,
                  L.ssm_causal_conv1d_bwd, L.ssm_ssd_fwd, L.ssm_lti_conv,
                  L.ssm_lti_conv_fft):
            f.restype = i32
        L.ssm_status_str.argtypes = [i32]
        L.ssm_status_str.restype = ctypes.c_char_p
        L.ssm_last_error.argtypes = []
        L.ssm_last_error.restype = ctypes.c_char_p
        L.ssm_abi_version.argtypes = []
        L.ssm_abi_version.restype = i32
        if L.ssm_abi_version() != ABI_VERSION:
            raise ImportError(f"{_SO} has ABI version {L.ssm_abi_version()}, this binding "
                              f"expects {ABI_VERSION}: rebuild it")
        _LIB = L
    return _LIB


def ssm_status_str(status: int) -> str:
    return lib().ssm_status_str(int(status)).decode()


def ssm_last_error() -> str:
    return lib().ssm_last_error().decode()


def ssm_abi_version() -> int:
    return int(lib().ssm_abi_version())


def check(status: int, where: str) -> None:
    if status != 0:
        raise SelscanError(status, where, ssm_last_error() or ssm_status_str(status))
