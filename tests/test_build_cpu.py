"""Compile-time checks of the HIP source (a syntax-only device pass, no GPU):
the shipped layouts compile, and a forward-scan layout whose B/C tiles and
carry rows cannot fit one CU's 160 KiB of LDS is rejected by the compiler
instead of faulting at launch (64 lanes per channel with 16-state tiles:
2 x 16 x 64 x 20 floats of tiles plus 2 x 8 x 64 floats of carry and A rows)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "selective_state_space_43_amd", "csrc", "selscan.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _syntax_check(*defines):
    if not (os.path.exists(HIPCC) or shutil.which(HIPCC)):
        pytest.skip("hipcc not available")
    cmd = [HIPCC, "--offload-arch=gfx950", "-std=c++17", "-fsyntax-only",
           "-I", os.path.join(ROOT, "include"), *defines, SRC]
    return subprocess.run(cmd, capture_output=True, text=True, timeout=300)


def test_shipped_layouts_compile():
    res = _syntax_check()
    assert res.returncode == 0, res.stderr[-3000:]


def test_forward_layout_over_lds_fails_to_compile():
    # SELSCAN_NT=32 gives the 64-lanes-per-channel layout (eight waves) 16-state tiles
    res = _syntax_check("-DSELSCAN_NT=32")
    assert res.returncode != 0
    assert "exceeds the LDS of one CU" in res.stderr
