"""ssm_ssd_fwd_noalloc (the Mamba-2 scan with its workspace in the library's
static scratch, for callers that cannot allocate) against ssm_ssd_fwd, the
entry point with a caller-owned workspace, through the C ABI: two calls in a
row, the second with a smaller input, each bit for bit equal to ssm_ssd_fwd
on the same inputs (the same kernels run), and within the bf16 bound of the
fp64 oracle.  Sizes beyond the scratch are refused."""
import numpy as np
import pytest

import oracle
import workloads as wl
from helpers import TOL, norm_err, to_dev, to_np

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ssm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_43_amd as m
    m.lib()
    return m


def _inputs(w, dev):
    x = wl.ssd_inputs(w, with_h0=True)
    return x, {k: to_dev(v, dev) for k, v in x.items() if v is not None}


def test_noalloc_matches_workspace_entry_point(ssm):
    dev = torch.device("cuda:0")
    # the second call is smaller: the scratch still holds the first call's data
    for w in (wl.SsdWorkload("big", 2, 3000, 8, 64, 2, 128, True, seed=4800),
              wl.SsdWorkload("small", 1, 700, 4, 64, 1, 64, True, seed=4801)):
        x, t = _inputs(w, dev)
        kw = dict(D=t["D"], z=t["z"], dt_bias=t["dt_bias"], dt_softplus=True, h0=t["h0"])
        y_ref, f_ref = ssm.ssm_ssd_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], w.nheads,
                                       w.ngroups, **kw)
        y = torch.empty_like(t["x"])
        fs = torch.empty_like(f_ref)
        ssm.ssm_ssd_fwd_noalloc(t["x"], t["dt"], t["A"], t["B"], t["C"], w.nheads, w.ngroups,
                                y, final_state=fs, **kw)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref) and torch.equal(fs, f_ref), w.name
        yr, fr = oracle.ssd(x["x"], x["dt"], x["A"], x["B"], x["C"], w.nheads, w.ngroups,
                            D=x["D"], z=x["z"], dt_bias=x["dt_bias"], dt_softplus=True,
                            h0=x["h0"])
        ey, es = norm_err(to_np(y), yr), norm_err(to_np(fs), fr)
        print(f"noalloc {w.name}: y {ey:.2e} state {es:.2e}", flush=True)
        assert ey <= TOL["bf16"] and es <= TOL["bf16"]


def test_noalloc_refuses_sizes_beyond_the_scratch(ssm):
    dev = torch.device("cuda:0")
    cap = ssm.ssm_ssd_scratch_bytes()
    # batch 16, L 65536, N 128, one group: far more workspace than the scratch
    assert ssm.ssm_ssd_workspace_size(16, 65536, 1, 128) > cap
    x = torch.empty((16, 64, 65536), dtype=torch.bfloat16, device=dev)
    dt = torch.empty((16, 1, 65536), dtype=torch.bfloat16, device=dev)
    B = torch.empty((16, 128, 65536), dtype=torch.bfloat16, device=dev)
    A = torch.full((1,), -1.0, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    with pytest.raises(ssm.SelscanError, match="SSM_E_SHAPE"):
        ssm.ssm_ssd_fwd_noalloc(x, dt, A, B, B, 1, 1, y)
