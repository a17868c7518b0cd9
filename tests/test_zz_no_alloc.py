"""lime_xor_fwd_noalloc (the user side with the library's own per-GPU scratch
array as its workspace) against lime_xor_fwd with a caller workspace, through
the C ABI: two calls in a row on the same GPU, the second with a smaller
input, so it runs on what the first left in the scratch array.  The two entry
points run the same kernels, so their outputs must be identical bit for bit;
a call that needs more workspace than the array holds is rejected before
anything is enqueued."""
import numpy as np
import pytest
import torch

import workloads as W
from parity_utils import dev, dev_weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import decoupled_linear_link_amd as lib
    return lib


def _run_both(L, w, hist_out):
    ui = W.user_inputs(w)
    off = ui["hist_offsets"]
    lc, hs, ho = dev(ui["links_ctx"]), dev(ui["hist"]), dev(off)
    wts = dev_weights(ui["weights"])
    max_n = int(np.diff(off).max())
    dt = torch.bfloat16
    need = L.xor_fwd_workspace_size(dt, w.B, w.ell, w.d, w.heads, w.dff, hs.shape[0], max_n)
    assert 0 < need <= L.NOALLOC_SCRATCH_BYTES, need
    # the caller workspace starts as 0xFF bytes (bf16 NaN patterns): neither
    # entry point may depend on what its workspace holds on entry
    ws = torch.full((need,), 255, dtype=torch.uint8, device="cuda")
    lp_a, lp_b = torch.empty_like(lc), torch.empty_like(lc)
    h_a = torch.empty_like(hs) if hist_out else None
    h_b = torch.empty_like(hs) if hist_out else None
    L.xor_fwd(lc, hs, ho, wts, heads=w.heads, phi=w.phi, max_N=max_n, links_pers=lp_a, hist_out=h_a,
              workspace=ws)
    L.xor_fwd_noalloc(lc, hs, ho, wts, heads=w.heads, phi=w.phi, max_N=max_n, links_pers=lp_b, hist_out=h_b)
    torch.cuda.synchronize()
    assert torch.isfinite(lp_b.float()).all()
    assert torch.equal(lp_a.view(torch.int16), lp_b.view(torch.int16)), "links_pers differ"
    if hist_out:
        assert torch.equal(h_a.view(torch.int16), h_b.view(torch.int16)), "hist_out differ"
    return need


def test_noalloc_matches_workspace_call_twice(L):
    # first call: the large-M user side (16 users x 1,024 rows, d = 128,
    # the streaming path with the fused attention), with hist_out
    big = W.workload("large_m")
    print(f"noalloc call 1: large_m user side B={big.B} N={big.N} d={big.d}", flush=True)
    n1 = _run_both(L, big, hist_out=True)
    # second call, smaller, on what the first left in the scratch array:
    # lifelong-shaped layers (ell = 64, d = 256, 8 heads) over 3 ragged users
    small = W.workload("lifelong").replace(B=3, N=(300, 1500), layers=2)
    print(f"noalloc call 2: lifelong-shaped B={small.B} N={small.N} d={small.d}", flush=True)
    n2 = _run_both(L, small, hist_out=False)
    assert n2 < n1


def test_noalloc_rejects_calls_beyond_the_scratch_array(L):
    # the long workload needs more workspace than the array: rejected on the
    # host with LIME_ERR_WORKSPACE, nothing enqueued (the tensors below are
    # never read)
    w = W.workload("long")
    total_n = w.B * w.N
    need = L.xor_fwd_workspace_size(torch.bfloat16, w.B, w.ell, w.d, w.heads, w.dff, total_n, w.N)
    assert need > L.NOALLOC_SCRATCH_BYTES
    lc = torch.zeros((w.B, w.ell, w.d), dtype=torch.bfloat16, device="cuda")
    hs = torch.zeros((total_n, w.d), dtype=torch.bfloat16, device="cuda")
    ho = torch.arange(0, total_n + 1, w.N, dtype=torch.int64, device="cuda")
    d = w.d
    wts = [{"w_qkv": torch.zeros((3 * d, d), dtype=torch.bfloat16, device="cuda"),
            "w_o": torch.zeros((d, d), dtype=torch.bfloat16, device="cuda"),
            "w_gate": torch.zeros((d, d), dtype=torch.bfloat16, device="cuda"),
            "w_up": torch.zeros((d, d), dtype=torch.bfloat16, device="cuda"),
            "w_down": torch.zeros((d, d), dtype=torch.bfloat16, device="cuda")}]
    lp = torch.full_like(lc, 7.0)
    with pytest.raises(L.LimeError) as e:
        L.xor_fwd_noalloc(lc, hs, ho, wts, heads=w.heads, phi=w.phi, max_N=w.N, links_pers=lp)
    assert e.value.status == 3
    torch.cuda.synchronize()
    assert (lp.float() == 7.0).all(), "a rejected call wrote its output"
