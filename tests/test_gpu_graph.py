"""The hot path captured in a HIP graph: every replay must reproduce the
eager result, with eager work and synchronisations between the replays.
Both user-side paths are covered (user-resident and streaming), as three
calls and as the bench's step (cache build, then lime_xor_fwd_score)."""
import numpy as np
import pytest
import torch

import workloads as W
from parity_utils import cache_inputs, dev, dev_weights, ids_for, user_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import decoupled_linear_link_amd as lib
    return lib


@pytest.mark.parametrize("combined", [False, True])
@pytest.mark.parametrize("max_n_hint", [None, 4096])
def test_graph_replays_match_eager(L, max_n_hint, combined):
    w = W.workload("ctr")
    ui, ci = user_inputs("ctr"), cache_inputs("ctr")
    off = ui["hist_offsets"]
    max_n = int(np.diff(off).max()) if max_n_hint is None else max_n_hint
    lc, hs, ho = dev(ui["links_ctx"]), dev(ui["hist"]), dev(off)
    wts = dev_weights(ui["weights"])
    items, keys = dev(ci["items"]), dev(ci["link_keys"])
    ids, coff = dev(ids_for("ctr")), dev(W.candidate_offsets(w))
    dt = torch.bfloat16
    lp = torch.empty_like(lc)
    cache = torch.empty((w.n_items, w.heads, w.ell), dtype=dt, device="cuda")
    out = torch.empty((ids.shape[0], w.d), dtype=dt, device="cuda")
    need = L.xor_fwd_workspace_size(dt, w.B, w.ell, w.d, w.heads, w.dff, hs.shape[0], max_n)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")

    def step():
        if combined:
            L.qk_cache_build(items, keys, phi=w.phi, cache=cache)
            L.xor_fwd_score(lc, hs, ho, wts, heads=w.heads, cache=cache, cand_ids=ids, cand_offsets=coff,
                            phi=w.phi, max_N=max_n, links_pers=lp, workspace=ws, out=out)
            return
        L.xor_fwd(lc, hs, ho, wts, heads=w.heads, phi=w.phi, max_N=max_n, links_pers=lp, workspace=ws)
        L.qk_cache_build(items, keys, phi=w.phi, cache=cache)
        L.cand_score(cache, lp, ids, coff, out=out)

    print(f"graph replays max_N hint={max_n_hint} combined={combined}", flush=True)
    step()
    torch.cuda.synchronize()
    ref = (lp.clone(), cache.clone(), out.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        # eager work between replays that overwrites every output
        lp.zero_()
        cache.fill_(1.0)
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want, name in zip((lp, cache, out), ref, ("links_pers", "cache", "scores")):
            assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"replay {rep}: {name}"
