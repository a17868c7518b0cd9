"""Uncached (cold-start) scoring: the cache formula evaluated per candidate,
then the weighted sum (LIME summary page, Table 10, "Uncached global"),
against the oracle on the same seeded inputs (sampled candidates for the
large workloads: each candidate's score depends on its own id and user)."""
import numpy as np
import pytest
import torch

import oracle.lime_oracle as O
import workloads as W
from parity_utils import assert_close, cache_inputs, dev, host_f64, ids_for

pytestmark = pytest.mark.gpu
SAMPLE = 16384


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import decoupled_linear_link_amd as lib
    return lib


@pytest.mark.parametrize("name", ["tiny", "ctr", "long", "large_m", "lifelong"])
def test_uncached_scoring(L, name):
    w = W.workload(name)
    ci = cache_inputs(name, stress=True)
    lp = W.links_pers(w, stress=True)
    ids, coff = ids_for(name), W.candidate_offsets(w)
    sc = W.scale_for(w)
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = L.cand_score_uncached(dev(ci["items"]), dev(ci["link_keys"]), dev(lp), dev(ids), dev(coff),
                                phi=w.phi, scale=sc, bad_id_count=bad)
    torch.cuda.synchronize()
    total = len(ids)
    sel = np.arange(total) if total <= SAMPLE else np.sort(np.random.default_rng(2).choice(total, SAMPLE, replace=False))
    users = np.searchsorted(coff, sel, side="right") - 1
    sub_off = W.offsets_from_lengths(np.bincount(users, minlength=w.B))
    uniq, inv = np.unique(ids[sel], return_inverse=True)
    ref, nb = O.cand_score_uncached(ci["items"][uniq], ci["link_keys"], sc, w.phi, lp, inv, sub_off)
    assert nb == 0 and int(bad.item()) == 0
    assert_close(host_f64(out[torch.from_numpy(sel).cuda()]), ref, w.dtype, f"uncached[{name}]")


@pytest.mark.parametrize("phi", ["softmax", "silu_mean"])
def test_uncached_ragged_users_bad_ids(L, phi):
    rng = np.random.default_rng(41)
    # (the matrix-core shapes take their heads in groups whose keys fit
    # LDS: 64, 256, 8 in four groups, 32, 256, 8 and 64, 128, 4 in two)
    for dt, B, ell, d, H, n in (("bf16", 21, 32, 64, 2, 300), ("bf16", 9, 32, 128, 4, 100),
                                ("f32", 5, 7, 48, 3, 60), ("bf16", 6, 64, 256, 8, 50),
                                ("bf16", 7, 32, 256, 8, 40), ("bf16", 5, 64, 128, 4, 70)):
        counts = rng.integers(0, 30, size=B)
        counts[1] = 0
        coff = W.offsets_from_lengths(counts)
        items = W.as_storage(rng.standard_normal((n, d)).astype(np.float32), dt)
        keys = W.as_storage(rng.standard_normal((H, ell, d)).astype(np.float32), dt)
        lp = W.as_storage(rng.standard_normal((B, ell, d)).astype(np.float32), dt)
        ids = rng.integers(0, n, size=int(coff[-1]))
        ids[::11] = -1
        ids[5::13] = n
        bad = torch.zeros(1, dtype=torch.int32, device="cuda")
        out = L.cand_score_uncached(dev(items), dev(keys), dev(lp), dev(ids), dev(coff), phi=phi,
                                    scale=0.25, bad_id_count=bad)
        torch.cuda.synchronize()
        ref, nb = O.cand_score_uncached(items, keys, 0.25, phi, lp, ids, coff)
        assert int(bad.item()) == nb > 0
        got = host_f64(out)
        assert np.all(got[(ids < 0) | (ids >= n)] == 0)
        assert_close(got, ref, dt, f"uncached {dt} {B,ell,d,H} {phi}")


def test_uncached_equals_cached_path(L):
    """Uncached scores equal scores from a GPU-built cache up to the cache's
    bf16 rounding."""
    w = W.workload("ctr")
    ci = cache_inputs("ctr", stress=True)
    lp = dev(W.links_pers(w, stress=True))
    ids, coff = dev(ids_for("ctr")), dev(W.candidate_offsets(w))
    items, keys = dev(ci["items"]), dev(ci["link_keys"])
    a = L.cand_score_uncached(items, keys, lp, ids, coff, phi=w.phi)
    b = L.cand_score(L.qk_cache_build(items, keys, phi=w.phi), lp, ids, coff)
    torch.cuda.synchronize()
    assert_close(host_f64(a), host_f64(b), "bf16", "uncached vs cached")
