"""Int8 QK cache and scoring from it (LIME summary page, Tables 10 and 12:
int8 lookup with dequantisation).  Codes are an integer decision taken in
float32 on both sides: they must match the oracle's exactly except where the
oracle's scaled value lies within 1e-3 of a rounding tie, where they may
differ by one.  Scales match to float32 precision (1e-5 relative);
dequantised rows and scores meet the usual tolerance."""
import numpy as np
import pytest
import torch

import oracle.lime_oracle as O
import workloads as W
from parity_utils import assert_close, cache_inputs, dev, host_f64, ids_for

pytestmark = pytest.mark.gpu
SAMPLE = 65536


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import decoupled_linear_link_amd as lib
    return lib


def _check_codes(codes_gpu, scale_gpu, ref_cache):
    q_ref, s_ref = O.quantize_i8(ref_cache)
    sr = s_ref.astype(np.float64)
    assert np.all(np.abs(scale_gpu.astype(np.float64) - sr) <= 1e-5 * sr + 1e-30), "scales"
    w32 = ref_cache.astype(np.float32)
    m = np.abs(w32).max(-1, keepdims=True)
    x = w32 * np.where(m > 0, np.float32(127) / m, np.float32(0))
    near_tie = np.abs(np.abs(x - np.floor(x)) - 0.5) < 1e-3
    diff = np.abs(codes_gpu.astype(int) - q_ref.astype(int))
    assert np.all(diff <= 1), "codes differ by more than one"
    assert np.all(diff[~near_tie] == 0), f"{int((diff[~near_tie] > 0).sum())} codes differ away from ties"


@pytest.mark.parametrize("name", ["tiny", "ctr", "long", "large_m", "lifelong"])
def test_int8_cache_build(L, name):
    w = W.workload(name)
    print(f"int8 cache build {name}: {w.n_items} items", flush=True)
    ci = cache_inputs(name, stress=True)
    sc = W.scale_for(w)
    codes, qs = L.qk_cache_build_i8(dev(ci["items"]), dev(ci["link_keys"]), phi=w.phi, scale=sc)
    torch.cuda.synchronize()
    n = w.n_items
    sel = np.arange(n) if n <= SAMPLE else np.sort(np.random.default_rng(0).choice(n, SAMPLE, replace=False))
    ref = O.qk_cache_build(ci["items"][sel], ci["link_keys"], sc, w.phi)
    idx = torch.from_numpy(sel).cuda()
    _check_codes(codes[idx].cpu().numpy(), qs[idx].cpu().numpy(), ref)


@pytest.mark.parametrize("phi", ["softmax", "silu_mean"])
def test_int8_cache_build_odd_shapes(L, phi):
    rng = np.random.default_rng(31)
    for dt in ("f32", "bf16"):
        for n, d, H, ell in ((77, 40, 3, 5), (300, 64, 2, 32), (129, 256, 8, 64), (65, 128, 4, 32)):
            items = W.as_storage(rng.standard_normal((n, d)).astype(np.float32), dt)
            keys = W.as_storage(rng.standard_normal((H, ell, d)).astype(np.float32), dt)
            codes, qs = L.qk_cache_build_i8(dev(items), dev(keys), phi=phi, scale=0.3)
            torch.cuda.synchronize()
            _check_codes(codes.cpu().numpy(), qs.cpu().numpy(), O.qk_cache_build(items, keys, 0.3, phi))


@pytest.mark.parametrize("name", ["tiny", "ctr", "large_m", "lifelong"])
def test_int8_scoring(L, name):
    """Scores from int8 codes and scales built by the oracle from a seeded
    stand-in cache."""
    w = W.workload(name)
    base = np.abs(W.normal(w.seed, "cache_stand_in", (w.n_items, w.heads, w.ell), 1.0 / w.ell))
    q, s = O.quantize_i8(base)
    lp = W.links_pers(w, stress=True)
    ids, coff = ids_for(name), W.candidate_offsets(w)
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = L.cand_score_i8(dev(q), dev(s), dev(lp), dev(ids), dev(coff), bad_id_count=bad)
    torch.cuda.synchronize()
    total = len(ids)
    sel = np.arange(total) if total <= SAMPLE else np.sort(np.random.default_rng(1).choice(total, SAMPLE, replace=False))
    users = np.searchsorted(coff, sel, side="right") - 1
    sub_off = W.offsets_from_lengths(np.bincount(users, minlength=w.B))
    uniq, inv = np.unique(ids[sel], return_inverse=True)
    ref, nb = O.cand_score_i8(q[uniq], s[uniq], lp, inv, sub_off)
    assert nb == 0 and int(bad.item()) == 0
    assert_close(host_f64(out[torch.from_numpy(sel).cuda()]), ref, w.dtype, f"int8 scores[{name}]")


def test_int8_end_to_end_ctr(L):
    """GPU int8 cache -> GPU int8 scores vs the oracle's int8 pipeline."""
    w = W.workload("ctr")
    ci = cache_inputs("ctr", stress=True)
    sc = W.scale_for(w)
    lp = W.links_pers(w, stress=True)
    ids, coff = ids_for("ctr"), W.candidate_offsets(w)
    codes, qs = L.qk_cache_build_i8(dev(ci["items"]), dev(ci["link_keys"]), phi=w.phi, scale=sc)
    out = L.cand_score_i8(codes, qs, dev(lp), dev(ids), dev(coff))
    torch.cuda.synchronize()
    uniq, inv = np.unique(ids, return_inverse=True)
    q, s = O.quantize_i8(O.qk_cache_build(ci["items"][uniq], ci["link_keys"], sc, w.phi))
    ref, _ = O.cand_score_i8(q, s, lp, inv, coff)
    assert_close(host_f64(out), ref, "bf16", "int8 end to end")
    # and close to the float cache's scores (within the int8 step)
    f_ref, _ = O.cand_score(O.qk_cache_build(ci["items"][uniq], ci["link_keys"], sc, w.phi), lp, inv, coff)
    assert_close(host_f64(out), f_ref, "bf16", "int8 vs float scores", tol=5e-2)
