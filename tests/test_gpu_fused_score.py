"""lime_xor_fwd_score (the user side and the scoring of each user's own
candidates in one call) against lime_xor_fwd followed by lime_cand_score:
links, scores, history rows and the bad-id count must be bit-identical.
Covers the user-resident path, where the scoring runs inside the user-side
kernel (ell = 32 and 64 with d = 64, ell = 64 with d = 128), the streaming path and
the float32 generic path, where the call runs the user side's kernels and
then the scoring kernel; ragged and
empty candidate lists, out-of-range ids, both phi.  One case is also checked
against the oracle."""
import numpy as np
import pytest
import torch

import oracle.lime_oracle as O
import workloads as W
from parity_utils import assert_close, dev, dev_weights, host_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import decoupled_linear_link_amd as lib
    return lib


# (dtype, ell, d, heads, layers, history lengths, candidate counts, max_N hint)
CASES = [
    ("bf16", 32, 64, 2, 2, [50, 0, 17, 64, 3], [0, 1, 17, 40, 16], None),     # user-resident
    ("bf16", 64, 128, 4, 2, [32, 5, 0], [33, 0, 16], None),                   # user-resident, ell = 64
    ("bf16", 64, 64, 2, 3, [30, 1, 0, 32], [40, 17, 0, 100], None),           # user-resident, ell = 64, d = 64
    ("bf16", 32, 128, 4, 1, [300, 40, 0, 9], [7, 0, 50, 1], None),            # streaming
    ("bf16", 32, 64, 2, 2, [50, 3, 20], [20, 20, 5], 4096),                   # streaming (max_N hint)
    ("f32", 8, 32, 1, 1, [10, 0, 7], [3, 5, 0], None),                        # generic
]


RESIDENT = {0, 1, 2}  # cases planned on the user-resident path (scored inside the kernel)


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _inputs(seed, dt, ell, d, layers, lens, counts, n_items=300):
    rng = np.random.default_rng(seed)
    B = len(lens)
    off = W.offsets_from_lengths(lens)
    lc = W.as_storage(rng.standard_normal((B, ell, d)).astype(np.float32), dt)
    hs = W.as_storage((rng.standard_normal((int(off[-1]), d)) * 0.7).astype(np.float32), dt)
    ws = [{k: W.as_storage((rng.standard_normal(s) * s[1] ** -0.5).astype(np.float32), dt)
           for k, s in (("w_qkv", (3 * d, d)), ("w_o", (d, d)), ("w_gate", (d, d)),
                        ("w_up", (d, d)), ("w_down", (d, d)))} for _ in range(layers)]
    coff = W.offsets_from_lengths(counts)
    ids = rng.integers(0, n_items, size=int(coff[-1])).astype(np.int64)
    if len(ids) > 4:
        ids[1] = -3
        ids[len(ids) // 2] = n_items
    return off, lc, hs, ws, coff, ids, rng


@pytest.mark.parametrize("phi", ["softmax", "silu_mean"])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_fused_equals_the_two_calls(L, case, phi):
    dt, ell, d, H, layers, lens, counts, hint = CASES[case]
    off, lc, hs, ws, coff, ids, rng = _inputs(900 + case, dt, ell, d, layers, lens, counts)
    n_items = 300
    items = W.as_storage(rng.standard_normal((n_items, d)).astype(np.float32), dt)
    keys = W.as_storage((rng.standard_normal((H, ell, d)) * d ** -0.5).astype(np.float32), dt)
    scale = (d // H) ** -0.5
    max_n = hint if hint is not None else max(lens)
    print(f"fused score case {case} {phi}: {dt} ell={ell} d={d} lens={lens} counts={counts}", flush=True)
    launches, plan = L.xor_fwd_plan(torch.bfloat16 if dt == "bf16" else torch.float32, len(lens), ell, d, H,
                                    layers, d, int(off[-1]), max_n)
    assert (launches == 1 and "user-resident" in plan) == (case in RESIDENT), plan
    cache = L.qk_cache_build(dev(items), dev(keys), phi=phi, scale=scale)
    args = (dev(lc), dev(hs) if hs.shape[0] else torch.empty((0, d), dtype=cache.dtype, device="cuda"),
            dev(off), dev_weights(ws))
    bad1 = torch.zeros(1, dtype=torch.int32, device="cuda")
    lp1, ho1 = L.xor_fwd(*args, heads=H, phi=phi, scale=scale, max_N=max_n, want_hist=True)
    out1 = L.cand_score(cache, lp1, dev(ids), dev(coff), bad_id_count=bad1)
    bad2 = torch.zeros(1, dtype=torch.int32, device="cuda")
    lp2, ho2, out2 = L.xor_fwd_score(*args, heads=H, cache=cache, cand_ids=dev(ids), cand_offsets=dev(coff),
                                     phi=phi, scale=scale, max_N=max_n, want_hist=True, bad_id_count=bad2)
    torch.cuda.synchronize()
    assert torch.equal(_bits(lp1), _bits(lp2)), "links_pers"
    assert torch.equal(_bits(ho1), _bits(ho2)), "hist_out"
    assert torch.equal(_bits(out1), _bits(out2)), "scores"
    assert int(bad1.item()) == int(bad2.item()) == (2 if len(ids) > 4 else 0)
    if case == 0:
        ref_lp, _ = O.xor_fwd(lc, hs, off, ws, H, scale, phi)
        ref, nbad = O.cand_score(O.qk_cache_build(items, keys, scale, phi), ref_lp, ids, coff)
        assert nbad == 2
        assert_close(host_f64(out2), ref, dt, f"fused scores against the oracle ({phi})")


def test_fused_without_candidates_and_twice_in_a_row(L):
    """total_M = 0 (links only), then a call with candidates on the same
    buffers, then a smaller one: each equals the two-call result."""
    dt, ell, d, H, layers = "bf16", 32, 64, 2, 2
    for k, counts in enumerate(([0, 0, 0], [30, 2, 17], [1, 0, 0])):
        off, lc, hs, ws, coff, ids, rng = _inputs(950, dt, ell, d, layers, [40, 12, 0], counts)
        cache = torch.from_numpy(rng.random((300, H, ell)).astype(np.float32) / ell).to(torch.bfloat16).cuda()
        args = (dev(lc), dev(hs), dev(off), dev_weights(ws))
        lp1, _ = L.xor_fwd(*args, heads=H, phi="silu_mean")
        out1 = L.cand_score(cache, lp1, dev(ids), dev(coff))
        lp2, _, out2 = L.xor_fwd_score(*args, heads=H, cache=cache, cand_ids=dev(ids), cand_offsets=dev(coff),
                                       phi="silu_mean")
        torch.cuda.synchronize()
        assert torch.equal(_bits(lp1), _bits(lp2)), f"links_pers, call {k}"
        assert out2.shape[0] == sum(counts)
        assert torch.equal(_bits(out1), _bits(out2)), f"scores, call {k}"


@pytest.mark.parametrize("name", ["ctr", "large_m"])
def test_fused_equals_the_two_calls_at_workload_size(L, name):
    """The bench's configuration (ctr: 256 users, 8,192 candidates, the
    user-resident path) and a streaming one (large-M users with a sample of
    their candidates): bit-identical to the two calls."""
    from parity_utils import cache_inputs, ids_for, user_inputs
    w = W.workload(name)
    ui, ci = user_inputs(name), cache_inputs(name)
    off = ui["hist_offsets"]
    scale = W.scale_for(w)
    ids, coff = ids_for(name), W.candidate_offsets(w)
    if name == "large_m":  # the first 4,096 candidates of every user
        per = np.minimum(np.diff(coff), 4096)
        ids = np.concatenate([ids[coff[b]:coff[b] + per[b]] for b in range(w.B)])
        coff = W.offsets_from_lengths(per)
    print(f"fused score at {name} size: B={w.B} candidates={len(ids)}", flush=True)
    cache = torch.empty((min(w.n_items, 1 << 20), w.heads, w.ell), dtype=torch.bfloat16, device="cuda")
    n_items = cache.shape[0]
    L.qk_cache_build(dev(ci["items"][:n_items]), dev(ci["link_keys"]), phi=w.phi, scale=scale, cache=cache)
    ids = np.where(ids < n_items, ids, ids % n_items)
    args = (dev(ui["links_ctx"]), dev(ui["hist"]), dev(off), dev_weights(ui["weights"]))
    max_n = int(np.diff(off).max())
    lp1, _ = L.xor_fwd(*args, heads=w.heads, phi=w.phi, scale=scale, max_N=max_n)
    out1 = L.cand_score(cache, lp1, dev(ids), dev(coff))
    lp2, _, out2 = L.xor_fwd_score(*args, heads=w.heads, cache=cache, cand_ids=dev(ids), cand_offsets=dev(coff),
                                   phi=w.phi, scale=scale, max_N=max_n)
    torch.cuda.synchronize()
    assert torch.equal(_bits(lp1), _bits(lp2)), "links_pers"
    assert torch.equal(_bits(out1), _bits(out2)), "scores"
