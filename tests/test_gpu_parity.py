"""Parity of the HIP path (through the C ABI) with the CPU oracle on the
same seeded inputs.  Small workloads are compared in full; the large ones on
samples the oracle can compute one by one (users, items, candidates are
independent of each other, so a sample is exact).  Bar: max|err| <= tol *
max|ref| with tol 1e-4 (float32) and 2e-2 (bf16)."""
import numpy as np
import pytest
import torch

import oracle.lime_oracle as O
import workloads as W
from parity_utils import (assert_close, cache_inputs, dev, dev_weights, host_f64, ids_for,
                          synthetic_cache, user_inputs)

pytestmark = pytest.mark.gpu

ALL = ["tiny", "ctr", "long", "large_m", "lifelong"]
SAMPLE = 65536


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import decoupled_linear_link_amd as lib
    return lib


def _sample(n, k=SAMPLE, seed=0):
    if n <= k:
        return np.arange(n)
    return np.sort(np.random.default_rng(seed).choice(n, k, replace=False))


def _oracle_scores(cache_st, lp_st, ids, coff, sel, n_items):
    """Oracle scores of the sampled candidates `sel` (sorted) only."""
    B = len(coff) - 1
    users = np.searchsorted(coff, sel, side="right") - 1
    sub_off = W.offsets_from_lengths(np.bincount(users, minlength=B))
    sid = ids[sel]
    ok = (sid >= 0) & (sid < n_items)
    uniq, inv = np.unique(sid[ok], return_inverse=True)
    remap = np.full(len(sid), -1, dtype=np.int64)
    remap[ok] = inv
    return O.cand_score(cache_st[uniq], lp_st, remap, sub_off, n_items=len(uniq))


# ------------------------------------------------------------ candidate scoring

@pytest.mark.parametrize("name", ALL)
def test_cand_score(L, name):
    w = W.workload(name)
    cache = synthetic_cache(name)
    lp = W.links_pers(w, stress=True)
    ids, coff = ids_for(name), W.candidate_offsets(w)
    print(f"cand_score {name}: total_M={len(ids)} n_items={w.n_items}", flush=True)
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = L.cand_score(dev(cache), dev(lp), dev(ids), dev(coff), bad_id_count=bad)
    torch.cuda.synchronize()
    sel = _sample(len(ids))
    ref, nbad = _oracle_scores(cache, lp, ids, coff, sel, w.n_items)
    assert nbad == 0 and int(bad.item()) == 0
    assert_close(host_f64(out[torch.from_numpy(sel).cuda()]), ref, w.dtype, f"cand_score[{name}]")


def test_cand_score_bad_ids_and_ragged_users(L):
    w = W.workload("ctr")
    cache = synthetic_cache("ctr")
    lp = W.links_pers(w, stress=True)
    rng = np.random.default_rng(5)
    counts = rng.integers(0, 70, size=w.B)
    counts[[0, 7]] = 0
    coff = W.offsets_from_lengths(counts)
    ids = rng.integers(0, w.n_items, size=int(coff[-1]))
    ids[::97] = -5
    ids[13::101] = w.n_items
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = L.cand_score(dev(cache), dev(lp), dev(ids), dev(coff), bad_id_count=bad)
    torch.cuda.synchronize()
    ref, nbad = _oracle_scores(cache, lp, ids, coff, np.arange(len(ids)), w.n_items)
    assert int(bad.item()) == nbad > 0
    got = host_f64(out)
    assert np.all(got[(ids < 0) | (ids >= w.n_items)] == 0)
    assert_close(got, ref, "bf16", "cand_score ragged/bad ids")


@pytest.mark.parametrize("ell,H", [(32, 1), (32, 4), (64, 2), (64, 8)])
def test_cand_score_bf16_ragged_users(L, ell, H):
    """Users whose candidate ranges start and end inside 16-candidate tiles,
    single-candidate and empty users, a partial last tile."""
    rng = np.random.default_rng(9 + ell + H)
    B, d, n = 37, 32 * H, 500
    counts = rng.integers(0, 40, size=B)
    counts[[3, 4, 5]] = [1, 0, 1]
    coff = W.offsets_from_lengths(counts)
    cache = W.as_storage(rng.random((n, H, ell)).astype(np.float32) / ell, "bf16")
    lp = W.as_storage(rng.standard_normal((B, ell, d)).astype(np.float32), "bf16")
    ids = rng.integers(0, n, size=int(coff[-1]))
    ids[::53] = n + 7
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = L.cand_score(dev(cache), dev(lp), dev(ids), dev(coff), bad_id_count=bad)
    torch.cuda.synchronize()
    ref, nbad = O.cand_score(cache, lp, ids, coff)
    assert int(bad.item()) == nbad
    assert_close(host_f64(out), ref, "bf16", f"cand_score bf16 ragged ell={ell} H={H}")


def test_cand_score_f32_small_odd_shapes(L):
    rng = np.random.default_rng(6)
    for B, ell, d, H, n in ((3, 5, 32, 2, 40), (2, 1, 64, 4, 7), (4, 33, 48, 3, 100)):
        cache = rng.random((n, H, ell)).astype(np.float32)
        lp = rng.standard_normal((B, ell, d)).astype(np.float32)
        coff = W.offsets_from_lengths(rng.integers(0, 9, size=B))
        ids = rng.integers(0, n, size=int(coff[-1]))
        out = L.cand_score(dev(cache), dev(lp), dev(ids), dev(coff))
        torch.cuda.synchronize()
        ref, _ = O.cand_score(cache, lp, ids, coff)
        if len(ids):
            assert_close(host_f64(out), ref, "f32", f"cand_score f32 {B,ell,d,H}")


# ------------------------------------------------------------ QK cache

@pytest.mark.parametrize("stress", [False, True])
@pytest.mark.parametrize("name", ALL)
def test_qk_cache_build(L, name, stress):
    w = W.workload(name)
    ci = cache_inputs(name, stress)
    scale = W.scale_for(w)
    print(f"qk_cache_build {name} stress={stress}: n_items={w.n_items}", flush=True)
    cache = L.qk_cache_build(dev(ci["items"]), dev(ci["link_keys"]), phi=w.phi, scale=scale)
    torch.cuda.synchronize()
    sel = _sample(w.n_items)
    ref = O.qk_cache_build(ci["items"][sel], ci["link_keys"], scale, w.phi)
    got = host_f64(cache[torch.from_numpy(sel).cuda()])
    assert_close(got, ref, w.dtype, f"qk_cache[{name}]")


@pytest.mark.parametrize("phi", ["softmax", "silu_mean"])
def test_qk_cache_build_odd_shapes(L, phi):
    rng = np.random.default_rng(7)
    for dt in ("f32", "bf16"):
        for n, d, H, ell in ((1, 8, 1, 1), (77, 40, 3, 5), (300, 64, 2, 33), (129, 256, 8, 64),
                                (77, 128, 4, 32), (1000, 64, 2, 32), (65, 256, 8, 32), (200, 128, 4, 64)):
            items = W.as_storage(rng.standard_normal((n, d)).astype(np.float32), dt)
            keys = W.as_storage(rng.standard_normal((H, ell, d)).astype(np.float32), dt)
            cache = L.qk_cache_build(dev(items), dev(keys), phi=phi, scale=0.3)
            torch.cuda.synchronize()
            ref = O.qk_cache_build(items, keys, 0.3, phi)
            assert_close(host_f64(cache), ref, dt, f"qk_cache {dt} {n,d,H,ell}")


@pytest.mark.parametrize("shape", [(256, 8, 64), (128, 4, 32), (64, 2, 32)])
def test_qk_cache_build_persistent_partial_tail(L, shape):
    """The matrix-core cache build with several item tiles per workgroup and
    a partial last tile (rows past the catalogue are neither read nor
    written): three and a bit rounds of 64- or 128-item tiles over a
    256-slot grid, checked against the oracle on the last rows and a
    sample, both phi."""
    d, H, ell = shape
    rng = np.random.default_rng(11)
    n = 3 * 256 * 128 + 77
    items = W.as_storage((rng.standard_normal((n, d)) * d ** -0.5).astype(np.float32), "bf16")
    keys = W.as_storage(rng.standard_normal((H, ell, d)).astype(np.float32), "bf16")
    sel = np.unique(np.concatenate([_sample(n, 2048, seed=3), np.arange(n - 300, n)]))
    for phi in ("softmax", "silu_mean"):
        print(f"qk_cache persistent tail n={n} d={d} H={H} ell={ell} {phi}", flush=True)
        cache = L.qk_cache_build(dev(items), dev(keys), phi=phi, scale=32 ** -0.5)
        torch.cuda.synchronize()
        ref = O.qk_cache_build(items[sel], keys, 32 ** -0.5, phi)
        got = host_f64(cache[torch.from_numpy(sel).cuda()])
        assert_close(got, ref, "bf16", f"qk_cache tail {shape} {phi}")


# ------------------------------------------------------------ user side

def _users_for(w, off):
    if w.B <= 256 and int(off[-1]) <= 20000:
        return list(range(w.B))
    lens = np.diff(off)
    longest = int(np.argmax(lens))
    other = int(np.random.default_rng(1).integers(0, w.B))
    return sorted({longest, other})


@pytest.mark.parametrize("name", ALL)
def test_xor_fwd(L, name):
    w = W.workload(name)
    ui = user_inputs(name)
    off = ui["hist_offsets"]
    print(f"xor_fwd {name}: B={w.B} total_N={int(off[-1])} layers={w.layers}", flush=True)
    lp, _ = L.xor_fwd(dev(ui["links_ctx"]), dev(ui["hist"]), dev(off), dev_weights(ui["weights"]),
                      heads=w.heads, phi=w.phi, scale=W.scale_for(w), max_N=int(np.diff(off).max()))
    torch.cuda.synchronize()
    users = _users_for(w, off)
    ref, _ = O.xor_fwd(ui["links_ctx"], ui["hist"], off, ui["weights"], w.heads, W.scale_for(w),
                       w.phi, users=users)
    assert_close(host_f64(lp)[users], ref, w.dtype, f"L^P[{name}]")


@pytest.mark.parametrize("case", ["streaming_d128", "streaming_d64", "resident_d64"])
def test_xor_fwd_rows_far_from_zero_mean(L, case):
    """Rows whose values sit far from zero relative to their spread (a
    per-row offset of 30-100 times the spread, on the context links and the
    history): the LayerNorm statistics must not lose the spread to
    cancellation.  Covers the LN of the fused attention kernel and of its
    link projection (streaming, d <= 128) and the user-resident kernel.  One
    layer: between layers the streaming path keeps the residual stream in
    bf16, whose rounding of rows this far from zero is not what is tested."""
    rng = np.random.default_rng(77)
    if case == "streaming_d128":
        B, ell, d, H, lens, max_n = 4, 32, 128, 4, [600, 0, 1500, 77], None
    elif case == "streaming_d64":
        B, ell, d, H, lens, max_n = 3, 32, 64, 2, [900, 31, 2], 4096
    else:
        B, ell, d, H, lens, max_n = 5, 32, 64, 2, [50, 0, 13, 1, 40], None
    off = W.offsets_from_lengths(lens)
    spread = 0.05

    def rows(n):
        mag = rng.uniform(30, 100, size=(n, 1)) * spread
        sign = np.where(rng.random((n, 1)) < 0.5, -1.0, 1.0)
        return (sign * mag + spread * rng.standard_normal((n, d))).astype(np.float32)

    lc = W.as_storage(rows(B * ell).reshape(B, ell, d), "bf16")
    hs = W.as_storage(rows(int(off[-1])), "bf16")
    ws = [{k: W.as_storage((rng.standard_normal(sh) * sh[1] ** -0.5).astype(np.float32), "bf16")
           for k, sh in (("w_qkv", (3 * d, d)), ("w_o", (d, d)), ("w_gate", (d, d)), ("w_up", (d, d)),
                         ("w_down", (d, d)))}]
    scale = (d // H) ** -0.5
    n_launch, plan = L.xor_fwd_plan(torch.bfloat16, B, ell, d, H, 1, d, int(off[-1]),
                                    max_n or int(max(lens)))
    assert (n_launch == 1) == (case == "resident_d64"), plan
    for phi in ("softmax", "silu_mean"):
        lp, ho = L.xor_fwd(dev(lc), dev(hs), dev(off), dev_weights(ws), heads=H, phi=phi, scale=scale,
                           max_N=max_n, want_hist=True)
        torch.cuda.synchronize()
        ref, href = O.xor_fwd(lc, hs, off, ws, H, scale, phi)
        assert_close(host_f64(lp), ref, "bf16", f"L^P far-from-zero rows {case} {phi}")
        assert_close(host_f64(ho), np.concatenate(href), "bf16", f"hist_out far-from-zero rows {case} {phi}")


@pytest.mark.parametrize("name", ["tiny", "ctr"])
@pytest.mark.parametrize("phi", ["softmax", "silu_mean"])
def test_xor_fwd_both_phis_with_history_out(L, name, phi):
    w = W.workload(name)
    ui = user_inputs(name, stress=True)
    off = ui["hist_offsets"]
    lp, ho = L.xor_fwd(dev(ui["links_ctx"]), dev(ui["hist"]), dev(off), dev_weights(ui["weights"]),
                       heads=w.heads, phi=phi, scale=W.scale_for(w), want_hist=True)
    torch.cuda.synchronize()
    ref, href = O.xor_fwd(ui["links_ctx"], ui["hist"], off, ui["weights"], w.heads, W.scale_for(w), phi)
    assert_close(host_f64(lp), ref, w.dtype, f"L^P[{name},{phi}]")
    assert_close(host_f64(ho), np.concatenate(href), w.dtype, f"hist_out[{name},{phi}]")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("phi", ["softmax", "silu_mean"])
def test_xor_fwd_ragged_empty_and_odd_shapes(L, dt, phi):
    """Ragged lengths including empty and single-row histories, ell not a
    multiple of 8, several splits per user, d_ff != d."""
    rng = np.random.default_rng(8)
    for B, ell, d, H, layers, dff, lens in (
            (5, 3, 32, 1, 2, 64, [0, 1, 700, 2, 1500]),
            (3, 32, 64, 2, 1, 32, [1100, 0, 5]),
            (2, 64, 256, 8, 1, 256, [130, 2049]),
            (6, 32, 64, 2, 2, 64, [0, 1, 77, 2, 1500, 33]),
            (4, 64, 128, 4, 2, 128, [17, 0, 640, 5])):
        off = W.offsets_from_lengths(lens)
        lc = W.as_storage(rng.standard_normal((B, ell, d)).astype(np.float32), dt)
        hs = W.as_storage((rng.standard_normal((int(off[-1]), d)) * 0.5).astype(np.float32), dt)
        ws = []
        for _ in range(layers):
            ws.append({k: W.as_storage((rng.standard_normal(s) * s[1] ** -0.5).astype(np.float32), dt)
                       for k, s in (("w_qkv", (3 * d, d)), ("w_o", (d, d)), ("w_gate", (dff, d)),
                                    ("w_up", (dff, d)), ("w_down", (d, dff)))})
        scale = (d // H) ** -0.5
        lp, ho = L.xor_fwd(dev(lc), dev(hs), dev(off), dev_weights(ws), heads=H, phi=phi, scale=scale,
                           max_N=int(max(lens)), want_hist=True)
        torch.cuda.synchronize()
        ref, href = O.xor_fwd(lc, hs, off, ws, H, scale, phi)
        assert_close(host_f64(lp), ref, dt, f"L^P odd {B,ell,d,H} {dt} {phi}")
        assert_close(host_f64(ho), np.concatenate(href), dt, f"hist_out odd {B,ell,d,H} {dt} {phi}")


@pytest.mark.parametrize("ell", [32, 64])
@pytest.mark.parametrize("want_hist", [False, True])
def test_xor_fwd_d256_many_users(L, ell, want_hist):
    """d = 256 with many users: the link rows' Q, K, V are projected once
    per (user, head) and every split of the user reads them; 37 users with
    ragged lengths (empty, single-row, and lengths around the split size)
    put users at every offset of a split group.  Two layers: a full one,
    then the last one links-only (without hist_out) or full (with it)."""
    rng = np.random.default_rng(11 + ell)
    B, d, H, layers = 37, 256, 8, 2
    lens = [int(x) for x in rng.integers(0, 300, B)]
    lens[0], lens[5], lens[17] = 0, 1, 64
    off = W.offsets_from_lengths(lens)
    lc = W.as_storage(rng.standard_normal((B, ell, d)).astype(np.float32), "bf16")
    hs = W.as_storage((rng.standard_normal((int(off[-1]), d)) * 0.5).astype(np.float32), "bf16")
    ws = [{k: W.as_storage((rng.standard_normal(s) * s[1] ** -0.5).astype(np.float32), "bf16")
           for k, s in (("w_qkv", (3 * d, d)), ("w_o", (d, d)), ("w_gate", (d, d)), ("w_up", (d, d)),
                        ("w_down", (d, d)))} for _ in range(layers)]
    scale = (d // H) ** -0.5
    print(f"xor_fwd d=256 B={B} ell={ell} total_N={int(off[-1])} want_hist={want_hist}", flush=True)
    for phi in ("softmax", "silu_mean"):
        lp, ho = L.xor_fwd(dev(lc), dev(hs), dev(off), dev_weights(ws), heads=H, phi=phi, scale=scale,
                           max_N=int(max(lens)), want_hist=want_hist)
        torch.cuda.synchronize()
        ref, href = O.xor_fwd(lc, hs, off, ws, H, scale, phi)
        assert_close(host_f64(lp), ref, "bf16", f"L^P d=256 B={B} ell={ell} {phi}")
        if want_hist:
            assert_close(host_f64(ho), np.concatenate(href), "bf16", f"hist_out d=256 B={B} ell={ell} {phi}")


def test_xor_fwd_max_n_too_small_stays_in_bounds(L):
    """max_N below the real maximum breaks the precondition: the call must
    still finish without fault and leave finite outputs."""
    w = W.workload("ctr")
    ui = user_inputs("ctr")
    off = ui["hist_offsets"]
    lp, _ = L.xor_fwd(dev(ui["links_ctx"]), dev(ui["hist"]), dev(off), dev_weights(ui["weights"]),
                      heads=w.heads, phi=w.phi, max_N=1)
    torch.cuda.synchronize()
    assert torch.isfinite(lp.float()).all()


@pytest.mark.parametrize("phi", ["softmax", "silu_mean"])
def test_xor_fwd_resident_and_streaming_paths(L, phi):
    """Small histories run on the user-resident kernel (one workgroup per user,
    all layers); a large max_N forces the streaming kernels.  Both match the
    oracle, on ragged users including empty and single-row histories."""
    rng = np.random.default_rng(10)
    for B, ell, d, H, layers, lens in ((7, 32, 64, 2, 3, [0, 1, 50, 13, 100, 64, 31]),
                                       (3, 64, 64, 2, 2, [5, 0, 40]),
                                       (4, 32, 128, 4, 2, [10, 0, 60, 3])):
        off = W.offsets_from_lengths(lens)
        lc = W.as_storage(rng.standard_normal((B, ell, d)).astype(np.float32), "bf16")
        hs = W.as_storage((rng.standard_normal((int(off[-1]), d)) * 0.5).astype(np.float32), "bf16")
        ws = [{k: W.as_storage((rng.standard_normal(s) * s[1] ** -0.5).astype(np.float32), "bf16")
               for k, s in (("w_qkv", (3 * d, d)), ("w_o", (d, d)), ("w_gate", (d, d)),
                            ("w_up", (d, d)), ("w_down", (d, d)))} for _ in range(layers)]
        scale = (d // H) ** -0.5
        ref, href = O.xor_fwd(lc, hs, off, ws, H, scale, phi)
        outs = []
        for max_n in (int(max(lens)), 4096):
            lp, ho = L.xor_fwd(dev(lc), dev(hs), dev(off), dev_weights(ws), heads=H, phi=phi,
                               scale=scale, max_N=max_n, want_hist=True)
            torch.cuda.synchronize()
            assert_close(host_f64(lp), ref, "bf16", f"L^P {B,ell,d,H} max_N={max_n} {phi}")
            assert_close(host_f64(ho), np.concatenate(href), "bf16", f"hist {B,ell,d,H} max_N={max_n} {phi}")
            outs.append(host_f64(lp))
        assert_close(outs[0], outs[1], "bf16", "resident vs streaming")


# ------------------------------------------------------------ whole path

@pytest.mark.parametrize("name", ["tiny", "ctr"])
def test_end_to_end(L, name):
    """user encoder -> QK cache -> candidate scores, all on the GPU, against
    the oracle's own pipeline on the same inputs."""
    w = W.workload(name)
    ui, ci = user_inputs(name), cache_inputs(name)
    ids, coff = ids_for(name), W.candidate_offsets(w)
    sc = W.scale_for(w)
    lp, _ = L.xor_fwd(dev(ui["links_ctx"]), dev(ui["hist"]), dev(ui["hist_offsets"]),
                      dev_weights(ui["weights"]), heads=w.heads, phi=w.phi, scale=sc)
    cache = L.qk_cache_build(dev(ci["items"]), dev(ci["link_keys"]), phi=w.phi, scale=sc)
    out = L.cand_score(cache, lp, dev(ids), dev(coff))
    torch.cuda.synchronize()
    lp_ref, _ = O.xor_fwd(ui["links_ctx"], ui["hist"], ui["hist_offsets"], ui["weights"], w.heads, sc, w.phi)
    uniq, inv = np.unique(ids, return_inverse=True)
    c_ref = O.qk_cache_build(ci["items"][uniq], ci["link_keys"], sc, w.phi)
    ref, _ = O.cand_score(c_ref, lp_ref, inv, coff)
    assert_close(host_f64(out), ref, w.dtype, f"end-to-end[{name}]")


def test_repeat_runs_are_bitwise_identical(L):
    w = W.workload("ctr")
    ui, ci = user_inputs("ctr"), cache_inputs("ctr")
    args = (dev(ui["links_ctx"]), dev(ui["hist"]), dev(ui["hist_offsets"]), dev_weights(ui["weights"]))
    a, _ = L.xor_fwd(*args, heads=w.heads, phi=w.phi)
    b, _ = L.xor_fwd(*args, heads=w.heads, phi=w.phi)
    items, keys = dev(ci["items"]), dev(ci["link_keys"])
    c1 = L.qk_cache_build(items, keys, phi=w.phi)
    c2 = L.qk_cache_build(items, keys, phi=w.phi)
    ids, coff = dev(ids_for("ctr")), dev(W.candidate_offsets(w))
    o1 = L.cand_score(c1, a, ids, coff)
    o2 = L.cand_score(c1, a, ids, coff)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(c1.view(torch.int16), c2.view(torch.int16))
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
