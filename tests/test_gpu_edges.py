"""Degenerate and limit cases through the C ABI, against the oracle:
every history empty (total_N = 0) on every user-side path and variant, a
single user, the largest shapes the header accepts (ell = 256; d = 1024 with
d_ff = 4096), and scoring with a single candidate and users without
candidates.  Same bar as the other parity tests."""
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


def _case(seed, B, ell, d, layers, dff, lens, dt):
    rng = np.random.default_rng(seed)
    off = W.offsets_from_lengths(lens)
    lc = W.as_storage(rng.standard_normal((B, ell, d)).astype(np.float32), dt)
    hs = W.as_storage((rng.standard_normal((int(off[-1]), d)) * 0.7).astype(np.float32), dt)
    ws = [{k: W.as_storage((rng.standard_normal(s) * s[1] ** -0.5).astype(np.float32), dt)
           for k, s in (("w_qkv", (3 * d, d)), ("w_o", (d, d)), ("w_gate", (dff, d)),
                        ("w_up", (dff, d)), ("w_down", (d, dff)))} for _ in range(layers)]
    return off, lc, hs, ws


def _hist_dev(hs, d, dt):
    if hs.shape[0] == 0:
        return torch.empty((0, d), dtype=torch.float32 if dt == "f32" else torch.bfloat16, device="cuda")
    return dev(hs)


# (dtype, B, ell, d, heads, layers, max_N hints): generic; resident and
# streaming matrix-core; d = 256 streaming
EMPTY_CASES = [("f32", 3, 8, 32, 2, 2, (None,)), ("bf16", 4, 32, 64, 2, 2, (None, 4096)),
               ("bf16", 2, 64, 256, 8, 1, (None,))]


@pytest.mark.parametrize("variant", ["xor", "mha", "xor_window"])
@pytest.mark.parametrize("case", range(len(EMPTY_CASES)))
def test_every_history_empty(L, case, variant):
    dt, B, ell, d, H, layers, hints = EMPTY_CASES[case]
    off, lc, hs, ws = _case(300 + case, B, ell, d, layers, d, [0] * B, dt)
    scale = (d // H) ** -0.5
    ref, _ = O.xor_fwd(lc, hs, off, ws, H, scale, "softmax", variant=variant)
    for hint in hints:
        max_n = 0 if hint is None else hint
        print(f"empty histories case {case} {variant} max_N={max_n}", flush=True)
        lp, _ = L.xor_fwd(dev(lc), _hist_dev(hs, d, dt), dev(off), dev_weights(ws), heads=H, phi="softmax",
                          scale=scale, max_N=max_n, variant=variant)
        torch.cuda.synchronize()
        assert_close(host_f64(lp), ref, dt, f"L^P empty histories case {case} {variant} max_N={max_n}")


@pytest.mark.parametrize("dt,ell,d,H", [("f32", 5, 32, 1), ("bf16", 32, 64, 2), ("bf16", 64, 128, 4),
                                        ("bf16", 32, 256, 8)])
def test_single_user(L, dt, ell, d, H):
    off, lc, hs, ws = _case(400 + ell + d, 1, ell, d, 2, d, [777], dt)
    scale = (d // H) ** -0.5
    ref, href = O.xor_fwd(lc, hs, off, ws, H, scale, "silu_mean")
    lp, ho = L.xor_fwd(dev(lc), dev(hs), dev(off), dev_weights(ws), heads=H, phi="silu_mean", scale=scale,
                       want_hist=True)
    torch.cuda.synchronize()
    assert_close(host_f64(lp), ref, dt, f"L^P single user {dt} {ell} {d} {H}")
    assert_close(host_f64(ho), href[0], dt, f"hist_out single user {dt} {ell} {d} {H}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(2, 256, 512, 4, 1024, [40, 3]), (1, 8, 1024, 8, 4096, [10])])
def test_largest_accepted_shapes(L, dt, shape):
    """ell = 256 (the limit) and d = 1024 with d_ff = 4096 (the limits), on the
    generic kernels (d_h = 128)."""
    B, ell, d, H, dff, lens = shape
    off, lc, hs, ws = _case(500 + ell, B, ell, d, 1, dff, lens, dt)
    scale = (d // H) ** -0.5
    for phi in ("softmax", "silu_mean"):
        ref, href = O.xor_fwd(lc, hs, off, ws, H, scale, phi)
        lp, ho = L.xor_fwd(dev(lc), dev(hs), dev(off), dev_weights(ws), heads=H, phi=phi, scale=scale,
                           want_hist=True)
        torch.cuda.synchronize()
        assert_close(host_f64(lp), ref, dt, f"L^P largest {shape[:5]} {dt} {phi}")
        assert_close(host_f64(ho), np.concatenate(href), dt, f"hist largest {shape[:5]} {dt} {phi}")
    # the QK cache and scoring at the same shape (a seeded L^P, so both sides
    # score the same input)
    rng = np.random.default_rng(7)
    items = W.as_storage(rng.standard_normal((37, d)).astype(np.float32), dt)
    keys = W.as_storage((rng.standard_normal((H, ell, d)) * d ** -0.5).astype(np.float32), dt)
    lp_in = W.as_storage(rng.standard_normal((B, ell, d)).astype(np.float32), dt)
    cache = L.qk_cache_build(dev(items), dev(keys), phi="softmax", scale=scale)
    ids = rng.integers(0, 37, size=11).astype(np.int64)
    coff = W.offsets_from_lengths([4, 7] if B == 2 else [11])
    out = L.cand_score(cache, dev(lp_in), dev(ids), dev(coff))
    torch.cuda.synchronize()
    c_ref = O.qk_cache_build(items, keys, scale, "softmax")
    assert_close(host_f64(cache), c_ref, dt, f"cache largest {dt}")
    s_ref, _ = O.cand_score(c_ref, lp_in, ids, coff)
    assert_close(host_f64(out), s_ref, dt, f"scores largest {dt}")


@pytest.mark.parametrize("dt,ell,d,H", [("f32", 6, 32, 2), ("bf16", 32, 64, 2), ("bf16", 64, 256, 8)])
def test_single_candidate_and_users_without_candidates(L, dt, ell, d, H):
    rng = np.random.default_rng(11)
    n = 50
    cache = W.as_storage(np.abs(rng.standard_normal((n, H, ell))).astype(np.float32) / ell, dt)
    lp = W.as_storage(rng.standard_normal((4, ell, d)).astype(np.float32), dt)
    for lens in ([0, 1, 0, 0], [0, 0, 0, 1], [1, 0, 0, 0]):
        coff = W.offsets_from_lengths(lens)
        ids = np.array([17], dtype=np.int64)
        out = L.cand_score(dev(cache), dev(lp), dev(ids), dev(coff))
        torch.cuda.synchronize()
        ref, _ = O.cand_score(cache, lp, ids, coff)
        assert_close(host_f64(out), ref, dt, f"single candidate {lens} {dt}")


@pytest.mark.parametrize("phi", ["softmax", "silu_mean"])
def test_streaming_splits_over_many_users(L, phi):
    """More users than the split plan scans in one pass (1024), ragged and
    partly empty histories, one user far longer than the rest (many splits
    against one), on the streaming kernels (a large max_N hint); the oracle
    checks users from both scan passes, the long user and empty ones."""
    rng = np.random.default_rng(21)
    B, ell, d, H = 1500, 32, 64, 2
    lens = rng.integers(0, 25, size=B)
    lens[::7] = 0
    lens[1234] = 3000
    off, lc, hs, ws = _case(600, B, ell, d, 1, d, lens.tolist(), "bf16")
    scale = (d // H) ** -0.5
    print(f"streaming splits: B={B} total_N={int(off[-1])} {phi}", flush=True)
    lp, ho = L.xor_fwd(dev(lc), dev(hs), dev(off), dev_weights(ws), heads=H, phi=phi, scale=scale,
                       max_N=4096, want_hist=True)
    torch.cuda.synchronize()
    users = [0, 1, 7, 500, 1023, 1024, 1025, 1234, 1400, B - 1]
    ref, href = O.xor_fwd(lc, hs, off, ws, H, scale, phi, users=users)
    assert_close(host_f64(lp)[users], ref, "bf16", f"L^P many users {phi}")
    hos = host_f64(ho)
    for u, hr in zip(users, href):
        if len(hr):
            assert_close(hos[off[u]:off[u + 1]], hr, "bf16", f"hist_out user {u} {phi}")


@pytest.mark.parametrize("max_n", [64, 4096])
def test_out_of_order_offsets_stay_in_bounds(L, max_n):
    """Offsets that break the prefix-sum precondition (decreasing, and
    summing past total_N) give unspecified outputs but must not fault: the
    user-resident kernel (max_N = 64) and the streaming kernels (4096), whose
    split plan then caps the splits.  The personalized links stay finite
    (rows outside a split never enter it, not even as 0 * nan); history rows
    that no split covers keep unspecified values, so hist_out is not
    checked."""
    B, ell, d, H = 4, 32, 64, 2
    off, lc, hs, ws = _case(700, B, ell, d, 2, d, [100, 100, 100, 100], "bf16")
    bad = np.array([0, 300, 100, 400, 400], dtype=np.int64)
    print(f"out-of-order offsets max_N={max_n}", flush=True)
    lp, ho = L.xor_fwd(dev(lc), dev(hs), dev(bad), dev_weights(ws), heads=H, phi="softmax",
                       max_N=max_n, want_hist=True)
    torch.cuda.synchronize()
    assert torch.isfinite(lp.float()).all()


@pytest.mark.parametrize("d,H,max_n", [(64, 2, 64), (64, 2, 4096), (128, 4, 4096), (256, 8, 4096)])
def test_non_finite_history_stays_with_its_user(L, d, H, max_n):
    """A user whose history holds non-finite values must not change other
    users' results: chunks that straddle user boundaries (lengths not
    multiples of 8) read the neighbour's rows and must mask them entirely.
    Users 0 and 2 are compared with the oracle; user 1 (nan and inf rows at
    both of its ends) is not checked."""
    lens = [37, 45, 50]
    off, lc, hs, ws = _case(800 + d, 3, 32, d, 2, d, lens, "bf16")
    bad = hs.copy()
    nan16, inf16 = np.uint16(0x7FC0), np.uint16(0x7F80)  # bf16 bit patterns
    bad[37] = nan16
    bad[38] = inf16
    bad[80] = inf16
    bad[81] = nan16
    scale = (d // H) ** -0.5
    print(f"non-finite neighbour d={d} max_N={max_n}", flush=True)
    lp, ho = L.xor_fwd(dev(lc), dev(bad), dev(off), dev_weights(ws), heads=H, phi="softmax", scale=scale,
                       max_N=max_n, want_hist=True)
    torch.cuda.synchronize()
    ref, href = O.xor_fwd(lc, hs, off, ws, H, scale, "softmax", users=[0, 2])
    got = host_f64(lp)
    assert_close(got[[0, 2]], ref, "bf16", f"L^P beside a non-finite user d={d} max_N={max_n}")
    hos = host_f64(ho)
    assert_close(hos[off[0]:off[1]], href[0], "bf16", f"hist_out user 0 d={d} max_N={max_n}")
    assert_close(hos[off[2]:off[3]], href[1], "bf16", f"hist_out user 2 d={d} max_N={max_n}")
