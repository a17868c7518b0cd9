"""Parity of the user-side variants through the C ABI with the CPU oracle:
LIME-MHA (links -> history only; history rows pass through) and
LIME-XOR+Window (history rows also attend their neighbours within the
window, one phi over the union).  Same bar as the other parity tests:
max|err| <= tol * max|ref| per output tensor, tol 1e-4 (float32) and 2e-2
(bf16).  Every path is covered: the generic kernels (float32, odd shapes,
windows wider than the matrix-core kernels serve), the user-resident
matrix-core kernel and the streaming matrix-core kernels."""
import numpy as np
import pytest
import torch

import oracle.lime_oracle as O
import workloads as W
from parity_utils import assert_close, dev, dev_weights, host_f64, user_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import decoupled_linear_link_amd as lib
    return lib


def _users(name, variant, off):
    """Users the oracle checks: all of them for the small workloads; for the
    large ones the longest and one other (LIME-MHA), or, for LIME-XOR+Window
    (whose oracle walks history rows one by one), the shortest and a second
    user: the last one in the packed history at long (equal lengths) and the
    longest at lifelong."""
    lens = np.diff(off)
    if name in ("tiny", "ctr"):
        return list(range(len(lens)))
    if variant == "xor_window":
        second = len(lens) - 1 if name == "long" else int(np.argmax(lens))
        return sorted({int(np.argmin(lens)), second})
    return sorted({int(np.argmax(lens)), int(np.random.default_rng(1).integers(0, len(lens)))})


@pytest.mark.parametrize("variant", ["mha", "xor_window"])
@pytest.mark.parametrize("name", ["tiny", "ctr", "long", "lifelong"])
def test_variant_on_workloads(L, name, variant):
    w = W.workload(name)
    ui = user_inputs(name)
    off = ui["hist_offsets"]
    sc = W.scale_for(w)
    print(f"xor_fwd variant={variant} {name}: B={w.B} total_N={int(off[-1])}", flush=True)
    lp, _ = L.xor_fwd(dev(ui["links_ctx"]), dev(ui["hist"]), dev(off), dev_weights(ui["weights"]),
                      heads=w.heads, phi=w.phi, scale=sc, max_N=int(np.diff(off).max()), variant=variant)
    torch.cuda.synchronize()
    users = _users(name, variant, off)
    ref, _ = O.xor_fwd(ui["links_ctx"], ui["hist"], off, ui["weights"], w.heads, sc, w.phi,
                       users=users, variant=variant)
    assert_close(host_f64(lp)[users], ref, w.dtype, f"L^P[{name},{variant}]")


@pytest.mark.parametrize("name", ["tiny", "ctr"])
@pytest.mark.parametrize("phi", ["softmax", "silu_mean"])
def test_window_both_phis_with_history_out(L, name, phi):
    w = W.workload(name)
    ui = user_inputs(name, stress=True)
    off = ui["hist_offsets"]
    sc = W.scale_for(w)
    lp, ho = L.xor_fwd(dev(ui["links_ctx"]), dev(ui["hist"]), dev(off), dev_weights(ui["weights"]),
                       heads=w.heads, phi=phi, scale=sc, want_hist=True, variant="xor_window")
    torch.cuda.synchronize()
    ref, href = O.xor_fwd(ui["links_ctx"], ui["hist"], off, ui["weights"], w.heads, sc, phi,
                          variant="xor_window")
    assert_close(host_f64(lp), ref, w.dtype, f"L^P[{name},{phi}]")
    assert_close(host_f64(ho), np.concatenate(href), w.dtype, f"hist_out[{name},{phi}]")


def _random_case(rng, B, ell, d, layers, dff, lens, dt):
    off = W.offsets_from_lengths(lens)
    lc = W.as_storage(rng.standard_normal((B, ell, d)).astype(np.float32), dt)
    hs = W.as_storage((rng.standard_normal((int(off[-1]), d)) * 0.7).astype(np.float32), dt)
    ws = [{k: W.as_storage((rng.standard_normal(s) * s[1] ** -0.5).astype(np.float32), dt)
           for k, s in (("w_qkv", (3 * d, d)), ("w_o", (d, d)), ("w_gate", (dff, d)),
                        ("w_up", (dff, d)), ("w_down", (d, dff)))} for _ in range(layers)]
    return off, lc, hs, ws


# (dtype, B, ell, d, heads, layers, d_ff, lengths, window, max_N hints)
# max_N = the real maximum gives the user-resident kernel where the rows fit;
# 4096 forces the streaming kernels.  Windows 17 (ell 32) and 40 (ell 64)
# are wider than the matrix-core kernels serve: generic kernels.
WINDOW_CASES = [
    ("f32", 5, 3, 32, 1, 2, 64, [0, 1, 70, 2, 150], 2, (None,)),
    ("f32", 3, 8, 32, 2, 1, 32, [9, 0, 40], 4, (None,)),
    ("bf16", 7, 32, 64, 2, 2, 64, [0, 1, 50, 13, 100, 17, 31], 16, (None, 4096)),
    ("bf16", 4, 32, 64, 2, 2, 64, [3, 0, 90, 40], 5, (None, 4096)),
    ("bf16", 4, 32, 128, 4, 2, 128, [10, 0, 60, 33], 1, (None, 4096)),
    ("bf16", 3, 64, 64, 2, 2, 64, [5, 0, 40], 32, (None, 4096)),
    ("bf16", 3, 64, 128, 4, 1, 128, [70, 1, 9], 7, (None, 4096)),
    ("bf16", 2, 64, 256, 8, 1, 256, [130, 600], 32, (None,)),
    ("bf16", 3, 32, 256, 8, 1, 256, [300, 0, 45], 16, (None,)),
    ("bf16", 3, 32, 64, 2, 1, 64, [3, 80, 41], 17, (None,)),
    ("bf16", 2, 64, 128, 4, 1, 128, [90, 7], 40, (None,)),
]


@pytest.mark.parametrize("phi", ["softmax", "silu_mean"])
@pytest.mark.parametrize("case", range(len(WINDOW_CASES)))
def test_window_ragged_paths_and_widths(L, case, phi):
    dt, B, ell, d, H, layers, dff, lens, win, hints = WINDOW_CASES[case]
    rng = np.random.default_rng(100 + case)
    off, lc, hs, ws = _random_case(rng, B, ell, d, layers, dff, lens, dt)
    scale = (d // H) ** -0.5
    ref, href = O.xor_fwd(lc, hs, off, ws, H, scale, phi, variant="xor_window", window=win)
    for hint in hints:
        max_n = int(max(lens)) if hint is None else hint
        print(f"window case {case}: {dt} B={B} ell={ell} d={d} H={H} lens={lens} window={win} "
              f"max_N={max_n} {phi}", flush=True)
        lp, ho = L.xor_fwd(dev(lc), dev(hs), dev(off), dev_weights(ws), heads=H, phi=phi, scale=scale,
                           max_N=max_n, want_hist=True, variant="xor_window", window=win)
        torch.cuda.synchronize()
        assert_close(host_f64(lp), ref, dt, f"L^P window case {case} max_N={max_n}")
        assert_close(host_f64(ho), np.concatenate(href), dt, f"hist_out window case {case} max_N={max_n}")


MHA_CASES = [
    ("f32", 4, 3, 32, 1, 3, 64, [0, 1, 200, 9], (None,)),
    ("bf16", 7, 32, 64, 2, 3, 64, [0, 1, 50, 13, 100, 64, 31], (None, 4096)),
    ("bf16", 3, 64, 128, 4, 2, 128, [70, 0, 9], (None, 4096)),
    ("bf16", 2, 64, 256, 8, 2, 256, [130, 1000], (None,)),
]


@pytest.mark.parametrize("phi", ["softmax", "silu_mean"])
@pytest.mark.parametrize("case", range(len(MHA_CASES)))
def test_mha_ragged_and_paths(L, case, phi):
    dt, B, ell, d, H, layers, dff, lens, hints = MHA_CASES[case]
    rng = np.random.default_rng(200 + case)
    off, lc, hs, ws = _random_case(rng, B, ell, d, layers, dff, lens, dt)
    scale = (d // H) ** -0.5
    ref, _ = O.xor_fwd(lc, hs, off, ws, H, scale, phi, variant="mha")
    for hint in hints:
        max_n = int(max(lens)) if hint is None else hint
        print(f"mha case {case}: {dt} B={B} ell={ell} d={d} H={H} lens={lens} max_N={max_n} {phi}",
              flush=True)
        lp, ho = L.xor_fwd(dev(lc), dev(hs), dev(off), dev_weights(ws), heads=H, phi=phi, scale=scale,
                           max_N=max_n, variant="mha")
        torch.cuda.synchronize()
        assert ho is None
        assert_close(host_f64(lp), ref, dt, f"L^P mha case {case} max_N={max_n}")


def test_mha_first_layer_equals_xor(L):
    """With one layer the link rows of LIME-MHA and LIME-XOR are the same
    computation; the two kernels' results agree bit for bit."""
    w = W.workload("ctr")
    ui = user_inputs("ctr")
    args = (dev(ui["links_ctx"]), dev(ui["hist"]), dev(ui["hist_offsets"]), dev_weights(ui["weights"][:1]))
    a, _ = L.xor_fwd(*args, heads=w.heads, phi=w.phi)
    b, _ = L.xor_fwd(*args, heads=w.heads, phi=w.phi, variant="mha")
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
