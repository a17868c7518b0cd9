"""The C ABI without a GPU: the library loads, exports every symbol the
header declares, and rejects every host-visible argument error before
enqueueing anything (no call here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lime.h")


@pytest.fixture(scope="module")
def L():
    import decoupled_linear_link_amd as pkg
    return pkg


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lime_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_three_calls():
    fns = declared_functions()
    for f in ("lime_xor_fwd", "lime_qk_cache_build", "lime_cand_score",
              "lime_xor_fwd_workspace_size", "lime_status_string", "lime_last_error"):
        assert f in fns


def test_library_exports_every_declared_symbol(L):
    for f in declared_functions():
        assert hasattr(L.lib, f), f"{f} not exported"
    assert sorted(L.EXPORTED) == declared_functions()


def test_library_is_gfx950_only(L):
    # the build targets exactly one architecture
    from decoupled_linear_link_amd import build
    assert build.ARCH == "gfx950"
    assert "--offload-arch=gfx950" in build.compile_flags()


def test_status_strings(L):
    for code, name in L.STATUS.items():
        assert L.lib.lime_status_string(code).decode() == name


# fake, never dereferenced device addresses (aligned and misaligned)
P = 0x7F0000000000
PM = P + 2


def _xor_args(**kw):
    a = dict(dtype=1, phi=1, scale=0.17, B=2, ell=32, d=64, heads=2, layers=1, d_ff=64,
             links_ctx=P, hist=P, off=P, total_N=100, max_N=50, w=None, lp=P, ho=None,
             ws=P, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return a


def _call_xor(L, a):
    if a["w"] is None:
        arr = (L.LayerWeights * max(1, a["layers"]))()
        for i in range(max(1, a["layers"])):
            arr[i] = L.LayerWeights(P, P, P, P, P)
        a["w"] = arr
    return L.lib.lime_xor_fwd(a["dtype"], a["phi"], a["scale"], a["B"], a["ell"], a["d"], a["heads"],
                              a["layers"], a["d_ff"], a["links_ctx"], a["hist"], a["off"],
                              a["total_N"], a["max_N"], a["w"], a["lp"], a["ho"], a["ws"],
                              a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), 1), (dict(phi=5), 1), (dict(scale=float("nan")), 1), (dict(B=0), 1),
    (dict(ell=0), 1), (dict(d=65), 1), (dict(heads=0), 1), (dict(layers=0), 1),
    (dict(total_N=-1), 1), (dict(links_ctx=None), 1), (dict(off=None), 1), (dict(lp=None), 1),
    (dict(hist=None), 1), (dict(links_ctx=PM), 1), (dict(ho=PM), 1),
    (dict(ell=300), 2), (dict(d=96, heads=1), 2), (dict(d=60, heads=2), 2), (dict(d_ff=60), 2),
    (dict(total_N=(1 << 34) + 1), 2),
    (dict(ws=None), 3), (dict(ws_bytes=1024), 3), (dict(ws=P + 16), 3),
])
def test_xor_fwd_rejects(L, kw, code):
    assert _call_xor(L, _xor_args(**kw)) == code
    assert L.lib.lime_last_error().decode() != ""


def _call_variant(L, variant, window, a):
    arr = (L.LayerWeights * max(1, a["layers"]))()
    for i in range(max(1, a["layers"])):
        arr[i] = L.LayerWeights(P, P, P, P, P)
    a["w"] = arr
    return L.lib.lime_xor_fwd_variant(variant, window, a["dtype"], a["phi"], a["scale"], a["B"], a["ell"],
                                      a["d"], a["heads"], a["layers"], a["d_ff"], a["links_ctx"], a["hist"],
                                      a["off"], a["total_N"], a["max_N"], a["w"], a["lp"], a["ho"], a["ws"],
                                      a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("variant,window,kw,code", [
    (3, 0, {}, 1), (-1, 0, {}, 1),            # bad variant
    (0, 4, {}, 1), (1, 2, {}, 1),             # window given where none applies
    (1, 0, dict(ho=P), 1),                    # LIME-MHA never writes history rows
    (2, 0, {}, 1), (2, -3, {}, 1), (2, 5000, {}, 1),
    (2, 16, dict(ws=None), 3), (1, 0, dict(ws_bytes=64), 3), (2, 16, dict(d=65), 1),
])
def test_xor_fwd_variant_rejects(L, variant, window, kw, code):
    a = _xor_args(**kw)
    assert _call_variant(L, variant, window, a) == code
    assert L.lib.lime_last_error().decode() != ""


def test_xor_fwd_null_weight(L):
    arr = (L.LayerWeights * 2)()
    arr[0] = L.LayerWeights(P, P, P, P, P)
    arr[1] = L.LayerWeights(P, None, P, P, P)
    assert _call_xor(L, _xor_args(layers=2, w=arr)) == 1


def test_workspace_size_is_monotone_and_zero_on_bad_sizes(L):
    f = L.lib.lime_xor_fwd_workspace_size
    a = f(1, 64, 32, 128, 4, 128, 64 * 4096, 4096)
    b = f(1, 64, 32, 128, 4, 128, 64 * 8192, 8192)
    assert 0 < a < b
    assert f(1, 0, 32, 128, 4, 128, 100, 10) == 0
    assert f(9, 4, 32, 128, 4, 128, 100, 10) == 0
    assert f(1, 8, 64, 256, 8, 256, (1 << 34) + 1, 16384) == 0  # beyond the row cap


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=3), 1), (dict(phi=9), 1), (dict(n=-1), 1), (dict(ell=0), 1), (dict(keys=None), 1),
    (dict(items=None), 1), (dict(cache=PM), 1), (dict(ell=257), 2), (dict(d=12), 2),
    (dict(scale=float("inf")), 1),
])
def test_qk_cache_build_rejects(L, kw, code):
    a = dict(dtype=1, phi=0, scale=0.5, n=10, d=64, H=2, ell=32, items=P, keys=P, cache=P)
    a.update(kw)
    st = L.lib.lime_qk_cache_build(a["dtype"], a["phi"], a["scale"], a["n"], a["d"], a["H"], a["ell"],
                                   a["items"], a["keys"], a["cache"], None)
    assert st == code


def test_qk_cache_build_empty_is_noop(L):
    # n_items = 0 returns before any launch
    assert L.lib.lime_qk_cache_build(1, 0, 0.5, 0, 64, 2, 32, None, P, None, None) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), 1), (dict(B=0), 1), (dict(d=65), 1), (dict(M=-3), 1), (dict(lp=None), 1),
    (dict(coff=None), 1), (dict(ids=None), 1), (dict(out=None), 1), (dict(cache=None), 1),
    (dict(ids=PM), 1), (dict(bad=P + 2), 1), (dict(ell=300), 2), (dict(d=96, H=1), 2),
])
def test_cand_score_rejects(L, kw, code):
    a = dict(dtype=1, B=2, ell=32, d=64, H=2, cache=P, n=100, lp=P, ids=P, coff=P, M=10, out=P, bad=None)
    a.update(kw)
    st = L.lib.lime_cand_score(a["dtype"], a["B"], a["ell"], a["d"], a["H"], a["cache"], a["n"], a["lp"],
                               a["ids"], a["coff"], a["M"], a["out"], a["bad"], None)
    assert st == code


def test_cand_score_empty_is_noop(L):
    assert L.lib.lime_cand_score(1, 2, 32, 64, 2, P, 100, P, None, P, 0, None, None, None) == 0


def test_product_path_does_not_use_the_oracle():
    """The package never imports the oracle and has no CPU fallback."""
    pkg = os.path.join(ROOT, "decoupled_linear_link_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in src.replace("oracle is", ""), f


@pytest.mark.parametrize("kw,skw,code", [
    ({}, dict(ids=None), 1), ({}, dict(cache=None), 1), ({}, dict(out=None), 1), ({}, dict(out=PM), 1),
    ({}, dict(bad=P + 2), 1), ({}, dict(M=-1), 1), ({}, dict(coff=None), 1),
    (dict(phi=5), {}, 1), (dict(layers=0), {}, 1), (dict(lp=None), {}, 1), (dict(ell=300), {}, 2),
    (dict(ws=None), {}, 3), (dict(ws_bytes=1024), {}, 3),
])
def test_xor_fwd_score_rejects(L, kw, skw, code):
    """Errors of either half (the user side or the scoring) return before
    anything is enqueued."""
    a = _xor_args(**kw)
    s = dict(cache=P, n=100, ids=P, coff=P, M=10, out=P, bad=None)
    s.update(skw)
    arr = (L.LayerWeights * max(1, a["layers"]))()
    for i in range(max(1, a["layers"])):
        arr[i] = L.LayerWeights(P, P, P, P, P)
    st = L.lib.lime_xor_fwd_score(a["dtype"], a["phi"], a["scale"], a["B"], a["ell"], a["d"], a["heads"],
                                  a["layers"], a["d_ff"], a["links_ctx"], a["hist"], a["off"], a["total_N"],
                                  a["max_N"], arr, a["lp"], a["ho"], a["ws"], a["ws_bytes"], s["cache"], s["n"],
                                  s["ids"], s["coff"], s["M"], s["out"], s["bad"], None)
    assert st == code
    assert L.lib.lime_last_error().decode() != ""


def test_binding_rejects_host_tensors(L):
    """Host tensors never reach the C ABI (their pointers are not device
    addresses)."""
    import torch
    bf = torch.bfloat16
    lp = torch.zeros((2, 32, 64), dtype=bf)
    ids = torch.zeros(4, dtype=torch.int64)
    coff = torch.tensor([0, 2, 4], dtype=torch.int64)
    with pytest.raises(ValueError, match="device tensor"):
        L.cand_score(torch.zeros((10, 2, 32), dtype=bf), lp, ids, coff)
    with pytest.raises(ValueError, match="device tensor"):
        L.qk_cache_build(torch.zeros((10, 64), dtype=bf), torch.zeros((2, 32, 64), dtype=bf))
    with pytest.raises(ValueError, match="device tensor"):
        L.xor_fwd(lp, torch.zeros((4, 64), dtype=bf), coff, [], heads=2)
