"""The Python binding rejects tensors whose shape, dtype, device or size does
not match what the kernels will index, before anything is enqueued (the C ABI
sees only pointers, so these checks can only be made here)."""
import pytest
import torch

pytestmark = pytest.mark.gpu

B, ELL, D, H, N, NI, M = 2, 32, 64, 2, 40, 100, 24


@pytest.fixture(scope="module")
def args():
    import decoupled_linear_link_amd as L
    torch.manual_seed(0)
    dt = torch.bfloat16
    c = lambda *s, dtype=dt: torch.randn(*s, device="cuda").to(dtype)  # noqa: E731
    w = [{"w_qkv": c(3 * D, D), "w_o": c(D, D), "w_gate": c(D, D), "w_up": c(D, D), "w_down": c(D, D)}]
    return dict(L=L, lc=c(B, ELL, D), hist=c(N, D),
                off=torch.tensor([0, 15, N], dtype=torch.int64, device="cuda"), w=w,
                items=c(NI, D), keys=c(H, ELL, D), cache=c(NI, H, ELL),
                ids=torch.randint(0, NI, (M,), device="cuda"),
                coff=torch.tensor([0, 10, M], dtype=torch.int64, device="cuda"))


def _bad_weights(a, key, shape):
    w = [dict(a["w"][0])]
    w[0][key] = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
    return w


def test_good_arguments_run(args):
    a, L = args, args["L"]
    lp, _ = L.xor_fwd(a["lc"], a["hist"], a["off"], a["w"], heads=H)
    L.cand_score(a["cache"], lp, a["ids"], a["coff"])
    torch.cuda.synchronize()


@pytest.mark.parametrize("key,shape", [("w_qkv", (D, D)), ("w_o", (D, 2 * D)), ("w_up", (2 * D, D)),
                                       ("w_down", (D, 2 * D)), ("w_qkv", (3 * D, D + 8))])
def test_xor_fwd_rejects_weight_shapes(args, key, shape):
    a, L = args, args["L"]
    with pytest.raises(ValueError):
        L.xor_fwd(a["lc"], a["hist"], a["off"], _bad_weights(a, key, shape), heads=H)


@pytest.mark.parametrize("which", ["links_pers_short", "links_pers_host", "links_pers_f32", "hist_out_short",
                                   "ws_small", "ws_f32", "ws_host"])
def test_xor_fwd_rejects_outputs_and_workspace(args, which):
    a, L = args, args["L"]
    kw = {}
    if which == "links_pers_short":
        kw["links_pers"] = torch.empty((B - 1, ELL, D), dtype=torch.bfloat16, device="cuda")
    elif which == "links_pers_host":
        kw["links_pers"] = torch.empty((B, ELL, D), dtype=torch.bfloat16)
    elif which == "links_pers_f32":
        kw["links_pers"] = torch.empty((B, ELL, D), dtype=torch.float32, device="cuda")
    elif which == "hist_out_short":
        kw["hist_out"] = torch.empty((N - 1, D), dtype=torch.bfloat16, device="cuda")
    elif which == "ws_small":
        kw["workspace"] = torch.empty(256, dtype=torch.uint8, device="cuda")
    elif which == "ws_f32":
        kw["workspace"] = torch.empty(1 << 20, dtype=torch.float32, device="cuda")
    elif which == "ws_host":
        kw["workspace"] = torch.empty(1 << 24, dtype=torch.uint8)
    with pytest.raises((ValueError, TypeError)):
        L.xor_fwd(a["lc"], a["hist"], a["off"], a["w"], heads=H, **kw)


@pytest.mark.parametrize("which", ["out_short", "out_f32", "out_host", "bad_i64", "bad_host"])
def test_cand_score_rejects_outputs(args, which):
    a, L = args, args["L"]
    lp = torch.zeros((B, ELL, D), dtype=torch.bfloat16, device="cuda")
    kw = {}
    if which == "out_short":
        kw["out"] = torch.empty((M - 1, D), dtype=torch.bfloat16, device="cuda")
    elif which == "out_f32":
        kw["out"] = torch.empty((M, D), dtype=torch.float32, device="cuda")
    elif which == "out_host":
        kw["out"] = torch.empty((M, D), dtype=torch.bfloat16)
    elif which == "bad_i64":
        kw["bad_id_count"] = torch.zeros(1, dtype=torch.int64, device="cuda")
    elif which == "bad_host":
        kw["bad_id_count"] = torch.zeros(1, dtype=torch.int32)
    with pytest.raises((ValueError, TypeError)):
        L.cand_score(a["cache"], lp, a["ids"], a["coff"], **kw)
    with pytest.raises((ValueError, TypeError)):
        L.xor_fwd_score(a["lc"], a["hist"], a["off"], a["w"], heads=H, cache=a["cache"], cand_ids=a["ids"],
                        cand_offsets=a["coff"], **kw)
    with pytest.raises((ValueError, TypeError)):
        L.cand_score_uncached(a["items"], a["keys"], lp, a["ids"], a["coff"], **kw)


@pytest.mark.parametrize("which", ["cache_short", "cache_f32", "codes_short", "qscale_short"])
def test_cache_build_rejects_outputs(args, which):
    a, L = args, args["L"]
    with pytest.raises((ValueError, TypeError)):
        if which == "cache_short":
            L.qk_cache_build(a["items"], a["keys"], cache=torch.empty((NI - 1, H, ELL), dtype=torch.bfloat16,
                                                                      device="cuda"))
        elif which == "cache_f32":
            L.qk_cache_build(a["items"], a["keys"], cache=torch.empty((NI, H, ELL), dtype=torch.float32,
                                                                      device="cuda"))
        elif which == "codes_short":
            L.qk_cache_build_i8(a["items"], a["keys"], codes=torch.empty((NI, H, ELL - 1), dtype=torch.int8,
                                                                         device="cuda"))
        else:
            L.qk_cache_build_i8(a["items"], a["keys"], qscale=torch.empty((NI,), dtype=torch.float32,
                                                                          device="cuda"))
