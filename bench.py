"""Benchmark of the LIME inference hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  lime_qk_cache_build (QK cache over the whole catalogue), then
  lime_xor_fwd_score  (user encoder over all B users and all layers, and the
                       scoring of all B*M candidates: lime_xor_fwd followed
                       by lime_cand_score in one call, one launch on the
                       user-resident path)
Inputs are resident in HBM before the timed region starts.  The step made of
the three separate calls is timed alongside (`ms_per_step_separate_calls`).

    python bench.py [--steps K] [--warmup W] [--workload ctr] [--no-cpu-baseline]

Prints ONE JSON line.  `value` = candidates scored per second of whole-step
time; users encoded/s and items cached/s are reported alongside.  The K
timed steps are captured in one HIP graph and replayed once (every kernel
of every step is a graph node; --no-graph launches them eagerly instead).  The `roofline` object is
for the kernel with the largest share of step time, its duration measured
with HIP events on the launch stream around a graph of K back-to-back calls
(per-call times are the median of 5 such graphs, the minimum alongside);
`scoring` has candidate scoring cold (each call after a 512 MiB write and a
512 MiB read that evict L2 and the Infinity Cache) and warm, for the
workload's ids and for a uniform-id control with no reuse; `cpu_baseline` is
the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="ctr")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="approximate CPU budget of the oracle baseline")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch the timed steps eagerly instead of replaying a HIP graph of one step")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip timing the int8 and uncached candidate-side variants")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (for HBM counter scaling)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards users and catalogue rows with no exchange, see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as W
    import decoupled_linear_link_amd as L

    w = W.workload(args.workload)
    dt = {"f32": torch.float32, "bf16": torch.bfloat16}[w.dtype]
    es = 4 if w.dtype == "f32" else 2
    scale = W.scale_for(w)

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    # ---- inputs, resident in HBM
    ui = W.user_inputs(w)
    ci = W.cache_inputs(w)
    ids = W.candidate_ids(w)
    coff = W.candidate_offsets(w)
    off = ui["hist_offsets"]
    total_N = int(off[-1])
    max_N = int(np.diff(off).max())
    lc, hs, hoff = dev(ui["links_ctx"]), dev(ui["hist"]), dev(off)
    wts = [{k: dev(v) for k, v in lw.items()} for lw in ui["weights"]]
    items, keys = dev(ci["items"]), dev(ci["link_keys"])
    ids_d, coff_d = dev(ids), dev(coff)
    lp = torch.empty_like(lc)
    cache = torch.empty((w.n_items, w.heads, w.ell), dtype=dt, device="cuda")
    out = torch.empty((len(ids), w.d), dtype=dt, device="cuda")
    ws_bytes = L.xor_fwd_workspace_size(dt, w.B, w.ell, w.d, w.heads, w.dff, total_N, max_N)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")

    def user(stream=None):
        L.xor_fwd(lc, hs, hoff, wts, heads=w.heads, phi=w.phi, scale=scale, max_N=max_N,
                  links_pers=lp, workspace=ws, stream=stream)

    def build(stream=None):
        L.qk_cache_build(items, keys, phi=w.phi, scale=scale, cache=cache, stream=stream)

    def score(stream=None):
        L.cand_score(cache, lp, ids_d, coff_d, out=out, stream=stream)

    def user_score(stream=None):
        L.xor_fwd_score(lc, hs, hoff, wts, heads=w.heads, cache=cache, cand_ids=ids_d, cand_offsets=coff_d,
                        phi=w.phi, scale=scale, max_N=max_N, links_pers=lp, workspace=ws, out=out,
                        stream=stream)

    def step():
        build()
        user_score()

    def step_separate():
        user()
        build()
        score()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    def capture(fn, reps):
        """A HIP graph of `reps` back-to-back calls of fn (kernels only, no
        allocation or memset inside)."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                fn()
        torch.cuda.synchronize()
        return g

    # one HIP graph holding exactly the K timed steps (every kernel of every
    # step is a node), so host launch costs do not pace the GPU
    graph = None if args.no_graph else capture(step, args.steps)
    if graph is not None:
        graph.replay()  # warm replay, outside the timed region
        torch.cuda.synchronize()

    # ---- timed region: exactly K steps
    t0 = time.perf_counter()
    if graph is not None:
        graph.replay()
    else:
        for _ in range(args.steps):
            step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / args.steps

    def time_calls(fn, reps, repeats=5):
        """Per-call milliseconds (median, min over `repeats`) from HIP events
        on the launch stream around a graph of `reps` back-to-back calls (no
        host gaps between the kernels; warm caches)."""
        g = capture(fn, reps)
        g.replay()
        ts = []
        for _ in range(repeats):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) / reps)
        del g
        return float(np.median(ts)), float(min(ts))

    # ---- the step made of the three separate calls, and the per-call
    # durations
    ms_sep = time_calls(step_separate, args.steps)[0]
    calls = {"lime_xor_fwd": user, "lime_qk_cache_build": build, "lime_cand_score": score,
             "lime_xor_fwd_score": user_score}
    call_ms, call_min_ms = {}, {}
    for k, fn in calls.items():
        call_ms[k], call_min_ms[k] = time_calls(fn, args.steps)

    # roofline of the kernel with the largest share of step time among the
    # calls that are one kernel launch (lime_xor_fwd is one launch on the
    # user-resident path)
    n_cand = len(ids)
    launches, plan = L.xor_fwd_plan(dt, w.B, w.ell, w.d, w.heads, w.layers, w.dff, total_N, max_N)
    algo = {
        "lime_qk_cache_build": dict(kernel="qk_cache", bound="hbm",
                                    bytes=w.n_items * (w.d + w.heads * w.ell) * es,
                                    flops=2.0 * w.n_items * w.d * w.heads * w.ell),
        "lime_cand_score": dict(kernel="cand_score", bound="hbm",
                                bytes=n_cand * (w.heads * w.ell * es + w.d * es + 8),
                                flops=2.0 * n_cand * w.ell * w.d),
    }
    # the step's single-launch calls: the cache build, and either the
    # user-resident kernel in its scoring form (lime_xor_fwd_score is one
    # launch) or the scoring kernel the call launches after the user side
    in_step = ["lime_qk_cache_build"]
    if launches == 1:
        cs = algo["lime_cand_score"]
        algo["lime_xor_fwd_score"] = dict(kernel="xor_fwd_resident_score", bound="mfma",
                                          bytes=(w.B * w.ell * 2 + total_N) * w.d * es + cs["bytes"],
                                          flops=xor_fwd_flops(w, np.diff(off)) + cs["flops"])
        in_step.append("lime_xor_fwd_score")
    else:
        in_step.append("lime_cand_score")
    single = {k: v for k, v in call_ms.items() if k in in_step}
    dom = max(single, key=single.get)
    a = algo[dom]
    t = single[dom] * 1e-3
    if a["bound"] == "hbm":
        achieved, peak, unit = a["bytes"] / t / 1e9, HBM_PEAK_GBS, "GB/s"
    else:
        achieved, peak, unit = a["flops"] / t / 1e12, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"
    roofline = {"kernel": a["kernel"], "bound": a["bound"], "achieved": round(achieved, 2),
                "peak": peak, "unit": unit, "frac": round(achieved / peak, 4),
                "traffic": traffic_from_profiles(w.name, a["kernel"]),
                "avg_launch_us": round(single[dom] * 1e3, 2),
                "algorithmic_bytes_per_launch": int(a["bytes"]),
                "algorithmic_flops_per_launch": float(a["flops"])}
    # the user side against its roofline: algorithmic flops of the call, and
    # the fused minimum of HBM bytes (every layer reads and writes each row of
    # the residual stream once: 2 (B ell + N) d s per layer), at the peaks
    t_user = call_ms["lime_xor_fwd"] * 1e-3
    u_flops = xor_fwd_flops(w, np.diff(off))
    u_bytes = 2.0 * w.layers * (w.B * w.ell + total_N) * w.d * es
    u_roof = max(u_bytes / (HBM_PEAK_GBS * 1e9), u_flops / (MFMA_BF16_PEAK_TFLOPS * 1e12))
    user_side = {"us": round(t_user * 1e6, 2), "users_per_s": round(w.B / t_user, 1),
                 "history_rows_per_s": round(total_N / t_user, 1),
                 "TFLOP/s": round(u_flops / t_user / 1e12, 2),
                 "fused_min_bytes": int(u_bytes), "fused_min_GB/s": round(u_bytes / t_user / 1e9, 1),
                 "roofline_us": round(u_roof * 1e6, 2), "frac": round(u_roof / t_user, 4),
                 "launches": launches}
    per_call = {}
    for k, v in algo.items():
        tk = call_ms[k] * 1e-3
        per_call[k] = {"us": round(call_ms[k] * 1e3, 2), "us_min": round(call_min_ms[k] * 1e3, 2),
                       "GB/s": round(v["bytes"] / tk / 1e9, 1),
                       "TFLOP/s": round(v["flops"] / tk / 1e12, 2)}

    # ---- scoring cold and with no id reuse.  Cold: every timed call follows
    # a 512 MiB write and then a 512 MiB read of another buffer, which evict
    # L2 and the 256 MB Infinity Cache and leave them clean (after the write
    # alone its dirty lines would be written back during the timed call);
    # the call is timed alone between HIP events, queued behind that work so
    # no host latency counts; median and min of 20.  The uniform-id control
    # draws the same number of candidates uniformly over the catalogue
    # (seeded), so nearly every gathered cache row is distinct and crosses HBM.
    scoring = None
    if not args.no_extras:
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        rbuf = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
        sink = []

        def cold_calls(fn, n=20):
            ts = []
            for _ in range(n):
                scratch.fill_(1)
                sink.append(rbuf.sum())
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                fn()
                e1.record()
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
            return float(np.median(ts)), float(min(ts))

        ids_u = dev(np.random.default_rng(20260).integers(0, w.n_items, size=n_cand, dtype=np.int64))

        def score_uniform():
            L.cand_score(cache, lp, ids_u, coff_d, out=out)

        cs_bytes = algo["lime_cand_score"]["bytes"]

        def entry(med, mn):
            return {"us": round(med * 1e3, 2), "us_min": round(mn * 1e3, 2),
                    "candidates_per_s": round(n_cand / (med * 1e-3), 1),
                    "GB/s": round(cs_bytes / (med * 1e-3) / 1e9, 1),
                    "frac_of_hbm_peak": round(cs_bytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}

        scoring = {"zipf_cold": entry(*cold_calls(score)),
                   "uniform_cold": entry(*cold_calls(score_uniform)),
                   "uniform_warm": entry(*time_calls(score_uniform, args.steps)),
                   "zipf_warm": entry(call_ms["lime_cand_score"], call_min_ms["lime_cand_score"])}
        del scratch, rbuf, sink

    # ---- the pages' other variants (not part of the step): the user-side
    # LIME-MHA and LIME-XOR+Window; int8 cache build and scoring, uncached
    # scoring (LIME summary page, Table 10 columns); each timed like the
    # calls above
    extras = {}
    if not args.no_extras:
        codes = torch.empty((w.n_items, w.heads, w.ell), dtype=torch.int8, device="cuda")
        qsc = torch.empty((w.n_items, w.heads), dtype=torch.float32, device="cuda")
        out2 = torch.empty_like(out)

        def build_i8():
            L.qk_cache_build_i8(items, keys, phi=w.phi, scale=scale, codes=codes, qscale=qsc)

        def score_i8():
            L.cand_score_i8(codes, qsc, lp, ids_d, coff_d, out=out2)

        def score_uncached():
            L.cand_score_uncached(items, keys, lp, ids_d, coff_d, phi=w.phi, scale=scale, out=out2)

        build_i8()
        torch.cuda.synchronize()
        hl = w.heads * w.ell
        ex_bytes = {
            "lime_qk_cache_build_i8": w.n_items * (w.d * es + hl + 4 * w.heads),
            "lime_cand_score_i8": n_cand * (hl + 4 * w.heads + w.d * es + 8),
            "lime_cand_score_uncached": n_cand * (w.d * es + w.d * es + 8),
        }
        lp2 = torch.empty_like(lp)

        def user_variant(variant):
            def run():
                L.xor_fwd(lc, hs, hoff, wts, heads=w.heads, phi=w.phi, scale=scale, max_N=max_N,
                          links_pers=lp2, workspace=ws, variant=variant)
            return run

        # the user-side variants (LIME-MHA; LIME-XOR+Window with ell/2
        # neighbours on each side), timed like the user side of the step
        for k, fn in (("lime_xor_fwd_variant[mha]", user_variant("mha")),
                      ("lime_xor_fwd_variant[xor_window]", user_variant("xor_window"))):
            fn()
            torch.cuda.synchronize()
            t_ms, t_min = time_calls(fn, args.steps)
            extras[k] = {"us": round(t_ms * 1e3, 2), "us_min": round(t_min * 1e3, 2),
                         "users_per_s": round(w.B / (t_ms * 1e-3), 1)}
        for k, fn in (("lime_qk_cache_build_i8", build_i8), ("lime_cand_score_i8", score_i8),
                      ("lime_cand_score_uncached", score_uncached)):
            t_ms, t_min = time_calls(fn, args.steps)
            extras[k] = {"us": round(t_ms * 1e3, 2), "us_min": round(t_min * 1e3, 2),
                         "GB/s": round(ex_bytes[k] / (t_ms * 1e-3) / 1e9, 1),
                         "per_s": round((w.n_items if "build" in k else n_cand) / (t_ms * 1e-3), 1)}

    # achievable HBM bandwidth next to the 8 TB/s peak: a plain 1 GiB
    # device-to-device copy (read + write bytes counted), timed like the calls
    # (skipped in counter-calibration runs, whose only copies must be the
    # calibration copies below)
    copy_gbs = None
    if not args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        copy_gbs = 2 * src.numel() * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
        del src, dst
    if a["bound"] == "hbm" and copy_gbs:
        roofline["achievable_copy_GBs"] = round(copy_gbs, 1)
        roofline["frac_of_copy"] = round(achieved / copy_gbs, 4)

    if args.copy_calibration:
        # a plain device copy of known size, for scaling the HBM byte counters
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    res = {
        "metric": "candidates scored/sec + user histories encoded/sec; % HBM/MFMA roofline",
        "value": n_cand / (ms_step * 1e-3),
        "unit": "candidates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "ms_per_step_separate_calls": round(ms_sep, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded; shapes and id law of the workload)",
        "config": {"workload": f"{w.name}: B={w.B} users, N={w.N}, ell={w.ell}, d={w.d}, "
                               f"heads={w.heads}, layers={w.layers}, catalogue={w.n_items}, "
                               f"M={w.M}/user, zipf={w.zipf}, phi={w.phi}",
                   "users": w.B, "history_rows": total_N, "catalogue_items": w.n_items,
                   "candidates": n_cand},
        "users_per_s": w.B / (ms_step * 1e-3),
        "items_per_s": w.n_items / (ms_step * 1e-3),
        "call_ms": {k: round(v, 4) for k, v in call_ms.items()},
        "user_side": user_side,
        "per_call": per_call,
        "scoring": scoring,
        "variants": extras,
        "xor_fwd_plan": plan,
        "launch": "eager" if args.no_graph else "one hip-graph replay of the K captured steps",
        "roofline": roofline,
        "hbm_copy_GBs": round(copy_gbs, 1) if copy_gbs else None,
    }

    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, ui, ci, ids, coff, scale, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def xor_fwd_flops(w, lens):
    """Algorithmic flops of one lime_xor_fwd call without hist_out: every
    layer projects all rows (QKV 6d^2, W_o 2d^2, gated MLP 6 d d_ff per row)
    and runs both XOR branches (8 ell N d per user); the last layer needs
    only the K,V projection of history rows (4d^2) and the link-side branch
    (4 ell N d)."""
    d, f, ell, L = w.d, w.dff, w.ell, w.layers
    N = float(np.sum(lens))
    rows_link = w.B * ell
    full = (rows_link + N) * (8 * d * d + 6 * d * f) + 8 * ell * N * d
    last = rows_link * (8 * d * d + 6 * d * f) + N * 4 * d * d + 4 * ell * N * d
    return (L - 1) * full + last


def traffic_from_profiles(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary
    profiles/<kernel>_<workload>_traffic.txt (FETCH_SIZE and WRITE_SIZE in
    KiB per dispatch, scaled by the copy-kernel factors recorded there), or
    None if there is none or the kernel sources changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    try:
        h = hashlib.sha256()
        csrc = os.path.join(ROOT, "decoupled_linear_link_amd", "csrc")
        for f in sorted(os.listdir(csrc)):
            h.update(open(os.path.join(csrc, f), "rb").read())
        if kv.get("sources_sha256") != h.hexdigest():
            return None
        return int(float(kv["fetch_kib"]) * 1024 * float(kv["fetch_factor"])
                   + float(kv["write_kib"]) * 1024 * float(kv["write_factor"]))
    except (KeyError, ValueError, OSError):
        return None


def cpu_baseline(w, ui, ci, ids, coff, scale, budget_s):
    """The oracle, as it stands, on a bounded sample of the same workload;
    per-part rates are scaled to one whole step."""
    import oracle.lime_oracle as O
    import workloads as W
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        pools = threadpool_info()
        cores = max([p.get("num_threads", 1) for p in pools] or [1])
        blas = ", ".join(f"{p.get('internal_api')} {p.get('version')} ({p.get('num_threads')} threads)"
                         for p in pools if p.get("user_api") == "blas") or "none"
    except Exception:
        cores = 1
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    off = ui["hist_offsets"]
    frac = 1.0 / 3.0
    # users: a prefix of users
    nu = max(1, min(w.B, 8))
    t0 = time.perf_counter()
    O.xor_fwd(ui["links_ctx"], ui["hist"], off, ui["weights"], w.heads, scale, w.phi, users=range(nu))
    t_user = (time.perf_counter() - t0) / nu
    nu2 = int(min(w.B, max(nu, budget_s * frac / max(t_user, 1e-9))))
    if nu2 > nu:
        t0 = time.perf_counter()
        O.xor_fwd(ui["links_ctx"], ui["hist"], off, ui["weights"], w.heads, scale, w.phi, users=range(nu2))
        t_user = (time.perf_counter() - t0) / nu2
        nu = nu2
    # items: a prefix of the catalogue
    ni = min(w.n_items, 20000)
    t0 = time.perf_counter()
    O.qk_cache_build(ci["items"][:ni], ci["link_keys"], scale, w.phi)
    t_item = (time.perf_counter() - t0) / ni
    ni2 = int(min(w.n_items, max(ni, budget_s * frac / max(t_item, 1e-12))))
    if ni2 > ni:
        t0 = time.perf_counter()
        c = O.qk_cache_build(ci["items"][:ni2], ci["link_keys"], scale, w.phi)
        t_item = (time.perf_counter() - t0) / ni2
        ni = ni2
    else:
        c = O.qk_cache_build(ci["items"][:ni], ci["link_keys"], scale, w.phi)
    # candidates: the first users' candidates, ids folded into the sampled rows
    lp = W.links_pers(w)
    nc_users = max(1, min(w.B, int(budget_s * frac / 1e-3 / max(1, w.M)) or 1))
    t0 = time.perf_counter()
    O.cand_score(c, lp[:nc_users], ids[: coff[nc_users]] % ni, coff[: nc_users + 1])
    t_cand = (time.perf_counter() - t0) / max(1, int(coff[nc_users]))
    n_cand = len(ids)
    t_step = t_user * w.B + t_item * w.n_items + t_cand * n_cand
    return {"value": n_cand / t_step, "unit": "candidates/s", "cores": int(cores), "kind": "oracle",
            "cpu_model": cpu_model, "blas": blas,
            "sample": f"{nu} users, {ni} catalogue items, {int(coff[nc_users])} candidates; "
                      "per-part times scaled to one whole step",
            "users_per_s": 1.0 / t_user, "items_per_s": 1.0 / t_item,
            "candidates_per_s": 1.0 / t_cand}


if __name__ == "__main__":
    main()
