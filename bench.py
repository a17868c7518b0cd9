"""Benchmark of the LIME inference hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  lime_qk_cache_build (the QK cache over the whole catalogue: the offline
                       stage), then
  lime_xor_fwd_score  (the online stage: user encoder over all B users and
                       all layers, and the scoring of all B*M candidates;
                       lime_xor_fwd followed by lime_cand_score in one call)
Inputs are resident in HBM before the timed region starts.  The default
workload is the largest one that fits one GPU (lifelong: 8 users with
8,192-16,384 history rows, ell = 64, d = 256, 8 heads, 4 layers, a 4M-item
catalogue, 65,536 candidates).

    python bench.py [--steps K] [--warmup W] [--workload lifelong] [--no-cpu-baseline]

Prints ONE JSON line.  `value` = candidates scored per second of whole-step
time; `online` has the rate of the online call alone (lime_xor_fwd_score),
without the catalogue rebuild.  The K timed steps are captured in one HIP
graph and replayed once.  Per-call times are HIP events on the launch
stream around a graph of K back-to-back calls (median of 5, minimum
alongside).  Per-kernel times come from a kernel trace of the library
(lime_trace_begin / lime_trace_end: every launch stamped with its own start
and end by the runtime), taken over eager calls after the timed region.

`rooflines` puts each kernel against max(algorithmic bytes / 8 TB/s,
algorithmic flops / peak); `roofline` is the kernel with the largest share
of the step's kernel time.  `scoring` has candidate scoring cold (each call
after a 512 MiB write and a 512 MiB read that evict L2 and the Infinity
Cache) and warm, for the workload's ids and for a uniform-id control with
no reuse; `cpu_baseline` is the CPU oracle timed on a bounded sample of the
same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}  # dense MFMA bf16; fp32 vector


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="lifelong")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="approximate CPU budget of the oracle baseline")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch the timed steps eagerly instead of replaying a HIP graph of them")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the cold-scoring, int8, uncached and user-side variant timings")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (for HBM counter scaling)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# --------------------------------------------------------------------------
# algorithmic work per launch (bytes each kernel must move, flops it must do)
# --------------------------------------------------------------------------

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


def kernel_work(w, es, total_N, n_cand):
    """name -> f(full) = (bytes, flops) of one launch of that kernel, where
    `full` says whether the layer also updates history rows (every layer but
    the last when hist_out is not requested).  Bytes are what the method
    must move (inputs read once, outputs written once), not what a kernel
    happens to move."""
    d, f, ell, H = w.d, w.dff, w.ell, w.heads
    N, nlr = float(total_N), float(w.B * ell)
    R = N + nlr

    def qkv(full):
        # read X; write Q (all rows, or links only), K and V
        q_rows = R if full else nlr
        return (R + q_rows + 2 * R) * d * es, 2.0 * d * d * (q_rows + 2 * R)

    def attn(full):
        # per user-layer 4 (N + ell) d s: read Q, K, V, write Y; the links-only
        # last layer reads K_E, V_E and the links' Q, K, V, writes Y_L
        if full:
            return 4 * R * d * es, 8.0 * ell * N * d
        return (2 * N + 4 * nlr) * d * es, 4.0 * ell * N * d

    def attn_fused(full):
        # the history rows' LN + QKV inside the attention: read X, write Y_E
        # (the links' Y comes from the split combine)
        if full:
            return (R + N) * d * es, 2.0 * d * 3 * d * R + 8.0 * ell * N * d
        return R * d * es, 2.0 * d * 2 * d * N + 2.0 * d * 3 * d * nlr + 4.0 * ell * N * d

    # the link operands of every (user, head): f16 registers of one wave
    lops_bytes = w.B * H * (2 * (ell // 16) + 2 * (ell // 32)) * 64 * 16

    def link_h(full):
        # d = 256: the link rows' Q, K, V (Q only in a links-only last layer)
        # from their LayerNorm rows, once per user and head
        if full:
            return nlr * d * es + lops_bytes, 2.0 * d * 3 * d * nlr
        return nlr * d * es + lops_bytes / 3, 2.0 * d * d * nlr

    def attn_h(full):
        # d = 256: the history rows' projection inside the attention, from
        # the LayerNorm rows the post block stored: read those rows and the
        # link operands, write Y_E (the links' Y comes from the split combine)
        if full:
            return 2 * N * d * es + lops_bytes, 2.0 * d * 3 * d * N + 8.0 * ell * N * d
        return N * d * es + lops_bytes / 3, 2.0 * d * 2 * d * N + 4.0 * ell * N * d

    def ln_rows(full):
        # the first layer's LayerNorm rows: read X, write them
        return 2 * R * d * es, 0.0

    def post(full):
        # read Y and X, write the new rows; at d = 256 a full layer's post
        # block also writes the next layer's LayerNorm rows (the operands of
        # the attention with the projection fused in)
        rows = R if full else nlr
        passes = 4 if (full and d == 256) else 3
        return passes * rows * d * es, rows * (2.0 * d * d + 6.0 * d * f)

    def combine(full):
        return nlr * d * es, 0.0

    user_bytes = (2 * nlr + N) * d * es

    def resident(full):
        return user_bytes, xor_fwd_flops(w, [total_N])

    def resident_score(full):
        cb, cf = cand(full)
        return user_bytes + cb, xor_fwd_flops(w, [total_N]) + cf

    def cache(full):
        return w.n_items * (d + H * ell) * es, 2.0 * w.n_items * d * H * ell

    def cand(full):
        return n_cand * (H * ell * es + d * es + 8), 2.0 * n_cand * ell * d

    return {"qkv_proj_stream": qkv, "qkv_proj_lds": qkv, "xor_attn": attn, "xor_attn_qkv": attn_fused,
            "xor_attn_h": attn_h, "link_qkv_h": link_h, "ln_rows": ln_rows,
            "xor_combine": combine, "post_block_stream": post, "post_block_lds": post,
            "xor_fwd_resident": resident, "xor_fwd_resident_score": resident_score,
            "qk_cache": cache, "cand_score": cand}


def against_roof(bytes_, flops, seconds, peak_tflops):
    """bound, roofline time and fraction: t_roof = max(bytes/BW, flops/peak)."""
    t_b = bytes_ / (HBM_PEAK_GBS * 1e9)
    t_f = flops / (peak_tflops * 1e12)
    t_roof = max(t_b, t_f)
    return {"bound": "hbm" if t_b >= t_f else ("mfma" if peak_tflops == PEAK_TFLOPS["bf16"] else "alu"),
            "roofline_us": round(t_roof * 1e6, 3),
            "frac": round(t_roof / seconds, 4),
            "GB/s": round(bytes_ / seconds / 1e9, 1), "frac_of_hbm_peak": round(t_b / seconds, 4),
            "TFLOP/s": round(flops / seconds / 1e12, 2), "frac_of_flops_peak": round(t_f / seconds, 4),
            "algorithmic_bytes": int(bytes_), "algorithmic_flops": float(flops)}


# the files that hold each kernel's code: a traffic summary is used only while
# their hash matches the one it records
_USER = ("common.h", "mfma_kernels.h", "user_kernels.h")
KERNEL_SOURCES = {
    "qk_cache": ("common.h", "mfma_kernels.h"),
    "cand_score": ("common.h", "mfma_kernels.h"),
    **{k: _USER for k in ("xor_attn_h", "link_qkv_h", "xor_attn_qkv", "xor_attn", "post_block_stream", "post_block_lds",
                          "qkv_proj_stream", "qkv_proj_lds", "ln_rows", "xor_combine", "xor_fwd_resident",
                          "xor_fwd_resident_score")},
}
ALL_SOURCES = ("common.h", "generic_kernels.h", "lime_api.hip", "mfma_kernels.h", "user_kernels.h")


def traffic_from_profiles(workload, kernel, last=False):
    """HBM bytes per launch of `kernel` from the committed counter summary
    profiles/<kernel>_<workload>_traffic.txt (FETCH_SIZE and WRITE_SIZE in
    KiB per dispatch, scaled by the copy-kernel factors recorded there; with
    `last`, a per-layer kernel's last-layer launches), or None if there is
    none or the kernel's sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    try:
        files = tuple(kv.get("sources", "").split()) or KERNEL_SOURCES.get(kernel, ALL_SOURCES)
        if kv.get("sources_sha256") != sources_sha256(files):
            return None
        pre = "last_" if last else ""
        if pre + "fetch_kib" not in kv:
            return None
        return int(float(kv[pre + "fetch_kib"]) * 1024 * float(kv["fetch_factor"])
                   + float(kv[pre + "write_kib"]) * 1024 * float(kv["write_factor"]))
    except (KeyError, ValueError, OSError):
        return None


def sources_sha256(files=ALL_SOURCES):
    """sha256 over the named files of the library's sources, in name order."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "decoupled_linear_link_amd", "csrc")
    for f in sorted(files):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()


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
    peak_tf = PEAK_TFLOPS[w.dtype]
    scale = W.scale_for(w)

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    # ---- inputs, resident in HBM
    log(f"generating the {w.name} inputs")
    t_gen = time.perf_counter()
    ui = W.user_inputs(w)
    ci = W.cache_inputs(w)
    ids = W.candidate_ids(w)
    coff = W.candidate_offsets(w)
    off = ui["hist_offsets"]
    lens = np.diff(off)
    total_N = int(off[-1])
    max_N = int(lens.max())
    lc, hs, hoff = dev(ui["links_ctx"]), dev(ui["hist"]), dev(off)
    wts = [{k: dev(v) for k, v in lw.items()} for lw in ui["weights"]]
    items, keys = dev(ci["items"]), dev(ci["link_keys"])
    ids_d, coff_d = dev(ids), dev(coff)
    lp = torch.empty_like(lc)
    cache = torch.empty((w.n_items, w.heads, w.ell), dtype=dt, device="cuda")
    out = torch.empty((len(ids), w.d), dtype=dt, device="cuda")
    ws_bytes = L.xor_fwd_workspace_size(dt, w.B, w.ell, w.d, w.heads, w.dff, total_N, max_N)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    log(f"inputs on the device ({time.perf_counter() - t_gen:.1f} s)")

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
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    if graph is not None:
        graph.replay()
    else:
        for _ in range(args.steps):
            step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / args.steps
    del graph

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

    # ---- per-call durations, and the step as three separate calls
    log("timing the calls")
    ms_sep = time_calls(step_separate, args.steps)[0]
    calls = {"lime_xor_fwd": user, "lime_qk_cache_build": build, "lime_cand_score": score,
             "lime_xor_fwd_score": user_score}
    call_ms, call_min_ms = {}, {}
    for k, fn in calls.items():
        call_ms[k], call_min_ms[k] = time_calls(fn, args.steps)

    # ---- per-kernel durations: a trace of eager steps (each launch stamped
    # with its own start and end on the GPU)
    log("tracing the kernels of the step")
    n_cand = len(ids)
    launches, plan = L.xor_fwd_plan(dt, w.B, w.ell, w.d, w.heads, w.layers, w.dff, total_N, max_N)
    work = kernel_work(w, es, total_N, n_cand)
    trace_steps = 5
    L.trace_begin(4096)
    for _ in range(trace_steps):
        step()
    torch.cuda.synchronize()
    recs, dropped = L.trace_end(4096)
    if dropped:
        log(f"trace dropped {dropped} launches")
    # each record: (name, ms, full) where full = the layer updates history
    # rows; layers are counted by the launch that opens each of them
    # (at d = 256 link_qkv_h opens a layer, xor_attn_h follows it)
    opens = ("qkv_proj_stream", "qkv_proj_lds", "xor_attn_qkv", "link_qkv_h")
    per_layer = ("xor_attn", "xor_attn_qkv", "xor_attn_h", "link_qkv_h", "qkv_proj_stream", "qkv_proj_lds", "post_block_stream",
                 "post_block_lds")
    per = {}
    layer = -1
    for name, ms in recs:
        if name == "split_plan":
            layer = -1  # a streaming user side starts
        elif name in opens:
            layer += 1
        full = layer < w.layers - 1
        key = f"{name}[{'full' if full else 'last'}]" if name in per_layer else name
        per.setdefault(key, {"name": name, "full": full, "ms": []})["ms"].append(ms)
    step_kernel_ms = sum(ms for _, ms in recs) / trace_steps
    rooflines = {}
    for key, v in per.items():
        t_mean = float(np.mean(v["ms"])) * 1e-3
        share = sum(v["ms"]) / trace_steps / step_kernel_ms
        entry = {"us": round(t_mean * 1e6, 2), "launches_per_step": len(v["ms"]) // trace_steps,
                 "share_of_step_kernel_time": round(share, 4)}
        if v["name"] in work:
            b, f = work[v["name"]](v["full"])
            entry.update(against_roof(b, f, t_mean, peak_tf))
            # measured HBM bytes per launch (committed counter summary), if current
            entry["traffic"] = traffic_from_profiles(w.name, v["name"],
                                                     last=v["name"] in per_layer and not v["full"])
        rooflines[key] = entry
    # the MFMA ceiling of the cache build: its intensity over the MFMA ridge
    if "qk_cache" in rooflines:
        r = rooflines["qk_cache"]
        ridge = peak_tf * 1e12 / (HBM_PEAK_GBS * 1e9)
        r["mfma_ceiling_at_hbm_peak"] = round(min(1.0, r["algorithmic_flops"] / r["algorithmic_bytes"] / ridge), 4)

    # ---- the headline roofline: the kernel with the largest share of the
    # step's kernel time.  A kernel that is a whole call (the cache build,
    # scoring) is timed by events around K back-to-back calls; the others by
    # their traced mean.
    dom = max((k for k in rooflines if "algorithmic_bytes" in rooflines[k]),
              key=lambda k: rooflines[k]["share_of_step_kernel_time"])
    whole_call = {"qk_cache": "lime_qk_cache_build", "cand_score": "lime_cand_score",
                  "xor_fwd_resident_score": "lime_xor_fwd_score"}
    dname = per[dom]["name"]
    t_dom = (call_ms[whole_call[dname]] * 1e-3) if dname in whole_call else rooflines[dom]["us"] * 1e-6
    b, f = work[dname](per[dom]["full"])
    rr = against_roof(b, f, t_dom, peak_tf)
    if rr["bound"] == "hbm":
        achieved, peak, unit = b / t_dom / 1e9, HBM_PEAK_GBS, "GB/s"
    else:
        achieved, peak, unit = f / t_dom / 1e12, peak_tf, "TFLOP/s"
    roofline = {"kernel": dname, "bound": rr["bound"], "achieved": round(achieved, 2), "peak": peak,
                "unit": unit, "frac": round(achieved / peak, 4),
                "traffic": traffic_from_profiles(w.name, dname),
                "avg_launch_us": round(t_dom * 1e6, 2), "traced_launch_us": rooflines[dom]["us"],
                "algorithmic_bytes_per_launch": int(b), "algorithmic_flops_per_launch": float(f),
                "other_bound_frac": rr["frac_of_flops_peak"] if rr["bound"] == "hbm" else rr["frac_of_hbm_peak"]}

    # ---- the user side against its roofline: algorithmic flops of the call
    # and the fused minimum of HBM bytes (every layer reads and writes each
    # row of the residual stream once: 2 (B ell + N) d s per layer)
    t_user = call_ms["lime_xor_fwd"] * 1e-3
    u_flops = xor_fwd_flops(w, lens)
    u_bytes = 2.0 * w.layers * (w.B * w.ell + total_N) * w.d * es
    u_roof = max(u_bytes / (HBM_PEAK_GBS * 1e9), u_flops / (peak_tf * 1e12))
    user_side = {"us": round(t_user * 1e6, 2), "users_per_s": round(w.B / t_user, 1),
                 "history_rows_per_s": round(total_N / t_user, 1),
                 "TFLOP/s": round(u_flops / t_user / 1e12, 2),
                 "fused_min_bytes": int(u_bytes), "fused_min_GB/s": round(u_bytes / t_user / 1e9, 1),
                 "roofline_us": round(u_roof * 1e6, 2), "frac": round(u_roof / t_user, 4),
                 "launches": launches}
    t_online = call_ms["lime_xor_fwd_score"] * 1e-3
    online = {"call": "lime_xor_fwd_score", "us": round(t_online * 1e6, 2),
              "candidates_per_s": round(n_cand / t_online, 1), "users_per_s": round(w.B / t_online, 1)}

    # ---- scoring cold and with no id reuse.  Cold: every timed call follows
    # a 512 MiB write and then a 512 MiB read of another buffer, which evict
    # L2 and the 256 MB Infinity Cache and leave them clean (after the write
    # alone its dirty lines would be written back during the timed call);
    # the call is timed alone between HIP events, queued behind that work so
    # no host latency counts; median and min of 20.  The uniform-id control
    # draws the same number of candidates uniformly over the catalogue
    # (seeded), so nearly every gathered cache row is distinct and crosses HBM.
    scoring = None
    cs_bytes, cs_flops = work["cand_score"](True)
    if not args.no_extras:
        log("timing cold and warm scoring")
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

        def entry(med, mn):
            e = {"us": round(med * 1e3, 2), "us_min": round(mn * 1e3, 2),
                 "candidates_per_s": round(n_cand / (med * 1e-3), 1)}
            e.update(against_roof(cs_bytes, cs_flops, med * 1e-3, peak_tf))
            return e

        scoring = {"zipf_cold": entry(*cold_calls(score)),
                   "uniform_cold": entry(*cold_calls(score_uniform)),
                   "uniform_warm": entry(*time_calls(score_uniform, args.steps)),
                   "zipf_warm": entry(call_ms["lime_cand_score"], call_min_ms["lime_cand_score"])}
        del scratch, rbuf, sink
        if "cand_score" in rooflines:
            rooflines["cand_score"]["cold_zipf"] = {k: scoring["zipf_cold"][k] for k in ("us", "frac", "GB/s")}
            rooflines["cand_score"]["cold_uniform"] = {k: scoring["uniform_cold"][k]
                                                       for k in ("us", "frac", "GB/s")}

    # ---- the pages' other variants (not part of the step): the user-side
    # LIME-MHA and LIME-XOR+Window; int8 cache build and scoring, uncached
    # scoring (LIME summary page, Table 10 columns); each timed like the
    # calls above
    extras = {}
    if not args.no_extras:
        log("timing the variants")
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
        del codes, qsc, out2, lp2

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
    if roofline["bound"] == "hbm" and copy_gbs:
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
        "data": "synthetic (seeded; shapes, length law and id law of the workload)",
        "config": {"workload": f"{w.name}: B={w.B} users, N={w.N}, ell={w.ell}, d={w.d}, "
                               f"heads={w.heads}, layers={w.layers}, catalogue={w.n_items}, "
                               f"M={w.M}/user, zipf={w.zipf}, phi={w.phi}",
                   "users": w.B, "history_rows": total_N, "catalogue_items": w.n_items,
                   "candidates": n_cand},
        "users_per_s": w.B / (ms_step * 1e-3),
        "items_per_s": w.n_items / (ms_step * 1e-3),
        "online": online,
        "call_ms": {k: round(v, 4) for k, v in call_ms.items()},
        "user_side": user_side,
        "roofline": roofline,
        "rooflines": rooflines,
        "step_kernel_ms_traced": round(step_kernel_ms, 4),
        "scoring": scoring,
        "variants": extras,
        "xor_fwd_plan": plan,
        "launch": "eager" if args.no_graph else "one hip-graph replay of the K captured steps",
        "hbm_copy_GBs": round(copy_gbs, 1) if copy_gbs else None,
    }

    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample")
        res["cpu_baseline"] = cpu_baseline(w, ui, ci, ids, coff, scale, args.cpu_seconds)
    print(json.dumps(res), flush=True)


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
    nu = 1
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
            "sample": f"{nu} of {w.B} users, {ni} of {w.n_items} catalogue items, {int(coff[nc_users])} of "
                      f"{n_cand} candidates; per-part times scaled to one whole step",
            "users_per_s": 1.0 / t_user, "items_per_s": 1.0 / t_item,
            "candidates_per_s": 1.0 / t_cand}


if __name__ == "__main__":
    main()
