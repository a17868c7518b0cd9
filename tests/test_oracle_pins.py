"""Pins of the CPU oracle to facts other than itself.

Each pin compares the oracle with something the pages or the mathematics
fix: the dense XOR-masked form of the attention (LIME notes, Key design 2,
XORA equation), library routines (torch's scaled_dot_product_attention,
layer_norm, softmax, silu, linear in float64 on the CPU), exact identities
(SiLU(s) - SiLU(-s) = s), closed-form special cases, brute force over
scalars on tiny inputs, and the cache-size arithmetic of the LIME summary
page, Table 12.  The LIME-MHA and LIME-XOR+Window variants are pinned the
same way: brute force from each variant's description, dense masked
attention, torch SDPA with an explicit boolean mask, and invariances
(window symmetry, locality, first-layer agreement with LIME-XOR).  The mutation tests at the end plant plausible mistakes in
the oracle and check that some pin fails for each.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle.lime_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _qkv(rng, rows, d, std=1.0):
    return [rng.standard_normal((rows, d)) * std for _ in range(3)]


def _weights(rng, d, dff, std=None):
    s = d ** -0.5 if std is None else std
    return {
        "w_qkv": rng.standard_normal((3 * d, d)) * s,
        "w_o": rng.standard_normal((d, d)) * s,
        "w_gate": rng.standard_normal((dff, d)) * s,
        "w_up": rng.standard_normal((dff, d)) * s,
        "w_down": rng.standard_normal((d, dff)) * s,
    }


# ---------------------------------------------------------------- pin functions

def pin_dense_equals_decoupled(seed=0):
    """max |decoupled - dense| over several tiny shapes, both phis."""
    rng = _rng(seed)
    err = 0.0
    for ell in (1, 3, 8):
        for n in (0, 1, 2, 7):
            for heads, d in ((1, 4), (2, 8)):
                for phi in ("softmax", "silu_mean"):
                    q, k, v = _qkv(rng, ell + n, d)
                    a = O.xor_attention(q, k, v, ell, heads, 0.7, phi)
                    b = O.xor_attention_dense(q, k, v, ell, heads, 0.7, phi)
                    err = max(err, float(np.abs(a - b).max()))
    return err


def pin_stack_dense_equals_decoupled(seed=1):
    """Whole multi-layer encoder: decoupled == dense-masked attention inside."""
    rng = _rng(seed)
    B, ell, d, heads = 3, 4, 8, 2
    lens = np.array([5, 0, 3])
    off = np.concatenate([[0], np.cumsum(lens)])
    lc = rng.standard_normal((B, ell, d))
    hs = rng.standard_normal((int(off[-1]), d))
    W = [_weights(rng, d, d) for _ in range(2)]
    err = 0.0
    for phi in ("softmax", "silu_mean"):
        a, ha = O.xor_fwd(lc, hs, off, W, heads, 0.5, phi)
        b, hb = O.xor_fwd(lc, hs, off, W, heads, 0.5, phi, dense=True)
        err = max(err, float(np.abs(a - b).max()))
        for x, y in zip(ha, hb):
            if x.size:
                err = max(err, float(np.abs(x - y).max()))
    return err


def pin_softmax_branches_vs_sdpa(seed=2):
    """Each branch with softmax equals torch's scaled_dot_product_attention."""
    rng = _rng(seed)
    ell, n, d, heads, scale = 5, 11, 12, 3, 0.37
    dh = d // heads
    q, k, v = _qkv(rng, ell + n, d)
    y = O.xor_attention(q, k, v, ell, heads, scale, "softmax")
    err = 0.0
    for h in range(heads):
        c = slice(h * dh, (h + 1) * dh)
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
        ye = F.scaled_dot_product_attention(t(q[ell:, c]), t(k[:ell, c]), t(v[:ell, c]), scale=scale)
        yl = F.scaled_dot_product_attention(t(q[:ell, c]), t(k[ell:, c]), t(v[ell:, c]), scale=scale)
        err = max(err, float(np.abs(y[ell:, c] - ye.numpy()).max()))
        err = max(err, float(np.abs(y[:ell, c] - yl.numpy()).max()))
    return err


def pin_silu_odd_identity(seed=3):
    """SiLU(s) - SiLU(-s) = s, so for silu_mean each branch satisfies
    att(Q) - att(-Q) = scale * Q K^T V / |A| (a plain linear-algebra form)."""
    rng = _rng(seed)
    ell, n, d, heads, scale = 4, 9, 8, 2, 0.8
    dh = d // heads
    q, k, v = _qkv(rng, ell + n, d, std=1.5)
    diff = (O.xor_attention(q, k, v, ell, heads, scale, "silu_mean")
            - O.xor_attention(-q, k, v, ell, heads, scale, "silu_mean"))
    ref = np.zeros_like(diff)
    for h in range(heads):
        c = slice(h * dh, (h + 1) * dh)
        ref[ell:, c] = scale * q[ell:, c] @ k[:ell, c].T @ v[:ell, c] / ell
        ref[:ell, c] = scale * q[:ell, c] @ k[ell:, c].T @ v[ell:, c] / n
    return float(np.abs(diff - ref).max())


def _torch_layer(x, lw, ell, heads, scale, phi):
    """One layer from torch library routines (float64, CPU)."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    x = t(x)
    d = x.shape[1]
    dh = d // heads
    h = F.layer_norm(x, (d,), eps=1e-5)
    qkv = F.linear(h, t(lw["w_qkv"]))
    q, k, v = qkv[:, :d], qkv[:, d:2 * d], qkv[:, 2 * d:]
    y = torch.zeros_like(x)
    for hd in range(heads):
        c = slice(hd * dh, (hd + 1) * dh)
        for rows, keys in ((slice(ell, None), slice(0, ell)), (slice(0, ell), slice(ell, None))):
            qq, kk, vv = q[rows, c], k[keys, c], v[keys, c]
            if kk.shape[0] == 0:
                continue
            if phi == "softmax":
                y[rows, c] = F.scaled_dot_product_attention(qq, kk, vv, scale=scale)
            else:
                y[rows, c] = F.silu(scale * qq @ kk.T) @ vv / kk.shape[0]
    x = x + F.linear(y, t(lw["w_o"]))
    g = F.layer_norm(x, (d,), eps=1e-5)
    x = x + F.linear(F.silu(F.linear(g, t(lw["w_gate"]))) * F.linear(g, t(lw["w_up"])), t(lw["w_down"]))
    return x.numpy()


def pin_layer_vs_torch(seed=4):
    rng = _rng(seed)
    err = 0.0
    for ell, n, d, dff, heads in ((3, 6, 8, 8, 2), (2, 0, 4, 8, 1), (4, 1, 12, 6, 3)):
        x = rng.standard_normal((ell + n, d))
        lw = _weights(rng, d, dff)
        for phi in ("softmax", "silu_mean"):
            a = O.xor_layer(x, lw, ell, heads, 0.6, phi)
            b = _torch_layer(x, lw, ell, heads, 0.6, phi)
            err = max(err, float(np.abs(a - b).max()))
    return err


def _brute_allowed(i, rows, ell, variant, window):
    """Keys row i may attend, written from the variant's description."""
    if variant == "mha" and i >= ell:
        return None  # history rows pass through the layer untouched
    keys = [j for j in range(rows) if (i < ell) != (j < ell)]
    if variant == "xor_window" and i >= ell:
        keys += [j for j in range(ell, rows) if j != i and abs(j - i) <= window]
    return keys


def _brute_layer(x, lw, ell, heads, scale, phi, variant="xor", window=0):
    """One layer by scalar loops (tiny inputs only)."""
    rows, d = len(x), len(x[0])
    dh = d // heads

    def ln(r):
        mu = sum(r) / d
        var = sum((u - mu) ** 2 for u in r) / d
        return [(u - mu) / math.sqrt(var + 1e-5) for u in r]

    def mv(W, r):
        return [sum(W[o][i] * r[i] for i in range(len(r))) for o in range(len(W))]

    def sig(u):
        return 1.0 / (1.0 + math.exp(-u))

    h = [ln(list(r)) for r in x]
    qkv = [mv(lw["w_qkv"], r) for r in h]
    y = [[0.0] * d for _ in range(rows)]
    passthrough = set()
    for i in range(rows):
        allowed = _brute_allowed(i, rows, ell, variant, window)
        if allowed is None:
            passthrough.add(i)
            continue
        if not allowed:
            continue
        for hd in range(heads):
            cs = range(hd * dh, (hd + 1) * dh)
            s = [scale * sum(qkv[i][c] * qkv[j][d + c] for c in cs) for j in allowed]
            if phi == "softmax":
                m = max(s)
                e = [math.exp(u - m) for u in s]
                w = [u / sum(e) for u in e]
            else:
                w = [u * sig(u) / len(allowed) for u in s]
            for c in cs:
                y[i][c] = sum(w[t] * qkv[allowed[t]][2 * d + c] for t in range(len(allowed)))
    x2 = [[x[i][c] + mv(lw["w_o"], y[i])[c] for c in range(d)] for i in range(rows)]
    out = []
    for i, r in enumerate(x2):
        if i in passthrough:
            out.append(list(x[i]))
            continue
        g = ln(r)
        gate, up = mv(lw["w_gate"], g), mv(lw["w_up"], g)
        mid = [gate[t] * sig(gate[t]) * up[t] for t in range(len(gate))]
        dn = mv(lw["w_down"], mid)
        out.append([r[c] + dn[c] for c in range(d)])
    return np.array(out)


def pin_layer_brute_force(seed=5):
    rng = _rng(seed)
    err = 0.0
    for ell, n, d, dff, heads in ((2, 3, 4, 4, 2), (3, 2, 6, 4, 3)):
        x = rng.standard_normal((ell + n, d))
        lw = _weights(rng, d, dff)
        lwl = {k: v.tolist() for k, v in lw.items()}
        for phi in ("softmax", "silu_mean"):
            a = O.xor_layer(x, lw, ell, heads, 0.9, phi)
            b = _brute_layer(x.tolist(), lwl, ell, heads, 0.9, phi)
            err = max(err, float(np.abs(a - b).max()))
    return err


def pin_variant_layer_brute_force(seed=9):
    """LIME-MHA and LIME-XOR+Window layers against scalar brute force."""
    rng = _rng(seed)
    err = 0.0
    for ell, n, d, dff, heads, window in ((2, 6, 4, 4, 2, 2), (3, 5, 6, 4, 3, 1), (2, 4, 4, 4, 1, 5)):
        x = rng.standard_normal((ell + n, d))
        lw = _weights(rng, d, dff)
        lwl = {k: v.tolist() for k, v in lw.items()}
        for phi in ("softmax", "silu_mean"):
            for variant in ("mha", "xor_window"):
                a = O.xor_layer(x, lw, ell, heads, 0.9, phi, variant=variant, window=window)
                b = _brute_layer(x.tolist(), lwl, ell, heads, 0.9, phi, variant, window)
                err = max(err, float(np.abs(a - b).max()))
    return err


def pin_variants_dense_equals_decoupled(seed=10):
    """Both variants: the decoupled form equals dense attention under the
    variant's mask, for single layers and whole stacks."""
    rng = _rng(seed)
    err = 0.0
    for ell in (1, 4):
        for n in (0, 1, 2, 7, 12):
            for heads, d in ((1, 4), (2, 8)):
                for phi in ("softmax", "silu_mean"):
                    q, k, v = _qkv(rng, ell + n, d)
                    for variant, window in (("mha", 0), ("xor_window", 1), ("xor_window", 3)):
                        a = O.xor_attention(q, k, v, ell, heads, 0.7, phi, variant, window)
                        b = O.xor_attention_dense(q, k, v, ell, heads, 0.7, phi, variant, window)
                        err = max(err, float(np.abs(a - b).max()))
    B, ell, d, heads = 3, 4, 8, 2
    off = np.array([0, 9, 9, 12])
    lc = rng.standard_normal((B, ell, d))
    hs = rng.standard_normal((12, d))
    W = [_weights(rng, d, d) for _ in range(2)]
    for phi in ("softmax", "silu_mean"):
        for variant in ("mha", "xor_window"):
            a, ha = O.xor_fwd(lc, hs, off, W, heads, 0.5, phi, variant=variant, window=2)
            b, hb = O.xor_fwd(lc, hs, off, W, heads, 0.5, phi, dense=True, variant=variant, window=2)
            err = max(err, float(np.abs(a - b).max()))
            for x, y in zip(ha, hb):
                if x.size:
                    err = max(err, float(np.abs(x - y).max()))
    return err


def pin_window_softmax_vs_sdpa(seed=11):
    """LIME-XOR+Window with softmax: every row equals torch's
    scaled_dot_product_attention over all rows with a boolean mask built
    from the variant's description (links <-> history, plus the history
    band 1 <= |i - j| <= w)."""
    rng = _rng(seed)
    ell, n, d, heads, scale, window = 3, 10, 8, 2, 0.6, 2
    dh = d // heads
    q, k, v = _qkv(rng, ell + n, d)
    y = O.xor_attention(q, k, v, ell, heads, scale, "softmax", "xor_window", window)
    rows = ell + n
    mask = torch.zeros((rows, rows), dtype=torch.bool)
    for i in range(rows):
        for j in range(rows):
            cross = (i < ell) != (j < ell)
            band = i >= ell and j >= ell and 1 <= abs(i - j) <= window
            mask[i, j] = cross or band
    err = 0.0
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    for h in range(heads):
        c = slice(h * dh, (h + 1) * dh)
        ref = F.scaled_dot_product_attention(t(q[:, c]), t(k[:, c]), t(v[:, c]), attn_mask=mask, scale=scale)
        err = max(err, float(np.abs(y[:, c] - ref.numpy()).max()))
    return err


def pin_cache_vs_torch(seed=6):
    """softmax cache == torch.softmax of the per-head logits; silu_mean
    cache == F.silu(logits) / ell; logits from an einsum over d."""
    rng = _rng(seed)
    n, d, H, ell, scale = 37, 16, 3, 5, 0.45
    T = rng.standard_normal((n, d))
    K = rng.standard_normal((H, ell, d))
    logits = torch.einsum("nd,hkd->nhk", torch.from_numpy(T), torch.from_numpy(K)) * scale
    err = float(np.abs(O.qk_cache_build(T, K, scale, "softmax") - torch.softmax(logits, -1).numpy()).max())
    err = max(err, float(np.abs(O.qk_cache_build(T, K, scale, "silu_mean")
                                - (F.silu(logits) / ell).numpy()).max()))
    return err


def pin_cache_silu_odd(seed=7):
    rng = _rng(seed)
    n, d, H, ell, scale = 20, 8, 2, 6, 0.9
    T = rng.standard_normal((n, d)) * 2
    K = rng.standard_normal((H, ell, d))
    diff = O.qk_cache_build(T, K, scale, "silu_mean") - O.qk_cache_build(-T, K, scale, "silu_mean")
    ref = np.stack([scale * T @ K[h].T / ell for h in range(H)], axis=1)
    return float(np.abs(diff - ref).max())


def _brute_cand(cache, lp, ids, off, n_items):
    B, ell, d = lp.shape
    H = cache.shape[1]
    dh = d // H
    out = np.zeros((len(ids), d))
    bad = 0
    for b in range(B):
        for i in range(off[b], off[b + 1]):
            m = int(ids[i])
            if not 0 <= m < n_items:
                bad += 1
                continue
            for c in range(d):
                h = c // dh
                out[i, c] = sum(cache[m, h, k] * lp[b, k, c] for k in range(ell))
    return out, bad


def pin_cand_brute_force(seed=8):
    rng = _rng(seed)
    n, B, ell, d, H = 50, 3, 4, 6, 2
    cache = rng.standard_normal((n, H, ell))
    lp = rng.standard_normal((B, ell, d))
    ids = rng.integers(-3, n + 3, size=23)
    off = np.array([0, 9, 9, 23])
    a, ba = O.cand_score(cache, lp, ids, off)
    b, bb = _brute_cand(cache, lp, ids, off, n)
    return float(np.abs(a - b).max()) + abs(ba - bb)


def _torch_bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns decoded by torch's own bfloat16 -> float64 cast."""
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def pin_bf16_decode():
    """The oracle's decode of bf16 storage (the bits both sides read) against
    torch's bfloat16 -> float64 conversion, over all 65,536 bit patterns:
    normals, subnormals, both zeros, both infinities and every NaN.  Returns
    the largest difference of finite values plus the number of patterns
    whose class (NaN, infinity, sign of zero) disagrees."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    a = O._f64(bits)
    b = _torch_bf16_to_f64(bits)
    if a.dtype != np.float64 or a.shape != b.shape:
        return float("inf")
    fin = np.isfinite(b)
    err = float(np.abs(a[fin] - b[fin]).max()) if fin.any() else 0.0
    bad = int(np.count_nonzero(np.isnan(a) != np.isnan(b)))
    bad += int(np.count_nonzero(np.isinf(a) != np.isinf(b)))
    inf = np.isinf(b)
    bad += int(np.count_nonzero(np.sign(a[inf]) != np.sign(b[inf])))
    zero = b == 0
    bad += int(np.count_nonzero(np.signbit(a[zero]) != np.signbit(b[zero])))
    return err + bad


def pin_bf16_inputs_decode_through_calls(seed=21):
    """The whole calls on bf16 storage arrays (uint16 bits, as the kernels
    read them) against the same calls on those inputs decoded by torch: the
    oracle must compute on exactly the values the bits stand for."""
    rng = _rng(seed)
    B, ell, d, H, n_items = 2, 4, 8, 2, 11
    lens = np.array([5, 3])
    off = np.concatenate([[0], np.cumsum(lens)])

    def bits(shape, std):
        x = (rng.standard_normal(shape) * std).astype(np.float32)
        u = x.view(np.uint32)
        return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)

    lc, hs = bits((B, ell, d), 1.0), bits((int(off[-1]), d), 1.0)
    W = [{k: bits(s, d ** -0.5) for k, s in (("w_qkv", (3 * d, d)), ("w_o", (d, d)), ("w_gate", (d, d)),
                                              ("w_up", (d, d)), ("w_down", (d, d)))}]
    T, K = bits((n_items, d), 1.0), bits((H, ell, d), 1.0)
    ids = rng.integers(0, n_items, size=7)
    coff = np.array([0, 4, 7])
    dec = _torch_bf16_to_f64
    err = 0.0
    for phi in ("softmax", "silu_mean"):
        lp_a, h_a = O.xor_fwd(lc, hs, off, W, H, 0.5, phi)
        lp_b, h_b = O.xor_fwd(dec(lc), dec(hs), off, [{k: dec(v) for k, v in W[0].items()}], H, 0.5, phi)
        c_a = O.qk_cache_build(T, K, 0.5, phi)
        c_b = O.qk_cache_build(dec(T), dec(K), 0.5, phi)
        err = max(err, float(np.abs(lp_a - lp_b).max()),
                  float(np.abs(np.concatenate(h_a) - np.concatenate(h_b)).max()),
                  float(np.abs(c_a - c_b).max()))
    cb = bits((n_items, H, ell), 1.0)
    lpb = bits((B, ell, d), 1.0)
    s_a, _ = O.cand_score(cb, lpb, ids, coff)
    s_b, _ = O.cand_score(dec(cb), dec(lpb), ids, coff)
    return max(err, float(np.abs(s_a - s_b).max()))


ALL_PINS = {
    "dense_equals_decoupled": (pin_dense_equals_decoupled, 1e-12),
    "stack_dense_equals_decoupled": (pin_stack_dense_equals_decoupled, 1e-11),
    "softmax_branches_vs_sdpa": (pin_softmax_branches_vs_sdpa, 1e-12),
    "silu_odd_identity": (pin_silu_odd_identity, 1e-11),
    "layer_vs_torch": (pin_layer_vs_torch, 1e-11),
    "layer_brute_force": (pin_layer_brute_force, 1e-11),
    "cache_vs_torch": (pin_cache_vs_torch, 1e-12),
    "cache_silu_odd": (pin_cache_silu_odd, 1e-12),
    "cand_brute_force": (pin_cand_brute_force, 1e-12),
    "variant_layer_brute_force": (pin_variant_layer_brute_force, 1e-11),
    "variants_dense_equals_decoupled": (pin_variants_dense_equals_decoupled, 1e-11),
    "window_softmax_vs_sdpa": (pin_window_softmax_vs_sdpa, 1e-12),
    "bf16_decode": (pin_bf16_decode, 0.0),
    "bf16_inputs_decode_through_calls": (pin_bf16_inputs_decode_through_calls, 0.0),
}


@pytest.mark.parametrize("name", sorted(ALL_PINS))
def test_pin(name):
    fn, tol = ALL_PINS[name]
    err = fn()
    assert err <= tol, f"{name}: {err}"


# ---------------------------------------------------------------- closed forms

def test_cache_uniform_when_all_keys_equal():
    rng = _rng(10)
    T = rng.standard_normal((9, 8))
    K = np.repeat(rng.standard_normal((2, 1, 8)), 5, axis=1)
    c = O.qk_cache_build(T, K, 0.5, "softmax")
    assert np.abs(c - 1 / 5).max() < 1e-15
    s = O.qk_cache_build(T, K, 0.5, "silu_mean")
    assert np.abs(s - s[:, :, :1]).max() == 0.0


def test_softmax_rows_sum_to_one():
    rng = _rng(11)
    c = O.qk_cache_build(rng.standard_normal((30, 8)) * 3, rng.standard_normal((3, 7, 8)), 1.0, "softmax")
    assert np.abs(c.sum(-1) - 1).max() < 1e-14 and (c >= 0).all()


def test_single_link_softmax_returns_links():
    """ell = 1 with softmax: every cached weight is 1, so O_i = L^P_b."""
    rng = _rng(12)
    cache = O.qk_cache_build(rng.standard_normal((40, 6)), rng.standard_normal((3, 1, 6)), 0.7, "softmax")
    assert np.all(cache == 1.0)
    lp = rng.standard_normal((2, 1, 6))
    ids = rng.integers(0, 40, size=10)
    out, bad = O.cand_score(cache, lp, ids, np.array([0, 4, 10]))
    assert bad == 0
    assert np.abs(out[:4] - lp[0, 0]).max() < 1e-15 and np.abs(out[4:] - lp[1, 0]).max() < 1e-15


def test_single_history_row_softmax():
    """N_b = 1 with softmax: each link's attention output is v of that row."""
    rng = _rng(13)
    q, k, v = _qkv(rng, 6, 8)
    y = O.xor_attention(q, k, v, 5, 2, 0.3, "softmax")
    assert np.abs(y[:5] - v[5]).max() < 1e-15


def test_empty_history_branch_is_zero():
    rng = _rng(14)
    q, k, v = _qkv(rng, 4, 8)
    for phi in ("softmax", "silu_mean"):
        assert np.all(O.xor_attention(q, k, v, 4, 2, 0.3, phi) == 0.0)
        assert np.all(O.xor_attention_dense(q, k, v, 4, 2, 0.3, phi) == 0.0)


def test_xor_mask_blocks():
    m = O.xor_mask(2, 5)
    assert not m[:2, :2].any() and not m[2:, 2:].any() and m[:2, 2:].all() and m[2:, :2].all()


def test_layer_identity_when_projections_zero():
    """W_o = 0 and W_down = 0 make the layer the identity (residual only)."""
    rng = _rng(15)
    lw = _weights(rng, 8, 8)
    lw["w_o"][:] = 0
    lw["w_down"][:] = 0
    x = rng.standard_normal((7, 8))
    assert np.all(O.xor_layer(x, lw, 3, 2, 0.5, "silu_mean") == x)


def test_history_permutation_invariance():
    """No history<->history and no positional term: permuting one user's
    history leaves L^P unchanged and permutes the history outputs."""
    rng = _rng(16)
    B, ell, d, heads = 2, 3, 8, 2
    off = np.array([0, 6, 10])
    lc = rng.standard_normal((B, ell, d))
    hs = rng.standard_normal((10, d))
    W = [_weights(rng, d, d) for _ in range(2)]
    perm = np.concatenate([rng.permutation(6), 6 + rng.permutation(4)])
    for phi in ("softmax", "silu_mean"):
        a, ha = O.xor_fwd(lc, hs, off, W, heads, 0.5, phi)
        b, hb = O.xor_fwd(lc, hs[perm], off, W, heads, 0.5, phi)
        assert np.abs(a - b).max() < 1e-12
        assert np.abs(ha[0][perm[:6]] - hb[0]).max() < 1e-12


def test_users_independent():
    rng = _rng(17)
    B, ell, d = 3, 2, 4
    off = np.array([0, 3, 5, 9])
    lc = rng.standard_normal((B, ell, d))
    hs = rng.standard_normal((9, d))
    W = [_weights(rng, d, d)]
    a, _ = O.xor_fwd(lc, hs, off, W, 1, 0.5, "softmax")
    b, _ = O.xor_fwd(lc[1:2], hs[3:5], np.array([0, 2]), W, 1, 0.5, "softmax")
    assert np.array_equal(a[1], b[0])


def test_candidate_independence_and_bad_ids():
    rng = _rng(18)
    n, B, ell, d, H = 30, 2, 4, 8, 2
    cache = rng.standard_normal((n, H, ell))
    lp = rng.standard_normal((B, ell, d))
    ids = rng.integers(0, n, size=12)
    off = np.array([0, 5, 12])
    full, bad = O.cand_score(cache, lp, ids, off)
    assert bad == 0
    # one candidate alone
    one, _ = O.cand_score(cache, lp[1:2], ids[7:8], np.array([0, 1]))
    assert np.array_equal(one[0], full[7])
    # permuted and duplicated candidate lists
    p = rng.permutation(7) + 5
    dup = np.concatenate([ids[p], ids[p[:3]]])
    pd, _ = O.cand_score(cache, lp[1:2], dup, np.array([0, len(dup)]))
    assert np.array_equal(pd[:7], full[p]) and np.array_equal(pd[7:], full[p[:3]])
    # out-of-range ids: zero rows, counted
    bad_ids = ids.copy()
    bad_ids[[1, 8]] = [-1, n]
    o2, nb = O.cand_score(cache, lp, bad_ids, off)
    assert nb == 2 and np.all(o2[[1, 8]] == 0) and np.array_equal(np.delete(o2, [1, 8], 0), np.delete(full, [1, 8], 0))


def test_cached_equals_recomputed():
    """Cached weights of a sampled id equal phi(scale K_L T_m) computed fresh
    for that item alone."""
    rng = _rng(19)
    T = rng.standard_normal((100, 8))
    K = rng.standard_normal((2, 4, 8))
    c = O.qk_cache_build(T, K, 0.5, "silu_mean")
    for m in (0, 17, 99):
        # equal up to the BLAS kernel's summation order
        assert np.abs(c[m] - O.qk_cache_build(T[m:m + 1], K, 0.5, "silu_mean")[0]).max() < 1e-15


def test_cache_size_matches_table12():
    """Cache bytes = items * heads * ell * bytes/elem reproduce the int8 cache
    sizes printed in the LIME summary page, Table 12 (100M items, 4 heads)."""
    with open(os.path.join(GOLDEN, "table12_int8_cache_size.json")) as f:
        g = json.load(f)
    rng = _rng(20)
    for ell_s, gb in g["int8_cache_gb_by_links"].items():
        ell = int(ell_s)
        c = O.qk_cache_build(rng.standard_normal((3, 8)), rng.standard_normal((g["heads"], ell, 8)), 1.0, "softmax")
        per_item = c.shape[1] * c.shape[2]  # one weight per (head, link)
        assert per_item * g["items"] * g["bytes_per_weight"] / 1e9 == pytest.approx(gb, rel=1e-9)


# ---------------------------------------------------------------- int8 cache, uncached scoring

def test_int8_codes_within_half_a_step():
    """|dequantised - w| <= scale/2 (the rounding bound), codes in [-127, 127],
    the largest magnitude of each row maps to +-127 exactly."""
    rng = _rng(21)
    w = np.concatenate([rng.standard_normal((50, 3, 32)) * 0.05,
                        np.abs(rng.standard_normal((5, 3, 32))) / 32], axis=0)
    w[7, 1] = 0.0
    q, s = O.quantize_i8(w)
    assert q.dtype == np.int8 and s.dtype == np.float32 and s.shape == (55, 3)
    w32 = w.astype(np.float32).astype(np.float64)
    err = np.abs(O.dequantize_i8(q, s) - w32)
    assert np.all(err <= s[..., None].astype(np.float64) * (0.5 + 1e-6) + 1e-12)
    assert np.all(np.abs(q.astype(int)) <= 127)
    mx = np.abs(q.astype(int)).max(-1)
    assert np.all(mx[s > 0] == 127) and np.all(q[7, 1] == 0) and s[7, 1] == 0


def test_int8_scoring_is_scoring_of_dequantised_cache():
    rng = _rng(22)
    cache = np.abs(rng.standard_normal((40, 2, 8))) / 8
    q, s = O.quantize_i8(cache)
    lp = rng.standard_normal((3, 8, 16))
    ids = rng.integers(0, 40, size=20)
    off = np.array([0, 5, 5, 20])
    a, _ = O.cand_score_i8(q, s, lp, ids, off)
    b, _ = _brute_cand(q.astype(np.float64) * s[..., None], lp, ids, off, 40)
    assert np.abs(a - b).max() < 1e-12
    # and within the quantisation error of the float scores
    c, _ = O.cand_score(cache, lp, ids, off)
    assert np.abs(a - c).max() <= (s.max() / 2) * np.abs(lp).sum(1).max() + 1e-12


def test_uncached_equals_cache_then_score():
    rng = _rng(23)
    T = rng.standard_normal((30, 8))
    K = rng.standard_normal((2, 4, 8))
    lp = rng.standard_normal((2, 4, 8))
    ids = rng.integers(-2, 32, size=11)
    off = np.array([0, 6, 11])
    for phi in ("softmax", "silu_mean"):
        a, na = O.cand_score_uncached(T, K, 0.4, phi, lp, ids, off)
        b, nb = _brute_cand(O.qk_cache_build(T, K, 0.4, phi), lp, ids, off, 30)
        assert na == nb == int(((ids < 0) | (ids >= 30)).sum())
        assert np.abs(a - b).max() < 1e-12


# ---------------------------------------------------------------- mutation tests

def test_window_zero_is_plain_xor():
    rng = _rng(30)
    ell, n, d, heads = 3, 7, 8, 2
    q, k, v = _qkv(rng, ell + n, d)
    for phi in ("softmax", "silu_mean"):
        a = O.xor_attention(q, k, v, ell, heads, 0.5, phi, "xor_window", 0)
        b = O.xor_attention(q, k, v, ell, heads, 0.5, phi)
        assert np.abs(a - b).max() < 1e-14


def test_mha_first_layer_links_equal_xor_and_history_passes():
    """In the first layer the link rows see only LN(E) and LN(L^C), so
    LIME-MHA and LIME-XOR agree on them; LIME-MHA leaves history rows as
    they came in, whatever the depth."""
    rng = _rng(31)
    B, ell, d, heads = 2, 4, 8, 2
    off = np.array([0, 6, 11])
    lc = rng.standard_normal((B, ell, d))
    hs = rng.standard_normal((11, d))
    W = [_weights(rng, d, d) for _ in range(3)]
    for phi in ("softmax", "silu_mean"):
        a, _ = O.xor_fwd(lc, hs, off, W[:1], heads, 0.5, phi, variant="mha")
        b, _ = O.xor_fwd(lc, hs, off, W[:1], heads, 0.5, phi)
        assert np.abs(a - b).max() < 1e-13
        _, ho = O.xor_fwd(lc, hs, off, W, heads, 0.5, phi, variant="mha")
        for bb, x in enumerate(ho):
            assert np.array_equal(x, hs[off[bb]:off[bb + 1]])


def test_window_reversal_symmetry():
    """The window reaches equally far before and after: reversing every
    history keeps L^P and reverses the history outputs."""
    rng = _rng(32)
    B, ell, d, heads = 2, 4, 8, 2
    lens = [9, 5]
    off = np.array([0, 9, 14])
    lc = rng.standard_normal((B, ell, d))
    hs = rng.standard_normal((14, d))
    rev = np.concatenate([hs[off[b]:off[b + 1]][::-1] for b in range(B)])
    W = [_weights(rng, d, d) for _ in range(2)]
    for phi in ("softmax", "silu_mean"):
        a, ha = O.xor_fwd(lc, hs, off, W, heads, 0.5, phi, variant="xor_window", window=2)
        b, hb = O.xor_fwd(lc, rev, off, W, heads, 0.5, phi, variant="xor_window", window=2)
        assert np.abs(a - b).max() < 1e-12
        for x, y, nb in zip(ha, hb, lens):
            assert x.shape[0] == nb and np.abs(x - y[::-1]).max() < 1e-12


def test_window_changes_history_rows_only_through_neighbours():
    """Perturbing history row j's key and value changes the attention
    output of every link row and of the history rows within w of j, and of
    no other row."""
    rng = _rng(33)
    ell, n, d, heads, window = 2, 12, 4, 1, 2
    q, k, v = _qkv(rng, ell + n, d)
    y0 = O.xor_attention(q, k, v, ell, heads, 0.5, "softmax", "xor_window", window)
    k2, v2 = k.copy(), v.copy()
    j = ell + 9
    k2[j] += 1.0
    v2[j] -= 1.0
    y1 = O.xor_attention(q, k2, v2, ell, heads, 0.5, "softmax", "xor_window", window)
    changed = np.nonzero(np.abs(y1 - y0).max(axis=1) > 0)[0]
    expect = set(range(ell)) | {i for i in range(ell, ell + n) if 1 <= abs(i - j) <= window}
    assert set(changed.tolist()) == expect


def test_default_window_gives_two_ell_keys():
    ell = 32
    w = O.default_window(ell)
    assert len(O.window_neighbours(100, 1000, w)) + ell == 2 * ell


def _mutations():
    def silu_norm_off(s, phi):
        n = s.shape[-1]
        if phi == "silu_mean" and n:
            return O.silu(s) / (n + 1)
        return ORIG["phi_weights"](s, phi)

    def no_max_shift_wrong_sum(s, phi):
        if phi == "softmax" and s.shape[-1]:
            e = np.exp(s)
            return e / (e.sum(axis=-1, keepdims=True) + 1e-3)
        return ORIG["phi_weights"](s, phi)

    def ln_unbiased(x, eps=1e-5):
        mu = x.mean(axis=-1, keepdims=True)
        return (x - mu) / np.sqrt(x.var(axis=-1, ddof=1, keepdims=True) + eps)

    def attend_wrong_scale(q, k, v, scale, phi):
        return ORIG["attend"](q, k, v, 1.0, phi)

    def attend_transposed_v(q, k, v, scale, phi):
        if k.shape[0] == 0:
            return np.zeros((q.shape[0], v.shape[1]))
        w = ORIG["phi_weights"](scale * (q @ k.T), phi)
        return w @ v[::-1]

    def silu_sign(s):
        return -s * O._sigmoid(-s)

    def window_with_self(p, n, window):
        q = np.arange(max(0, p - window), min(n, p + window + 1))
        return q

    def window_one_sided(p, n, window):
        return np.arange(max(0, p - window), p)

    def bf16_wrong_shift(a):
        a = np.asarray(a)
        if a.dtype == np.uint16:
            return (a.astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64)
        return a.astype(np.float64)

    def bf16_read_as_half(a):
        a = np.asarray(a)
        if a.dtype == np.uint16:
            return a.view(np.float16).astype(np.float64)
        return a.astype(np.float64)

    return {
        "bf16 decode shifted by 15 bits": ("_f64", bf16_wrong_shift),
        "bf16 bits read as float16": ("_f64", bf16_read_as_half),
        "window includes the row itself": ("window_neighbours", window_with_self),
        "window reaches only backwards": ("window_neighbours", window_one_sided),
        "silu normaliser off by one": ("phi_weights", silu_norm_off),
        "softmax denominator perturbed": ("phi_weights", no_max_shift_wrong_sum),
        "LayerNorm with unbiased variance": ("layer_norm", ln_unbiased),
        "attention scale dropped": ("attend", attend_wrong_scale),
        "values taken from the wrong rows": ("attend", attend_transposed_v),
        "SiLU sign error": ("silu", silu_sign),
    }


ORIG = {k: getattr(O, k) for k in ("phi_weights", "layer_norm", "attend", "silu", "window_neighbours")}


@pytest.mark.parametrize("name", sorted(_mutations()))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = _mutations()[name]
    monkeypatch.setattr(O, attr, fn)
    failed = []
    for pin, (f, tol) in ALL_PINS.items():
        try:
            err = f()
        except Exception:
            err = float("inf")
        if not err <= tol:
            failed.append(pin)
    assert failed, f"no pin caught: {name}"
