"""CPU oracle for the LIME inference hot path (NumPy, float64).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the bench's CPU
baseline leg use it.  It shares no code with the HIP path; the two meet only
through the seeded inputs of the ``workloads`` module.

Everything here is the plain definition, written slowly and in float64:
inputs are decoded exactly from their storage type and nothing is rounded
afterwards.  Sources (the LIME pages):

* LIME notes (papernotes.org), "Key design 1": the candidate side computes
  O = MHA(T, L, L^P; J) = phi(T L^T) L^P with an all-ones mask J, phi being
  a scaled softmax or SiLU; the weights phi(T L^T) depend on the item and
  the global links only, so they are computed offline into a QK cache and
  each candidate's output is a lookup plus an ell-wide weighted sum
  ("complete example", steps 1 and 3).
* LIME notes, "Key design 2": XOR attention over X = E (+) L^C equals the
  sum of two cross attentions, history -> context links and context links
  -> history, with no history<->history or link<->link terms (the XORA
  equation; its mask is the exclusive-or of block membership).  Layers are
  stacked with residuals and a gated MLP.
* LIME notes, "Loss / training strategy": LayerNorm is applied before the
  query/key projections; softmax is used for single-layer attention and
  SiLU for deep stacks.
* LIME summary page, Table 12 caption: the cache holds, per item, one
  weight per (head, link).

Readings where the pages are silent (each is a choice of this oracle):

* XOR mask = [i is a link] xor [j is a link] (the printed symbol is an AND,
  which would keep exactly the block the text says is removed).
* phi = "softmax": softmax over the keys a row may attend; phi =
  "silu_mean": SiLU(s) divided by the number of keys the row may attend
  (ell for history rows and for the cache, N_b for link rows).  A row with
  no keys (empty history) outputs 0.
* scale is an explicit argument (usually 1/sqrt(d_h)), used by both phis.
* Heads are column slices of width d_h = d / heads.
* Layer = pre-LN (no affine, eps 1e-5, population variance) -> shared
  W_qkv -> XOR attention -> W_o + residual -> pre-LN -> SwiGLU MLP
  (SiLU(G Wg^T) * (G Wu^T)) Wd^T + residual.  No positional terms, no final
  LN.  Weights are [out, in] (y = x @ W.T); W_qkv rows are Q, K, V.
* The candidate-side query/key projections fold into a per-head key tensor
  link_keys[h] in R^{ell x d}; values are the head slices of L^P.
* An out-of-range candidate id yields a zero output row and is counted.
* Int8 cache (the pages give "Int8 lookup+dequant" and int8 cache sizes,
  LIME summary page, Tables 10 and 12, but no scheme): symmetric codes in
  [-127, 127] with one float32 scale per (item, head), scale = max|w|/127,
  code = round-half-even(w * 127/max|w|).  Codes are an integer decision
  made in float32, as the kernel makes it.
* Uncached scoring (the pages' "Uncached global" column, Table 10; the
  cold-start fallback in the limitations section) is the cache formula
  evaluated per candidate and then the same weighted sum.

* LIME-MHA (LIME summary page, Fig. 2; LIME notes, experiments table:
  "single-layer decoupled"): only the links -> history cross attention
  runs; history rows are not updated by any layer and pass through.  The
  link rows keep the rest of the layer (W_o + residual, gated MLP).
* LIME-XOR+Window (LIME notes, Key design 3; Table 13): besides the ell
  links, history row p also attends the history rows q with
  1 <= |p - q| <= w (its neighbours before and after, itself excluded),
  under one joint phi over the union.  The default half-width w = ell / 2
  gives each row 2 ell keys, the context size the notes state.  The
  silu_mean normaliser counts the union.  Link rows are unchanged.

Parity unpinned: the layer internals beyond attention (LN placement, the
SwiGLU MLP, residual order) are readings; they are pinned only by brute
force against this module's own definitions, not by any number the pages
print.  The pages print no input/output values for any function.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "layer_norm", "silu", "phi_weights", "attend", "xor_attention",
    "xor_attention_dense", "xor_mask", "xor_layer", "xor_fwd",
    "qk_cache_build", "cand_score", "quantize_i8", "dequantize_i8",
    "cand_score_i8", "cand_score_uncached", "VARIANTS", "window_neighbours",
    "default_window",
]

# user-side variants: plain XOR attention, LIME-MHA (links -> history only),
# LIME-XOR+Window (history rows also see a local window of history rows)
VARIANTS = ("xor", "mha", "xor_window")

LN_EPS = 1e-5


def _f64(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.uint16:  # bf16 bit patterns
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def layer_norm(x: np.ndarray, eps: float = LN_EPS) -> np.ndarray:
    """Per-row LayerNorm without affine parameters (LIME notes, training
    strategy: LN before the QK projections)."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps)


def _sigmoid(s: np.ndarray) -> np.ndarray:
    # 1 / (1 + exp(-s)) written so that neither tail overflows
    return np.exp(-np.logaddexp(0.0, -s))


def silu(s: np.ndarray) -> np.ndarray:
    return s * _sigmoid(s)


def phi_weights(s: np.ndarray, phi: str) -> np.ndarray:
    """Attention weights over the last axis, which holds exactly the keys
    the row may attend (LIME notes, Key design 1: phi is a scaled softmax or
    SiLU; reading: SiLU is divided by the number of allowed keys)."""
    n = s.shape[-1]
    if n == 0:
        return s.copy()
    if phi == "softmax":
        e = np.exp(s - s.max(axis=-1, keepdims=True))
        return e / e.sum(axis=-1, keepdims=True)
    if phi == "silu_mean":
        return silu(s) / n
    raise ValueError(phi)


def attend(q, k, v, scale: float, phi: str) -> np.ndarray:
    """Cross attention of queries q [nq, dh] to keys k / values v [nk, dh]."""
    if k.shape[0] == 0:
        return np.zeros((q.shape[0], v.shape[1]))
    return phi_weights(scale * (q @ k.T), phi) @ v


def default_window(n_links: int) -> int:
    """Half-width of the LIME-XOR+Window neighbourhood: ell / 2 on each
    side, so that a history row sees ell links plus ell neighbours."""
    return max(1, n_links // 2)


def window_neighbours(p: int, n: int, window: int) -> np.ndarray:
    """History positions q in [0, n) with 1 <= |p - q| <= window."""
    q = np.arange(max(0, p - window), min(n, p + window + 1))
    return q[q != p]


def xor_attention(q, k, v, n_links: int, heads: int, scale: float, phi: str,
                  variant: str = "xor", window: int = 0) -> np.ndarray:
    """Decoupled XOR attention for one user (LIME notes, Key design 2, XORA
    equation): rows [0, n_links) are the context links, the rest history.
    History rows attend to the links only; link rows attend to the history
    only.  variant "mha" drops the history -> links branch (history rows get
    no attention output); "xor_window" lets history row p also attend the
    history rows of ``window_neighbours`` with one phi over the union (LIME
    notes, Key design 3)."""
    if variant not in VARIANTS:
        raise ValueError(variant)
    rows, d = q.shape
    dh = d // heads
    n = rows - n_links
    y = np.zeros((rows, d))
    L, E = slice(0, n_links), slice(n_links, rows)
    for h in range(heads):
        c = slice(h * dh, (h + 1) * dh)
        y[L, c] = attend(q[L, c], k[E, c], v[E, c], scale, phi)   # MHA(L^C, E, E)
        if variant == "xor":
            y[E, c] = attend(q[E, c], k[L, c], v[L, c], scale, phi)   # MHA(E, L^C, L^C)
        elif variant == "xor_window":
            for p in range(n):
                keys = np.concatenate([np.arange(n_links), n_links + window_neighbours(p, n, window)])
                i = n_links + p
                y[i:i + 1, c] = attend(q[i:i + 1, c], k[keys, c], v[keys, c], scale, phi)
    return y


def xor_mask(n_links: int, rows: int, variant: str = "xor", window: int = 0) -> np.ndarray:
    """M[i, j] = [i is a link] xor [j is a link] (block anti-diagonal).
    "mha" keeps only the link rows of it; "xor_window" adds the history
    band 1 <= |i - j| <= window."""
    is_link = np.arange(rows) < n_links
    m = is_link[:, None] ^ is_link[None, :]
    if variant == "mha":
        m &= is_link[:, None]
    elif variant == "xor_window":
        i = np.arange(rows)
        dist = np.abs(i[:, None] - i[None, :])
        m |= (~is_link[:, None]) & (~is_link[None, :]) & (dist >= 1) & (dist <= window)
    elif variant != "xor":
        raise ValueError(variant)
    return m


def xor_attention_dense(q, k, v, n_links: int, heads: int, scale: float, phi: str,
                        variant: str = "xor", window: int = 0) -> np.ndarray:
    """The same attention as dense masked self-attention over the whole
    concatenated sequence (the form the XOR mask defines)."""
    rows, d = q.shape
    dh = d // heads
    m = xor_mask(n_links, rows, variant, window)
    cnt = m.sum(axis=1, keepdims=True)
    y = np.zeros((rows, d))
    for h in range(heads):
        c = slice(h * dh, (h + 1) * dh)
        s = scale * (q[:, c] @ k[:, c].T)
        if phi == "softmax":
            s = np.where(m, s, -np.inf)
            mx = s.max(axis=1, keepdims=True)
            mx = np.where(np.isfinite(mx), mx, 0.0)
            e = np.where(m, np.exp(s - mx), 0.0)
            den = e.sum(axis=1, keepdims=True)
            w = np.divide(e, den, out=np.zeros_like(e), where=den > 0)
        else:
            w = np.where(m, silu(s), 0.0)
            w = np.divide(w, cnt, out=np.zeros_like(w), where=cnt > 0)
        y[:, c] = w @ v[:, c]
    return y


def xor_layer(x, lw: dict, n_links: int, heads: int, scale: float, phi: str,
              dense: bool = False, variant: str = "xor", window: int = 0) -> np.ndarray:
    """One LIME-XOR layer (LIME notes, Key design 2: residual + gated MLP;
    training strategy: LN before the projections).  ``lw`` holds float64
    weights in [out, in] layout.  With variant "mha" the history rows pass
    through unchanged."""
    d = x.shape[1]
    h = layer_norm(x)
    qkv = h @ lw["w_qkv"].T
    q, k, v = qkv[:, :d], qkv[:, d:2 * d], qkv[:, 2 * d:]
    att = xor_attention_dense if dense else xor_attention
    y = att(q, k, v, n_links, heads, scale, phi, variant, window)
    x1 = x + y @ lw["w_o"].T
    g = layer_norm(x1)
    out = x1 + (silu(g @ lw["w_gate"].T) * (g @ lw["w_up"].T)) @ lw["w_down"].T
    if variant == "mha":
        out[n_links:] = x[n_links:]
    return out


def xor_fwd(links_ctx, hist, hist_offsets, weights, heads: int, scale: float, phi: str,
            users=None, dense: bool = False, variant: str = "xor", window: int | None = None):
    """User-side encoder: stacked XOR layers over [L^C_b ; E_b] for each user.

    links_ctx [B, ell, d], hist [sum N, d], hist_offsets [B+1], weights a
    list of per-layer dicts.  Returns (links_pers [B', ell, d], hist_out list
    of [N_b, d] arrays) for the users in ``users`` (default all).  variant
    and window select LIME-MHA or LIME-XOR+Window (window defaults to
    ell / 2 for the latter)."""
    lc = _f64(links_ctx)
    hs = hist
    off = np.asarray(hist_offsets, dtype=np.int64)
    W = [{k: _f64(v) for k, v in lw.items()} for lw in weights]
    B, ell, _ = lc.shape
    if variant not in VARIANTS:
        raise ValueError(variant)
    if variant == "xor_window":
        window = default_window(ell) if window is None else int(window)
    else:
        window = 0
    users = range(B) if users is None else users
    lp, ho = [], []
    for b in users:
        x = np.concatenate([lc[b], _f64(hs[off[b]:off[b + 1]])], axis=0)
        for lw in W:
            x = xor_layer(x, lw, ell, heads, scale, phi, dense=dense, variant=variant, window=window)
        lp.append(x[:ell])
        ho.append(x[ell:])
    return np.stack(lp), ho


def qk_cache_build(items, link_keys, scale: float, phi: str) -> np.ndarray:
    """QK cache: cache[m, h, :] = phi(scale * link_keys[h] @ T_m) over the
    ell links of head h (LIME notes, Key design 1 and the offline stage of
    the framework; LIME summary page, Table 12: per item, per head, ell
    weights)."""
    t = _f64(items)
    kl = _f64(link_keys)
    H, ell, _ = kl.shape
    out = np.empty((t.shape[0], H, ell))
    for h in range(H):
        out[:, h, :] = phi_weights(scale * (t @ kl[h].T), phi)
    return out


def cand_score(cache, links_pers, cand_ids, cand_offsets, n_items: int | None = None):
    """Candidate scoring: O_i = phi(T_i L^T) L^P_b, i.e. the cached weights
    of item id_i times user b's personalised links, per head (LIME notes,
    complete example step 3: a lookup plus an ell-wide weighted sum).

    Returns (O [total_M, d], number of out-of-range ids)."""
    c = _f64(cache)
    lp = _f64(links_pers)
    ids = np.asarray(cand_ids, dtype=np.int64)
    off = np.asarray(cand_offsets, dtype=np.int64)
    n_items = c.shape[0] if n_items is None else n_items
    B, ell, d = lp.shape
    H = c.shape[1]
    dh = d // H
    out = np.zeros((ids.shape[0], d))
    bad = 0
    lp_heads = lp.reshape(B, ell, H, dh)
    for b in range(B):
        sl = slice(off[b], off[b + 1])
        m = ids[sl]
        ok = (m >= 0) & (m < n_items)
        bad += int((~ok).sum())
        w = c[m[ok]]                                          # [n_ok, H, ell]
        o = np.einsum("nhk,khc->nhc", w, lp_heads[b])         # per head: w_h @ L^P_b[:, h]
        blk = np.zeros((m.shape[0], d))
        blk[ok] = o.reshape(-1, d)
        out[sl] = blk
    return out, bad


def quantize_i8(cache):
    """Symmetric int8 codes and float32 scales per (item, head) of a cache
    [n, H, ell] (reading: scheme unstated on the pages).  The decision is
    taken in float32: w32 = float32(w), m = max|w32|, code = rint(w32 *
    (127/m)) clipped to [-127, 127], scale = m/127; an all-zero row gets
    scale 0 and codes 0."""
    w = np.asarray(cache, dtype=np.float64).astype(np.float32)
    m = np.abs(w).max(axis=-1, keepdims=True)
    with np.errstate(divide="ignore"):
        inv = np.where(m > 0, np.float32(127.0) / m, np.float32(0.0)).astype(np.float32)
    q = np.clip(np.rint((w * inv).astype(np.float32)), -127, 127).astype(np.int8)
    scale = (m[..., 0] / np.float32(127.0)).astype(np.float32)
    return q, scale


def dequantize_i8(codes, scales):
    return np.asarray(codes, dtype=np.float64) * np.asarray(scales, dtype=np.float64)[..., None]


def cand_score_i8(codes, scales, links_pers, cand_ids, cand_offsets, n_items=None):
    """Scoring from the int8 cache: dequantise the gathered rows, then the
    same weighted sum as cand_score (LIME summary page, Table 10: int8
    lookup + dequant)."""
    return cand_score(dequantize_i8(codes, scales), links_pers, cand_ids, cand_offsets,
                      n_items=n_items)


def cand_score_uncached(items, link_keys, scale: float, phi: str, links_pers, cand_ids,
                        cand_offsets):
    """Scoring without a cache: the cache row of each candidate's item is
    computed on the spot (LIME summary page, Table 10, "Uncached global"),
    then the weighted sum.  Out-of-range ids give zero rows and are
    counted."""
    t = np.asarray(items)
    ids = np.asarray(cand_ids, dtype=np.int64)
    n = t.shape[0]
    ok = (ids >= 0) & (ids < n)
    uniq, inv = np.unique(ids[ok], return_inverse=True)
    rows = qk_cache_build(t[uniq], link_keys, scale, phi)
    remap = np.full(ids.shape[0], -1, dtype=np.int64)
    remap[ok] = inv
    return cand_score(rows, links_pers, remap, cand_offsets, n_items=len(uniq))
