"""Seeded synthetic inputs for the LIME inference hot path.

This module is shared by the CPU oracle and the HIP path's tests and bench.
It holds none of the method's arithmetic: it only draws random numbers,
rounds them to the storage type, samples candidate ids and builds jagged
offsets.  Both sides receive the identical bytes it produces.

Workload shapes follow the problem sizes of the LIME pages (LIME summary
page, Table 8 hyper-parameters and Tables 10/12 candidate-side scaling;
LIME notes on papernotes.org, "complete example" section).  The recipe:

* Every tensor has its own random stream, keyed by (seed, tensor name,
  chunk index) through ``numpy.random.SeedSequence`` and drawn with PCG64,
  so any tensor can be regenerated alone and large tensors are drawn in
  parallel chunks.
* Embeddings and weights are N(0, 1/d) (std d**-0.5; ``W_down`` uses
  d_ff**-0.5).  "Stress" mode draws the link keys and the context links at
  unit variance so that the attention nonlinearity is actually exercised.
* Values are drawn in float32 and, for bf16 workloads, rounded to bf16 with
  round-to-nearest-even.  bf16 tensors are held as uint16 bit patterns.
* Candidate ids are uniform for the tiny workload and otherwise follow a
  finite Zipf(s) law over ranks 1..n_items (inverse CDF of the cumulative
  k**-s), mapped to ids through a seeded permutation so hot ids are not
  adjacent; draws are with replacement.
* Ragged history lengths (lifelong workload) are uniform integers in the
  stated range; offsets are their exclusive prefix sum.
"""
from __future__ import annotations

import dataclasses
import hashlib
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "workload", "normal", "round_bf16", "bf16_to_f32",
    "as_storage", "storage_to_f64", "lengths", "offsets_from_lengths",
    "candidate_ids", "candidate_offsets", "layer_weights", "user_inputs",
    "cache_inputs", "links_pers", "scale_for",
]

_CHUNK = 1 << 22


@dataclasses.dataclass(frozen=True)
class Workload:
    """One named problem size.  ``N`` is an int or an inclusive (lo, hi) range."""
    name: str
    index: int
    dtype: str          # "f32" or "bf16"
    B: int
    N: object
    ell: int
    d: int
    heads: int
    layers: int
    n_items: int
    M: int
    zipf: float | None  # None means uniform ids
    phi: str            # "softmax" or "silu_mean"
    d_ff: int = 0       # 0 means d_ff = d

    @property
    def seed(self) -> int:
        return 1000 + self.index

    @property
    def dff(self) -> int:
        return self.d_ff or self.d

    @property
    def dh(self) -> int:
        return self.d // self.heads

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 1, "f32", B=4, N=64, ell=8, d=32, heads=1, layers=1,
                     n_items=1000, M=16, zipf=None, phi="softmax"),
    "ctr": Workload("ctr", 2, "bf16", B=256, N=50, ell=32, d=64, heads=2, layers=2,
                    n_items=100_000, M=32, zipf=1.1, phi="silu_mean"),
    "long": Workload("long", 3, "bf16", B=64, N=4096, ell=32, d=128, heads=4, layers=4,
                     n_items=1_000_000, M=1024, zipf=1.1, phi="silu_mean"),
    "large_m": Workload("large_m", 4, "bf16", B=16, N=1024, ell=32, d=128, heads=4, layers=2,
                        n_items=10_000_000, M=65536, zipf=1.05, phi="silu_mean"),
    "lifelong": Workload("lifelong", 5, "bf16", B=8, N=(8192, 16384), ell=64, d=256, heads=8,
                         layers=4, n_items=4_000_000, M=8192, zipf=1.1, phi="silu_mean"),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def scale_for(w: Workload) -> float:
    """The default attention scale, 1/sqrt(d_h)."""
    return float(w.dh) ** -0.5


# --------------------------------------------------------------------------
# random streams
# --------------------------------------------------------------------------

def _key(name: str) -> int:
    return int.from_bytes(hashlib.blake2b(name.encode(), digest_size=8).digest(), "little")


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal(seed: int, name: str, shape, std: float) -> np.ndarray:
    """float32 N(0, std**2) array, reproducible per (seed, name) and chunked."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    out = np.empty(n, dtype=np.float32)
    k = _key(name)
    chunks = [(i, min(n, i + _CHUNK)) for i in range(0, n, _CHUNK)]

    def fill(ci):
        lo, hi = chunks[ci]
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, k, ci])))
        g.standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])
        out[lo:hi] *= np.float32(std)

    if len(chunks) <= 1:
        for ci in range(len(chunks)):
            fill(ci)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(len(chunks))))
    return out.reshape(shape)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float32 values."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def as_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values -> storage array (float32, or uint16 bf16 bits)."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return round_bf16(x)
    raise ValueError(dtype)


def storage_to_f64(a: np.ndarray) -> np.ndarray:
    """Decode a storage array (float32 or uint16 bf16 bits) to float64."""
    if a.dtype == np.uint16:
        return bf16_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------
# shapes and ids
# --------------------------------------------------------------------------

def lengths(w: Workload, B: int | None = None) -> np.ndarray:
    B = w.B if B is None else B
    if isinstance(w.N, tuple):
        lo, hi = w.N
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, _key("lengths")])))
        return g.integers(lo, hi + 1, size=B, dtype=np.int64)
    return np.full(B, int(w.N), dtype=np.int64)


def offsets_from_lengths(lens) -> np.ndarray:
    lens = np.asarray(lens, dtype=np.int64)
    off = np.zeros(len(lens) + 1, dtype=np.int64)
    np.cumsum(lens, out=off[1:])
    return off


def candidate_ids(w: Workload, total: int | None = None, uniform: bool = False) -> np.ndarray:
    """int64 candidate ids, ``total`` of them (default B*M), with replacement."""
    total = w.B * w.M if total is None else int(total)
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, _key("ids")])))
    if w.zipf is None or uniform:
        return g.integers(0, w.n_items, size=total, dtype=np.int64)
    ranks = np.arange(1, w.n_items + 1, dtype=np.float64)
    cdf = np.cumsum(ranks ** (-float(w.zipf)))
    cdf /= cdf[-1]
    u = g.random(total)
    r = np.minimum(np.searchsorted(cdf, u, side="right"), w.n_items - 1)
    pg = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, _key("perm")])))
    perm = pg.permutation(w.n_items).astype(np.int64)
    return perm[r]


def candidate_offsets(w: Workload, B: int | None = None) -> np.ndarray:
    B = w.B if B is None else B
    return offsets_from_lengths(np.full(B, w.M, dtype=np.int64))


# --------------------------------------------------------------------------
# tensors of one workload
# --------------------------------------------------------------------------

def layer_weights(w: Workload) -> list[dict]:
    """Per-layer weights in [out, in] row-major layout (y = x @ W.T), storage dtype."""
    d, f = w.d, w.dff
    out = []
    for l in range(w.layers):
        lw = {
            "w_qkv": normal(w.seed, f"w_qkv.{l}", (3 * d, d), d ** -0.5),
            "w_o": normal(w.seed, f"w_o.{l}", (d, d), d ** -0.5),
            "w_gate": normal(w.seed, f"w_gate.{l}", (f, d), d ** -0.5),
            "w_up": normal(w.seed, f"w_up.{l}", (f, d), d ** -0.5),
            "w_down": normal(w.seed, f"w_down.{l}", (d, f), f ** -0.5),
        }
        out.append({k: as_storage(v, w.dtype) for k, v in lw.items()})
    return out


def user_inputs(w: Workload, stress: bool = False) -> dict:
    """links_ctx [B, ell, d], hist [sum N, d], hist_offsets [B+1], weights."""
    lens = lengths(w)
    off = offsets_from_lengths(lens)
    std_l = 1.0 if stress else w.d ** -0.5
    links = normal(w.seed, "links_ctx", (w.B, w.ell, w.d), std_l)
    hist = normal(w.seed, "hist", (int(off[-1]), w.d), w.d ** -0.5)
    return {
        "links_ctx": as_storage(links, w.dtype),
        "hist": as_storage(hist, w.dtype),
        "hist_offsets": off,
        "weights": layer_weights(w),
    }


def cache_inputs(w: Workload, stress: bool = False, n_items: int | None = None) -> dict:
    """items [n_items, d] and link_keys [heads, ell, d] in storage dtype."""
    n = w.n_items if n_items is None else int(n_items)
    std_k = 1.0 if stress else w.d ** -0.5
    keys = normal(w.seed, "link_keys", (w.heads, w.ell, w.d), std_k)
    items = normal(w.seed, "items", (n, w.d), w.d ** -0.5)
    return {"items": as_storage(items, w.dtype), "link_keys": as_storage(keys, w.dtype)}


def links_pers(w: Workload, stress: bool = False) -> np.ndarray:
    """A stand-in personalised-link tensor [B, ell, d] for scoring-only tests."""
    std = 1.0 if stress else w.d ** -0.5
    return as_storage(normal(w.seed, "links_pers", (w.B, w.ell, w.d), std), w.dtype)
