"""Helpers shared by the GPU parity tests: moving seeded inputs to the
device bit-exactly, decoding results, and the tolerance rule
max|gpu - ref| <= tol * max|ref| per output tensor (1e-4 for float32 and
2e-2 for bf16 element types)."""
from __future__ import annotations

import functools

import numpy as np
import torch

import workloads as W

TOL = {"f32": 1e-4, "bf16": 2e-2}


def dev(a: np.ndarray) -> torch.Tensor:
    """Storage array (float32, uint16 bf16 bits, int64, int32) -> device tensor."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def host_f64(t: torch.Tensor) -> np.ndarray:
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    den = float(np.abs(ref).max())
    if den == 0.0:
        return float(np.abs(got).max())
    return float(np.abs(got - ref).max()) / den


def assert_close(got, ref, dtype: str, what: str, tol: float | None = None):
    tol = TOL[dtype] if tol is None else tol
    e = rel_err(got, ref)
    assert e <= tol, f"{what}: max|err|/max|ref| = {e:.3e} > {tol:.1e}"
    return e


def dev_weights(ws):
    return [{k: dev(v) for k, v in lw.items()} for lw in ws]


@functools.lru_cache(maxsize=4)
def user_inputs(name: str, stress: bool = False):
    return W.user_inputs(W.workload(name), stress=stress)


@functools.lru_cache(maxsize=1)
def _items(name: str):
    return W.cache_inputs(W.workload(name))["items"]


@functools.lru_cache(maxsize=4)
def _keys(name: str, stress: bool):
    return W.cache_inputs(W.workload(name), stress=stress, n_items=1)["link_keys"]


def cache_inputs(name: str, stress: bool = False):
    """items (shared by both stress modes) and the link keys."""
    return {"items": _items(name), "link_keys": _keys(name, stress)}


@functools.lru_cache(maxsize=2)
def synthetic_cache(name: str):
    """A seeded stand-in QK cache [n_items, heads, ell] for scoring-only
    tests (non-negative weights of the magnitude phi produces)."""
    w = W.workload(name)
    x = np.abs(W.normal(w.seed, "cache_stand_in", (w.n_items, w.heads, w.ell), 1.0 / w.ell))
    return W.as_storage(x, w.dtype)


@functools.lru_cache(maxsize=2)
def ids_for(name: str):
    return W.candidate_ids(W.workload(name))
