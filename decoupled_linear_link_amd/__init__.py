"""Python binding of liblime.so, the LIME inference hot path for MI355X.

Argument marshalling only: every step of the computation runs in the HIP
kernels of liblime.so.  Tensors are torch device tensors; calls enqueue on
torch's current stream and return without synchronising.  The functions
mirror the C ABI in include/lime.h:

    xor_fwd          -> lime_xor_fwd          (user side, LIME-XOR layers;
                        variant="mha" / "xor_window" -> lime_xor_fwd_variant)
    qk_cache_build   -> lime_qk_cache_build   (offline QK cache)
    cand_score       -> lime_cand_score       (online candidate scoring)

Importing works without a GPU (the library loads); calling needs one.
There is no fallback: if the library is missing the import fails.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "LimeError", "lib", "lib_path", "xor_fwd", "xor_fwd_workspace_size", "xor_fwd_plan", "qk_cache_build",
    "qk_cache_build_i8", "cand_score", "cand_score_i8", "cand_score_uncached", "PHI", "DTYPE", "VARIANT", "EXPORTED",
    "trace_begin", "trace_end", "xor_fwd_noalloc", "NOALLOC_SCRATCH_BYTES",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "_lib", "liblime.so")

if not os.path.exists(lib_path):
    raise ImportError(
        f"{lib_path} is missing: build it first with "
        "`python decoupled_linear_link_amd/build.py` (hipcc, gfx950)")

lib = ctypes.CDLL(lib_path)

PHI = {"softmax": 0, "silu_mean": 1}
VARIANT = {"xor": 0, "mha": 1, "xor_window": 2}
DTYPE = {torch.float32: 0, torch.bfloat16: 1}
STATUS = {0: "LIME_OK", 1: "LIME_ERR_INVALID_ARG", 2: "LIME_ERR_UNSUPPORTED",
          3: "LIME_ERR_WORKSPACE", 4: "LIME_ERR_HIP"}

# every symbol include/lime.h declares
EXPORTED = ("lime_xor_fwd", "lime_xor_fwd_variant", "lime_xor_fwd_score", "lime_xor_fwd_workspace_size",
            "lime_xor_fwd_plan",
            "lime_qk_cache_build", "lime_qk_cache_build_i8", "lime_cand_score", "lime_cand_score_i8",
            "lime_cand_score_uncached", "lime_status_string", "lime_last_error",
            "lime_trace_begin", "lime_trace_end", "lime_xor_fwd_noalloc")

# bytes of the library's scratch array (LIME_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 << 20


class LayerWeights(ctypes.Structure):
    _fields_ = [("w_qkv", ctypes.c_void_p), ("w_o", ctypes.c_void_p), ("w_gate", ctypes.c_void_p),
                ("w_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p)]


_vp, _i32, _i64, _f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float

lib.lime_status_string.restype = ctypes.c_char_p
lib.lime_status_string.argtypes = [ctypes.c_int]
lib.lime_last_error.restype = ctypes.c_char_p
lib.lime_last_error.argtypes = []
lib.lime_xor_fwd_workspace_size.restype = ctypes.c_size_t
lib.lime_xor_fwd_workspace_size.argtypes = [ctypes.c_int, _i32, _i32, _i32, _i32, _i32, _i64, _i32]
lib.lime_xor_fwd_plan.restype = ctypes.c_int32
lib.lime_xor_fwd_plan.argtypes = [ctypes.c_int, _i32, _i32, _i32, _i32, _i32, _i32, _i64, _i32, _i32,
                                  ctypes.c_char_p, ctypes.c_size_t]
lib.lime_xor_fwd.restype = ctypes.c_int
lib.lime_xor_fwd.argtypes = [ctypes.c_int, ctypes.c_int, _f32, _i32, _i32, _i32, _i32, _i32, _i32,
                             _vp, _vp, _vp, _i64, _i32, ctypes.POINTER(LayerWeights), _vp, _vp,
                             _vp, ctypes.c_size_t, _vp]
lib.lime_xor_fwd_noalloc.restype = ctypes.c_int
lib.lime_xor_fwd_noalloc.argtypes = lib.lime_xor_fwd.argtypes[:-3] + [_vp]
lib.lime_xor_fwd_variant.restype = ctypes.c_int
lib.lime_xor_fwd_variant.argtypes = [ctypes.c_int, _i32] + lib.lime_xor_fwd.argtypes
lib.lime_xor_fwd_score.restype = ctypes.c_int
lib.lime_xor_fwd_score.argtypes = lib.lime_xor_fwd.argtypes[:-1] + [_vp, _i64, _vp, _vp, _i64, _vp, _vp, _vp]
lib.lime_qk_cache_build.restype = ctypes.c_int
lib.lime_qk_cache_build.argtypes = [ctypes.c_int, ctypes.c_int, _f32, _i64, _i32, _i32, _i32,
                                    _vp, _vp, _vp, _vp]
lib.lime_qk_cache_build_i8.restype = ctypes.c_int
lib.lime_qk_cache_build_i8.argtypes = [ctypes.c_int, ctypes.c_int, _f32, _i64, _i32, _i32, _i32,
                                       _vp, _vp, _vp, _vp, _vp]
lib.lime_cand_score_i8.restype = ctypes.c_int
lib.lime_cand_score_i8.argtypes = [ctypes.c_int, _i32, _i32, _i32, _i32, _vp, _vp, _i64, _vp, _vp, _vp,
                                   _i64, _vp, _vp, _vp]
lib.lime_cand_score_uncached.restype = ctypes.c_int
lib.lime_cand_score_uncached.argtypes = [ctypes.c_int, ctypes.c_int, _f32, _i32, _i32, _i32, _i32, _vp, _i64,
                                         _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp]
lib.lime_cand_score.restype = ctypes.c_int
lib.lime_cand_score.argtypes = [ctypes.c_int, _i32, _i32, _i32, _i32, _vp, _i64, _vp, _vp, _vp,
                                _i64, _vp, _vp, _vp]


lib.lime_trace_begin.restype = ctypes.c_int
lib.lime_trace_begin.argtypes = [_i32]
lib.lime_trace_end.restype = ctypes.c_int32
lib.lime_trace_end.argtypes = [ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_float), _i32,
                               ctypes.POINTER(_i32)]


class LimeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib.lime_last_error().decode()
        super().__init__(f"{where}: {STATUS.get(status, status)}: {msg}")


def _check(st: int, where: str):
    if st != 0:
        raise LimeError(st, where)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _dtype(t):
    try:
        return DTYPE[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16") from None


def _want(t, name, dtype=None, dims=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if dims is not None and t.dim() != dims:
        raise ValueError(f"{name} must have {dims} dims, got {t.dim()}")


def _want_shape(t, name, dtype, shape, device):
    """A tensor the kernels index with sizes taken from the other arguments:
    a contiguous device tensor of exactly this dtype and shape, on the same
    device (the C ABI sees only its pointer)."""
    _want(t, name, dtype, len(shape))
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the other arguments on {device}")


def _want_workspace(ws, need, device):
    _want(ws, "workspace", torch.uint8, 1)
    if ws.device != device:
        raise ValueError(f"workspace is on {ws.device}, the other arguments on {device}")
    if ws.numel() < need:
        raise ValueError(f"workspace holds {ws.numel()} bytes, the call needs {need}")


def _same_device(dev, **tensors):
    for name, t in tensors.items():
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other arguments on {dev}")


def _out_rows(out, M, d, dtype, device):
    """The [M, d] score rows: allocated here, or checked when the caller
    passes them (the kernels write M*d elements)."""
    if out is None:
        return torch.empty((M, d), dtype=dtype, device=device)
    _want_shape(out, "out", dtype, (M, d), device)
    return out


def _want_bad(bad, device):
    if bad is not None:
        _want_shape(bad, "bad_id_count", torch.int32, tuple(bad.shape), device)
        if bad.numel() < 1:
            raise ValueError("bad_id_count must hold at least one int32")


def trace_begin(capacity: int = 4096):
    """Open a kernel trace (lime_trace_begin): every launch the library
    makes until trace_end() records its own start and end on the GPU."""
    _check(lib.lime_trace_begin(int(capacity)), "lime_trace_begin")


def trace_end(capacity: int = 4096):
    """Close the trace: [(kernel name, milliseconds)] in launch order, and
    the number of launches past the capacity."""
    names = (ctypes.c_char_p * capacity)()
    ms = (ctypes.c_float * capacity)()
    dropped = _i32(0)
    n = lib.lime_trace_end(names, ms, capacity, ctypes.byref(dropped))
    if n < 0:
        raise RuntimeError(f"lime_trace_end: {lib.lime_last_error().decode()}")
    return [(names[i].decode(), float(ms[i])) for i in range(min(n, capacity))], int(dropped.value)


def xor_fwd_workspace_size(dtype, B, ell, d, heads, d_ff, total_N, max_N) -> int:
    return int(lib.lime_xor_fwd_workspace_size(DTYPE[dtype], B, ell, d, heads, d_ff, total_N, max_N))


def xor_fwd_plan(dtype, B, ell, d, heads, layers, d_ff, total_N, max_N, with_hist=False):
    """(number of kernel launches, description) of the plan lime_xor_fwd uses."""
    buf = ctypes.create_string_buffer(512)
    n = lib.lime_xor_fwd_plan(DTYPE[dtype], B, ell, d, heads, layers, d_ff, total_N, max_N,
                              int(bool(with_hist)), buf, 512)
    return int(n), buf.value.decode()


def _xor_args(links_ctx, hist, hist_offsets, weights, heads, phi, scale, max_N, want_hist, links_pers,
              hist_out, workspace, with_workspace=True):
    """Checks and marshals the user-side arguments: (argument tuple without
    the stream, links_pers, hist_out, what must stay alive until the call:
    the layer array and the workspace).  with_workspace=False leaves the
    workspace and its size out of the tuple (lime_xor_fwd_noalloc)."""
    _want(links_ctx, "links_ctx", dims=3)
    dt = links_ctx.dtype
    _want(hist, "hist", dt, 2)
    _want(hist_offsets, "hist_offsets", torch.int64, 1)
    B, ell, d = links_ctx.shape
    if hist.shape[1] != d or hist_offsets.shape[0] != B + 1:
        raise ValueError("shape mismatch between links_ctx, hist and hist_offsets")
    total_N = hist.shape[0]
    if max_N is None:
        lens = hist_offsets.diff()
        max_N = int(lens.max().item()) if B > 0 else 0
    dev = links_ctx.device
    for t, name in ((hist, "hist"), (hist_offsets, "hist_offsets")):
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, links_ctx on {dev}")
    layers = len(weights)
    if layers < 1:
        raise ValueError("weights must hold at least one layer")
    _want(weights[0]["w_gate"], "weights[0].w_gate", dt, 2)
    d_ff = weights[0]["w_gate"].shape[0]
    # the kernels read every weight with the sizes d and d_ff: each must have
    # exactly its [out, in] shape
    shapes = {"w_qkv": (3 * d, d), "w_o": (d, d), "w_gate": (d_ff, d), "w_up": (d_ff, d), "w_down": (d, d_ff)}
    arr = (LayerWeights * layers)()
    for i, lw in enumerate(weights):
        for k, shp in shapes.items():
            _want_shape(lw[k], f"weights[{i}].{k}", dt, shp, dev)
        arr[i] = LayerWeights(*(lw[k].data_ptr() for k in ("w_qkv", "w_o", "w_gate", "w_up", "w_down")))
    if scale is None:
        scale = (d // heads) ** -0.5
    if links_pers is None:
        links_pers = torch.empty_like(links_ctx)
    else:
        _want_shape(links_pers, "links_pers", dt, (B, ell, d), dev)
    if want_hist and hist_out is None:
        hist_out = torch.empty_like(hist)
    elif hist_out is not None:
        _want_shape(hist_out, "hist_out", dt, (total_N, d), dev)
    args = (DTYPE[dt], PHI[phi], scale, B, ell, d, heads, layers, d_ff,
            _ptr(links_ctx), _ptr(hist), _ptr(hist_offsets), total_N, max_N, arr,
            _ptr(links_pers), _ptr(hist_out))
    if not with_workspace:
        return args, links_pers, hist_out, (arr,)
    need = xor_fwd_workspace_size(dt, B, ell, d, heads, d_ff, total_N, max_N)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    else:
        _want_workspace(workspace, need, dev)
    return args + (_ptr(workspace), workspace.numel()), links_pers, hist_out, (arr, workspace)


def xor_fwd(links_ctx, hist, hist_offsets, weights, heads: int, phi: str = "silu_mean",
            scale: float | None = None, max_N: int | None = None, want_hist: bool = False,
            links_pers=None, hist_out=None, workspace=None, stream=None,
            variant: str = "xor", window: int | None = None):
    """Stacked LIME-XOR layers.  links_ctx [B, ell, d], hist [total_N, d],
    hist_offsets [B+1] int64 (device), weights: list of per-layer dicts with
    w_qkv [3d, d], w_o [d, d], w_gate/w_up [d_ff, d], w_down [d, d_ff].
    variant "mha" (LIME-MHA, links -> history only) or "xor_window"
    (LIME-XOR+Window, window neighbours on each side, default ell // 2).
    Returns (links_pers [B, ell, d], hist_out [total_N, d] or None)."""
    if variant not in VARIANT:
        raise ValueError(f"variant must be one of {sorted(VARIANT)}")
    args, links_pers, hist_out, keep = _xor_args(links_ctx, hist, hist_offsets, weights, heads, phi, scale,
                                                max_N, want_hist, links_pers, hist_out, workspace)
    args = args + (_stream(stream),)
    ell = links_ctx.shape[1]
    if variant == "xor" and window is None:
        _check(lib.lime_xor_fwd(*args), "lime_xor_fwd")
    else:
        if window is None:
            window = max(1, ell // 2) if variant == "xor_window" else 0
        _check(lib.lime_xor_fwd_variant(VARIANT[variant], int(window), *args), "lime_xor_fwd_variant")
    return links_pers, hist_out


def xor_fwd_noalloc(links_ctx, hist, hist_offsets, weights, heads: int, phi: str = "silu_mean",
                    scale: float | None = None, max_N: int | None = None, want_hist: bool = False,
                    links_pers=None, hist_out=None, stream=None):
    """xor_fwd (the XOR variant) through lime_xor_fwd_noalloc: the library
    allocates nothing and uses its fixed per-GPU scratch array as the
    workspace (calls that need more than NOALLOC_SCRATCH_BYTES of it are
    rejected).  Pass links_pers (and hist_out) to allocate nothing here
    either.  Returns (links_pers, hist_out or None)."""
    args, links_pers, hist_out, keep = _xor_args(links_ctx, hist, hist_offsets, weights, heads, phi, scale,
                                                max_N, want_hist, links_pers, hist_out, None,
                                                with_workspace=False)
    _check(lib.lime_xor_fwd_noalloc(*args, _stream(stream)), "lime_xor_fwd_noalloc")
    return links_pers, hist_out


def xor_fwd_score(links_ctx, hist, hist_offsets, weights, heads: int, cache, cand_ids, cand_offsets,
                  phi: str = "silu_mean", scale: float | None = None, max_N: int | None = None,
                  want_hist: bool = False, links_pers=None, hist_out=None, workspace=None, out=None,
                  bad_id_count=None, stream=None):
    """xor_fwd (the XOR variant) followed by cand_score of every user's
    candidates with the links it produced, as one call.  Returns
    (links_pers, hist_out or None, scores [total_M, d])."""
    args, links_pers, hist_out, keep = _xor_args(links_ctx, hist, hist_offsets, weights, heads, phi, scale,
                                                max_N, want_hist, links_pers, hist_out, workspace)
    _want(cache, "cache", links_ctx.dtype, 3)
    _want(cand_ids, "cand_ids", torch.int64, 1)
    _want(cand_offsets, "cand_offsets", torch.int64, 1)
    n_items, H, ell = cache.shape
    B, ell2, d = links_ctx.shape
    if ell2 != ell or H != heads or cand_offsets.shape[0] != B + 1:
        raise ValueError("shape mismatch between cache, links_ctx, heads and cand_offsets")
    _same_device(links_ctx.device, cache=cache, cand_ids=cand_ids, cand_offsets=cand_offsets)
    M = cand_ids.shape[0]
    out = _out_rows(out, M, d, cache.dtype, links_ctx.device)
    _want_bad(bad_id_count, links_ctx.device)
    _check(lib.lime_xor_fwd_score(*args, _ptr(cache), n_items, _ptr(cand_ids), _ptr(cand_offsets), M,
                                  _ptr(out), _ptr(bad_id_count), _stream(stream)), "lime_xor_fwd_score")
    return links_pers, hist_out, out


def qk_cache_build(items, link_keys, phi: str = "silu_mean", scale: float | None = None,
                   cache=None, stream=None):
    """QK cache [n_items, heads, ell] from items [n_items, d] and link_keys
    [heads, ell, d]."""
    _want(items, "items", dims=2)
    _want(link_keys, "link_keys", items.dtype, 3)
    n, d = items.shape
    H, ell, d2 = link_keys.shape
    if d2 != d:
        raise ValueError("items and link_keys disagree on d")
    _same_device(items.device, link_keys=link_keys)
    if scale is None:
        scale = (d // H) ** -0.5 if d % H == 0 else d ** -0.5
    if cache is None:
        cache = torch.empty((n, H, ell), dtype=items.dtype, device=items.device)
    else:
        _want_shape(cache, "cache", items.dtype, (n, H, ell), items.device)
    _check(lib.lime_qk_cache_build(_dtype(items), PHI[phi], scale, n, d, H, ell, _ptr(items),
                                   _ptr(link_keys), _ptr(cache), _stream(stream)),
           "lime_qk_cache_build")
    return cache


def cand_score(cache, links_pers, cand_ids, cand_offsets, out=None, bad_id_count=None,
               stream=None):
    """Scores [total_M, d] for candidates cand_ids [total_M] (int64) split by
    cand_offsets [B+1] (int64) over users with links_pers [B, ell, d]."""
    _want(cache, "cache", dims=3)
    _want(links_pers, "links_pers", cache.dtype, 3)
    _want(cand_ids, "cand_ids", torch.int64, 1)
    _want(cand_offsets, "cand_offsets", torch.int64, 1)
    n_items, H, ell = cache.shape
    B, ell2, d = links_pers.shape
    if ell2 != ell or cand_offsets.shape[0] != B + 1:
        raise ValueError("shape mismatch between cache, links_pers and cand_offsets")
    _same_device(cache.device, links_pers=links_pers, cand_ids=cand_ids, cand_offsets=cand_offsets)
    M = cand_ids.shape[0]
    out = _out_rows(out, M, d, cache.dtype, cache.device)
    _want_bad(bad_id_count, cache.device)
    _check(lib.lime_cand_score(_dtype(cache), B, ell, d, H, _ptr(cache), n_items, _ptr(links_pers),
                               _ptr(cand_ids), _ptr(cand_offsets), M, _ptr(out),
                               _ptr(bad_id_count), _stream(stream)), "lime_cand_score")
    return out


def qk_cache_build_i8(items, link_keys, phi: str = "silu_mean", scale: float | None = None,
                      codes=None, qscale=None, stream=None):
    """Int8 QK cache: (codes [n_items, heads, ell] int8, qscale [n_items,
    heads] float32)."""
    _want(items, "items", dims=2)
    _want(link_keys, "link_keys", items.dtype, 3)
    n, d = items.shape
    H, ell, d2 = link_keys.shape
    if d2 != d:
        raise ValueError("items and link_keys disagree on d")
    if scale is None:
        scale = (d // H) ** -0.5 if d % H == 0 else d ** -0.5
    _same_device(items.device, link_keys=link_keys)
    if codes is None:
        codes = torch.empty((n, H, ell), dtype=torch.int8, device=items.device)
    else:
        _want_shape(codes, "codes", torch.int8, (n, H, ell), items.device)
    if qscale is None:
        qscale = torch.empty((n, H), dtype=torch.float32, device=items.device)
    else:
        _want_shape(qscale, "qscale", torch.float32, (n, H), items.device)
    _check(lib.lime_qk_cache_build_i8(_dtype(items), PHI[phi], scale, n, d, H, ell, _ptr(items),
                                      _ptr(link_keys), _ptr(codes), _ptr(qscale), _stream(stream)),
           "lime_qk_cache_build_i8")
    return codes, qscale


def cand_score_i8(codes, qscale, links_pers, cand_ids, cand_offsets, out=None, bad_id_count=None,
                  stream=None):
    """Scores [total_M, d] from the int8 cache."""
    _want(codes, "codes", torch.int8, 3)
    _want(qscale, "qscale", torch.float32, 2)
    _want(links_pers, "links_pers", dims=3)
    _want(cand_ids, "cand_ids", torch.int64, 1)
    _want(cand_offsets, "cand_offsets", torch.int64, 1)
    n_items, H, ell = codes.shape
    B, ell2, d = links_pers.shape
    if ell2 != ell or cand_offsets.shape[0] != B + 1 or tuple(qscale.shape) != (n_items, H):
        raise ValueError("shape mismatch between codes, qscale, links_pers and cand_offsets")
    _same_device(codes.device, qscale=qscale, links_pers=links_pers, cand_ids=cand_ids, cand_offsets=cand_offsets)
    M = cand_ids.shape[0]
    out = _out_rows(out, M, d, links_pers.dtype, links_pers.device)
    _want_bad(bad_id_count, links_pers.device)
    _check(lib.lime_cand_score_i8(_dtype(links_pers), B, ell, d, H, _ptr(codes), _ptr(qscale), n_items,
                                  _ptr(links_pers), _ptr(cand_ids), _ptr(cand_offsets), M, _ptr(out),
                                  _ptr(bad_id_count), _stream(stream)), "lime_cand_score_i8")
    return out


def cand_score_uncached(items, link_keys, links_pers, cand_ids, cand_offsets, phi: str = "silu_mean",
                        scale: float | None = None, out=None, bad_id_count=None, stream=None):
    """Scores [total_M, d] computed from the item rows without a cache."""
    _want(items, "items", dims=2)
    _want(link_keys, "link_keys", items.dtype, 3)
    _want(links_pers, "links_pers", items.dtype, 3)
    _want(cand_ids, "cand_ids", torch.int64, 1)
    _want(cand_offsets, "cand_offsets", torch.int64, 1)
    n_items, d = items.shape
    H, ell, d2 = link_keys.shape
    B, ell2, d3 = links_pers.shape
    if d2 != d or d3 != d or ell2 != ell or cand_offsets.shape[0] != B + 1:
        raise ValueError("shape mismatch between items, link_keys, links_pers and cand_offsets")
    _same_device(items.device, link_keys=link_keys, links_pers=links_pers, cand_ids=cand_ids,
                 cand_offsets=cand_offsets)
    if scale is None:
        scale = (d // H) ** -0.5
    M = cand_ids.shape[0]
    out = _out_rows(out, M, d, items.dtype, items.device)
    _want_bad(bad_id_count, items.device)
    _check(lib.lime_cand_score_uncached(_dtype(items), PHI[phi], scale, B, ell, d, H, _ptr(items), n_items,
                                        _ptr(link_keys), _ptr(links_pers), _ptr(cand_ids), _ptr(cand_offsets),
                                        M, _ptr(out), _ptr(bad_id_count), _stream(stream)),
           "lime_cand_score_uncached")
    return out
