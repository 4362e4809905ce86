"""Python binding of libfk: exact Lloyd k-means on MI355X (gfx950).

A thin ctypes layer over the C ABI in ``include/fk.h``: the functions carry the
same names, check tensor dtypes, devices and shapes, pass raw pointers and the
current torch stream, and raise ``FkError`` on a non-zero status.  Every step
of the computation runs in the HIP kernels of ``libfk.so``; torch is used only
for device memory and streams.  If ``libfk.so`` has not been built, ``load()``
raises -- there is no fallback path.

The workspace is cached per (device, stream) and reused by every call on that
stream that does not pass its own ``workspace`` (calls on one stream run in
order, so they may share it).
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfk.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "fk.h")

METRICS = {"l2": 0, "cosine": 1, "inner_product": 2, "spherical": 3}
SCORES = {"fp32": 0, "split_bf16": 1}
PHASES = ("prep", "assign", "recheck", "sort", "reduce", "finalize", "h2d")
MAX_K = 65536
MAX_D = 4096


class FkError(RuntimeError):
    """A non-zero fk_status, with the library's message."""

    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__(f"{_status_name(status)}: {message}")


class _Profile(ctypes.Structure):
    _fields_ = [("calls", ctypes.c_int64 * len(PHASES)), ("ms", ctypes.c_double * len(PHASES)),
                ("rechecked", ctypes.c_int64), ("paired", ctypes.c_int64), ("windowed", ctypes.c_int64),
                ("assigned", ctypes.c_int64)]


class _FitInfo(ctypes.Structure):
    _fields_ = [("k_used", ctypes.c_int32), ("iterations", ctypes.c_int32), ("last_shift", ctypes.c_double)]


_lib = None


def load():
    """Load libfk.so (raises FkError if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise FkError(-1, f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.fk_workspace_size.argtypes = [I64, I32, I32, I32, I64]
    lib.fk_workspace_size.restype = SZ
    lib.fk_assign.argtypes = [P, I64, I32, P, I32, I32, I32, P, P, P, SZ, P]
    lib.fk_sort_inverse.argtypes = [P, I64, I32, P, P, P, SZ, P]
    lib.fk_update.argtypes = [P, I64, I32, P, I32, I32, P, P, P, P, SZ, P]
    lib.fk_lloyd_iter.argtypes = [P, I64, I32, P, I32, I32, I32, P, P, P, P, P, SZ, P]
    lib.fk_lloyd_iter_noalloc.argtypes = [P, I64, I32, P, I32, I32, I32, P, P, P, P, P]
    lib.fk_lloyd_iter_stream.argtypes = [P, I64, I32, P, I32, I32, I32, I64, P, P, P, P, SZ, P]
    lib.fk_fit_workspace_size.argtypes = [I64, I32, I32, I32]
    lib.fk_fit_workspace_size.restype = SZ
    lib.fk_fit.argtypes = [P, I64, I32, I32, I32, I32, P, ctypes.c_uint64, I32, ctypes.c_double, P, P, P,
                           ctypes.POINTER(_FitInfo), P, SZ, P]
    lib.fk_ivf_workspace_size.argtypes = [I64, I32, I32, I32]
    lib.fk_ivf_workspace_size.restype = SZ
    lib.fk_ivf_build.argtypes = [P, I64, I32, I32, I32, I32, I32, P, ctypes.c_uint64, P, P, P, P,
                                 ctypes.POINTER(ctypes.c_int32), P, SZ, P]
    lib.fk_knn_workspace_size.argtypes = [I64, I32, I64, I32, I32]
    lib.fk_knn_workspace_size.restype = SZ
    lib.fk_knn.argtypes = [P, I64, I32, P, I64, I32, I32, I32, P, P, P, SZ, P]
    for f in ("fk_assign", "fk_sort_inverse", "fk_update", "fk_lloyd_iter", "fk_lloyd_iter_noalloc", "fk_lloyd_iter_stream",
              "fk_fit", "fk_ivf_build", "fk_knn", "fk_profile_enable", "fk_profile_read"):
        getattr(lib, f).restype = ctypes.c_int
    lib.fk_status_str.argtypes = [I32]
    lib.fk_status_str.restype = ctypes.c_char_p
    lib.fk_last_error.argtypes = []
    lib.fk_last_error.restype = ctypes.c_char_p
    lib.fk_profile_enable.argtypes = [I32]
    lib.fk_profile_read.argtypes = [ctypes.POINTER(_Profile)]
    _lib = lib
    return lib


def declared_symbols() -> list:
    """Names of the functions include/fk.h declares."""
    with open(HEADER_PATH) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fk_[a-z_]+)\s*\(", text)))


def _status_name(s: int) -> str:
    if _lib is None:
        return f"status {s}"
    return _lib.fk_status_str(s).decode()


def fk_status_str(status: int) -> str:
    return load().fk_status_str(int(status)).decode()


def _check(status: int):
    if status != 0:
        raise FkError(status, load().fk_last_error().decode())


def _metric(m) -> int:
    if isinstance(m, int):
        return m
    try:
        return METRICS[m]
    except KeyError:
        raise ValueError(f"unknown metric {m!r}") from None


def _score(s) -> int:
    if isinstance(s, int):
        return s
    try:
        return SCORES[s]
    except KeyError:
        raise ValueError(f"unknown score mode {s!r}") from None


def _dev(t, name, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _host_pinned(t, name, dtype, shape=None):
    if not isinstance(t, torch.Tensor) or t.is_cuda:
        raise ValueError(f"{name} must be a host tensor")
    if t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous {dtype}")
    if not t.is_pinned():
        raise ValueError(f"{name} must be pinned (pin_memory=True)")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


_ws_cache = {}


def _workspace(nbytes: int, device, workspace=None):
    """(pointer, size) of a 256-byte aligned device workspace of >= nbytes."""
    if workspace is not None:
        _dev(workspace, "workspace", torch.uint8)
        return workspace.data_ptr(), workspace.numel()
    dev_index = device.index if device.index is not None else torch.cuda.current_device()
    key = (dev_index, torch.cuda.current_stream(dev_index).cuda_stream)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes + 256:
        _ws_cache.pop(key, None)
        buf = torch.empty(max(nbytes, 1) + 256, dtype=torch.uint8, device=device)
        _ws_cache[key] = buf
    base = buf.data_ptr()
    pad = (-base) % 256
    return base + pad, buf.numel() - pad


def fk_workspace_size(N: int, d: int, K: int, metric="l2", chunk_rows: int = 0) -> int:
    n = load().fk_workspace_size(int(N), int(d), int(K), _metric(metric), int(chunk_rows))
    if n == 0:
        raise FkError(1, f"sizes outside the limits: N={N} d={d} K={K} chunk_rows={chunk_rows}")
    return int(n)


def _ws_args(N, d, K, metric, device, workspace, chunk_rows=0):
    need = load().fk_workspace_size(int(N), int(d), int(K), _metric(metric), int(chunk_rows))
    if need == 0:
        need = 256  # sizes invalid: the library reports which
    p, n = _workspace(need, device, workspace)
    return ctypes.c_void_p(p), ctypes.c_size_t(n)


def fk_assign(X, C, metric="l2", assign=None, min_dist=None, with_min_dist=False, workspace=None, score="fp32"):
    """FlashAssign: returns (assign int32[N], min_dist float32[N] or None).
    score: "fp32" or "split_bf16" (same exact result, different speed)."""
    _dev(X, "X", torch.float32)
    _dev(C, "C", torch.float32)
    if X.dim() != 2 or C.dim() != 2 or X.shape[1] != C.shape[1]:
        raise ValueError("X[N,d] and C[K,d] must be 2-D with the same d")
    N, d = X.shape
    K = C.shape[0]
    if assign is None:
        assign = torch.empty(N, dtype=torch.int32, device=X.device)
    _dev(assign, "assign", torch.int32, (N,))
    if min_dist is None and with_min_dist:
        min_dist = torch.empty(N, dtype=torch.float32, device=X.device)
    if min_dist is not None:
        _dev(min_dist, "min_dist", torch.float32, (N,))
    ws, wsn = _ws_args(N, d, K, metric, X.device, workspace)
    _check(load().fk_assign(_ptr(X), N, d, _ptr(C), K, _metric(metric), _score(score), _ptr(assign),
                            _ptr(min_dist), ws, wsn, _stream(X.device)))
    return assign, min_dist


def fk_sort_inverse(assign, K: int, perm=None, offsets=None, workspace=None):
    """Inverse index: returns (perm int32[N], offsets int32[K+1])."""
    _dev(assign, "assign", torch.int32)
    N = assign.numel()
    if perm is None:
        perm = torch.empty(N, dtype=torch.int32, device=assign.device)
    if offsets is None:
        offsets = torch.empty(K + 1, dtype=torch.int32, device=assign.device)
    _dev(perm, "perm", torch.int32, (N,))
    _dev(offsets, "offsets", torch.int32, (K + 1,))
    ws, wsn = _ws_args(N, 1, K, "l2", assign.device, workspace)
    _check(load().fk_sort_inverse(_ptr(assign), N, int(K), _ptr(perm), _ptr(offsets), ws, wsn,
                                  _stream(assign.device)))
    return perm, offsets


def fk_update(X, assign, C_prev, metric="l2", C_out=None, counts=None, workspace=None):
    """Sort-Inverse Update: returns (C_out float32[K,d], counts int32[K])."""
    _dev(X, "X", torch.float32)
    _dev(C_prev, "C_prev", torch.float32)
    N, d = X.shape
    K = C_prev.shape[0]
    _dev(assign, "assign", torch.int32, (N,))
    if C_out is None:
        C_out = torch.empty_like(C_prev)
    if counts is None:
        counts = torch.empty(K, dtype=torch.int32, device=X.device)
    _dev(C_out, "C_out", torch.float32, (K, d))
    _dev(counts, "counts", torch.int32, (K,))
    ws, wsn = _ws_args(N, d, K, metric, X.device, workspace)
    _check(load().fk_update(_ptr(X), N, d, _ptr(assign), K, _metric(metric), _ptr(C_prev), _ptr(C_out),
                            _ptr(counts), ws, wsn, _stream(X.device)))
    return C_out, counts


def fk_lloyd_iter(X, C_in, metric="l2", assign=None, C_out=None, counts=None, min_dist=None, with_min_dist=False,
                  workspace=None, score="fp32"):
    """One Lloyd iteration: returns (assign, C_out, counts, min_dist or None)."""
    _dev(X, "X", torch.float32)
    _dev(C_in, "C_in", torch.float32)
    if X.dim() != 2 or C_in.dim() != 2 or X.shape[1] != C_in.shape[1]:
        raise ValueError("X[N,d] and C[K,d] must be 2-D with the same d")
    N, d = X.shape
    K = C_in.shape[0]
    if assign is None:
        assign = torch.empty(N, dtype=torch.int32, device=X.device)
    if C_out is None:
        C_out = torch.empty_like(C_in)
    if counts is None:
        counts = torch.empty(K, dtype=torch.int32, device=X.device)
    if min_dist is None and with_min_dist:
        min_dist = torch.empty(N, dtype=torch.float32, device=X.device)
    _dev(assign, "assign", torch.int32, (N,))
    _dev(C_out, "C_out", torch.float32, (K, d))
    _dev(counts, "counts", torch.int32, (K,))
    if min_dist is not None:
        _dev(min_dist, "min_dist", torch.float32, (N,))
    ws, wsn = _ws_args(N, d, K, metric, X.device, workspace)
    _check(load().fk_lloyd_iter(_ptr(X), N, d, _ptr(C_in), K, _metric(metric), _score(score), _ptr(assign),
                                _ptr(min_dist), _ptr(C_out), _ptr(counts), ws, wsn, _stream(X.device)))
    return assign, C_out, counts, min_dist


NOALLOC_SCRATCH_BYTES = 128 << 20  # FK_NOALLOC_SCRATCH_BYTES of include/fk.h


def fk_lloyd_iter_noalloc(X, C_in, assign, C_out, counts, metric="l2", min_dist=None, score="fp32"):
    """One Lloyd iteration that allocates nothing: the library's static
    per-device scratch replaces the workspace (sizes up to
    NOALLOC_SCRATCH_BYTES of workspace; calls that overlap on one device
    race).  Every output is the caller's.  Returns (assign, C_out, counts,
    min_dist)."""
    _dev(X, "X", torch.float32)
    _dev(C_in, "C_in", torch.float32)
    if X.dim() != 2 or C_in.dim() != 2 or X.shape[1] != C_in.shape[1]:
        raise ValueError("X[N,d] and C[K,d] must be 2-D with the same d")
    N, d = X.shape
    K = C_in.shape[0]
    _dev(assign, "assign", torch.int32, (N,))
    _dev(C_out, "C_out", torch.float32, (K, d))
    _dev(counts, "counts", torch.int32, (K,))
    if min_dist is not None:
        _dev(min_dist, "min_dist", torch.float32, (N,))
    _check(load().fk_lloyd_iter_noalloc(_ptr(X), N, d, _ptr(C_in), K, _metric(metric), _score(score), _ptr(assign),
                                        _ptr(min_dist), _ptr(C_out), _ptr(counts), _stream(X.device)))
    return assign, C_out, counts, min_dist


def fk_lloyd_iter_stream(X_host, C_in, chunk_rows: int, metric="l2", assign_host=None, C_out=None, counts=None,
                         workspace=None, score="fp32"):
    """Out-of-core iteration from pinned host X: returns (C_out, counts).
    assign_host, if given, must be a pinned int32[N] host tensor."""
    _host_pinned(X_host, "X_host", torch.float32)
    _dev(C_in, "C_in", torch.float32)
    N, d = X_host.shape
    K = C_in.shape[0]
    if assign_host is not None:
        _host_pinned(assign_host, "assign_host", torch.int32, (N,))
    if C_out is None:
        C_out = torch.empty_like(C_in)
    if counts is None:
        counts = torch.empty(K, dtype=torch.int32, device=C_in.device)
    _dev(C_out, "C_out", torch.float32, (K, d))
    _dev(counts, "counts", torch.int32, (K,))
    ws, wsn = _ws_args(N, d, K, metric, C_in.device, workspace, chunk_rows=chunk_rows)
    _check(load().fk_lloyd_iter_stream(_ptr(X_host), N, d, _ptr(C_in), K, _metric(metric), _score(score),
                                       int(chunk_rows), _ptr(assign_host), _ptr(C_out), _ptr(counts), ws, wsn,
                                       _stream(C_in.device)))
    return C_out, counts


def fk_fit_workspace_size(N: int, d: int, K: int, metric="l2") -> int:
    n = load().fk_fit_workspace_size(int(N), int(d), int(K), _metric(metric))
    if n == 0:
        raise FkError(1, f"sizes outside the limits: N={N} d={d} K={K}")
    return int(n)


def fk_fit(X, C_init=None, n_iter: int = 20, metric="l2", K=None, seed: int = 0, tol: float = -1.0, assign=None,
           C_out=None, counts=None, workspace=None, score="fp32", with_info=False):
    """Lloyd k-means: up to n_iter iterations from C_init, or (C_init None)
    from K' = min(K, N) rows of X drawn with `seed`; with tol >= 0 it stops
    once no centroid moves by more than tol (squared L2).  Returns (C_out
    [K', d], assign, counts [K']) and, with with_info, a dict with k_used,
    iterations and last_shift as well."""
    _dev(X, "X", torch.float32)
    if X.dim() != 2:
        raise ValueError("X must be 2-D")
    N, d = X.shape
    if C_init is not None:
        _dev(C_init, "C_init", torch.float32)
        if C_init.dim() != 2 or C_init.shape[1] != d:
            raise ValueError("C_init must be [K, d] with the d of X")
        K = C_init.shape[0]
    elif K is None:
        raise ValueError("give C_init or K")
    K = int(K)
    Ku = K if C_init is not None else min(K, int(N))
    if assign is None:
        assign = torch.empty(N, dtype=torch.int32, device=X.device)
    if C_out is None:
        C_out = torch.empty((max(Ku, 1), d), dtype=torch.float32, device=X.device)
    if counts is None:
        counts = torch.empty(max(Ku, 1), dtype=torch.int32, device=X.device)
    _dev(assign, "assign", torch.int32, (N,))
    _dev(C_out, "C_out", torch.float32)
    _dev(counts, "counts", torch.int32)
    if C_out.numel() < Ku * d or counts.numel() < Ku:
        raise ValueError("C_out and counts must hold K' rows")
    need = load().fk_fit_workspace_size(int(N), int(d), K, _metric(metric)) or 256
    p, n = _workspace(need, X.device, workspace)
    info = _FitInfo()
    _check(load().fk_fit(_ptr(X), N, d, K, _metric(metric), _score(score), _ptr(C_init), int(seed) & (2 ** 64 - 1),
                         int(n_iter), float(tol), _ptr(C_out), _ptr(assign), _ptr(counts), ctypes.byref(info),
                         ctypes.c_void_p(p), ctypes.c_size_t(n), _stream(X.device)))
    out = (C_out[:info.k_used], assign, counts[:info.k_used])
    if with_info:
        return out + ({"k_used": int(info.k_used), "iterations": int(info.iterations),
                       "last_shift": float(info.last_shift)},)
    return out


def fk_ivf_workspace_size(N: int, d: int, nlist: int, metric="l2") -> int:
    n = load().fk_ivf_workspace_size(int(N), int(d), int(nlist), _metric(metric))
    if n == 0:
        raise FkError(1, f"sizes outside the limits: N={N} d={d} nlist={nlist}")
    return int(n)


def fk_ivf_build(X, nlist: int, init_idx=None, n_iter: int = 20, metric="l2", seed: int = 0, workspace=None,
                 score="fp32"):
    """IVF-Flat build: returns a dict with centroids [nl, d], offsets [nl+1],
    ids [N] and data [N, d] (rows grouped by cell), where nl = min(nlist, N)
    (the library clamps it as the FlashLib guide does); init_idx holds the
    quantizer's initial rows (host ints, at least nl of them), or None for
    nl rows drawn with `seed`."""
    import numpy as np
    _dev(X, "X", torch.float32)
    if X.dim() != 2:
        raise ValueError("X must be 2-D")
    N, d = X.shape
    nlist = int(nlist)
    idx = None
    if init_idx is not None:
        idx = np.ascontiguousarray(np.asarray(init_idx, dtype=np.int32))
        if idx.ndim != 1 or idx.shape[0] < min(nlist, int(N)):
            raise ValueError(f"init_idx has {idx.shape[0]} entries, {min(nlist, int(N))} needed")
    dev = X.device
    rows = max(1, min(nlist, int(N)))
    out = {"centroids": torch.empty((rows, d), dtype=torch.float32, device=dev),
           "offsets": torch.empty(rows + 1, dtype=torch.int32, device=dev),
           "ids": torch.empty(N, dtype=torch.int32, device=dev),
           "data": torch.empty((N, d), dtype=torch.float32, device=dev)}
    need = load().fk_ivf_workspace_size(int(N), int(d), nlist, _metric(metric)) or 256
    p, n = _workspace(need, dev, workspace)
    nl = ctypes.c_int32(0)
    _check(load().fk_ivf_build(_ptr(X), N, d, nlist, _metric(metric), _score(score), int(n_iter),
                               None if idx is None else ctypes.c_void_p(idx.ctypes.data), int(seed) & (2 ** 64 - 1),
                               _ptr(out["centroids"]), _ptr(out["offsets"]), _ptr(out["ids"]), _ptr(out["data"]),
                               ctypes.byref(nl), ctypes.c_void_p(p), ctypes.c_size_t(n), _stream(dev)))
    out["nlist"] = int(nl.value)
    return out


def fk_knn_workspace_size(M: int, d: int, Ndb: int, k: int, metric="l2") -> int:
    n = load().fk_knn_workspace_size(int(M), int(d), int(Ndb), int(k), _metric(metric))
    if n == 0:
        raise FkError(1, f"sizes outside the limits: M={M} d={d} Ndb={Ndb} k={k}")
    return int(n)


def fk_knn(Q, DB, k: int, metric="l2", idx=None, dist=None, workspace=None, score="fp32"):
    """Exact k nearest database rows of every query: returns (idx [M, k] int32,
    dist [M, k] fp32), nearest first (lower row index first on equal
    distances); with k above the database size the library clamps it as the
    FlashLib backend does and the columns past Ndb hold -1 and +inf."""
    _dev(Q, "Q", torch.float32)
    _dev(DB, "DB", torch.float32)
    if Q.dim() != 2 or DB.dim() != 2 or Q.shape[1] != DB.shape[1]:
        raise ValueError("Q[M,d] and DB[Ndb,d] must be 2-D with the same d")
    M, d = Q.shape
    Ndb = DB.shape[0]
    k = int(k)
    if idx is None:
        idx = torch.empty((M, k), dtype=torch.int32, device=Q.device)
    if dist is None:
        dist = torch.empty((M, k), dtype=torch.float32, device=Q.device)
    _dev(idx, "idx", torch.int32, (M, k))
    _dev(dist, "dist", torch.float32, (M, k))
    need = load().fk_knn_workspace_size(int(M), int(d), int(Ndb), k, _metric(metric)) or 256
    p, n = _workspace(need, Q.device, workspace)
    _check(load().fk_knn(_ptr(Q), M, d, _ptr(DB), Ndb, k, _metric(metric), _score(score), _ptr(idx), _ptr(dist),
                         ctypes.c_void_p(p), ctypes.c_size_t(n), _stream(Q.device)))
    return idx, dist


def fk_profile_enable(on: bool = True):
    _check(load().fk_profile_enable(1 if on else 0))


def fk_profile_read() -> dict:
    """Waits for the pending phase events; returns per-phase calls and
    milliseconds, the near-tie points settled by an fp64 compare of two
    centroids ("paired"), of the centroids within their error window
    ("windowed"), or against all K ("rechecked"), and the points assigned."""
    p = _Profile()
    _check(load().fk_profile_read(ctypes.byref(p)))
    return {"calls": {ph: int(p.calls[i]) for i, ph in enumerate(PHASES)},
            "ms": {ph: float(p.ms[i]) for i, ph in enumerate(PHASES)},
            "rechecked": int(p.rechecked), "paired": int(p.paired), "windowed": int(p.windowed),
            "assigned": int(p.assigned)}
