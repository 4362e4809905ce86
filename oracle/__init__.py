"""fp64 CPU oracle for one exact Lloyd k-means iteration (ctypes over oracle.c).

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product path
(the HIP library and its Python binding) never imports, loads or calls it, and
the two share no code.

The oracle computes the plain definition of a Lloyd iteration (Flash-KMeans
article, lumevalley.com article 3696, section "Why being fast took so long":
assign every point to its nearest centroid, then reduce-sum each cluster and
divide by its size; section "Two kernels rewrite the GPU pipeline": the maths
is unchanged and exact).  Cosine is L2 on L2-normalised rows with a zero norm
replaced by 1 (LEANN FlashLib backend guide, mhpn.cn, paragraph "distance
metric").  Every function below names the step it follows; the arithmetic is
all in ``oracle.c``.

Pins: every function here is checked in ``tests/test_oracle_pins.py`` against
brute force, exact rational arithmetic, closed forms and library routines that
do not share its code.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

METRICS = {"l2": 0, "cosine": 1, "inner_product": 2, "spherical": 3}

_CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared"]


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc into liboracle.so next to it."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *_CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.fko_assign.argtypes = [P, I64, I64, P, I64, ctypes.c_int, P, P, P]
        lib.fko_assign.restype = ctypes.c_int
        lib.fko_update.argtypes = [P, I64, I64, P, I64, ctypes.c_int, P, P, P]
        lib.fko_update.restype = ctypes.c_int
        lib.fko_lloyd_iter.argtypes = [P, I64, I64, P, I64, ctypes.c_int, P, P, P, P, P, P]
        lib.fko_lloyd_iter.restype = ctypes.c_int
        lib.fko_normalize_rows.argtypes = [P, I64, I64, P]
        lib.fko_normalize_rows.restype = ctypes.c_int
        lib.fko_knn.argtypes = [P, I64, I64, P, I64, I64, ctypes.c_int, P, P]
        lib.fko_knn.restype = ctypes.c_int
        lib.fko_num_threads.argtypes = []
        lib.fko_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f32(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    if a.ndim != 2:
        raise ValueError("expected a 2-D array")
    return a


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def num_threads() -> int:
    """OpenMP threads the assignment step uses (OMP_NUM_THREADS or all cores)."""
    return int(_load().fko_num_threads())


def assign(X, C, metric: str = "l2"):
    """Assignment step: for each row x_i of X, D_ik = ||x_i - c_k||^2 (fp64,
    direct difference; inner product: D_ik = -x_i.c_k, the dot product summed
    in increasing j), a_i = lowest index attaining the minimum, D1 = that
    minimum, D2 = the minimum over the other centroids (inf when K == 1).

    Returns (a int32[N], D1 float64[N], D2 float64[N]).
    """
    X = _f32(X)
    C = _f32(C)
    N, d = X.shape
    K, dc = C.shape
    if dc != d:
        raise ValueError("X and C differ in d")
    a = np.empty(N, np.int32)
    D1 = np.empty(N, np.float64)
    D2 = np.empty(N, np.float64)
    rc = _load().fko_assign(_ptr(X), N, d, _ptr(C), K, METRICS[metric], _ptr(a), _ptr(D1), _ptr(D2))
    if rc != 0:
        raise ValueError("oracle assign rejected its arguments")
    return a, D1, D2


def update(X, a, C_in, metric: str = "l2"):
    """Update step: counts n_k, and C_new[k] = mean of the (normalised, for
    cosine) rows assigned to k, summed in fp64 in increasing i; a cluster with
    no rows keeps C_in[k].  Returns (C_new float64[K,d], counts int64[K])."""
    X = _f32(X)
    C_in = _f32(C_in)
    a = np.ascontiguousarray(a, dtype=np.int32)
    N, d = X.shape
    K = C_in.shape[0]
    if a.shape != (N,) or C_in.shape[1] != d:
        raise ValueError("shape mismatch")
    C_out = np.empty((K, d), np.float64)
    counts = np.empty(K, np.int64)
    rc = _load().fko_update(_ptr(X), N, d, _ptr(a), K, METRICS[metric], _ptr(C_in), _ptr(C_out), _ptr(counts))
    if rc != 0:
        raise ValueError("oracle update rejected its arguments (label outside [0, K)?)")
    return C_out, counts


def lloyd_iter(X, C_in, metric: str = "l2"):
    """One iteration from C_in: assignment, update, and the objective
    J = sum_i D1_i under C_in.  Returns a dict with a, D1, D2, C (float64),
    counts (int64), J."""
    X = _f32(X)
    C_in = _f32(C_in)
    N, d = X.shape
    K = C_in.shape[0]
    a = np.empty(N, np.int32)
    D1 = np.empty(N, np.float64)
    D2 = np.empty(N, np.float64)
    C_out = np.empty((K, d), np.float64)
    counts = np.empty(K, np.int64)
    J = ctypes.c_double(0.0)
    rc = _load().fko_lloyd_iter(_ptr(X), N, d, _ptr(C_in), K, METRICS[metric], _ptr(a), _ptr(D1),
                                _ptr(D2), _ptr(C_out), _ptr(counts), ctypes.byref(J))
    if rc != 0:
        raise ValueError("oracle iteration rejected its arguments")
    return {"a": a, "D1": D1, "D2": D2, "C": C_out, "counts": counts, "J": J.value}


def normalize_rows(X):
    """The rows as the cosine metric sees them: promoted to fp64, divided by
    their L2 norm (zero norm taken as 1), rounded once to fp32."""
    X = _f32(X)
    N, d = X.shape
    out = np.empty_like(X)
    if _load().fko_normalize_rows(_ptr(X), N, d, _ptr(out)) != 0:
        raise ValueError("oracle normalisation rejected its arguments")
    return out


_MASK64 = (1 << 64) - 1


class _SplitMix64:
    """SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
    generators", OOPSLA 2014): the state advances by the golden-ratio
    increment 0x9E3779B97F4A7C15 and each output is the new state passed
    through the variant-13 mix (xor-shifts by 30, 27 and 31 with multipliers
    0xBF58476D1CE4E5B9 and 0x94D049BB133111EB), all modulo 2^64.  The output
    is a function of the seed and the draw's position only."""

    def __init__(self, seed: int):
        self.st = seed & _MASK64

    def next(self) -> int:
        self.st = (self.st + 0x9E3779B97F4A7C15) & _MASK64
        z = self.st
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
        return z ^ (z >> 31)

    def below(self, m: int) -> int:
        """Uniform integer in [0, m): draws at or above the largest multiple
        of m that fits in 2^64 are rejected, the rest taken modulo m."""
        limit = (1 << 64) - ((1 << 64) % m)
        while True:
            r = self.next()
            if r < limit:
                return r % m


def splitmix64(seed: int, n: int) -> list:
    """The first n outputs of SplitMix64 seeded with `seed`."""
    g = _SplitMix64(seed)
    return [g.next() for _ in range(int(n))]


def sample_rows(N: int, K: int, seed: int) -> np.ndarray:
    """K distinct row indices of [0, N) drawn with `seed`: the first K
    positions of a Fisher-Yates shuffle of 0..N-1 (Durstenfeld's form: step i
    swaps position i with a uniform position in [i, N)), the shuffled array
    held as a map of the positions moved, numbers from SplitMix64 above.  The
    FlashLib guide's k-means takes a seed (paragraph "参数速查": seed 0) and
    samples its initial centroids from the rows; the pages name no generator,
    so this published one is the reading.  Requires 1 <= K <= N."""
    N, K = int(N), int(K)
    if not (1 <= K <= N):
        raise ValueError("need 1 <= K <= N")
    rng = _SplitMix64(seed)
    moved = {}
    out = np.empty(K, np.int64)
    for i in range(K):
        j = i + rng.below(N - i)
        vi = moved.get(i, i)
        vj = moved.get(j, j)
        moved[j] = vi
        moved[i] = vj
        out[i] = vj
    return out


def centroid_shift(C_old, C_new) -> float:
    """The largest squared L2 distance, in fp64, between a centroid's fp32
    value before and after an iteration: the fit's stopping measure."""
    D = np.asarray(C_new, np.float64) - np.asarray(C_old, np.float64)
    return float((D * D).sum(1).max())


def fit(X, C_init, n_iter: int, metric: str = "l2", tol=None):
    """Lloyd k-means: the iteration above repeated from C_init, at most n_iter
    times.  Between iterations the centroids are held in fp32, the precision
    of C in the problem statement (Flash-KMeans article, "Why being fast took
    so long": X and C are the inputs of every iteration).  With tol >= 0 the
    fit stops after the first iteration whose centroid_shift is at or below
    tol (tol = 0: once an iteration leaves every centroid unchanged, a fixed
    point).  Returns (C float32, a of the last iteration, counts of the last
    iteration, [J per iteration]); len(J) is the number of iterations run."""
    if n_iter < 1:
        raise ValueError("n_iter must be at least 1")
    C = _f32(C_init)
    Js = []
    for _ in range(int(n_iter)):
        r = lloyd_iter(X, C, metric)
        Js.append(r["J"])
        C_new = r["C"].astype(np.float32)
        stop = tol is not None and tol >= 0 and centroid_shift(C, C_new) <= tol
        C = C_new
        if stop:
            break
    return C, r["a"], r["counts"], Js


def fit_seeded(X, K: int, n_iter: int, seed: int, metric: str = "l2", tol=None):
    """The fit from K' = min(K, N) rows drawn by sample_rows(N, K', seed)
    (the FlashLib guide clamps the cluster count to the row count, paragraph
    "nlist 与 nprobe").  Returns fit()'s tuple plus the indices drawn."""
    X = _f32(X)
    idx = sample_rows(X.shape[0], min(int(K), X.shape[0]), seed)
    return fit(X, X[idx], n_iter, metric, tol) + (idx,)


def ivf_build(X, init_idx, n_iter: int, metric: str = "l2", nlist=None, seed=None):
    """IVF-Flat build as the LEANN FlashLib guide describes it (paragraphs
    "工作原理" and "参数速查"): for cosine the rows are normalised first; a
    coarse quantizer is trained by n_iter Lloyd iterations (L2) from the rows
    init_idx (or, with init_idx None, from min(nlist, N) rows drawn by
    sample_rows with `seed`: the guide clamps nlist to N, paragraph "nlist 与
    nprobe"); every row is then assigned to its nearest final centroid, and
    the rows are grouped by cell (CSR offsets, the row ids of each cell in
    increasing order, and the rows themselves).  Returns a dict with
    centroids, labels, offsets, ids, data."""
    Xu = normalize_rows(X) if metric == "cosine" else _f32(X)
    if init_idx is None:
        init_idx = sample_rows(Xu.shape[0], min(int(nlist), Xu.shape[0]), seed)
    init_idx = np.asarray(init_idx, np.int64)
    C, _, _, _ = fit(Xu, Xu[init_idx], n_iter, "l2")
    a, _, _ = assign(Xu, C, "l2")
    ids = np.argsort(a, kind="stable").astype(np.int32)
    counts = np.bincount(a, minlength=C.shape[0])
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return {"centroids": C, "labels": a, "offsets": offsets, "ids": ids, "data": Xu[ids]}


def knn(Q, DB, k: int, metric: str = "l2"):
    """Exact k nearest neighbours by brute force (LEANN FlashLib guide,
    paragraph "何时使用": the exact GPU k-NN backend): for each query, the k
    database rows first in (fp64 distance, row index) order, the distance
    being the assignment step's (cosine: both rows normalised; inner
    product: -q.x).  The backend clamps k to the database size; here a k
    above Ndb gives Ndb neighbours followed by index -1 at distance +inf.
    Returns (idx int32[M, k], dist float64[M, k])."""
    Q = _f32(Q)
    DB = _f32(DB)
    M, d = Q.shape
    Ndb, dd = DB.shape
    if dd != d:
        raise ValueError("Q and DB differ in d")
    kk = min(int(k), Ndb)
    idx = np.empty((M, kk), np.int32)
    dist = np.empty((M, kk), np.float64)
    rc = _load().fko_knn(_ptr(Q), M, d, _ptr(DB), Ndb, kk, METRICS[metric], _ptr(idx), _ptr(dist))
    if rc != 0:
        raise ValueError("oracle knn rejected its arguments")
    if kk < k:
        idx = np.concatenate([idx, np.full((M, k - kk), -1, np.int32)], axis=1)
        dist = np.concatenate([dist, np.full((M, k - kk), np.inf)], axis=1)
    return idx, dist


def relative_gap(D1, D2):
    """g_i = (D2_i - D1_i) / D1_i: the top-2 gap relative to the best distance
    (inf when D1 == 0 < D2, 0 when D1 == D2).  Points with g above a threshold
    have an assignment that any exact method must reproduce."""
    D1 = np.asarray(D1, np.float64)
    D2 = np.asarray(D2, np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        g = (D2 - D1) / D1
    g = np.where(D1 == 0, np.where(D2 > 0, np.inf, 0.0), g)
    return g
