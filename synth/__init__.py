"""Seeded synthetic workloads: Gaussian mixtures of the shapes the Flash-KMeans
pages measure on.

This module only draws inputs.  It holds none of the k-means arithmetic and is
shared, read-only, by the tests, the oracle checks and the benchmark.

Recipe (all draws from numpy ``default_rng`` / PCG64):
  * component means: ``default_rng([seed, 0])``; uniform in [-1, 1]^d or
    standard normal, float64, then cast to float32;
  * mixture weights: equal, or Zipf  w_j proportional to (j + 1)^-s;
  * rows are drawn in fixed blocks of ``BLOCK`` rows (always whole blocks,
    the tail of the last one being dropped); block b uses its own
    generator ``default_rng([seed, 2, b])`` and draws, in this order, the
    labels (``integers`` for equal weights, ``choice(p=w)`` otherwise), then
    ``standard_normal((rows, d), float32)`` noise; a row is
    ``mean[label] + sigma * noise`` in float32;
  * when ``normalize`` is set, each row is divided by its L2 norm in float64
    and stored as float32 (the IVF coarse-quantizer shape: cosine reduced to
    L2 on unit vectors);
  * initial centroids: the first K rows, or the rows
    ``default_rng([seed, 1]).choice(N, K, replace=False)`` in drawn order;
  * k-NN queries: rows of the same mixture drawn as above, block b with
    ``default_rng([seed, 3, b])``; means "zero" makes every row plain
    standard normal noise (the FlashLib guide's ``randn`` example).

Because every block has its own generator, any row range can be generated on
its own, in parallel, and gives the same bytes as a full generation.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

BLOCK = 65536


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    N: int
    d: int
    K: int
    sigma: float
    means: str          # "uniform" | "normal"
    weights: str        # "equal" | "zipf"
    zipf_s: float
    seed: int
    init: str           # "first" | "sample"
    iters: int
    normalize: bool
    metric: str = "l2"
    chunk_rows: int = 0  # rows per host->device chunk for the out-of-core shape
    queries: int = 0     # k-NN shapes: query rows
    k: int = 0           # k-NN shapes: neighbours per query

    def scaled(self, N: int) -> "Workload":
        """Same recipe with fewer rows (the first N rows of the full set are
        identical to those of the scaled one)."""
        return dataclasses.replace(self, N=int(N))


WORKLOADS = {
    # 65,536 x 16, K=64: means U[-1,1]^16, sigma 0.1, equal weights, seed 0,
    # initial centroids = first K rows, 10 iterations.
    "tiny_d16_k64": Workload("tiny_d16_k64", 65536, 16, 64, 0.1, "uniform", "equal", 0.0, 0, "first", 10, False),
    # 1,048,576 x 128, K=1024: means N(0,I), sigma 0.3, equal, seed 1, 20 iterations.
    "gmm_1m_d128_k1024": Workload("gmm_1m_d128_k1024", 1048576, 128, 1024, 0.3, "normal", "equal", 0.0, 1, "sample", 20, False),
    # IVF coarse-quantizer training shape: 1,000,000 x 768, K=4096, sigma 0.5,
    # rows L2-normalised, seed 0, 20 iterations.
    "ivf_1m_d768_k4096": Workload("ivf_1m_d768_k4096", 1000000, 768, 4096, 0.5, "normal", "equal", 0.0, 0, "sample", 20, True),
    # Skewed large K: 16,777,216 x 128, K=32,768, Zipf(1.2) weights, sigma 0.2,
    # seed 2, 5 iterations.
    "zipf_16m_d128_k32768": Workload("zipf_16m_d128_k32768", 16777216, 128, 32768, 0.2, "normal", "zipf", 1.2, 2, "sample", 5, False),
    # Out-of-core headline shape: 1e9 x 128, K=32,768, equal weights, sigma 0.2,
    # seed 3, one iteration, 2^26-row host->device chunks.
    "ooc_1b_d128_k32768": Workload("ooc_1b_d128_k32768", 1000000000, 128, 32768, 0.2, "normal", "equal", 0.0, 3, "sample", 1, False, "l2", 1 << 26),
    # Exact k-NN, the FlashLib guide's example: a 1,000,000 x 128 standard
    # normal database, 10,000 standard normal queries, 10 neighbours, seed 4.
    "knn_1m_d128_q10k": Workload("knn_1m_d128_q10k", 1000000, 128, 1, 1.0, "zero", "equal", 0.0, 4, "first", 1, False, "l2", 0, 10000, 10),
    # Exact k-NN on the guide's benchmark corpus shape: 1,000,000 x 768, a
    # mixture of 8,192 Gaussians (more components than the IVF's 4,096 cells),
    # sigma 0.5, 10,000 queries from the same mixture, 10 neighbours, seed 5.
    "knn_1m_d768_q10k": Workload("knn_1m_d768_q10k", 1000000, 768, 8192, 0.5, "normal", "equal", 0.0, 5, "first", 1, False, "l2", 0, 10000, 10),
}


def means(w: Workload) -> np.ndarray:
    """Component means, float32 [K, d]."""
    rng = np.random.default_rng([w.seed, 0])
    if w.means == "zero":
        m = np.zeros((w.K, w.d))
    elif w.means == "uniform":
        m = rng.uniform(-1.0, 1.0, size=(w.K, w.d))
    else:
        m = rng.standard_normal((w.K, w.d))
    return m.astype(np.float32)


def weights(w: Workload):
    """Mixture weights (None for equal weights)."""
    if w.weights == "equal":
        return None
    r = np.arange(1, w.K + 1, dtype=np.float64) ** (-w.zipf_s)
    return r / r.sum()


def _block(w: Workload, mu: np.ndarray, p, b: int, lo: int, hi: int, out: np.ndarray, stream: int = 2):
    """Rows [lo, hi) of block b (lo, hi relative to the block start) into out
    (stream 2: the rows of X, stream 3: the k-NN queries)."""
    rng = np.random.default_rng([w.seed, stream, b])
    n = BLOCK  # always a whole block, so a scaled workload is a prefix of the full one
    if p is None:
        labels = rng.integers(0, w.K, size=n)
    else:
        labels = rng.choice(w.K, size=n, p=p)
    noise = rng.standard_normal((n, w.d), dtype=np.float32)
    labels = labels[lo:hi]
    noise = noise[lo:hi]
    x = mu[labels]
    x += np.float32(w.sigma) * noise
    if w.normalize:
        x64 = x.astype(np.float64)
        x64 /= np.linalg.norm(x64, axis=1, keepdims=True)
        x = x64.astype(np.float32)
    out[...] = x
    return labels


def rows(w: Workload, start: int = 0, stop: int | None = None, out: np.ndarray | None = None,
         threads: int | None = None, return_labels: bool = False):
    """Rows [start, stop) of the workload's X as float32 [stop-start, d].

    ``out`` may be a preallocated (e.g. pinned) float32 array.  Blocks are
    generated in parallel threads; the bytes do not depend on the thread count.
    """
    stop = w.N if stop is None else int(stop)
    start = int(start)
    if not (0 <= start <= stop <= w.N):
        raise ValueError("row range outside the workload")
    n = stop - start
    if out is None:
        out = np.empty((n, w.d), np.float32)
    elif out.shape != (n, w.d) or out.dtype != np.float32:
        raise ValueError("out has the wrong shape or dtype")
    labels = np.empty(n, np.int64) if return_labels else None
    mu = means(w)
    p = weights(w)
    jobs = []
    b0 = start // BLOCK
    b1 = (stop + BLOCK - 1) // BLOCK
    for b in range(b0, b1):
        lo = max(start, b * BLOCK)
        hi = min(stop, (b + 1) * BLOCK)
        jobs.append((b, lo - b * BLOCK, hi - b * BLOCK, lo - start, hi - start))
    if threads is None:
        threads = min(16, os.cpu_count() or 1)

    def run(job):
        b, lo, hi, o0, o1 = job
        lab = _block(w, mu, p, b, lo, hi, out[o0:o1])
        if labels is not None:
            labels[o0:o1] = lab

    if threads <= 1 or len(jobs) <= 1:
        for j in jobs:
            run(j)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(run, jobs))
    return (out, labels) if return_labels else out


def queries(w: Workload, M: int | None = None) -> np.ndarray:
    """The first M (default: w.queries) k-NN query rows, float32 [M, d]: the
    same mixture as the rows of X, from their own generators."""
    M = w.queries if M is None else int(M)
    out = np.empty((M, w.d), np.float32)
    mu = means(w)
    p = weights(w)
    for b in range((M + BLOCK - 1) // BLOCK):
        lo = b * BLOCK
        hi = min(M, lo + BLOCK)
        _block(w, mu, p, b, 0, hi - lo, out[lo:hi], stream=3)
    return out


def init_indices(w: Workload) -> np.ndarray:
    """Row indices of the initial centroids."""
    if w.init == "first":
        if w.K > w.N:
            raise ValueError("K > N with first-K initialisation")
        return np.arange(w.K, dtype=np.int64)
    rng = np.random.default_rng([w.seed, 1])
    return np.asarray(rng.choice(w.N, size=w.K, replace=False), dtype=np.int64)


def gather_rows(w: Workload, idx: np.ndarray, X: np.ndarray | None = None) -> np.ndarray:
    """Rows idx of X, from X when given, else generated block by block."""
    idx = np.asarray(idx, dtype=np.int64)
    if X is not None:
        return np.ascontiguousarray(X[idx])
    out = np.empty((len(idx), w.d), np.float32)
    blocks = idx // BLOCK
    for b in np.unique(blocks):
        sel = np.nonzero(blocks == b)[0]
        lo = int(b) * BLOCK
        hi = min(w.N, lo + BLOCK)
        blk = rows(w, lo, hi, threads=1)
        out[sel] = blk[idx[sel] - lo]
    return out


def initial_centroids(w: Workload, X: np.ndarray | None = None) -> np.ndarray:
    return gather_rows(w, init_indices(w), X)


def adversarial(seed: int, N: int, d: int, K: int, kind: str = "gauss"):
    """Small seeded inputs for edge cases: returns (X, C) float32.

    kinds: "gauss" (random), "dup" (C has duplicated rows, so exact ties),
    "pairs" (C[1::2] copies C[0::2], so nearly every point has an exact
    two-way tie), "dup3" (every centroid has two copies, so three-way ties), "dup40" (40
    copies of one row, so ties wider than any fixed candidate list),
    "grid" (small integers: many exact ties), "far" (large offset, so the
    expanded distance form cancels badly), "zero" (some zero rows in X and C).
    """
    rng = np.random.default_rng([seed, 7, N, d, K])
    if kind == "grid":
        X = rng.integers(-3, 4, size=(N, d)).astype(np.float32)
        C = rng.integers(-3, 4, size=(K, d)).astype(np.float32)
    else:
        X = rng.standard_normal((N, d)).astype(np.float32)
        C = rng.standard_normal((K, d)).astype(np.float32)
    if kind == "dup" and K >= 2:
        src = rng.integers(0, K, size=K // 2)
        dst = rng.integers(0, K, size=K // 2)
        C[dst] = C[src]
    if kind == "pairs" and K >= 2:
        C[1::2] = C[0::2][: len(C[1::2])]
    if kind == "dup3" and K >= 3:
        C[1::3] = C[0::3][: len(C[1::3])]
        C[2::3] = C[0::3][: len(C[2::3])]
    if kind == "dup40" and K >= 2:
        C[: min(K, 40)] = C[0]
        X[: N // 2] = C[0] + np.float32(0.01) * X[: N // 2]
    if kind == "far":
        X += np.float32(100.0)
        C += np.float32(100.0)
    if kind == "zero":
        X[rng.integers(0, N, size=max(1, N // 16))] = 0
        C[rng.integers(0, K, size=max(1, K // 8))] = 0
    return X, C
