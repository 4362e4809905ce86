"""GPU parity of the k-means fit driver and the IVF-Flat build against the
oracle: the fit is the iteration repeated (bitwise equal to chaining
fk_lloyd_iter, and equal to the oracle's fit on separated data), and the IVF
lists are every row assigned to its nearest final centroid (bit-exact against
the oracle under the GPU's own centroids), grouped by cell in increasing row
order, with the rows themselves copied bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import centroid_rel_err, dev, host, log

pytestmark = pytest.mark.gpu

SCORES = ["fp32", "split_bf16"]


@pytest.mark.parametrize("score", SCORES)
@pytest.mark.parametrize("n_iter", [1, 4, 5])
def test_fit_equals_chained_iterations(gpu_lib, score, n_iter):
    fk = gpu_lib
    w = synth.WORKLOADS["gmm_1m_d128_k1024"].scaled(30001)
    X = synth.rows(w)
    C0 = X[synth.init_indices(w)[:200]].copy()
    log(f"fit n_iter={n_iter} score={score}")
    Xd = dev(X)
    C, a, n = fk.fk_fit(Xd, dev(C0), n_iter, score=score)
    Cc = dev(C0)
    for _ in range(n_iter):
        ac, Cc, nc, _ = fk.fk_lloyd_iter(Xd, Cc, score=score)
    np.testing.assert_array_equal(host(C).view(np.uint32), host(Cc).view(np.uint32))
    np.testing.assert_array_equal(host(a), host(ac))
    np.testing.assert_array_equal(host(n), host(nc))


@pytest.mark.parametrize("score", SCORES)
@pytest.mark.parametrize("metric", ["l2", "cosine"])
def test_fit_matches_oracle_fit(gpu_lib, score, metric):
    """Separated clusters keep the trajectories of the GPU and the oracle
    together (no near ties for fp32 centroid rounding to flip)."""
    fk = gpu_lib
    rng = np.random.default_rng(41)
    K, d, N = 40, 24, 12003
    centers = rng.standard_normal((K, d)) * 20
    labels = rng.integers(0, K, size=N)
    X = (centers[labels] + rng.standard_normal((N, d))).astype(np.float32)
    C0 = X[rng.choice(N, K, replace=False)]
    C_ref, a_ref, n_ref, _ = oracle.fit(X, C0, 6, metric)
    C, a, n = fk.fk_fit(dev(X), dev(C0), 6, metric=metric, score=score)
    np.testing.assert_array_equal(host(a), a_ref)
    np.testing.assert_array_equal(host(n), n_ref)
    assert centroid_rel_err(host(C), C_ref.astype(np.float64), n_ref) <= 1e-6


def _check_ivf(out, X, init, n_iter, metric, score, fk):
    """The IVF outputs against the oracle, step by step under the GPU's own
    centroids (so that fp32 centroid rounding cannot move the trajectory)."""
    N, d = X.shape
    nl = out["nlist"]
    Xu = oracle.normalize_rows(X) if metric == "cosine" else X
    C = host(out["centroids"])
    # the quantizer is the fit from the initial rows (same kernels: bitwise)
    C_fit, _, _ = fk.fk_fit(dev(Xu), dev(Xu[init[:nl]]), n_iter, score=score)
    np.testing.assert_array_equal(C.view(np.uint32), host(C_fit).view(np.uint32))
    # the lists: every row under the final centroids, exact
    a_ref, _, _ = oracle.assign(Xu, C)
    ids = host(out["ids"])
    offs = host(out["offsets"])
    np.testing.assert_array_equal(ids, np.argsort(a_ref, kind="stable").astype(np.int32))
    np.testing.assert_array_equal(offs, np.concatenate([[0], np.cumsum(np.bincount(a_ref, minlength=nl))]))
    np.testing.assert_array_equal(host(out["data"]).view(np.uint32), Xu[ids].view(np.uint32))


@pytest.mark.parametrize("score", SCORES)
@pytest.mark.parametrize("metric", ["l2", "cosine"])
@pytest.mark.parametrize("N,d,nlist", [(20011, 96, 300), (4097, 48, 64), (777, 130, 50)])
def test_ivf_build_matches_oracle(gpu_lib, N, d, nlist, metric, score):
    fk = gpu_lib
    w = synth.WORKLOADS["ivf_1m_d768_k4096"].scaled(N)
    X = synth.rows(w)[:, :d].copy() * np.float32(3.0)   # not unit rows: cosine has work to do
    X[5] = 0.0
    init = np.random.default_rng([7, N]).choice(N, nlist, replace=False).astype(np.int32)
    log(f"ivf N={N} d={d} nlist={nlist} metric={metric} score={score}")
    out = fk.fk_ivf_build(dev(X), nlist, init, n_iter=4, metric=metric, score=score)
    _check_ivf(out, X, init, 4, metric, score, fk)
    # and against the oracle's whole build where the trajectory is stable:
    # the first iteration's centroids agree to fp32 rounding
    if metric == "l2":
        C1_ref, _, n1, _ = oracle.fit(X, X[init], 1)
        C1, _, _ = fk.fk_fit(dev(X), dev(X[init]), 1, score=score)
        assert centroid_rel_err(host(C1), C1_ref.astype(np.float64), n1) <= 1e-6


def test_ivf_build_clamps_nlist_to_n(gpu_lib):
    fk = gpu_lib
    rng = np.random.default_rng(43)
    X = rng.standard_normal((37, 16)).astype(np.float32)
    out = fk.fk_ivf_build(dev(X), 100, np.arange(37, dtype=np.int32), n_iter=2)
    assert out["nlist"] == 37
    # every row is its own centroid's only member
    offs = host(out["offsets"])
    np.testing.assert_array_equal(np.diff(offs), np.ones(37, np.int64))
    _check_ivf(out, X, np.arange(37, dtype=np.int32), 2, "l2", "fp32", fk)


def test_ivf_build_rejects_bad_init(gpu_lib):
    fk = gpu_lib
    X = torch.zeros((10, 8), device="cuda")
    with pytest.raises(fk.FkError, match="init_idx"):
        fk.fk_ivf_build(X, 3, np.array([0, 4, 10], np.int32), n_iter=1)
    with pytest.raises(fk.FkError, match="n_iter"):
        fk.fk_ivf_build(X, 3, np.array([0, 4, 9], np.int32), n_iter=0)
