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


# ------------------------------------------------ seeded draw, tolerance, spherical

def _separated(seed, K=40, d=24, N=12003, scale=20.0):
    rng = np.random.default_rng(seed)
    centers = rng.standard_normal((K, d)) * scale
    labels = rng.integers(0, K, size=N)
    return (centers[labels] + rng.standard_normal((N, d))).astype(np.float32)


@pytest.mark.parametrize("score", SCORES)
def test_fit_draws_the_oracles_rows(gpu_lib, score):
    """With no initial centroids the library draws K rows with SplitMix64 and
    a Fisher-Yates shuffle from the seed: one iteration equals the oracle's
    iteration from oracle.sample_rows' rows, and the whole seeded fit the
    oracle's seeded fit (separated data keeps the trajectories together)."""
    fk = gpu_lib
    X = _separated(51)
    Xd = dev(X)
    for seed in (0, 1, 12345678901234567):
        idx = oracle.sample_rows(X.shape[0], 40, seed)
        C1, _, _ = fk.fk_fit(Xd, None, 1, K=40, seed=seed, score=score)
        C1c, _, _ = fk.fk_fit(Xd, dev(X[idx]), 1, score=score)
        assert host(C1).tobytes() == host(C1c).tobytes()
    C_ref, a_ref, n_ref, _, _ = oracle.fit_seeded(X, 40, 6, 5)
    C, a, n, info = fk.fk_fit(Xd, None, 6, K=40, seed=5, score=score, with_info=True)
    assert info == {"k_used": 40, "iterations": 6, "last_shift": -1.0}
    np.testing.assert_array_equal(host(a), a_ref)
    np.testing.assert_array_equal(host(n), n_ref)
    assert centroid_rel_err(host(C), C_ref.astype(np.float64), n_ref) <= 1e-6


def test_fit_clamps_k_to_n(gpu_lib):
    fk = gpu_lib
    X = np.random.default_rng(52).standard_normal((50, 7)).astype(np.float32)
    C, a, n, info = fk.fk_fit(dev(X), None, 3, K=80, seed=2, with_info=True)
    assert info["k_used"] == 50 and tuple(C.shape) == (50, 7)
    C_ref, a_ref, n_ref, _, idx = oracle.fit_seeded(X, 80, 3, 2)
    np.testing.assert_array_equal(host(a), a_ref)
    np.testing.assert_array_equal(host(n), np.ones(50))
    np.testing.assert_array_equal(host(C)[host(a)], X)


@pytest.mark.parametrize("score", SCORES)
@pytest.mark.parametrize("metric", ["l2", "cosine", "spherical"])
def test_fit_tolerance(gpu_lib, score, metric):
    """tol = 0 stops at the fixed point the oracle's fit reaches, in as many
    iterations; a huge tol stops after one; tol < 0 runs them all."""
    fk = gpu_lib
    X = _separated(53)
    C0 = X[np.random.default_rng(54).choice(X.shape[0], 40, replace=False)]
    Xd, C0d = dev(X), dev(C0)
    C_ref, a_ref, n_ref, J = oracle.fit(X, C0, 50, metric, tol=0.0)
    assert len(J) < 50
    C, a, n, info = fk.fk_fit(Xd, C0d, 50, metric=metric, tol=0.0, score=score, with_info=True)
    assert info["iterations"] == len(J) and info["last_shift"] == 0.0
    np.testing.assert_array_equal(host(a), a_ref)
    np.testing.assert_array_equal(host(n), n_ref)
    assert centroid_rel_err(host(C), C_ref.astype(np.float64), n_ref) <= 1e-6
    _, _, _, info = fk.fk_fit(Xd, C0d, 50, metric=metric, tol=1e30, score=score, with_info=True)
    assert info["iterations"] == 1 and info["last_shift"] > 0
    Cf, _, _ = fk.fk_fit(Xd, C0d, 1, metric=metric, score=score)
    C1, _, _, info = fk.fk_fit(Xd, C0d, 7, metric=metric, tol=-1.0, score=score, with_info=True)
    assert info["iterations"] == 7


@pytest.mark.parametrize("score", SCORES)
@pytest.mark.parametrize("N,d,K", [(20011, 96, 300), (3000, 768, 64), (5000, 17, 40)])
def test_spherical_iteration_matches_oracle(gpu_lib, score, N, d, K):
    """Spherical k-means: cosine assignment, then every centroid (an empty
    one's kept centroid too) divided by its norm."""
    fk = gpu_lib
    w = synth.WORKLOADS["ivf_1m_d768_k4096"].scaled(N)
    X = synth.rows(w)[:, :d].copy() * np.float32(2.5)
    X[3] = 0.0
    C = X[np.random.default_rng([N, d]).choice(N, K, replace=False)].copy()
    C[1] = 0.0                  # a zero centroid (the zero-norm guard)
    C[4] = C[2]                 # a duplicate: ties go to index 2, cluster 4 stays empty
    Xd = dev(X)
    Cd = dev(C)
    for it in range(3):
        a, C1, n, md = fk.fk_lloyd_iter(Xd, Cd, metric="spherical", with_min_dist=True, score=score)
        r = oracle.lloyd_iter(X, host(Cd), "spherical")
        np.testing.assert_array_equal(host(a), r["a"])
        np.testing.assert_array_equal(host(n), r["counts"])
        assert centroid_rel_err(host(C1), r["C"], np.ones_like(r["counts"])) <= 1e-6
        nrm = np.linalg.norm(host(C1).astype(np.float64), axis=1)
        assert np.all((np.abs(nrm - 1) < 1e-6) | (nrm == 0))
        Cd = C1
    # streamed chunks give the same iteration
    Xh = torch.empty(X.shape, dtype=torch.float32, pin_memory=True)
    Xh.numpy()[...] = X
    a, C1, n, _ = fk.fk_lloyd_iter(Xd, dev(C), metric="spherical", score=score)
    C_s, n_s = fk.fk_lloyd_iter_stream(Xh, dev(C), 4099, metric="spherical", score=score)
    np.testing.assert_array_equal(host(n_s), host(n))
    assert centroid_rel_err(host(C_s), host(C1).astype(np.float64), np.ones(K)) <= 1e-6


@pytest.mark.parametrize("metric", ["l2", "cosine"])
def test_ivf_build_seeded_draw(gpu_lib, metric):
    """With no initial rows the build draws min(nlist, N) rows from the seed,
    the oracle's sample_rows rows; nlist above N gives N cells."""
    fk = gpu_lib
    X = np.random.default_rng(55).standard_normal((5001, 40)).astype(np.float32)
    Xd = dev(X)
    out = fk.fk_ivf_build(Xd, 64, None, n_iter=3, metric=metric, seed=99)
    ref = fk.fk_ivf_build(Xd, 64, oracle.sample_rows(5001, 64, 99).astype(np.int32), n_iter=3, metric=metric)
    for k in ("centroids", "offsets", "ids", "data"):
        assert host(out[k]).tobytes() == host(ref[k]).tobytes()
    assert out["nlist"] == 64
    small = dev(X[:30])
    out = fk.fk_ivf_build(small, 64, None, n_iter=2, metric=metric, seed=3)
    assert out["nlist"] == 30 and tuple(out["centroids"].shape) == (30, 40)
    np.testing.assert_array_equal(host(out["offsets"]), np.arange(31))
