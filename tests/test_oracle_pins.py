"""Pins for the fp64 oracle: each test checks it against something that does
not share its code -- a hand-worked example, exact rational arithmetic, a
closed form, a library routine, or an invariant of the mathematics -- chosen
so that a dropped term, a wrong sign or index, or a transposed operand in the
oracle fails at least one of them.  All run on the CPU."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.cluster.vq
import scipy.spatial.distance

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- worked examples

def test_hand_worked_l2_example():
    g = _golden("hand_2d_l2.json")
    X = np.array(g["X"], np.float32)
    C = np.array(g["C"], np.float32)
    r = oracle.lloyd_iter(X, C, "l2")
    assert r["a"].tolist() == g["a"]
    assert r["D1"].tolist() == g["D1"]
    assert r["D2"].tolist() == g["D2"]
    assert r["counts"].tolist() == g["counts"]
    assert r["C"].tolist() == g["C_new"]
    assert r["J"] == g["J"]


def test_hand_worked_cosine_example():
    g = _golden("hand_2d_cosine.json")
    X = np.array(g["X"], np.float32)
    C = np.array(g["C"], np.float32)
    r = oracle.lloyd_iter(X, C, "cosine")
    assert r["a"].tolist() == g["a"]
    np.testing.assert_allclose(r["D1"], g["D1"], rtol=0, atol=1e-15)
    assert r["counts"].tolist() == g["counts"]
    np.testing.assert_allclose(r["C"], np.array(g["C_new"]), rtol=0, atol=1e-15)


# ---------------------------------------------------------------- assignment

def _second_smallest(D):
    if D.shape[1] == 1:
        return np.full(D.shape[0], np.inf)
    return np.partition(D, 1, axis=1)[:, 1]


@pytest.mark.parametrize("N,d,K,seed", [(200, 5, 7, 0), (300, 16, 64, 1), (50, 1, 3, 2), (97, 33, 1, 3), (64, 128, 40, 4)])
def test_assign_matches_cdist_bruteforce(N, d, K, seed):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((N, d)).astype(np.float32)
    C = rng.standard_normal((K, d)).astype(np.float32)
    a, D1, D2 = oracle.assign(X, C)
    D = scipy.spatial.distance.cdist(X.astype(np.float64), C.astype(np.float64), "sqeuclidean")
    np.testing.assert_array_equal(a, np.argmin(D, axis=1))
    np.testing.assert_allclose(D1, D.min(axis=1), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(D2, _second_smallest(D), rtol=1e-12, atol=1e-12)
    # scipy's vector quantiser is a second, independent argmin
    code, dist = scipy.cluster.vq.vq(X.astype(np.float64), C.astype(np.float64), check_finite=True)
    np.testing.assert_array_equal(a, code)
    np.testing.assert_allclose(np.sqrt(D1), dist, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", range(4))
def test_assign_exact_integers_with_planted_ties(seed):
    """Small-integer data: every fp64 operation of the oracle is exact, so its
    distances must equal exact integer arithmetic, and ties must go to the
    lowest index."""
    rng = np.random.default_rng([seed, 11])
    N, d, K = 60, 4, 9
    X = rng.integers(-3, 4, size=(N, d))
    C = rng.integers(-3, 4, size=(K, d))
    C[5] = C[2]            # duplicated centroid: exact ties everywhere it is nearest
    C[8] = C[0]
    a, D1, D2 = oracle.assign(X.astype(np.float32), C.astype(np.float32))
    nties = 0
    for i in range(N):
        D = [sum(Fraction(int(X[i, j] - C[k, j])) ** 2 for j in range(d)) for k in range(K)]
        m = min(D)
        k_best = D.index(m)          # lowest index attaining the minimum
        rest = D[:k_best] + D[k_best + 1:]
        assert a[i] == k_best
        assert D1[i] == float(m)
        assert D2[i] == float(min(rest))
        nties += D.count(m) > 1
    assert nties > 0


def test_assign_one_dimensional_voronoi_closed_form():
    """In 1-D with sorted centroids, the cell boundaries are the midpoints;
    points exactly on a midpoint go to the lower index."""
    c = np.array([-8.0, -2.0, 0.0, 4.0, 10.0, 16.0], np.float32)   # midpoints -5,-1,2,7,13
    mids = (c[:-1] + c[1:]) / 2
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.uniform(-20, 25, 400), mids, mids + 0.5, mids - 0.5]).astype(np.float32)
    a, _, _ = oracle.assign(x[:, None], c[:, None])
    expect = np.searchsorted(mids, x, side="left")
    np.testing.assert_array_equal(a, expect)


def test_assign_self_assignment():
    rng = np.random.default_rng(6)
    X = rng.standard_normal((500, 12)).astype(np.float32)
    S = rng.choice(500, 37, replace=False)
    a, D1, _ = oracle.assign(X, X[S])
    np.testing.assert_array_equal(a[S], np.arange(37))
    assert np.all(D1[S] == 0.0)
    assert np.all(D1 >= 0.0)


def test_assign_order_of_operands_matters_not():
    """D is symmetric in the difference: swapping the roles of a single point
    and a single centroid gives the same distance (guards a transposed
    operand in the row/column indexing)."""
    rng = np.random.default_rng(7)
    X = rng.standard_normal((30, 7)).astype(np.float32)
    C = rng.standard_normal((11, 7)).astype(np.float32)
    _, D1, _ = oracle.assign(X, C)
    a, _, _ = oracle.assign(X, C)
    for i in range(30):
        _, d_back, _ = oracle.assign(C[a[i]:a[i] + 1], X[i:i + 1])
        assert d_back[0] == D1[i]


# ---------------------------------------------------------------- update

@pytest.mark.parametrize("seed", range(3))
def test_update_exact_rational_means(seed):
    rng = np.random.default_rng([seed, 12])
    N, d, K = 80, 3, 6
    X = rng.integers(-50, 51, size=(N, d))
    a = rng.integers(0, K - 1, size=N).astype(np.int32)     # cluster K-1 stays empty
    C_in = rng.standard_normal((K, d)).astype(np.float32)
    C, counts = oracle.update(X.astype(np.float32), a, C_in)
    for k in range(K):
        members = X[a == k]
        assert counts[k] == len(members)
        for j in range(d):
            if len(members):
                assert C[k, j] == float(Fraction(int(members[:, j].sum()), len(members)))
            else:
                assert C[k, j] == float(C_in[k, j])
    assert counts.sum() == N


def test_update_k1_is_global_mean():
    rng = np.random.default_rng(13)
    X = rng.standard_normal((1000, 9)).astype(np.float32)
    C, counts = oracle.update(X, np.zeros(1000, np.int32), np.zeros((1, 9), np.float32))
    assert counts.tolist() == [1000]
    exact = [float(sum(Fraction(float(v)) for v in X[:, j]) / 1000) for j in range(9)]
    np.testing.assert_allclose(C[0], exact, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("metric", ["l2", "cosine"])
def test_update_matches_add_at(metric):
    rng = np.random.default_rng(14)
    N, d, K = 2000, 17, 50
    X = rng.standard_normal((N, d)).astype(np.float32)
    X[::97] = 0.0
    a = rng.integers(0, K, size=N).astype(np.int32)
    a[a == 7] = 8            # cluster 7 empty
    C_in = rng.standard_normal((K, d)).astype(np.float32)
    C, counts = oracle.update(X, a, C_in, metric)
    Xd = X.astype(np.float64)
    if metric == "cosine":
        n = np.linalg.norm(Xd, axis=1, keepdims=True)
        n[n == 0] = 1.0
        Xd = Xd / n
    sums = np.zeros((K, d))
    np.add.at(sums, a, Xd)
    cnt = np.bincount(a, minlength=K)
    np.testing.assert_array_equal(counts, cnt)
    expect = np.where(cnt[:, None] > 0, sums / np.maximum(cnt, 1)[:, None], C_in.astype(np.float64))
    np.testing.assert_allclose(C, expect, rtol=1e-12, atol=1e-14)
    assert C[7].tolist() == C_in[7].astype(np.float64).tolist()


def test_update_rejects_out_of_range_labels():
    X = np.zeros((4, 2), np.float32)
    with pytest.raises(ValueError):
        oracle.update(X, np.array([0, 1, 2, 3], np.int32), np.zeros((3, 2), np.float32))
    with pytest.raises(ValueError):
        oracle.update(X, np.array([0, -1, 0, 0], np.int32), np.zeros((3, 2), np.float32))


def test_one_iteration_matches_sklearn_lloyd():
    """scikit-learn's Lloyd k-means, run for exactly one iteration from the
    same centroids, is an independent implementation of the same step."""
    from sklearn.cluster import KMeans
    w = synth.WORKLOADS["gmm_1m_d128_k1024"]
    X = synth.rows(w.scaled(20000), threads=1)[:, :16].copy()
    rng = np.random.default_rng(15)
    C0 = X[rng.choice(len(X), 24, replace=False)]
    r = oracle.lloyd_iter(X, C0)
    assert r["counts"].min() > 0          # sklearn would relocate an empty cluster
    km = KMeans(n_clusters=24, init=C0.astype(np.float64), n_init=1, max_iter=1, algorithm="lloyd", tol=0.0)
    km.fit(X.astype(np.float64))
    np.testing.assert_allclose(r["C"], km.cluster_centers_, rtol=1e-9, atol=1e-11)


# ---------------------------------------------------------------- iteration

def test_objective_non_increasing_and_counts_sum_to_n():
    w = synth.WORKLOADS["zipf_16m_d128_k32768"]
    X = synth.rows(w.scaled(6000), threads=1)[:, :8].copy()
    rng = np.random.default_rng(16)
    C = X[rng.choice(len(X), 40, replace=False)]
    Js = []
    for _ in range(15):
        r = oracle.lloyd_iter(X, C)
        assert r["counts"].sum() == len(X)
        Js.append(r["J"])
        C = r["C"].astype(np.float32)
    for j0, j1 in zip(Js, Js[1:]):
        assert j1 <= j0 * (1 + 1e-6)
    assert Js[-1] < Js[0]


def test_fixed_point_on_planted_separated_clusters():
    rng = np.random.default_rng(17)
    K, d = 6, 5
    centers = rng.standard_normal((K, d)) * 50
    labels = rng.integers(0, K, size=600)
    X = (centers[labels] + rng.standard_normal((600, d)) * 0.1).astype(np.float32)
    C = X[[np.nonzero(labels == k)[0][0] for k in range(K)]]
    for _ in range(3):
        r = oracle.lloyd_iter(X, C)
        C = r["C"].astype(np.float32)
    np.testing.assert_array_equal(r["a"], labels)
    r2 = oracle.lloyd_iter(X, C)
    np.testing.assert_array_equal(r2["a"], labels)
    np.testing.assert_allclose(r2["C"], r["C"], rtol=1e-7, atol=1e-6)


def test_row_permutation_invariance():
    rng = np.random.default_rng(18)
    X = rng.standard_normal((700, 6)).astype(np.float32)
    C = X[:20].copy()
    perm = rng.permutation(700)
    r = oracle.lloyd_iter(X, C)
    rp = oracle.lloyd_iter(X[perm], C)
    np.testing.assert_array_equal(rp["a"], r["a"][perm])
    np.testing.assert_array_equal(rp["counts"], r["counts"])
    np.testing.assert_allclose(rp["C"], r["C"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(rp["J"], r["J"], rtol=1e-12)


# ---------------------------------------------------------------- cosine

def test_cosine_equals_inner_product_on_unit_centroids():
    """On unit vectors, squared L2 order equals inner-product order."""
    rng = np.random.default_rng(19)
    X = rng.standard_normal((400, 10)).astype(np.float32) * 3
    C = rng.standard_normal((15, 10))
    C = (C / np.linalg.norm(C, axis=1, keepdims=True)).astype(np.float32)
    a, D1, D2 = oracle.assign(X, C, "cosine")
    S = X.astype(np.float64) @ C.astype(np.float64).T
    ok = oracle.relative_gap(D1, D2) > 1e-9
    np.testing.assert_array_equal(a[ok], np.argmax(S, axis=1)[ok])
    # and squared distances of unit vectors are 2 - 2 cos
    cos = S / np.linalg.norm(X.astype(np.float64), axis=1, keepdims=True)
    Cn = C.astype(np.float64) / np.linalg.norm(C.astype(np.float64), axis=1, keepdims=True)
    cos = (X.astype(np.float64) / np.linalg.norm(X.astype(np.float64), axis=1, keepdims=True)) @ Cn.T
    np.testing.assert_allclose(D1, 2 - 2 * cos.max(axis=1), rtol=0, atol=1e-12)


def test_cosine_scale_invariance_and_zero_rows():
    rng = np.random.default_rng(20)
    X = rng.standard_normal((300, 8)).astype(np.float32)
    X[::10] = 0.0
    C = rng.standard_normal((12, 8)).astype(np.float32)
    a1, D1, _ = oracle.assign(X, C, "cosine")
    a2, _, _ = oracle.assign(X * np.float32(4.0), C * np.float32(0.5), "cosine")
    np.testing.assert_array_equal(a1, a2)
    # a zero row stays zero, so it is at distance ||c^||^2 = 1 (to rounding)
    # from every normalised centroid
    np.testing.assert_allclose(D1[::10], 1.0, rtol=0, atol=1e-15)
    # with centroids that normalise exactly (scaled axis vectors) that is an
    # exact tie, which goes to centroid 0
    Cax = (np.eye(8, dtype=np.float32) * np.arange(1, 9, dtype=np.float32)[:, None])[::-1].copy()
    a3, D13, D23 = oracle.assign(X, Cax, "cosine")
    assert np.all(a3[::10] == 0)
    assert np.all(D13[::10] == 1.0) and np.all(D23[::10] == 1.0)


def test_relative_gap_definition():
    g = oracle.relative_gap(np.array([1.0, 0.0, 0.0, 2.0]), np.array([1.5, 0.0, 3.0, 2.0]))
    assert g[0] == 0.5 and g[1] == 0.0 and np.isinf(g[2]) and g[3] == 0.0


# ---------------------------------------------------------- fit and IVF build

def test_fit_reaches_exact_cluster_means_on_planted_integer_clusters():
    """Integer points in far-apart clusters, one initial centroid per cluster:
    from the second iteration on every point is in its own cluster, so the
    fit's centroids are the exact cluster means rounded to fp32 (the sums of
    small integers are exact in fp64; each mean is the correctly rounded fp64
    quotient, as float(Fraction) gives it, then fp32)."""
    rng = np.random.default_rng(31)
    K, d, n = 7, 4, 350
    centers = rng.integers(-1000, 1000, size=(K, d)) * 10
    labels = rng.integers(0, K, size=n)
    X = (centers[labels] + rng.integers(-3, 4, size=(n, d))).astype(np.float32)
    init = [int(np.nonzero(labels == k)[0][0]) for k in range(K)]
    C, a, counts, Js = oracle.fit(X, X[init], 4)
    np.testing.assert_array_equal(a, labels)
    np.testing.assert_array_equal(counts, np.bincount(labels, minlength=K))
    for k in range(K):
        rows = X[labels == k].astype(np.int64)
        for j in range(d):
            exact = Fraction(int(rows[:, j].sum()), len(rows))
            assert C[k, j] == np.float32(float(exact)), (k, j)
    assert all(j1 <= j0 for j0, j1 in zip(Js, Js[1:]))


def test_fit_one_iteration_is_the_iteration_rounded_to_fp32():
    rng = np.random.default_rng(32)
    X = rng.standard_normal((500, 6)).astype(np.float32)
    C0 = X[:9].copy()
    C, a, counts, Js = oracle.fit(X, C0, 1)
    r = oracle.lloyd_iter(X, C0)
    np.testing.assert_array_equal(a, r["a"])
    np.testing.assert_array_equal(C, r["C"].astype(np.float32))
    assert Js == [r["J"]]


def test_normalize_rows_unit_norm_direction_and_zero_rows():
    rng = np.random.default_rng(33)
    X = (rng.standard_normal((300, 11)) * rng.uniform(0.01, 100, size=(300, 1))).astype(np.float32)
    X[7] = 0.0
    Y = oracle.normalize_rows(X)
    n = np.linalg.norm(Y.astype(np.float64), axis=1)
    n[7] = 1.0
    np.testing.assert_allclose(n, 1.0, rtol=0, atol=4e-7)
    assert not Y[7].any()
    # the same direction: each row is a positive multiple of the input row
    ratio = Y.astype(np.float64) / np.where(X == 0, 1, X)
    ok = np.delete(np.arange(300), 7)
    np.testing.assert_allclose(ratio[ok], (1.0 / np.linalg.norm(X[ok].astype(np.float64), axis=1))[:, None]
                               * np.ones((1, 11)), rtol=2e-7)
    # and the assignment under cosine is the L2 assignment of the normalised
    # rows, up to the fp32 rounding of those rows (it can only flip points
    # whose two best distances are within a few fp32 ulps)
    C = X[rng.choice(300, 12, replace=False)]
    Cn = oracle.normalize_rows(C)
    a_cos, D1, D2 = oracle.assign(X, C, "cosine")
    a_l2, _, _ = oracle.assign(Y, Cn, "l2")
    flips = a_cos != a_l2
    assert (oracle.relative_gap(D1, D2)[flips] < 1e-5).all()
    assert flips.mean() < 0.05


@pytest.mark.parametrize("metric", ["l2", "cosine"])
def test_ivf_build_layout_by_brute_force(metric):
    """Every cell's list is the rows assigned to it, in increasing row order
    (checked with plain loops), the offsets delimit them, and the data rows
    are those rows."""
    rng = np.random.default_rng(34)
    X = rng.standard_normal((420, 5)).astype(np.float32)
    init = rng.choice(420, 13, replace=False)
    r = oracle.ivf_build(X, init, 3, metric)
    Xu = oracle.normalize_rows(X) if metric == "cosine" else X
    C, _, _, _ = oracle.fit(Xu, Xu[init], 3)
    np.testing.assert_array_equal(r["centroids"], C)
    a, _, _ = oracle.assign(Xu, C)
    np.testing.assert_array_equal(r["labels"], a)
    pos = 0
    for k in range(13):
        members = [i for i in range(420) if a[i] == k]
        assert r["offsets"][k] == pos
        assert list(r["ids"][pos:pos + len(members)]) == members
        pos += len(members)
    assert r["offsets"][13] == 420 == pos
    np.testing.assert_array_equal(r["data"], Xu[r["ids"]])


# ------------------------------------------------------------ inner product

@pytest.mark.parametrize("N,d,K,seed", [(300, 5, 17, 51), (64, 33, 3, 52), (1000, 2, 40, 53)])
def test_inner_product_assign_matches_bruteforce(N, d, K, seed):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((N, d)).astype(np.float32)
    C = rng.standard_normal((K, d)).astype(np.float32)
    a, D1, D2 = oracle.assign(X, C, "inner_product")
    S = X.astype(np.float64) @ C.astype(np.float64).T
    np.testing.assert_array_equal(a, S.argmax(1))
    np.testing.assert_allclose(D1, -S.max(1), rtol=1e-12, atol=1e-12)
    part = np.sort(S, axis=1)
    np.testing.assert_allclose(D2, -part[:, -2], rtol=1e-12, atol=1e-12)


def test_inner_product_exact_integer_ties_lowest_index():
    rng = np.random.default_rng(54)
    X = rng.integers(-4, 5, size=(200, 6)).astype(np.float32)
    base = rng.integers(-3, 4, size=(5, 6))
    C = np.concatenate([base, base[[2, 0]]]).astype(np.float32)     # rows 5, 6 copy rows 2, 0
    a, _, _ = oracle.assign(X, C, "inner_product")
    dots = [[sum(Fraction(int(x[j])) * int(c[j]) for j in range(6)) for c in C] for x in X]
    expect = [max(range(7), key=lambda k: (row[k], -k)) for row in dots]
    np.testing.assert_array_equal(a, expect)


def test_inner_product_on_unit_centroids_is_l2_order():
    """With unit-norm centroids, -2 x.c = ||x - c||^2 - ||x||^2 - 1, so the
    largest inner product is the nearest centroid."""
    rng = np.random.default_rng(55)
    X = rng.standard_normal((400, 9)).astype(np.float32)
    C = oracle.normalize_rows(rng.standard_normal((25, 9)).astype(np.float32))
    a_ip, D1, D2 = oracle.assign(X, C, "inner_product")
    a_l2, E1, E2 = oracle.assign(X, C, "l2")
    close = oracle.relative_gap(E1, E2) < 1e-6
    np.testing.assert_array_equal(a_ip[~close], a_l2[~close])


def test_inner_product_update_is_plain_mean():
    rng = np.random.default_rng(56)
    X = rng.standard_normal((300, 4)).astype(np.float32)
    a = rng.integers(0, 9, size=300).astype(np.int32)
    C0 = rng.standard_normal((9, 4)).astype(np.float32)
    C_ip, n_ip = oracle.update(X, a, C0, "inner_product")
    C_l2, n_l2 = oracle.update(X, a, C0, "l2")
    np.testing.assert_array_equal(C_ip, C_l2)
    np.testing.assert_array_equal(n_ip, n_l2)


# ---- exact k nearest neighbours (LEANN FlashLib guide, paragraph "何时使用":
# the exact GPU k-NN backend)

def _lex_topk(D, k):
    """k first columns of each row of D in (value, column) order."""
    cols = np.arange(D.shape[1])
    return np.stack([np.lexsort((cols, row))[:k] for row in D])


@pytest.mark.parametrize("metric", ["l2", "inner_product"])
@pytest.mark.parametrize("k", [1, 5, 17])
def test_knn_exact_integers_with_ties(metric, k):
    """Integer rows: every distance is an exact integer in fp64, so the order
    is fixed exactly (int64 arithmetic here), with many ties that must go to
    the lower row index."""
    rng = np.random.default_rng(60 + k)
    Q = rng.integers(-3, 4, size=(40, 5))
    base = rng.integers(-3, 4, size=(30, 5))
    DB = np.concatenate([base, base[::3], base[:7]])              # duplicated rows: exact ties
    if metric == "l2":
        D = ((Q[:, None, :] - DB[None, :, :]) ** 2).sum(-1)
    else:
        D = -(Q[:, None, :] * DB[None, :, :]).sum(-1)
    idx, dist = oracle.knn(Q.astype(np.float32), DB.astype(np.float32), k, metric)
    expect = _lex_topk(D, k)
    np.testing.assert_array_equal(idx, expect)
    np.testing.assert_array_equal(dist, np.take_along_axis(D, expect, 1).astype(np.float64))


@pytest.mark.parametrize("seed", [0, 1])
def test_knn_matches_cdist_where_ranks_are_clear(seed):
    """Continuous data against scipy's direct-difference distances: the order
    of the k first rows, and every row left out being at least as far."""
    rng = np.random.default_rng(70 + seed)
    Q = rng.standard_normal((60, 12)).astype(np.float32)
    DB = rng.standard_normal((500, 12)).astype(np.float32)
    k = 10
    idx, dist = oracle.knn(Q, DB, k)
    D = scipy.spatial.distance.cdist(Q.astype(np.float64), DB.astype(np.float64), "sqeuclidean")
    order = np.argsort(D, axis=1, kind="stable")
    srt = np.take_along_axis(D, order, 1)
    clear = (np.diff(srt[:, :k + 1], axis=1) > 1e-9 * srt[:, 1:k + 1]).all(1)
    assert clear.mean() > 0.9
    np.testing.assert_array_equal(idx[clear], order[clear, :k])
    np.testing.assert_allclose(dist, np.take_along_axis(D, idx.astype(np.int64), 1), rtol=1e-12)
    assert (np.diff(dist, axis=1) >= 0).all()


def test_knn_k1_is_the_assignment_and_k_eq_n_is_a_full_sort():
    rng = np.random.default_rng(80)
    Q = rng.standard_normal((50, 6)).astype(np.float32)
    DB = rng.standard_normal((23, 6)).astype(np.float32)
    a, D1, _ = oracle.assign(Q, DB)
    idx, dist = oracle.knn(Q, DB, 1)
    np.testing.assert_array_equal(idx[:, 0], a)
    np.testing.assert_array_equal(dist[:, 0], D1)
    idx, dist = oracle.knn(Q, DB, 23)
    assert all(sorted(r) == list(range(23)) for r in idx.tolist())
    assert (np.diff(dist, axis=1) >= 0).all()


def test_knn_cosine_is_largest_cosine_similarity():
    """For unit rows ||q - x||^2 = 2 - 2 cos(q, x): nearest is most similar,
    whatever the rows' lengths (zero rows count as having norm 1)."""
    rng = np.random.default_rng(81)
    Q = (rng.standard_normal((40, 7)) * rng.uniform(0.1, 9, (40, 1))).astype(np.float32)
    DB = (rng.standard_normal((200, 7)) * rng.uniform(0.1, 9, (200, 1))).astype(np.float32)
    DB[5] = 0.0
    k = 6
    idx, dist = oracle.knn(Q, DB, k, "cosine")
    q = Q.astype(np.float64)
    x = DB.astype(np.float64)
    nq = np.linalg.norm(q, axis=1, keepdims=True)
    nx = np.linalg.norm(x, axis=1, keepdims=True)
    nx[nx == 0] = 1.0
    cs = (q / nq) @ (x / nx).T
    order = np.argsort(-cs, axis=1, kind="stable")
    srt = np.take_along_axis(-cs, order, 1)
    clear = (np.diff(srt[:, :k + 1], axis=1) > 1e-9).all(1)
    assert clear.mean() > 0.9
    np.testing.assert_array_equal(idx[clear], order[clear, :k])
    np.testing.assert_allclose(dist, 2.0 - 2.0 * np.take_along_axis(cs, idx.astype(np.int64), 1), atol=1e-12)


def test_knn_clamps_k_to_database_size():
    """k above the database size (the FlashLib backend clamps top_k to it):
    every row, nearest first, then index -1 at distance +inf; k = 0 is
    rejected."""
    rng = np.random.default_rng(82)
    Q = rng.integers(-3, 4, (5, 3)).astype(np.float32)
    DB = rng.integers(-3, 4, (4, 3)).astype(np.float32)
    idx, dist = oracle.knn(Q, DB, 7)
    full, fd = oracle.knn(Q, DB, 4)
    np.testing.assert_array_equal(idx[:, :4], full)
    np.testing.assert_array_equal(dist[:, :4], fd)
    assert (idx[:, 4:] == -1).all() and np.isinf(dist[:, 4:]).all()
    exact = ((Q[:, None, :].astype(np.int64) - DB[None].astype(np.int64)) ** 2).sum(-1)
    np.testing.assert_array_equal(np.sort(exact, axis=1), dist[:, :4])
    with pytest.raises(ValueError):
        oracle.knn(Q, DB, 0)


# ---------------------------------------------------- seeded draw, fit, spherical

def test_splitmix64_first_outputs():
    """SplitMix64 from seed 0 starts 0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4,
    0x06C45D188009454F (the values the generator's reference C code gives,
    widely used to check implementations)."""
    assert oracle.splitmix64(0, 3) == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    # the output is a function of (seed, position): seeding one step later
    # by the increment gives the same stream shifted by one
    assert oracle.splitmix64(0x9E3779B97F4A7C15, 2) == oracle.splitmix64(0, 3)[1:]


def test_sample_rows_distinct_in_range_and_uniform():
    for N, K, seed in [(1, 1, 0), (10, 10, 3), (1000, 17, 5), (2 ** 31 - 1, 64, 9)]:
        idx = oracle.sample_rows(N, K, seed)
        assert len(idx) == K and len(set(idx.tolist())) == K
        assert idx.min() >= 0 and idx.max() < N
    assert sorted(oracle.sample_rows(10, 10, 3).tolist()) == list(range(10))
    # every ordered pair of distinct rows of 5 is equally likely: 20 cells,
    # 40,000 draws, chi-square with 19 degrees of freedom below its 0.999
    # quantile (43.8); a shuffle that never picks the last row, or picks
    # from [i, N - 1) only, fails this
    cnt = np.zeros((5, 5))
    for seed in range(40000):
        i, j = oracle.sample_rows(5, 2, seed)
        cnt[i, j] += 1
    obs = cnt[~np.eye(5, dtype=bool)]
    chi2 = ((obs - 2000.0) ** 2 / 2000.0).sum()
    assert chi2 < 43.8, chi2
    with pytest.raises(ValueError):
        oracle.sample_rows(3, 4, 0)


def test_fit_tolerance_zero_stops_at_a_fixed_point():
    """tol = 0 stops once an iteration leaves every centroid unchanged; the
    result equals running all the iterations (the iteration is then at a
    fixed point), with fewer of them run."""
    rng = np.random.default_rng(83)
    X = np.concatenate([rng.normal(m, 0.05, (50, 2)) for m in ([0, 0], [3, 0], [0, 3])]).astype(np.float32)
    C0 = X[[0, 50, 100]]
    C_all, a_all, n_all, J_all = oracle.fit(X, C0, 30)
    C_t, a_t, n_t, J_t = oracle.fit(X, C0, 30, tol=0.0)
    assert len(J_t) < 30 and len(J_all) == 30
    assert C_t.tobytes() == C_all.tobytes()
    np.testing.assert_array_equal(a_t, a_all)
    np.testing.assert_array_equal(n_t, n_all)
    # an infinite tolerance stops after one iteration
    C_1, _, _, J_1 = oracle.fit(X, C0, 30, tol=np.inf)
    assert len(J_1) == 1
    assert C_1.tobytes() == oracle.lloyd_iter(X, C0)["C"].astype(np.float32).tobytes()


def test_centroid_shift_closed_form():
    C0 = np.array([[0, 0], [1, 1]], np.float32)
    C1 = np.array([[3, 4], [1, 2]], np.float32)
    assert oracle.centroid_shift(C0, C1) == 25.0


def test_fit_seeded_clamps_k_to_n():
    """K above N: N clusters from every row; distinct rows are then each
    their own centroid and the objective is zero."""
    X = np.arange(14, dtype=np.float32).reshape(7, 2)
    C, a, n, J, idx = oracle.fit_seeded(X, 10, 3, seed=4)
    assert C.shape == (7, 2) and sorted(idx.tolist()) == list(range(7))
    assert J[-1] == 0.0 and (n == 1).all()
    np.testing.assert_array_equal(C[a], X)


def test_spherical_update_closed_form():
    """Spherical centroids are the normalised mean of the normalised rows:
    rows (2, 0) and (0, 5) give (1/sqrt2, 1/sqrt2); a zero mean stays zero;
    an empty cluster returns its given centroid normalised."""
    X = np.array([[2, 0], [0, 5], [1, 0], [-3, 0]], np.float32)
    a = np.array([0, 0, 1, 1], np.int32)
    C_in = np.array([[9, 9], [9, 9], [0, -4]], np.float32)
    C, n = oracle.update(X, a, C_in, "spherical")
    np.testing.assert_array_equal(n, [2, 2, 0])
    assert np.allclose(C[0], [2 ** -0.5, 2 ** -0.5], rtol=0, atol=4e-16)
    assert (C[1] == 0).all()
    np.testing.assert_array_equal(C[2], [0, -1])


def test_spherical_centroid_maximises_cosine_sum():
    """The spherical centroid of a cluster is the unit vector c maximising
    sum_i xhat_i . c: no other unit vector (random ones, and small
    perturbations of c) does better; the iteration's objective sum_i
    (1 - xhat_i . c_{a_i}) does not increase."""
    rng = np.random.default_rng(84)
    X = (rng.standard_normal((300, 5)) + [2, 0, 0, 0, 0]).astype(np.float32)
    a = np.zeros(300, np.int32)
    C, _ = oracle.update(X, a, X[:1], "spherical")
    c = C[0]
    assert abs(np.linalg.norm(c) - 1) < 1e-12
    xh = X.astype(np.float64) / np.linalg.norm(X.astype(np.float64), axis=1, keepdims=True)
    best = (xh @ c).sum()
    for _ in range(200):
        v = c + 1e-3 * rng.standard_normal(5)
        v /= np.linalg.norm(v)
        assert (xh @ v).sum() <= best + 1e-9
        w = rng.standard_normal(5)
        w /= np.linalg.norm(w)
        assert (xh @ w).sum() <= best + 1e-9
    Xm = np.concatenate([rng.standard_normal((200, 6)) + m for m in np.eye(6) * 3]).astype(np.float32)
    Cc = Xm[rng.choice(len(Xm), 6, replace=False)]
    obj = []
    for _ in range(8):
        r = oracle.lloyd_iter(Xm, Cc, "spherical")
        Cc = r["C"].astype(np.float32)
        assert np.allclose(np.linalg.norm(r["C"], axis=1), 1.0, atol=1e-12)
        obj.append(r["J"])
    # under cosine assignment J = sum (2 - 2 xhat.c) with unit c (every
    # centroid after the first iteration is unit length)
    assert all(j1 <= j0 * (1 + 1e-12) for j0, j1 in zip(obj[1:], obj[2:]))


def test_ivf_build_seeded_and_clamped():
    """With no initial rows the quantizer starts from sample_rows(N,
    min(nlist, N), seed); nlist above N gives N cells of one row each."""
    rng = np.random.default_rng(85)
    X = rng.standard_normal((300, 4)).astype(np.float32)
    r1 = oracle.ivf_build(X, None, 3, nlist=16, seed=11)
    r2 = oracle.ivf_build(X, oracle.sample_rows(300, 16, 11), 3)
    for k in ("centroids", "offsets", "ids"):
        np.testing.assert_array_equal(r1[k], r2[k])
    small = X[:9]
    r = oracle.ivf_build(small, None, 2, nlist=40, seed=1)
    assert r["centroids"].shape == (9, 4)
    np.testing.assert_array_equal(r["offsets"], np.arange(10))
