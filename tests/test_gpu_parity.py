"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs.  Shapes span several tiles and ragged tails in N, d and
K, plus the degenerate cases (K=1, K>N, N=1, duplicated centroids, exact ties
on integer grids, zero rows, a large common offset)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import centroid_rel_err, check_min_dist, check_update, dev, host, log

pytestmark = pytest.mark.gpu

SHAPES = [
    (1, 1, 1), (5, 3, 7), (64, 4, 1), (1000, 16, 64), (4097, 128, 33), (3000, 100, 1000), (2049, 129, 65),
    (777, 768, 300), (500, 20, 4097), (300, 2048, 17), (2000, 31, 129), (130, 64, 3), (1025, 2, 2),
]


SCORES = ["fp32", "split_bf16"]


@pytest.mark.parametrize("score", SCORES)
@pytest.mark.parametrize("N,d,K", SHAPES)
@pytest.mark.parametrize("kind", ["gauss", "dup", "dup3", "dup40", "grid", "far", "zero"])
def test_assign_matches_oracle(gpu_lib, N, d, K, kind, score):
    fk = gpu_lib
    log(f"assign N={N} d={d} K={K} kind={kind} score={score}")
    X, C = synth.adversarial(3, N, d, K, kind)
    a_ref, D1, D2 = oracle.assign(X, C)
    a, md = fk.fk_assign(dev(X), dev(C), with_min_dist=True, score=score)
    a = host(a)
    np.testing.assert_array_equal(a, a_ref)
    check_min_dist(host(md), D1)


@pytest.mark.parametrize("score", SCORES)
@pytest.mark.parametrize("N,d,K", [(1000, 16, 64), (3001, 128, 257), (400, 768, 100), (999, 7, 5)])
@pytest.mark.parametrize("kind", ["gauss", "zero", "dup"])
def test_assign_cosine_matches_oracle(gpu_lib, N, d, K, kind, score):
    fk = gpu_lib
    log(f"cosine assign N={N} d={d} K={K} kind={kind} score={score}")
    X, C = synth.adversarial(4, N, d, K, kind)
    X[::3] *= np.float32(7.0)
    a_ref, D1, _ = oracle.assign(X, C, "cosine")
    a, md = fk.fk_assign(dev(X), dev(C), metric="cosine", with_min_dist=True, score=score)
    np.testing.assert_array_equal(host(a), a_ref)
    check_min_dist(host(md), D1)


@pytest.mark.parametrize("N,d,K", [(1, 4, 1), (1000, 16, 64), (5000, 128, 1024), (4096 * 3 + 5, 8, 300),
                                   (2048 * 5 + 7, 65, 40), (300, 768, 4096), (20000, 3, 2), (9000, 1030, 7),
                                   (2048 * 3 + 3, 100, 77), (4097, 68, 5)])
@pytest.mark.parametrize("metric", ["l2", "cosine"])
def test_update_matches_oracle(gpu_lib, N, d, K, metric):
    fk = gpu_lib
    log(f"update N={N} d={d} K={K} {metric}")
    rng = np.random.default_rng([N, d, K])
    X = rng.standard_normal((N, d)).astype(np.float32)
    # skewed labels, with some clusters left empty
    w = (np.arange(1, K + 1) ** -1.2)
    w /= w.sum()
    a = rng.choice(K, size=N, p=w).astype(np.int32)
    C_prev = rng.standard_normal((K, d)).astype(np.float32)
    C_out, counts = fk.fk_update(dev(X), dev(a), dev(C_prev), metric=metric)
    check_update(X, a, C_prev, host(C_out), host(counts), metric)


@pytest.mark.parametrize("score", SCORES)
@pytest.mark.parametrize("kind,path", [("dup", "paired"), ("dup3", "windowed"), ("dup40", "rechecked")])
def test_each_near_tie_path_is_taken(gpu_lib, kind, path, score):
    """Exact ties between 2, 3 and 40 copies of a centroid send points down
    each of the three fp64 paths (two-way compare, window compare, all K);
    the result must match the oracle on every one."""
    fk = gpu_lib
    X, C = synth.adversarial(6, 3000, 24, 200, kind)
    a_ref, _, _ = oracle.assign(X, C)
    fk.fk_profile_enable(True)
    a, _ = fk.fk_assign(dev(X), dev(C), score=score)
    prof = fk.fk_profile_read()
    fk.fk_profile_enable(False)
    np.testing.assert_array_equal(host(a), a_ref)
    assert prof[path] > 0, prof


@pytest.mark.parametrize("score", SCORES)
@pytest.mark.parametrize("metric", ["l2", "cosine"])
@pytest.mark.parametrize("d", [64, 201, 768, 1000])
@pytest.mark.parametrize("kind,path", [("dup", "paired"), ("dup3", "windowed"), ("dup40", "rechecked")])
def test_short_list_paths(gpu_lib, kind, path, d, metric, score):
    """Short near-tie lists (3,000 points) take the checks built for them:
    the window pass split over several tile slices of K = 600 centroids,
    each with its own candidate lists, and the fp64 distances summed by
    32-lane groups that pass the running sum from lane to lane (d <= 768;
    d = 1000 takes one lane per point), including a d that is not a multiple
    of four.  Every label must equal the oracle's."""
    fk = gpu_lib
    X, C = synth.adversarial(7, 3000, d, 600, kind)
    a_ref, _, _ = oracle.assign(X, C, metric)
    fk.fk_profile_enable(True)
    a, _ = fk.fk_assign(dev(X), dev(C), metric=metric, score=score)
    prof = fk.fk_profile_read()
    fk.fk_profile_enable(False)
    np.testing.assert_array_equal(host(a), a_ref)
    assert prof[path] > 0, prof


NEAR_TIE_CAP_MIN = 65536  # the window pass collects candidates for max(N/8, 65,536) listed points


@pytest.mark.parametrize("score", SCORES)
@pytest.mark.parametrize("metric", ["l2", "cosine", "inner_product"])
@pytest.mark.parametrize("d", [32, 128])
@pytest.mark.parametrize("kind", ["pairs", "dup3"])
def test_near_tie_paths_at_scale(gpu_lib, kind, d, metric, score):
    """200,000 points against 24 centroids that come in exact copies: with
    pairs nearly every point is an exact two-way tie, with three copies a
    three-way tie, so the pair list or the window list holds far more than
    65,536 points.  That takes the LDS-staged fp64 checks (d <= 128), and the
    window points past the candidate slots (max(N/8, 65,536) of them) go to
    the all-K rescoring.  Every label must equal the oracle's."""
    fk = gpu_lib
    N, K = 200000, 24
    log(f"near ties at scale: {kind} N={N} d={d} K={K} {metric} {score}")
    X, C = synth.adversarial(11, N, d, K, kind)
    a_ref, D1, _ = oracle.assign(X, C, metric)
    fk.fk_profile_enable(True)
    a, md = fk.fk_assign(dev(X), dev(C), metric=metric, with_min_dist=True, score=score)
    prof = fk.fk_profile_read()
    fk.fk_profile_enable(False)
    np.testing.assert_array_equal(host(a), a_ref)
    check_min_dist(host(md), D1)
    cap = max(N // 8, NEAR_TIE_CAP_MIN)
    if kind == "pairs":
        assert prof["paired"] >= NEAR_TIE_CAP_MIN, prof
    else:
        assert prof["windowed"] >= N - 100, prof
        assert prof["rechecked"] >= prof["windowed"] - cap, prof


@pytest.mark.parametrize("score", SCORES)
def test_window_list_beyond_cap(gpu_lib, score):
    """600,000 points, d = 24, 300 centroids in groups of three copies: every
    point is a three-way tie, the window list holds all of them, and the
    points past the 75,000 candidate slots are rescored against all K."""
    fk = gpu_lib
    N, d, K = 600000, 24, 300
    X, C = synth.adversarial(12, N, d, K, "dup3")
    a_ref, _, _ = oracle.assign(X, C)
    fk.fk_profile_enable(True)
    a, _ = fk.fk_assign(dev(X), dev(C), score=score)
    prof = fk.fk_profile_read()
    fk.fk_profile_enable(False)
    np.testing.assert_array_equal(host(a), a_ref)
    assert prof["rechecked"] > max(N // 8, NEAR_TIE_CAP_MIN), prof


@pytest.mark.parametrize("score", SCORES)
def test_window_list_over_several_grid_rounds(gpu_lib, score):
    """About 160,000 window points, more than one round of the window pass's
    persistent grid (625 slot groups of 256 on 512 workgroups) and under half
    the candidate slots: the pass cuts the centroid tiles into slices and the
    LDS-staged fp64 check merges several candidate lists per point.  Points
    around 8 of 200 well-separated centres, each centre present three times
    over, are exact three-way ties; every label must equal the oracle's
    (lowest index among the copies)."""
    fk = gpu_lib
    rng = np.random.default_rng(13)
    N, d, G = 4_000_000, 16, 200
    centres = (4.0 * rng.standard_normal((G, d))).astype(np.float32)
    C = np.concatenate([centres, centres[:8], centres[:8]])
    C = C[rng.permutation(len(C))]
    X = (centres[rng.integers(0, G, N)] + 0.3 * rng.standard_normal((N, d))).astype(np.float32)
    log(f"window list over several grid rounds: N={N} d={d} K={len(C)} {score}")
    a_ref, _, _ = oracle.assign(X, C)
    fk.fk_profile_enable(True)
    a, _ = fk.fk_assign(dev(X), dev(C), score=score)
    prof = fk.fk_profile_read()
    fk.fk_profile_enable(False)
    np.testing.assert_array_equal(host(a), a_ref)
    cap = max(N // 8, NEAR_TIE_CAP_MIN)
    assert 512 * 256 < prof["windowed"] <= cap // 2, prof
    assert prof["rechecked"] == 0, prof


@pytest.mark.parametrize("d", [64, 100])
def test_update_single_giant_cluster(gpu_lib, d):
    """Every point in one cluster: the cluster crosses every segment boundary
    (d = 100: rows read two per 16-byte load, one per half-wave, with an odd
    row count, so the last pair of the last segment has one row)."""
    fk = gpu_lib
    N, K = 200001, 5
    rng = np.random.default_rng(9)
    X = rng.standard_normal((N, d)).astype(np.float32)
    a = np.full(N, 3, np.int32)
    C_prev = rng.standard_normal((K, d)).astype(np.float32)
    C_out, counts = fk.fk_update(dev(X), dev(a), dev(C_prev))
    check_update(X, a, C_prev, host(C_out), host(counts))


@pytest.mark.parametrize("d", [33, 128, 300])
def test_update_sparse_labels(gpu_lib, d):
    """Labels on a few scattered clusters: cluster 0, long runs of ids and the
    last ids are empty, one cluster holds half the rows (it crosses many
    segment boundaries) and a few hold one row each.  The reduction writes
    the cluster offsets at each key change and the centroids of the clusters
    it completes; the empty ones must keep C_prev and count 0."""
    fk = gpu_lib
    N, K = 150001, 5000
    rng = np.random.default_rng(d)
    ids = np.array([3, 4, 17, 2000, 4990] + list(range(500, 540)), np.int32)
    a = rng.choice(ids, size=N).astype(np.int32)
    a[rng.choice(N, N // 2, replace=False)] = 2000
    a[rng.choice(N, 3, replace=False)] = np.array([1, 1234, 4998], np.int32)
    X = rng.standard_normal((N, d)).astype(np.float32)
    C_prev = rng.standard_normal((K, d)).astype(np.float32)
    log(f"update sparse labels d={d}")
    C_out, counts = fk.fk_update(dev(X), dev(a), dev(C_prev))
    check_update(X, a, C_prev, host(C_out), host(counts))


def test_update_empty_input(gpu_lib):
    fk = gpu_lib
    C_prev = np.random.default_rng(1).standard_normal((9, 5)).astype(np.float32)
    X = torch.empty((0, 5), dtype=torch.float32, device="cuda:0")
    a = torch.empty(0, dtype=torch.int32, device="cuda:0")
    C_out, counts = fk.fk_update(X, a, dev(C_prev))
    assert host(counts).tolist() == [0] * 9
    assert np.array_equal(host(C_out), C_prev)


@pytest.mark.parametrize("N,K", [(0, 5), (1, 1), (100, 1), (4096, 256), (4097, 257), (10000, 2), (70000, 1024),
                                 (300000, 32768), (50000, 65536), (8191, 255), (20000001, 40000),
                                 (2048, 2048), (2049, 2049), (1048576, 1024), (2097151, 2048), (2097152, 70),
                                 (4194303, 2047), (4194304, 4096), (3000000, 65536)])
def test_sort_inverse_matches_stable_argsort(gpu_lib, N, K):
    fk = gpu_lib
    log(f"sort N={N} K={K}")
    rng = np.random.default_rng([N, K])
    a = rng.integers(0, K, size=N).astype(np.int32)
    if N > 100:
        a[: N // 3] = K - 1      # a long run of one key, and skew
    perm, offsets = fk.fk_sort_inverse(dev(a), K) if N > 0 else fk.fk_sort_inverse(
        torch.empty(0, dtype=torch.int32, device="cuda:0"), K)
    perm = host(perm)
    offsets = host(offsets)
    np.testing.assert_array_equal(perm, np.argsort(a, kind="stable"))
    expect = np.concatenate([[0], np.cumsum(np.bincount(a, minlength=K))])
    np.testing.assert_array_equal(offsets, expect)


@pytest.mark.parametrize("score", SCORES)
@pytest.mark.parametrize("name,N,iters", [("tiny_d16_k64", 65536, 3), ("gmm_1m_d128_k1024", 60000, 3),
                                          ("ivf_1m_d768_k4096", 12000, 2), ("zipf_16m_d128_k32768", 33000, 2)])
def test_lloyd_iterations_step_level(gpu_lib, name, N, iters, score):
    """Step-level protocol: at every iteration the oracle is given the GPU's
    own centroids; assignments and counts must match exactly and centroids to
    1e-6 relative, and the objective must not increase."""
    fk = gpu_lib
    w = synth.WORKLOADS[name].scaled(N)
    log(f"iterations {name} N={N}")
    X = synth.rows(w)
    C = synth.initial_centroids(w, X)
    Xd = dev(X)
    Cd = dev(C)
    Js = []
    for t in range(iters):
        a, C1, counts, md = fk.fk_lloyd_iter(Xd, Cd, with_min_dist=True, score=score)
        ref = oracle.lloyd_iter(X, C)
        a_h = host(a)
        np.testing.assert_array_equal(a_h, ref["a"])
        np.testing.assert_array_equal(host(counts), ref["counts"])
        err = centroid_rel_err(host(C1), ref["C"], ref["counts"])
        assert err <= 1e-6, err
        assert host(counts).sum() == N
        Js.append(ref["J"])
        C = host(C1).copy()
        Cd = C1
    for j0, j1 in zip(Js, Js[1:]):
        assert j1 <= j0 * (1 + 1e-6)


@pytest.mark.parametrize("score", SCORES)
def test_determinism_bitwise(gpu_lib, score):
    fk = gpu_lib
    w = synth.WORKLOADS["zipf_16m_d128_k32768"].scaled(300000)
    X = synth.rows(w)
    C = synth.initial_centroids(w, X)
    Xd, Cd = dev(X), dev(C)
    r1 = [host(t) for t in fk.fk_lloyd_iter(Xd, Cd, with_min_dist=True, score=score)]
    r2 = [host(t) for t in fk.fk_lloyd_iter(Xd, Cd, with_min_dist=True, score=score)]
    for u, v in zip(r1, r2):
        assert u.tobytes() == v.tobytes()


def test_scores_agree(gpu_lib):
    """Both scoring modes give the same exact assignment, counts and centroids."""
    fk = gpu_lib
    w = synth.WORKLOADS["gmm_1m_d128_k1024"].scaled(200000)
    X = synth.rows(w)
    C = synth.initial_centroids(w, X)
    Xd, Cd = dev(X), dev(C)
    r1 = [host(t) for t in fk.fk_lloyd_iter(Xd, Cd, score="fp32")[:3]]
    r2 = [host(t) for t in fk.fk_lloyd_iter(Xd, Cd, score="split_bf16")[:3]]
    for u, v in zip(r1, r2):
        assert u.tobytes() == v.tobytes()


def test_k_larger_than_n(gpu_lib):
    fk = gpu_lib
    X, C = synth.adversarial(5, 50, 12, 200)
    a, C1, counts, _ = fk.fk_lloyd_iter(dev(X), dev(C))
    ref = oracle.lloyd_iter(X, C)
    np.testing.assert_array_equal(host(a), ref["a"])
    np.testing.assert_array_equal(host(counts), ref["counts"])
    assert (host(counts) == 0).sum() >= 150
    check_update(X, ref["a"], C, host(C1), host(counts))


def test_error_paths_on_device(gpu_lib):
    fk = gpu_lib
    X = torch.zeros((100, 8), device="cuda:0")
    C = torch.zeros((4, 8), device="cuda:0")
    with pytest.raises(fk.FkError) as e:
        fk.fk_assign(X, C, metric=4)
    assert e.value.status == 1
    with pytest.raises(fk.FkError) as e:
        fk.fk_ivf_build(X, 4, np.arange(4, dtype=np.int32), metric="inner_product")
    assert e.value.status == 2
    with pytest.raises(fk.FkError) as e:
        fk.fk_assign(X, C, score=5)
    assert e.value.status == 1
    small = torch.empty(1024, dtype=torch.uint8, device="cuda:0")
    with pytest.raises(fk.FkError) as e:
        fk.fk_assign(X, C, workspace=small)
    assert e.value.status == 3
    host_x = torch.zeros((100, 8))          # pageable
    import ctypes
    lib = fk.load()
    ws = torch.empty(fk.fk_workspace_size(100, 8, 4, "l2", 50) + 256, dtype=torch.uint8, device="cuda:0")
    base = ws.data_ptr() + (-ws.data_ptr()) % 256
    out = torch.empty((4, 8), device="cuda:0")
    cnt = torch.empty(4, dtype=torch.int32, device="cuda:0")
    st = lib.fk_lloyd_iter_stream(ctypes.c_void_p(host_x.data_ptr()), 100, 8, ctypes.c_void_p(C.data_ptr()), 4, 0, 0, 50,
                                  None, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(cnt.data_ptr()),
                                  ctypes.c_void_p(base), ws.numel() - 256, None)
    assert st == 1 and b"pinned" in lib.fk_last_error()


# ------------------------------------------------------------ inner product

@pytest.mark.parametrize("score", SCORES)
@pytest.mark.parametrize("N,d,K", [(1000, 16, 64), (4097, 128, 33), (2049, 129, 65), (777, 768, 300), (5, 3, 7),
                                   (3000, 100, 1000)])
@pytest.mark.parametrize("kind", ["gauss", "dup", "dup3", "grid", "zero"])
def test_inner_product_assign_matches_oracle(gpu_lib, N, d, K, kind, score):
    fk = gpu_lib
    log(f"ip assign N={N} d={d} K={K} kind={kind} score={score}")
    X, C = synth.adversarial(5, N, d, K, kind)
    a_ref, D1, _ = oracle.assign(X, C, "inner_product")
    a, md = fk.fk_assign(dev(X), dev(C), metric="inner_product", with_min_dist=True, score=score)
    np.testing.assert_array_equal(host(a), a_ref)
    check_min_dist(host(md), D1)


@pytest.mark.parametrize("score", SCORES)
def test_inner_product_iteration(gpu_lib, score):
    fk = gpu_lib
    w = synth.WORKLOADS["gmm_1m_d128_k1024"].scaled(20011)
    X = synth.rows(w)
    C = X[synth.init_indices(w)[:300]].copy()
    Xd, Cd = dev(X), dev(C)
    for it in range(3):
        a, Cn, n, _ = fk.fk_lloyd_iter(Xd, Cd, metric="inner_product", score=score)
        a = host(a)
        a_ref, _, _ = oracle.assign(X, host(Cd), "inner_product")
        np.testing.assert_array_equal(a, a_ref)
        check_update(X, a, host(Cd), host(Cn), host(n), "inner_product")
        Cd = Cn
