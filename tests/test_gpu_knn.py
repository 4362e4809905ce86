"""GPU parity of the exact k-NN (fk_knn) against the oracle's brute force:
the neighbour indices bit-exact (nearest first, lower row index first on
equal distances) and the distances equal to the oracle's fp64 distances
rounded to fp32, across the kernel's shapes (d from 5 to 200, resident and
chunked query blocks, 16 and 32 candidates), both score modes, the three
metrics, ragged query and database sizes, databases smaller than the
candidate list, and exact ties wider than it (the all-rows fallback)."""
import dataclasses

import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import dev, host, log

pytestmark = pytest.mark.gpu

SCORES = ["fp32", "split_bf16"]


def _check(fk, Q, DB, k, metric, score):
    idx, dist = fk.fk_knn(dev(Q), dev(DB), k, metric=metric, score=score)
    i_ref, d_ref = oracle.knn(Q, DB, k, metric)
    gi, gd = host(idx), host(dist)
    np.testing.assert_array_equal(gi, i_ref)
    # distances bit for bit (inner product: -0 for a zero dot product)
    np.testing.assert_array_equal(gd.view(np.uint32), d_ref.astype(np.float32).view(np.uint32))


@pytest.mark.parametrize("score", SCORES)
@pytest.mark.parametrize("d", [5, 16, 32, 48, 100, 128, 200])
@pytest.mark.parametrize("k", [1, 10, 13, 24])
def test_knn_shapes(gpu_lib, score, d, k):
    rng = np.random.default_rng(1000 + d * 31 + k)
    M, Ndb = 1100, 3001          # several query blocks and tiles, ragged tails
    Q = rng.standard_normal((M, d)).astype(np.float32)
    DB = rng.standard_normal((Ndb, d)).astype(np.float32)
    log(f"knn d={d} k={k} score={score}")
    _check(gpu_lib, Q, DB, k, "l2", score)


@pytest.mark.parametrize("score", SCORES)
@pytest.mark.parametrize("metric", ["l2", "cosine", "inner_product"])
@pytest.mark.parametrize("k", [3, 10, 20])
def test_knn_metrics_on_a_mixture(gpu_lib, score, metric, k):
    w = synth.WORKLOADS["knn_1m_d768_q10k"]
    w = dataclasses.replace(w, d=64, K=64).scaled(65536)
    DB = synth.rows(w, 0, 5000)
    Q = synth.queries(w, 700)
    log(f"knn mixture metric={metric} k={k} score={score}")
    _check(gpu_lib, Q, DB, k, metric, score)


@pytest.mark.parametrize("score", SCORES)
@pytest.mark.parametrize("Ndb,k", [(1, 1), (5, 3), (5, 5), (16, 16), (31, 20), (40, 24)])
def test_knn_database_smaller_than_the_candidate_list(gpu_lib, score, Ndb, k):
    rng = np.random.default_rng(Ndb * 100 + k)
    Q = rng.standard_normal((300, 24)).astype(np.float32)
    DB = rng.standard_normal((Ndb, 24)).astype(np.float32)
    log(f"knn small database Ndb={Ndb} k={k} score={score}")
    _check(gpu_lib, Q, DB, k, "l2", score)


@pytest.mark.parametrize("score", SCORES)
@pytest.mark.parametrize("kind", ["dup", "dup3", "dup40", "grid", "far", "zero"])
@pytest.mark.parametrize("k", [4, 17])
def test_knn_ties_and_edge_inputs(gpu_lib, score, kind, k):
    """Duplicated rows give exact ties (40 copies of one row: wider than the
    candidate list, so the query is ranked against every row), integer grids
    many ties, a far offset cancellation, zero rows zero distances."""
    X, C = synth.adversarial(91, 900, 20, 300, kind)
    log(f"knn ties kind={kind} k={k} score={score}")
    _check(gpu_lib, X, C, k, "l2", score)
    _check(gpu_lib, X, C, k, "inner_product", score)


@pytest.mark.parametrize("score", SCORES)
def test_knn_every_query_falls_back(gpu_lib, score):
    """A database of one row repeated: every candidate ties, every query goes
    to the all-rows fp64 ranking, which must give rows 0..k-1."""
    rng = np.random.default_rng(7)
    DB = np.repeat(rng.standard_normal((1, 32)).astype(np.float32), 2000, axis=0)
    Q = rng.standard_normal((600, 32)).astype(np.float32)
    idx, dist = gpu_lib.fk_knn(dev(Q), dev(DB), 12, score=score)
    np.testing.assert_array_equal(host(idx), np.tile(np.arange(12, dtype=np.int32), (600, 1)))
    _check(gpu_lib, Q, DB, 12, "l2", score)


def test_knn_empty_queries_and_clamped_k(gpu_lib):
    DB = np.random.default_rng(3).standard_normal((7, 16)).astype(np.float32)
    idx, dist = gpu_lib.fk_knn(dev(np.zeros((0, 16), np.float32)), dev(DB), 5)
    assert tuple(idx.shape) == (0, 5) and tuple(dist.shape) == (0, 5)
    Q = np.random.default_rng(4).standard_normal((9, 16)).astype(np.float32)
    idx, dist = gpu_lib.fk_knn(dev(Q), dev(DB), 10)   # k clamped to Ndb = 7 in the library
    assert tuple(idx.shape) == (9, 10)
    assert (host(idx)[:, 7:] == -1).all() and np.isinf(host(dist)[:, 7:]).all()
    _check(gpu_lib, Q, DB, 10, "l2", "fp32")
    _check(gpu_lib, Q, DB, 10, "cosine", "split_bf16")
    DB1 = DB[:1]
    _check(gpu_lib, Q, DB1, 24, "inner_product", "fp32")
    _check(gpu_lib, Q, DB1, 60, "l2", "split_bf16")  # k beyond the limit, but Ndb = 1


def test_knn_repeatable_and_workspace_reuse(gpu_lib):
    rng = np.random.default_rng(11)
    Q = rng.standard_normal((2000, 96)).astype(np.float32)
    DB = rng.standard_normal((4000, 96)).astype(np.float32)
    a = [host(t) for t in gpu_lib.fk_knn(dev(Q), dev(DB), 10, score="split_bf16")]
    b = [host(t) for t in gpu_lib.fk_knn(dev(Q[:500]), dev(DB), 10, score="split_bf16")]
    c = [host(t) for t in gpu_lib.fk_knn(dev(Q), dev(DB), 10, score="split_bf16")]
    np.testing.assert_array_equal(a[0], c[0])
    np.testing.assert_array_equal(a[1].view(np.uint32), c[1].view(np.uint32))
    np.testing.assert_array_equal(a[0][:500], b[0])


@pytest.mark.parametrize("score", SCORES)
@pytest.mark.parametrize("d,k", [(32, 10), (128, 10), (128, 20), (200, 5)])
def test_knn_database_slices(gpu_lib, score, d, k):
    """A database of 20,001 rows is cut into 5 slices (4,096 rows each, the
    last ragged): the slices' candidate lists are merged per query."""
    rng = np.random.default_rng(2000 + d + k)
    Q = rng.standard_normal((700, d)).astype(np.float32)
    DB = rng.standard_normal((20001, d)).astype(np.float32)
    log(f"knn slices d={d} k={k} score={score}")
    _check(gpu_lib, Q, DB, k, "l2", score)


@pytest.mark.parametrize("score", SCORES)
def test_knn_ties_across_slices(gpu_lib, score):
    """Copies of the same rows in different slices: equal distances across
    slices must still come out lower index first."""
    rng = np.random.default_rng(12)
    base = rng.standard_normal((4096, 24)).astype(np.float32)
    DB = np.concatenate([base, base[::-1], base, base[:1000]])        # 13,288 rows, 4 slices
    Q = np.concatenate([base[::37] + np.float32(0.01), rng.standard_normal((200, 24)).astype(np.float32)])
    log(f"knn ties across slices score={score}")
    _check(gpu_lib, Q, DB, 7, "l2", score)
    _check(gpu_lib, Q, DB, 16, "inner_product", score)


@pytest.mark.parametrize("score", SCORES)
@pytest.mark.parametrize("metric", ["l2", "cosine", "inner_product"])
@pytest.mark.parametrize("kind", ["near_first", "far_first", "repeated"])
def test_knn_sample_threshold(gpu_lib, score, kind, metric):
    """With several database slices, a first sweep over the first 4096 rows
    gives each query a score at or below its L-th best, and the slices' lists
    start full of it.  The first rows either hold the true neighbours (a
    tight threshold), lie far away (a loose one), or the database repeats a
    few rows (the threshold ties with many rows, and with the L-th best)."""
    rng = np.random.default_rng({"near_first": 1, "far_first": 2, "repeated": 3}[kind])
    d, Ndb, M = 48, 24001, 900
    Q = rng.standard_normal((M, d)).astype(np.float32)
    if kind == "repeated":
        base = rng.standard_normal((11, d)).astype(np.float32)
        DB = base[rng.integers(0, 11, size=Ndb)]
    else:
        DB = rng.standard_normal((Ndb, d)).astype(np.float32) * np.float32(3.0)
        if kind == "near_first":
            DB[:M] = Q + np.float32(0.01) * rng.standard_normal((M, d)).astype(np.float32)
        else:
            DB[:4096] += np.float32(50.0)
    log(f"knn sample threshold {kind} {metric} score={score}")
    for k in (5, 20):
        _check(gpu_lib, Q, DB, k, metric, score)
