"""The seeded workload generators: determinism, block independence, and the
statistics the recipe promises (CPU only, small row counts)."""
import numpy as np
import pytest

import synth


def test_same_seed_same_bytes_and_threads_do_not_matter():
    w = synth.WORKLOADS["gmm_1m_d128_k1024"].scaled(200000)
    a = synth.rows(w, threads=1)
    b = synth.rows(w, threads=4)
    assert a.dtype == np.float32 and a.shape == (200000, 128)
    assert a.tobytes() == b.tobytes()


def test_row_ranges_match_full_generation():
    w = synth.WORKLOADS["tiny_d16_k64"]
    full = synth.rows(w)
    part = synth.rows(w, 1000, 60001)
    np.testing.assert_array_equal(part, full[1000:60001])
    idx = np.array([5, 65535, 3, 40000])
    np.testing.assert_array_equal(synth.gather_rows(w, idx), full[idx])


def test_scaled_prefix_is_the_full_prefix():
    w = synth.WORKLOADS["zipf_16m_d128_k32768"]
    small = synth.rows(w.scaled(70000), threads=2)
    prefix = synth.rows(w, 0, 70000, threads=2)
    np.testing.assert_array_equal(small, prefix)


def test_mixture_statistics():
    w = synth.WORKLOADS["tiny_d16_k64"]
    X, lab = synth.rows(w, return_labels=True)
    mu = synth.means(w)
    assert mu.min() >= -1 and mu.max() <= 1
    resid = X - mu[lab]
    assert abs(resid.std() - 0.1) < 0.002
    assert abs(resid.mean()) < 0.002
    counts = np.bincount(lab, minlength=64)
    assert counts.min() > 800 and counts.max() < 1250      # equal weights, 1024 expected


def test_zipf_weights_and_frequencies():
    w = synth.WORKLOADS["zipf_16m_d128_k32768"]
    p = synth.weights(w)
    assert abs(p.sum() - 1) < 1e-12
    assert abs(p[0] / p[1] - 2 ** 1.2) < 1e-9
    assert 0.19 < p[0] < 0.21                    # the top component holds about 20%
    _, lab = synth.rows(w.scaled(400000), return_labels=True, threads=2)
    freq = np.bincount(lab, minlength=w.K) / 400000
    assert abs(freq[0] - p[0]) < 0.005
    assert abs(freq[1] - p[1]) < 0.005


def test_normalised_rows_are_unit():
    w = synth.WORKLOADS["ivf_1m_d768_k4096"].scaled(3000)
    X = synth.rows(w)
    n = np.linalg.norm(X.astype(np.float64), axis=1)
    assert np.all(np.abs(n - 1) < 1e-6)


def test_initial_centroids():
    w = synth.WORKLOADS["gmm_1m_d128_k1024"]
    idx = synth.init_indices(w)
    assert len(idx) == 1024 and len(np.unique(idx)) == 1024 and idx.max() < w.N
    t = synth.WORKLOADS["tiny_d16_k64"]
    np.testing.assert_array_equal(synth.init_indices(t), np.arange(64))
    C = synth.initial_centroids(w.scaled(w.N), None)[:3]
    np.testing.assert_array_equal(C, synth.gather_rows(w, idx[:3]))


def test_out_of_core_shape():
    w = synth.WORKLOADS["ooc_1b_d128_k32768"]
    assert w.N == 10 ** 9 and w.chunk_rows == 1 << 26
    blk = synth.rows(w, w.N - 10, w.N)
    assert blk.shape == (10, 128)


@pytest.mark.parametrize("kind", ["gauss", "dup", "grid", "far", "zero"])
def test_adversarial_inputs(kind):
    X, C = synth.adversarial(1, 100, 7, 9, kind)
    X2, C2 = synth.adversarial(1, 100, 7, 9, kind)
    assert X.dtype == np.float32 and X.shape == (100, 7) and C.shape == (9, 7)
    assert X.tobytes() == X2.tobytes() and C.tobytes() == C2.tobytes()


def test_knn_queries_are_seeded_prefixes_and_differ_from_rows():
    w = synth.WORKLOADS["knn_1m_d128_q10k"]
    q = synth.queries(w, 3000)
    np.testing.assert_array_equal(q[:1000], synth.queries(w, 1000))
    np.testing.assert_array_equal(q, synth.queries(w, 3000))
    x = synth.rows(w.scaled(70000), 0, 3000)
    assert not np.array_equal(q, x)
    # the "zero" means: plain standard normal draws
    assert abs(float(q.mean())) < 0.01 and abs(float(q.std()) - 1.0) < 0.01
    assert synth.queries(w).shape == (w.queries, w.d)
