"""Parity at the workloads' full sizes, in the launch configuration bench.py
times (fk_lloyd_iter through the C ABI, X and C resident in HBM).

The oracle cannot score every point against every centroid at these sizes, so
the assignment is checked exactly on a seeded sample of points (the oracle
scores each sampled point against all K); the update is checked in full by
running the oracle's update on the GPU's own assignment (O(Nd)); counts are
checked in full against bincount of the GPU assignment and against the
oracle's update.  The out-of-core shape runs at a scaled N (its 10^9 rows need
512 GB of pinned host memory, more than a GPU-box command may hold) with the
configured 2^26-row chunks and a ragged last chunk."""
import time

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import centroid_rel_err, check_min_dist, dev, host, log

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]


def _sample(N, n, seed):
    rng = np.random.default_rng([seed, 99])
    return np.sort(rng.choice(N, size=min(n, N), replace=False))


@pytest.mark.parametrize("score", ["fp32", "split_bf16"])
@pytest.mark.parametrize("name,nsample", [("gmm_1m_d128_k1024", 4096), ("ivf_1m_d768_k4096", 1024),
                                          ("zipf_16m_d128_k32768", 2048)])
def test_full_size_iteration(gpu_lib, name, nsample, score):
    fk = gpu_lib
    w = synth.WORKLOADS[name]
    log(f"full size {name}: generating N={w.N}")
    X = synth.rows(w)
    C = synth.initial_centroids(w, X)
    Xd, Cd = dev(X), dev(C)
    # one warm-up iteration moves the centroids off the sampled points, as in
    # the timed steps of the benchmark
    _, C1d, _, _ = fk.fk_lloyd_iter(Xd, Cd, score=score)
    C1 = host(C1d).copy()
    log(f"full size {name}: second iteration")
    a, C2d, counts, md = fk.fk_lloyd_iter(Xd, C1d, with_min_dist=True, score=score)
    a = host(a)
    counts = host(counts)
    C2 = host(C2d)
    md = host(md)
    assert counts.sum() == w.N
    np.testing.assert_array_equal(counts, np.bincount(a, minlength=w.K))
    idx = _sample(w.N, nsample, w.seed)
    log(f"full size {name}: oracle on {len(idx)} sampled points")
    a_ref, D1, D2 = oracle.assign(X[idx], C1)
    np.testing.assert_array_equal(a[idx], a_ref)
    check_min_dist(md[idx], D1, X[idx], C1, score=score)
    log(f"full size {name}: oracle update on the GPU assignment")
    C_ref, n_ref = oracle.update(X, a, C1)
    np.testing.assert_array_equal(counts, n_ref)
    err = centroid_rel_err(C2, C_ref, n_ref)
    assert err <= 1e-6, err
    empty = n_ref == 0
    assert np.array_equal(C2[empty].view(np.uint32), C1[empty].view(np.uint32))


@pytest.mark.parametrize("score", ["fp32", "split_bf16"])
def test_out_of_core_scaled(gpu_lib, score):
    fk = gpu_lib
    w0 = synth.WORKLOADS["ooc_1b_d128_k32768"]
    N = (1 << 26) + (1 << 25) + 777          # two chunks of 2^26 rows, the second ragged
    w = w0.scaled(N)
    log(f"out of core: N={N}, chunk {w.chunk_rows}")
    Xh = torch.empty((N, w.d), dtype=torch.float32, pin_memory=True)
    X = Xh.numpy()
    synth.rows(w, out=X)
    C = X[synth.init_indices(w)].copy()
    ah = torch.empty(N, dtype=torch.int32, pin_memory=True)
    Cd = dev(C)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    C1d, cnt = fk.fk_lloyd_iter_stream(Xh, Cd, w.chunk_rows, assign_host=ah, score=score)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    log(f"out of core ({score}): one iteration in {dt:.2f} s including PCIe ({N * w.d * 4 / dt / 1e9:.1f} GB/s of X)")
    a = ah.numpy()
    counts = host(cnt)
    assert counts.sum() == N
    np.testing.assert_array_equal(counts, np.bincount(a, minlength=w.K))
    idx = _sample(N, 1024, 3)
    a_ref, _, _ = oracle.assign(X[idx], C)
    np.testing.assert_array_equal(a[idx], a_ref)
    C_ref, n_ref = oracle.update(X, a, C)
    np.testing.assert_array_equal(counts, n_ref)
    assert centroid_rel_err(host(C1d), C_ref, n_ref) <= 1e-6


@pytest.mark.parametrize("score", ["fp32", "split_bf16"])
def test_ivf_build_full_size(gpu_lib, score):
    """The IVF-Flat build at the 1M x 768, nlist = 4096, niter = 20 shape
    (rows pre-normalised, L2), in the configuration bench.py --ivf-build
    times: sampled list positions must hold a row whose exact nearest final
    centroid (oracle, fp64) is the position's cell, the row copied bit for
    bit; ids must be a permutation, increasing within each cell."""
    fk = gpu_lib
    w = synth.WORKLOADS["ivf_1m_d768_k4096"]
    X = synth.rows(w)
    init = synth.init_indices(w).astype(np.int32)
    Xd = dev(X)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    out = fk.fk_ivf_build(Xd, w.K, init, n_iter=20, score=score)
    torch.cuda.synchronize()
    log(f"ivf build ({score}): {time.perf_counter() - t0:.2f} s")
    C = host(out["centroids"])
    ids_t = out["ids"].long()
    assert torch.equal(torch.sort(ids_t).values, torch.arange(w.N, device=ids_t.device))
    offs = host(out["offsets"]).astype(np.int64)
    assert offs[0] == 0 and offs[-1] == w.N and (np.diff(offs) >= 0).all()
    ids = host(out["ids"])
    cell = np.searchsorted(offs, np.arange(w.N), side="right") - 1
    same_cell = cell[1:] == cell[:-1]
    assert (np.diff(ids.astype(np.int64))[same_cell] > 0).all()
    pos = _sample(w.N, 1024, 5)
    a_ref, _, _ = oracle.assign(X[ids[pos]], C)
    np.testing.assert_array_equal(a_ref, cell[pos])
    data = host(out["data"][torch.from_numpy(pos).to(Xd.device)])
    np.testing.assert_array_equal(data.view(np.uint32), X[ids[pos]].view(np.uint32))


@pytest.mark.parametrize("score", ["fp32", "split_bf16"])
@pytest.mark.parametrize("name,nsample", [("knn_1m_d128_q10k", 96), ("knn_1m_d768_q10k", 24)])
def test_knn_full_size(gpu_lib, name, nsample, score):
    """Exact k-NN at the full shapes, in the configuration bench.py --knn
    times (all queries in one call): a seeded sample of queries checked
    exactly against the oracle's brute force over the whole database; for
    every query the distances must be non-decreasing and equal the fp64
    distance of the reported row rounded to fp32 (checked on the GPU)."""
    fk = gpu_lib
    w = synth.WORKLOADS[name]
    DB = synth.rows(w)
    Q = synth.queries(w)
    DBd, Qd = dev(DB), dev(Q)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    idx, dist = fk.fk_knn(Qd, DBd, w.k, metric=w.metric, score=score)
    torch.cuda.synchronize()
    log(f"knn {name} ({score}): {1e3 * (time.perf_counter() - t0):.1f} ms")
    assert bool((dist[:, 1:] >= dist[:, :-1]).all())
    rows = DBd[idx.long()].double()                          # [M, k, d]
    D = ((Qd.double()[:, None, :] - rows) ** 2).sum(-1)
    # a different summation order: equal to within a few fp64 ulps
    assert bool(((D.float() - dist).abs() <= 1e-5 * dist.abs() + 1e-30).all())
    qs = _sample(Q.shape[0], nsample, 17)
    i_ref, d_ref = oracle.knn(Q[qs], DB, w.k, w.metric)
    np.testing.assert_array_equal(host(idx)[qs], i_ref)
    np.testing.assert_array_equal(host(dist)[qs], d_ref.astype(np.float32))
