"""Parity at the workloads' full sizes, in the launch configuration bench.py
times (fk_lloyd_iter through the C ABI, X and C resident in HBM).

Every label of every point is compared with the oracle's.  The oracle's own
Lloyd trajectory on each workload, from the workload's initial centroids, is
stored as digests in tests/golden/fullsize_<workload>.json (written by
tests/golden/make_fullsize_digests.py, which calls only the oracle and the
seeded generator): per iteration, a hash of the labels of every 65,536-row
block, a hash of the counts, the objective per block and a hash of the next
centroids.  The test walks the same trajectory: at iteration t the GPU
iterates from the oracle's C_t; its labels must hash to the oracle's in every
block and its counts to the oracle's counts; with the labels equal, the
oracle's update of them (O(Nd), run here) is the oracle's C_{t+1}, whose hash
must match the stored one, and the GPU's new centroids must be within 1e-6
relative of it.  The objective sum of the GPU's min_dist must match the
oracle's per block within the summed per-point bound.  A block that differs
is rescored by the oracle in full to report the mismatches.

The out-of-core shape runs at a scaled N (its 10^9 rows need 512 GB of pinned
host memory, more than a GPU-box command may hold) with the configured
2^26-row chunks and a ragged last chunk, sampled."""
import hashlib
import json
import os
import time

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import centroid_rel_err, dev, host, log, objective_tol

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _sample(N, n, seed):
    rng = np.random.default_rng([seed, 99])
    return np.sort(rng.choice(N, size=min(n, N), replace=False))


def _digest(a):
    return hashlib.blake2b(np.ascontiguousarray(a).tobytes(), digest_size=16).hexdigest()


def _trajectory(name):
    path = os.path.join(GOLDEN, f"fullsize_{name}.json")
    with open(path) as f:
        return json.load(f)


@pytest.mark.parametrize("score", ["fp32", "split_bf16"])
@pytest.mark.parametrize("name", ["tiny_d16_k64", "gmm_1m_d128_k1024", "ivf_1m_d768_k4096", "zipf_16m_d128_k32768"])
def test_full_size_oracle_trajectory(gpu_lib, name, score):
    fk = gpu_lib
    doc = _trajectory(name)
    w = synth.WORKLOADS[name]
    assert (doc["N"], doc["d"], doc["K"]) == (w.N, w.d, w.K)
    B = doc["block_rows"]
    log(f"full size {name} ({score}): generating N={w.N}, {len(doc['iterations'])} stored oracle iterations")
    X = synth.rows(w)
    C = synth.initial_centroids(w, X)
    assert _digest(C) == doc["initial_centroids_hash"], "the seeded inputs differ from those the oracle ran on"
    Xd = dev(X)
    worst_err = 0.0
    for it in doc["iterations"]:
        t = it["t"]
        assert _digest(C) == it["centroids_hash"]
        t0 = time.perf_counter()
        a_d, C1d, counts_d, md_d = fk.fk_lloyd_iter(Xd, dev(C), with_min_dist=True, score=score)
        a, C1, counts, md = host(a_d), host(C1d), host(counts_d), host(md_d)
        gpu_s = time.perf_counter() - t0
        blocks = [_digest(a[b:b + B].astype("<i4")) for b in range(0, w.N, B)]
        bad = [i for i, (u, v) in enumerate(zip(blocks, it["label_blocks"])) if u != v]
        if bad:
            lines = []
            for i in bad[:4]:
                lo, hi = i * B, min(w.N, (i + 1) * B)
                a_ref, D1, D2 = oracle.assign(X[lo:hi], C)
                miss = np.nonzero(a[lo:hi] != a_ref)[0]
                g = oracle.relative_gap(D1[miss], D2[miss])
                lines.append(f"block {i}: {len(miss)} labels differ, rows {lo + miss[:5]}, gaps {g[:5]}")
            pytest.fail(f"{name} iteration {t}: {len(bad)} of {len(blocks)} label blocks differ from the "
                        f"oracle's; " + "; ".join(lines))
        assert _digest(counts.astype("<i4")) == it["counts_hash"], f"iteration {t}: counts differ from the oracle's"
        if it["counts"] is not None:
            np.testing.assert_array_equal(counts, it["counts"])
        # the labels equal the oracle's, so its update of them is the oracle's own C_{t+1}
        C_ref, n_ref = oracle.update(X, a, C, w.metric)
        np.testing.assert_array_equal(counts, n_ref)
        C_next = C_ref.astype(np.float32)
        assert _digest(C_next) == it["next_centroids_hash"]
        err = centroid_rel_err(C1, C_ref, n_ref)
        assert err <= 1e-6, f"iteration {t}: centroid rel err {err}"
        empty = n_ref == 0
        assert np.array_equal(C1[empty].view(np.uint32), C[empty].view(np.uint32))
        worst_err = max(worst_err, err)
        # objective: the GPU's fp32 min_dist summed per block against the oracle's D1 sums
        J_gpu = 0.0
        for i, Jb in enumerate(it["J_blocks"]):
            lo, hi = i * B, min(w.N, (i + 1) * B)
            s = float(md[lo:hi].astype(np.float64).sum())
            tol = objective_tol(md[lo:hi])
            assert abs(s - Jb) <= tol, f"iteration {t} block {i}: objective {s} vs oracle {Jb} (tol {tol})"
            J_gpu += s
        log(f"VALIDATION {json.dumps({'workload': name, 'score': score, 'iteration': t, 'N': w.N, 'label_mismatches': 0, 'blocks': len(blocks), 'counts_equal': True, 'exempt_g_le_1e-5': it['gap']['le_1e-05'], 'g_le_1e-7': it['gap']['le_1e-07'], 'exact_ties': it['gap']['eq_0'], 'empty': it['empty'], 'max_centroid_rel_err': err, 'J_oracle': it['J'], 'J_gpu_fp32_min_dist': J_gpu, 'gpu_iter_s_incl_copies': round(gpu_s, 3)})}")
        C = C_next


@pytest.mark.parametrize("score", ["fp32", "split_bf16"])
def test_out_of_core_scaled(gpu_lib, score):
    fk = gpu_lib
    w0 = synth.WORKLOADS["ooc_1b_d128_k32768"]
    N = (1 << 26) + (1 << 25) + 777          # two chunks of 2^26 rows, the second ragged
    w = w0.scaled(N)
    log(f"out of core: N={N}, chunk {w.chunk_rows}")
    # hand back pinned blocks that earlier tests in this process left cached
    # before asking for 51.5 GB of pinned rows
    import gc
    gc.collect()
    torch._C._host_emptyCache()
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
    # give back the pinned rows and the chunked workspace at once
    del Xh, ah, X
    fk._ws_cache.clear()
    torch.cuda.empty_cache()
    torch._C._host_emptyCache()


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
