"""The allocation-free Lloyd iteration (fk_lloyd_iter_noalloc), called
through the C ABI, against fk_lloyd_iter on the same inputs: two calls in a
row, the second smaller, must give bit-identical assignments, min_dist,
centroids and counts (the second call also against the oracle's labels and
counts); sizes beyond the static scratch are rejected."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import dev, host, log

pytestmark = pytest.mark.gpu


def _noalloc(lib, X, C, metric, score):
    N, d = X.shape
    K = C.shape[0]
    a = torch.full((N,), -1, dtype=torch.int32, device=X.device)
    md = torch.full((N,), float("nan"), dtype=torch.float32, device=X.device)
    C1 = torch.full((K, d), float("nan"), dtype=torch.float32, device=X.device)
    n = torch.full((K,), -1, dtype=torch.int32, device=X.device)
    P = ctypes.c_void_p
    st = lib.fk_lloyd_iter_noalloc(P(X.data_ptr()), N, d, P(C.data_ptr()), K, metric, score, P(a.data_ptr()),
                                   P(md.data_ptr()), P(C1.data_ptr()), P(n.data_ptr()),
                                   P(torch.cuda.current_stream().cuda_stream))
    if st != 0:
        free, total = torch.cuda.mem_get_info()
        pytest.fail(f"status {st}: {lib.fk_last_error()} (device memory free {free / 2**30:.1f} of "
                    f"{total / 2**30:.1f} GiB, torch reserved {torch.cuda.memory_reserved() / 2**30:.1f} GiB)")
    torch.cuda.synchronize()
    return a, md, C1, n


@pytest.mark.parametrize("score", ["fp32", "split_bf16"])
@pytest.mark.parametrize("metric", ["l2", "cosine"])
def test_noalloc_matches_lloyd_iter(gpu_lib, metric, score):
    fk = gpu_lib
    lib = fk.load()
    w = synth.WORKLOADS["gmm_1m_d128_k1024"].scaled(300000)
    Xall = synth.rows(w)
    C = synth.initial_centroids(w, Xall)
    for N in (300000, 70001):  # the second call is smaller: the scratch keeps the first call's contents
        log(f"noalloc {metric} {score} N={N}")
        X = Xall[:N]
        Xd, Cd = dev(X), dev(C)
        a, md, C1, n = _noalloc(lib, Xd, Cd, fk.METRICS[metric], fk.SCORES[score])
        ra, rC, rn, rmd = fk.fk_lloyd_iter(Xd, Cd, metric=metric, with_min_dist=True, score=score)
        for u, v in ((a, ra), (md, rmd), (C1, rC), (n, rn)):
            assert host(u).tobytes() == host(v).tobytes()
        if N < 100000:
            a_ref, _, _ = oracle.assign(X, C, metric)
            np.testing.assert_array_equal(host(a), a_ref)
            np.testing.assert_array_equal(host(n), np.bincount(a_ref, minlength=w.K))


def test_noalloc_rejects_sizes_beyond_scratch(gpu_lib):
    fk = gpu_lib
    lib = fk.load()
    N, d, K = 3000000, 128, 4096
    assert fk.fk_workspace_size(N, d, K) > fk.NOALLOC_SCRATCH_BYTES
    X = torch.zeros((N, d), dtype=torch.float32, device="cuda:0")
    C = torch.zeros((K, d), dtype=torch.float32, device="cuda:0")
    a = torch.empty(N, dtype=torch.int32, device="cuda:0")
    C1 = torch.empty((K, d), dtype=torch.float32, device="cuda:0")
    n = torch.empty(K, dtype=torch.int32, device="cuda:0")
    with pytest.raises(fk.FkError) as e:
        fk.fk_lloyd_iter_noalloc(X, C, a, C1, n)
    assert e.value.status == 3 and "scratch" in str(e.value)
