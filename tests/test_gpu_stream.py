"""Out-of-core iteration (pinned host X streamed in chunks) against the
in-core iteration and the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import centroid_rel_err, dev, host, log

pytestmark = pytest.mark.gpu


def _pinned(a):
    t = torch.empty(a.shape, dtype=torch.from_numpy(a[:0]).dtype, pin_memory=True)
    t.numpy()[...] = a
    return t


@pytest.mark.parametrize("score", ["fp32", "split_bf16"])
@pytest.mark.parametrize("metric", ["l2", "cosine"])
@pytest.mark.parametrize("chunk", [100000, 65537, 300000, 300005, 4096])
def test_stream_equals_in_core(gpu_lib, chunk, metric, score):
    fk = gpu_lib
    w = synth.WORKLOADS["ooc_1b_d128_k32768"].scaled(300000)
    K = 2048
    log(f"stream chunk={chunk} {metric}")
    X = synth.rows(w)
    C = X[synth.init_indices(w)[:K]].copy()
    a_ic, C_ic, n_ic, _ = fk.fk_lloyd_iter(dev(X), dev(C), metric=metric, score=score)
    Xh = _pinned(X)
    ah = torch.empty(w.N, dtype=torch.int32, pin_memory=True)
    C_s, n_s = fk.fk_lloyd_iter_stream(Xh, dev(C), chunk, metric=metric, assign_host=ah, score=score)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ah.numpy(), host(a_ic))
    np.testing.assert_array_equal(host(n_s), host(n_ic))
    err = centroid_rel_err(host(C_s), host(C_ic).astype(np.float64), host(n_ic))
    assert err <= 1e-6, err
    # and against the oracle on a sample of points
    idx = np.random.default_rng(0).choice(w.N, 500, replace=False)
    a_ref, _, _ = oracle.assign(X[idx], C, metric)
    np.testing.assert_array_equal(ah.numpy()[idx], a_ref)


def test_stream_without_assignment_output(gpu_lib):
    fk = gpu_lib
    w = synth.WORKLOADS["tiny_d16_k64"]
    X = synth.rows(w)
    C = synth.initial_centroids(w, X)
    C_s, n_s = fk.fk_lloyd_iter_stream(_pinned(X), dev(C), 10000)
    ref = oracle.lloyd_iter(X, C)
    np.testing.assert_array_equal(host(n_s), ref["counts"])
    assert centroid_rel_err(host(C_s), ref["C"], ref["counts"]) <= 1e-6


@pytest.mark.parametrize("score", ["fp32", "split_bf16"])
@pytest.mark.parametrize("d,chunk", [(200, 20000), (37, 7777), (100, 9999)])
def test_stream_other_widths(gpu_lib, d, chunk, score):
    """Streamed chunks of rows with d > 128 (points streamed through the
    assignment kernel in 64-dim chunks), with a ragged d, and with d = 100
    (the reduction reads those rows two per 16-byte load and adds each
    batch's sums to the running ones): the batches' sums, counts and offsets
    add up to the in-core iteration and the oracle."""
    fk = gpu_lib
    rng = np.random.default_rng(d)
    N, K = 50001, 300
    X = rng.standard_normal((N, d)).astype(np.float32)
    C = X[rng.choice(N, K, replace=False)].copy()
    log(f"stream d={d} chunk={chunk} score={score}")
    a_ic, C_ic, n_ic, _ = fk.fk_lloyd_iter(dev(X), dev(C), score=score)
    ah = torch.empty(N, dtype=torch.int32, pin_memory=True)
    C_s, n_s = fk.fk_lloyd_iter_stream(_pinned(X), dev(C), chunk, assign_host=ah, score=score)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ah.numpy(), host(a_ic))
    np.testing.assert_array_equal(host(n_s), host(n_ic))
    ref = oracle.lloyd_iter(X, C)
    np.testing.assert_array_equal(ah.numpy(), ref["a"])
    np.testing.assert_array_equal(host(n_s), ref["counts"])
    assert centroid_rel_err(host(C_s), ref["C"], ref["counts"]) <= 1e-6


def test_stream_calls_from_two_threads(gpu_lib):
    """Two host threads stream at once, each on its own stream with its own
    workspace: both results equal the in-core iteration (the library
    enqueues the calls one at a time on the shared copy stream)."""
    import threading
    fk = gpu_lib
    w = synth.WORKLOADS["ooc_1b_d128_k32768"].scaled(120000)
    X = synth.rows(w)
    C = X[synth.init_indices(w)[:500]].copy()
    Xh = _pinned(X)
    Cd = dev(C)
    a_ic, C_ic, n_ic, _ = fk.fk_lloyd_iter(dev(X), Cd)
    torch.cuda.synchronize()
    chunk = 30001
    nbytes = fk.fk_workspace_size(w.N, w.d, 500, "l2", chunk) + 256
    res = [None, None]

    def run(i):
        s = torch.cuda.Stream()
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
        ah = torch.empty(w.N, dtype=torch.int32, pin_memory=True)
        with torch.cuda.stream(s):
            for _ in range(3):
                C_s, n_s = fk.fk_lloyd_iter_stream(Xh, Cd, chunk, assign_host=ah, workspace=ws)
        s.synchronize()
        res[i] = (ah.numpy().copy(), host(C_s), host(n_s))

    ts = [threading.Thread(target=run, args=(i,)) for i in range(2)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    for a, Cs, n in res:
        np.testing.assert_array_equal(a, host(a_ic))
        np.testing.assert_array_equal(n, host(n_ic))
        assert centroid_rel_err(Cs, host(C_ic).astype(np.float64), host(n_ic)) <= 1e-6
