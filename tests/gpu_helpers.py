"""Shared helpers of the GPU parity tests: moving seeded inputs to the device,
and the comparisons against the oracle, with the tolerances they use.

Tolerances
  * assignments, counts, permutations, offsets: bit-exact;
  * centroids: relative L2 error per non-empty centroid <= 1e-6.  The bar the
    method is held to is 1e-4; the library sums in fp64 and rounds once to
    fp32, so its error is about 2^-24 relative, and 1e-6 leaves ample room for
    the different fp64 summation order;
  * empty centroids: bitwise equal to the centroid that was passed in;
  * min_dist (fp32 output): |d_gpu - D1| <= 3 (d+4) 2^-24 (||x||^2 + M +
    2 ||x|| sqrt(M)), M = max ||c||^2: the fp32 rounding bound of the expanded
    distance, three times over; with split-bf16 scoring (3d+4) replaces
    (d+4) and the dropped bf16 remainders add 3 * 2.3e-5 ||x|| sqrt(M).
"""
import sys

import numpy as np
import torch

import oracle


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def centroid_rel_err(C_gpu, C_ref, counts):
    C_gpu = np.asarray(C_gpu, np.float64)
    C_ref = np.asarray(C_ref, np.float64)
    ne = counts > 0
    if not ne.any():
        return 0.0
    num = np.linalg.norm(C_gpu[ne] - C_ref[ne], axis=1)
    den = np.linalg.norm(C_ref[ne], axis=1)
    err = np.where(den > 0, num / np.where(den > 0, den, 1), num)
    return float(err.max())


def min_dist_tol(X, C, metric="l2", score="fp32"):
    """Per-point bound on |min_dist_gpu - D1_oracle| (see the module notes)."""
    X = np.asarray(X, np.float64)
    C = np.asarray(C, np.float64)
    d = X.shape[1]
    if metric == "inner_product":
        # min_dist = -max x.c: the score's own bound, three times over
        xn = np.sqrt((X * X).sum(1))
        sqM = np.sqrt((C * C).sum(1).max())
        tol = 3 * (d + 4) * 2.0 ** -24 * xn * sqM + 1e-30
        if score == "split_bf16":
            tol += 3 * 4.7e-5 * xn * sqM
        return tol
    if metric == "cosine":
        nx = np.linalg.norm(X, axis=1, keepdims=True)
        nx[nx == 0] = 1
        X = X / nx
        nc = np.linalg.norm(C, axis=1, keepdims=True)
        nc[nc == 0] = 1
        C = C / nc
    xn = (X * X).sum(1)
    M = (C * C).sum(1).max()
    n = 3 * d + 4 if score == "split_bf16" else d + 4
    tol = 3 * n * 2.0 ** -24 * (xn + M + 2 * np.sqrt(xn * M)) + 1e-30
    if score == "split_bf16":
        tol += 3 * 2.3e-5 * np.sqrt(xn * M)
    return tol


def check_min_dist(d1_gpu, D1, X, C, metric="l2", score="fp32"):
    tol = min_dist_tol(X, C, metric, score)
    err = np.abs(np.asarray(d1_gpu, np.float64) - D1)
    bad = err > tol
    assert not bad.any(), f"min_dist off at {np.nonzero(bad)[0][:5]}: err {err[bad][:5]} tol {tol[bad][:5]}"


def check_update(X, a, C_prev, C_out, counts, metric="l2"):
    """GPU update output against the oracle run on the same assignment."""
    C_ref, n_ref = oracle.update(X, a, C_prev, metric)
    np.testing.assert_array_equal(counts, n_ref)
    np.testing.assert_array_equal(counts, np.bincount(a, minlength=len(C_prev)))
    err = centroid_rel_err(C_out, C_ref, n_ref)
    assert err <= 1e-6, f"centroid rel err {err}"
    empty = n_ref == 0
    assert np.array_equal(np.asarray(C_out)[empty].view(np.uint32), np.asarray(C_prev)[empty].view(np.uint32))
    return err
