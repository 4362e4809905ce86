"""Shared helpers of the GPU parity tests: moving seeded inputs to the device,
and the comparisons against the oracle, with the tolerances they use.

Tolerances
  * assignments, counts, permutations, offsets: bit-exact;
  * centroids: relative L2 error per non-empty centroid <= 1e-6.  The bar the
    method is held to is 1e-4; the library sums in fp64 and rounds once to
    fp32, so its error is about 2^-24 relative, and 1e-6 leaves ample room for
    the different fp64 summation order;
  * empty centroids: bitwise equal to the centroid that was passed in;
  * min_dist (fp32 output): bit-exact against the oracle's fp64 D1 rounded
    to fp32 (the library takes it by the same definition, in the same order);
  * sums of min_dist over many points against the oracle's fp64 sums of D1:
    2^-23 of the sum (each term rounded once to fp32, 2^-24 relative).
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


def objective_tol(d1_gpu):
    """Bound on |sum(min_dist_gpu) - sum(D1_oracle)| (see the module notes)."""
    return 2.0 ** -23 * float(np.abs(np.asarray(d1_gpu, np.float64)).sum()) + 1e-300


def check_min_dist(d1_gpu, D1):
    """min_dist equals the oracle's D1 rounded to fp32, bit for bit."""
    want = np.asarray(D1, np.float64).astype(np.float32)
    got = np.asarray(d1_gpu, np.float32)
    bad = got.view(np.uint32) != want.view(np.uint32)
    assert not bad.any(), f"min_dist differs at {np.nonzero(bad)[0][:5]}: {got[bad][:5]} vs {want[bad][:5]}"


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
