"""Write the oracle's own Lloyd trajectory on the full-size workloads as
compact digests (tests/golden/fullsize_<workload>.json).

Every value written here comes from the fp64 CPU oracle (``oracle``) run on
the seeded inputs (``synth``); nothing comes from the HIP library.  The
oracle starts from the workload's initial centroids C_0 and runs the plain
iteration of the Flash-KMeans article (lumevalley.com article 3696, section
"Why being fast took so long": nearest centroid under the N x K squared
distances, then per-cluster sums divided by the cluster size), carrying the
centroids in fp32 between iterations: C_{t+1} = fp32(oracle means under C_t).

Per iteration t the file holds
  * ``label_blocks``: a BLAKE2b-128 hash of the oracle's int32 labels of each
    65,536-row block (little-endian bytes), so a test can compare every label
    of an N-row assignment with the oracle's and name the block that differs;
  * ``counts_hash`` (the int32 cluster sizes) and, for K <= 4096, the counts;
  * ``J`` (the objective sum_i D1_i under C_t) and, per block, the sum of D1;
  * ``gap``: how many points have a relative top-2 gap g = (D2 - D1) / D1 at
    or below 1e-5, 1e-6, 1e-7 and exactly 0 (an exact tie), the points the
    1e-5 exemption would cover;
  * ``next_centroids_hash``: the hash of C_{t+1} as fp32 bytes, which a test
    that rebuilds C_{t+1} from the oracle's update can check it against;
  * ``empty``: clusters with no point.

Usage (each workload is independent; iterations resume from the state saved
under --state):
    python tests/golden/make_fullsize_digests.py WORKLOAD [--iters T] [--state DIR]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

BLOCK = 65536
GAP_LEVELS = (1e-5, 1e-6, 1e-7)


def digest(a: np.ndarray) -> str:
    return hashlib.blake2b(np.ascontiguousarray(a).tobytes(), digest_size=16).hexdigest()


def label_block_hashes(a: np.ndarray) -> list:
    a = np.ascontiguousarray(a, dtype="<i4")
    return [digest(a[b:b + BLOCK]) for b in range(0, len(a), BLOCK)]


def dumps(doc: dict) -> str:
    """JSON with one line per top-level key and one line per iteration."""
    lines = []
    for k, v in doc.items():
        if k == "iterations":
            items = ",\n  ".join(json.dumps(it) for it in v)
            lines.append(f'"{k}": [\n  {items}\n ]')
        else:
            lines.append(f"{json.dumps(k)}: {json.dumps(v)}")
    return "{\n " + ",\n ".join(lines) + "\n}\n"


def out_path(name: str) -> str:
    return os.path.join(HERE, f"fullsize_{name}.json")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("workload")
    ap.add_argument("--iters", type=int, default=None, help="iterations to have in the file (default: the workload's)")
    ap.add_argument("--state", default=os.path.join(ROOT, "_work", "oracle_state"),
                    help="where the fp32 centroids of the last stored iteration are kept, to resume")
    args = ap.parse_args()
    w = synth.WORKLOADS[args.workload]
    T = w.iters if args.iters is None else args.iters
    path = out_path(w.name)
    if os.path.exists(path):
        with open(path) as f:
            doc = json.load(f)
    else:
        doc = {
            "about": ("The fp64 CPU oracle's own Lloyd trajectory on this workload from its initial centroids, "
                      "as digests; written by tests/golden/make_fullsize_digests.py, which calls only the "
                      "oracle and the seeded input generator."),
            "workload": w.name, "N": w.N, "d": w.d, "K": w.K, "metric": w.metric, "block_rows": BLOCK,
            "initial_centroids_hash": None, "iterations": [],
        }
    os.makedirs(args.state, exist_ok=True)
    state = os.path.join(args.state, f"{w.name}_C.npy")
    t0 = time.time()
    X = synth.rows(w)
    C0 = synth.initial_centroids(w, X)
    doc["initial_centroids_hash"] = digest(C0)
    done = len(doc["iterations"])
    if done == 0:
        C = C0
    else:
        C = np.load(state)
        if digest(C) != doc["iterations"][-1]["next_centroids_hash"]:
            raise SystemExit("saved centroids do not match the stored trajectory; delete the file to restart")
    print(f"{w.name}: X generated in {time.time() - t0:.1f} s, {done} iterations stored, "
          f"{oracle.num_threads()} oracle threads", flush=True)
    for t in range(done, T):
        t1 = time.time()
        r = oracle.lloyd_iter(X, C, w.metric)
        dt = time.time() - t1
        a = r["a"]
        counts = r["counts"].astype(np.int32)
        g = oracle.relative_gap(r["D1"], r["D2"])
        C_next = r["C"].astype(np.float32)
        blocks_J = [float(r["D1"][b:b + BLOCK].sum()) for b in range(0, w.N, BLOCK)]
        it = {
            "t": t,
            "centroids_hash": digest(C),
            "label_blocks": label_block_hashes(a),
            "counts_hash": digest(counts.astype("<i4")),
            "counts": counts.tolist() if w.K <= 4096 else None,
            "J": r["J"],
            "J_blocks": blocks_J,
            "gap": {f"le_{lv:g}": int((g <= lv).sum()) for lv in GAP_LEVELS} | {"eq_0": int((g == 0).sum())},
            "empty": int((counts == 0).sum()),
            "next_centroids_hash": digest(C_next),
            "oracle_seconds": round(dt, 1),
            "oracle_threads": oracle.num_threads(),
        }
        doc["iterations"].append(it)
        doc["host"] = {"cpu": platform.processor() or platform.machine(), "numpy": np.__version__}
        tmp = path + ".tmp"
        with open(tmp, "w") as f:
            f.write(dumps(doc))
        os.replace(tmp, path)
        np.save(state, C_next)
        print(f"{w.name}: iteration {t} in {dt:.1f} s, J = {r['J']:.9g}, gap<=1e-5: {it['gap']['le_1e-05']}, "
              f"empty {it['empty']}", flush=True)
        C = C_next


if __name__ == "__main__":
    main()
