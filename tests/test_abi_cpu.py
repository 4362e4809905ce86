"""The C-ABI library on the CPU: it loads, exports every symbol include/fk.h
declares, names its status codes, sizes workspaces, and rejects bad arguments
before touching any device (so no GPU is needed here)."""
import ctypes
import os

import pytest

import exact_lloyd_means_flashassign_amd as fk

OK, INVALID, UNSUPPORTED, WORKSPACE, NO_DEVICE, HIPERR = range(6)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fk.LIB_PATH):
        from exact_lloyd_means_flashassign_amd import build
        build.build()
    return fk.load()


def test_every_declared_symbol_is_exported(lib):
    names = fk.declared_symbols()
    expected = {"fk_workspace_size", "fk_assign", "fk_sort_inverse", "fk_update", "fk_lloyd_iter",
                "fk_lloyd_iter_stream", "fk_status_str", "fk_last_error", "fk_profile_enable", "fk_profile_read",
                "fk_fit_workspace_size", "fk_fit", "fk_ivf_workspace_size", "fk_ivf_build",
                "fk_knn_workspace_size", "fk_knn"}
    assert expected <= set(names)
    raw = ctypes.CDLL(fk.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n


def test_status_names(lib):
    names = [fk.fk_status_str(i) for i in range(6)]
    assert names == ["FK_OK", "FK_ERR_INVALID_ARG", "FK_ERR_UNSUPPORTED", "FK_ERR_WORKSPACE",
                     "FK_ERR_NO_DEVICE", "FK_ERR_HIP"]
    assert fk.fk_status_str(99) == "FK_ERR_UNKNOWN"


def test_workspace_sizes(lib):
    a = fk.fk_workspace_size(1000, 128, 1024)
    b = fk.fk_workspace_size(100000, 128, 1024)
    assert 0 < a < b
    assert fk.fk_workspace_size(0, 16, 64) > 0
    assert fk.fk_workspace_size(1000, 128, 1024, "cosine") > a
    s = fk.fk_workspace_size(10 ** 9, 128, 32768, "l2", chunk_rows=1 << 20)
    assert s > 2 * (1 << 20) * 128 * 4          # two chunk buffers
    # the zipf 16M x 128, K=32768 shape fits comfortably in 288 GB
    assert fk.fk_workspace_size(1 << 24, 128, 32768) < 2 * 10 ** 9
    for bad in [(-1, 16, 4), (10, 0, 4), (10, 16, 0), (10, 16, 65537), (10, 4097, 4), (2 ** 31, 4, 4)]:
        assert lib.fk_workspace_size(*bad, 0, 0) == 0
    assert lib.fk_workspace_size(10, 4, 4, 2, 0) > 0             # inner product
    assert lib.fk_workspace_size(10, 4, 4, 3, 0) > 0             # spherical
    assert lib.fk_workspace_size(10, 4, 4, 4, 0) == 0            # no such metric


P = ctypes.c_void_p


def _fake(addr):
    return P(addr)


def _call_assign(lib, N=100, d=8, K=4, metric=0, X=0x10000, C=0x20000, a=0x30000, ws=0x100000, wsn=1 << 30, score=0):
    return lib.fk_assign(_fake(X) if X else None, N, d, _fake(C) if C else None, K, metric, score,
                         _fake(a) if a else None, None, _fake(ws) if ws else None, wsn, None)


def test_validation_happens_before_any_device_call(lib):
    assert _call_assign(lib, N=-1) == INVALID
    assert _call_assign(lib, d=0) == INVALID
    assert _call_assign(lib, d=5000) == INVALID
    assert _call_assign(lib, K=0) == INVALID
    assert _call_assign(lib, K=70000) == INVALID
    assert _call_assign(lib, metric=7) == INVALID
    assert b"metric" in lib.fk_last_error()
    assert _call_assign(lib, score=2) == INVALID
    assert b"score" in lib.fk_last_error()
    assert _call_assign(lib, X=0) == INVALID
    assert _call_assign(lib, C=0) == INVALID
    assert _call_assign(lib, a=0) == INVALID
    assert _call_assign(lib, X=0x10004) == INVALID                # X not 16-byte aligned
    assert _call_assign(lib, ws=0) == WORKSPACE
    assert _call_assign(lib, ws=0x100010) == WORKSPACE            # not 256-byte aligned
    assert _call_assign(lib, wsn=100) == WORKSPACE
    assert b"needed" in lib.fk_last_error()


def test_update_and_iter_reject_aliasing(lib):
    K, d = 16, 8
    C = 0x200000
    st = lib.fk_update(_fake(0x10000), 10, d, _fake(0x30000), K, 0, _fake(C), _fake(C + 64), _fake(0x40000),
                       _fake(0x1000000), 1 << 30, None)
    assert st == INVALID and b"overlaps" in lib.fk_last_error()
    st = lib.fk_lloyd_iter(_fake(0x10000), 10, d, _fake(C), K, 0, 0, _fake(0x30000), None, _fake(C), _fake(0x40000),
                           _fake(0x1000000), 1 << 30, None)
    assert st == INVALID
    st = lib.fk_lloyd_iter(_fake(0x10000), 10, d, _fake(C), K, 0, 0, _fake(0x30000), None, None, _fake(0x40000),
                           _fake(0x1000000), 1 << 30, None)
    assert st == INVALID


def test_stream_rejects_bad_chunks(lib):
    st = lib.fk_lloyd_iter_stream(_fake(0x10000), 100, 8, _fake(0x20000), 4, 0, 0, 0, None, _fake(0x30000),
                                  _fake(0x40000), _fake(0x1000000), 1 << 30, None)
    assert st == INVALID and b"chunk_rows" in lib.fk_last_error()


def test_sort_inverse_validation(lib):
    assert lib.fk_sort_inverse(None, 10, 4, _fake(0x10000), _fake(0x20000), _fake(0x100000), 1 << 30, None) == INVALID
    assert lib.fk_sort_inverse(_fake(0x10000), 10, 4, _fake(0x20000), None, _fake(0x100000), 1 << 30, None) == INVALID
    assert lib.fk_sort_inverse(_fake(0x10000), 10, 0, _fake(0x20000), _fake(0x30000), _fake(0x100000), 1 << 30,
                               None) == INVALID


@pytest.mark.skipif(__import__("torch").cuda.device_count() > 0, reason="a device is visible")
def test_no_device_is_reported(lib):
    assert _call_assign(lib) == NO_DEVICE
    assert b"no HIP device" in lib.fk_last_error()


def test_binding_rejects_host_tensors(lib):
    import torch
    X = torch.zeros(10, 4)
    with pytest.raises(ValueError):
        fk.fk_assign(X, X[:2].clone())


def test_profile_api_without_device(lib):
    fk.fk_profile_enable(True)
    r = fk.fk_profile_read()
    assert r["rechecked"] == 0 and all(v == 0 for v in r["calls"].values())
    fk.fk_profile_enable(False)


def test_fit_and_ivf_validation(lib):
    ws = _fake(0x1000000)
    info = fk._FitInfo()

    def fit(N=100, K=4, C_init=_fake(0x20000), n_iter=3, tol=-1.0, C_out=_fake(0x30000), metric=0):
        return lib.fk_fit(_fake(0x10000), N, 8, K, metric, 0, C_init, 0, n_iter, tol, C_out, _fake(0x40000),
                          _fake(0x50000), ctypes.byref(info), ws, 1 << 30, None)
    # n_iter < 1, aliasing of C_out and C_init, a draw from no rows, NaN tol, unknown metric
    assert fit(n_iter=0) == INVALID and b"n_iter" in lib.fk_last_error()
    assert fit(C_out=_fake(0x20000 + 16)) == INVALID and b"overlaps" in lib.fk_last_error()
    assert fit(N=0, C_init=None) == INVALID and b"N=0" in lib.fk_last_error()
    assert fit(tol=float("nan")) == INVALID and b"NaN" in lib.fk_last_error()
    assert fit(metric=4) == INVALID
    assert fk.fk_fit_workspace_size(1000, 16, 10) > fk.fk_workspace_size(1000, 16, 10)
    assert fk.fk_fit_workspace_size(1000, 16, 10, "spherical") > 0
    # fk_ivf_build: an initial index out of range, n_iter < 1, no rows, unsupported metrics
    idx = (ctypes.c_int32 * 4)(0, 1, 2, 99)
    args = dict(X=_fake(0x10000), cent=_fake(0x20000), offs=_fake(0x30000), ids=_fake(0x40000), data=_fake(0x800000))

    def ivf(N, nlist, n_iter, init, metric=0):
        return lib.fk_ivf_build(args["X"], N, 8, nlist, metric, 0, n_iter, init, 0, args["cent"], args["offs"],
                                args["ids"], args["data"], None, ws, 1 << 30, None)
    assert ivf(50, 4, 2, idx) == INVALID and b"init_idx[3]" in lib.fk_last_error()
    assert ivf(500, 4, 0, idx) == INVALID and b"n_iter" in lib.fk_last_error()
    assert ivf(0, 4, 2, None) == INVALID and b"N >= 1" in lib.fk_last_error()
    assert ivf(500, 4, 2, idx, metric=2) == UNSUPPORTED and b"inner product" in lib.fk_last_error()
    assert ivf(500, 4, 2, idx, metric=3) == UNSUPPORTED
    assert lib.fk_ivf_workspace_size(10, 8, 11, 0) == lib.fk_ivf_workspace_size(10, 8, 10, 0) > 0
    assert lib.fk_ivf_workspace_size(0, 8, 11, 0) == 0
    assert fk.fk_ivf_workspace_size(1000, 16, 10, "cosine") > fk.fk_ivf_workspace_size(1000, 16, 10)


def test_knn_validation(lib):
    ws = _fake(0x1000000)
    Q, DB, idx, dist = _fake(0x10000), _fake(0x20000), _fake(0x30000), _fake(0x40000)

    def knn(M=10, d=8, Ndb=100, k=5, metric=0, score=0, q=Q, db=DB, wsb=1 << 30):
        return lib.fk_knn(q, M, d, db, Ndb, k, metric, score, idx, dist, ws, wsb, None)
    assert knn(k=0) == INVALID
    assert knn(k=25) == INVALID and b"k=25" in lib.fk_last_error()
    assert knn(Ndb=0) == INVALID
    assert knn(d=0) == INVALID
    assert knn(M=-1) == INVALID
    assert knn(metric=4) == INVALID
    assert knn(metric=3) == UNSUPPORTED and b"spherical" in lib.fk_last_error()
    assert knn(score=2) == INVALID
    assert knn(q=None) == INVALID
    assert knn(db=_fake(0x20004)) == INVALID and b"aligned" in lib.fk_last_error()
    assert knn(wsb=16) == WORKSPACE
    # the split copy of a 2^22 x 512 database is 8 GiB: beyond a buffer resource
    assert knn(d=512, Ndb=1 << 22, score=1) == UNSUPPORTED and b"4 GiB" in lib.fk_last_error()
    # k above the database size is clamped; k above the limit with a big database is not
    assert lib.fk_knn_workspace_size(10, 8, 4, 5, 0) == lib.fk_knn_workspace_size(10, 8, 4, 4, 0) > 0
    assert lib.fk_knn_workspace_size(10, 8, 4, 60, 0) > 0
    assert lib.fk_knn_workspace_size(10, 8, 100, 25, 0) == 0
    a = fk.fk_knn_workspace_size(10000, 128, 1 << 20, 10)
    assert a > (1 << 20) * 128 * 4                # the database's bf16 copy
    assert fk.fk_knn_workspace_size(10000, 128, 1 << 20, 10, "cosine") > a + (1 << 20) * 128 * 12
    assert fk.fk_knn_workspace_size(10000, 128, 1 << 20, 20) > a  # 32 candidates per query


def test_microbenchmark_library_exports():
    """The on-box microbenchmarks the benchmark loads are built beside libfk."""
    path = os.path.join(os.path.dirname(fk.LIB_PATH), "libfk_micro.so")
    assert os.path.exists(path), "run __graft_entry__.build() first"
    m = ctypes.CDLL(path)
    for name in ("fkm_stream_copy", "fkm_stream_read", "fkm_gather_rows", "fkm_mfma"):
        assert hasattr(m, name), name
