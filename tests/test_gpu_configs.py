"""GPU parity at the full sizes of the five workloads, in the same launch
configuration the benchmark times (the library picks launches from the data;
plans are built the same way).  The oracle runs on the host cores over the
whole output except where stated (sampled rows for the largest SpMM).
"""
import numpy as np
import pytest
import torch

import oracle
import unstructured_sparse_linear_amd as S
from unstructured_sparse_linear_amd import gen
from helpers import assert_close, csr_dev, dev, host, host_f64

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    S.lib()
    yield
    S.clear_plan_caches()
    torch.cuda.synchronize()


_W = {}


def workload(cfg, dt=None):
    key = (cfg, dt)
    if key not in _W:
        _W.clear()
        _W[key] = gen.make_config(cfg, dt=dt)
    return _W[key]


def on_device(A):
    v, ro, ci = csr_dev(A)
    ri = S.sort_rows_by_nnz(ro, A.n)
    assert np.array_equal(host(ri), oracle.row_idx(A.row_offsets, np.int16 if A.m <= 32767
                                                     else np.int32))
    return v, ro, ri, ci


def check_spmm(A, B, dt, sample_rows=None):
    v, ro, ri, ci = on_device(A)
    C = S.spmm(v, ro, ri, ci, dev(B, dt), A.m)
    Ch = host_f64(C)
    if sample_rows is None:
        ref = oracle.spmm(A.m, A.row_offsets, A.col_idx, A.values, dt, B, dt)
        return assert_close(Ch, ref, dt, "spmm")
    errs = []
    for r0, r1 in sample_rows:
        sl = gen.csr_row_slab(A, r0, r1)
        ref = oracle.spmm(sl.m, sl.row_offsets, sl.col_idx, sl.values, dt, B, dt)
        errs.append(assert_close(Ch[r0:r1], ref, dt, f"spmm rows {r0}:{r1}"))
    return max(errs)


def check_sddmm(M, Ad, BT, dt, backend):
    _, ro, ci = csr_dev(M)
    ri = S.sort_rows_by_nnz(ro, M.n)
    out = S.sddmm(ro, ri, ci, dev(Ad, dt), dev(BT, dt), backend=backend)
    ref = oracle.sddmm(M.row_offsets, M.col_idx, Ad, BT, dt)
    return assert_close(host_f64(out), ref, dt, f"sddmm {backend}")


def check_transpose(A):
    v, ro, ci = csr_dev(A)
    vT, roT, ciT = S.csr_transpose(v, ro, ci, A.m, A.n)
    ev, ero, eci = oracle.csr_transpose(A.m, A.n, A.row_offsets, A.col_idx, A.values)
    assert np.array_equal(host(roT), ero)
    assert np.array_equal(host(ciT), eci)
    assert np.array_equal(host(vT).view(np.uint8), ev.view(np.uint8))


def check_csr_add(A, W, dt):
    v, ro, ri, ci = on_device(A)
    Wd = dev(W, dt)
    S.csr_add(v, ro, ri, ci, Wd)
    ref = oracle.csr_add(A.row_offsets, A.col_idx, A.values, dt, W, dt)
    assert np.array_equal(host(Wd).view(np.uint8), ref.view(np.uint8))


def test_config1_all_ops():
    w = workload(1)
    A = w.get("A")
    check_spmm(A, w.get("B"), "f32")
    for backend in ("sputnik", "structure_aware"):
        check_sddmm(A, w.get("Ad"), w.get("BT"), "f32", backend)
    check_transpose(A)
    check_csr_add(A, w.get("W"), "f32")


def test_config2_spmm_and_csr_add():
    w = workload(2)
    check_spmm(w.get("A"), w.get("B"), "f16")
    check_csr_add(w.get("A"), w.get("W"), "f16")


def test_config2_sddmm_and_transpose():
    w = workload(2)
    for backend in ("sputnik", "structure_aware"):
        check_sddmm(w.get("mask"), w.get("Ad"), w.get("BT"), "f16", backend)
    check_transpose(w.get("A"))


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_config3_sddmm(dt):
    w = workload(3, dt)
    M = w.get("mask")
    _, ro, ci = csr_dev(M)
    info = S.SddmmPlan(ro, ci, M.m, M.n).info()
    assert info["dense_rows"] == 205 and info["dense_cols"] == 550
    assert info["tiled_nnz"] + info["rest_nnz"] == M.nnz
    for backend in ("structure_aware", "sputnik"):
        check_sddmm(M, w.get("Ad"), w.get("BT"), dt, backend)


def test_config3_derived_ops():
    w = workload(3, "f16")
    A = w.get("A")
    check_spmm(A, w.get("B"), "f16")
    check_transpose(A)
    check_csr_add(A, w.get("W"), "f16")


def test_config4_spmv_spmm():
    w = workload(4)
    A = w.get("A")
    check_spmm(A, w.get("B1"), "f32")
    check_spmm(A, w.get("B"), "f32")


def test_config4_cg():
    # conjugate gradients on the full banded SPD matrix, b = the SpMV vector
    w = workload(4)
    A = w.get("A")
    b = w.get("B1")[:, 0].astype(np.float32)
    v, ro, ci = csr_dev(A)
    ri = S.sort_rows_by_nnz(ro, A.n)
    x, k, rel = S.cg(v, ro, ri, ci, dev(b), rtol=1e-6, max_iter=1000)
    _, kr, _ = oracle.cg(A.m, A.row_offsets, A.col_idx, A.values, "f32", b, rtol=1e-6,
                         max_iter=1000)
    assert abs(k - kr) <= 1 and rel <= 1e-6
    r = b.astype(np.float64) - oracle.csr_matvec(A.m, A.row_offsets, A.col_idx,
                                                 A.values.astype(np.float64), host_f64(x))
    assert np.linalg.norm(r) <= 2e-6 * np.linalg.norm(b.astype(np.float64))


def test_config4_sddmm_transpose_csr_add():
    w = workload(4)
    A = w.get("A")
    for backend in ("sputnik", "structure_aware"):
        check_sddmm(A, w.get("Ad"), w.get("BT"), "f32", backend)
    check_transpose(A)
    slab = gen.csr_row_slab(A, 0, 8192)     # W is one slab of 8192 rows
    check_csr_add(slab, w.get("W"), "f32")


def test_config5_spmm_sddmm():
    w = workload(5)
    A = w.get("A")
    check_spmm(A, w.get("B"), "bf16")
    for backend in ("structure_aware", "sputnik"):
        check_sddmm(A, w.get("Ad"), w.get("BT"), "bf16", backend)


def test_config5_transpose_csr_add():
    w = workload(5)
    A = w.get("A")
    check_transpose(A)
    check_csr_add(A, w.get("W"), "bf16")
    w.drop("W")
