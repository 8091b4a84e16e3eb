"""Randomized GPU parity (hypothesis): small CSR matrices -- empty rows,
columns in any order inside a row, both index widths, every value format --
with integer-valued data, through the library against the float64 oracle,
for which every result is exact: SpMM (N = 1 takes the SpMV kernels), SDDMM
(both backends, dense tiles included), csr_add, csr_transpose, the
transpose's permutation and the row order (spops README sections "Sparse
Matrix Multiplication (SpMM)", "Sampled Dense-Dense Matrix Multiplication
(SDDMM)", "Sparse Addition", "CSR Transpose", "Usage")."""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings, strategies as st

import oracle
import unstructured_sparse_linear_amd as S
from unstructured_sparse_linear_amd import gen
from helpers import TORCH_DT, csr_dev, dev, host, host_f64

pytestmark = pytest.mark.gpu

SETTINGS = settings(max_examples=40, deadline=None,
                    suppress_health_check=[HealthCheck.function_scoped_fixture])
DTYPES = ["f32", "f16", "bf16"]


@st.composite
def small_csr(draw, max_m=40, max_n=48):
    m = draw(st.integers(1, max_m))
    n = draw(st.integers(1, max_n))
    dense_rows = draw(st.integers(0, 3))     # a few full rows: tiles for the SDDMM plan
    rows = []
    for r in range(m):
        if r < dense_rows:
            cols = list(range(n))
            if draw(st.booleans()):
                cols = cols[::-1]
        else:
            cols = draw(st.lists(st.integers(0, n - 1), unique=True, max_size=min(n, 6)))
        rows.append(cols)
    A = gen.csr_from_row_lists(m, n, rows)
    if draw(st.booleans()):
        A = gen.CSR(A.m, A.n, A.row_offsets, A.col_idx.astype(np.int32))
    dt = draw(st.sampled_from(DTYPES))
    vals = np.array(draw(st.lists(st.integers(-8, 8), min_size=A.nnz, max_size=A.nnz)),
                    dtype=np.float32)
    return A.with_values(gen.f32_to_storage(vals, dt), dt)


def ints(draw, shape, dt):
    rng = np.random.default_rng(draw(st.integers(0, 2 ** 31)))
    return gen.f32_to_storage(rng.integers(-8, 9, size=shape).astype(np.float32), dt)


@SETTINGS
@given(data=st.data())
def test_spmm(data):
    A = data.draw(small_csr())
    dt = A.val_dtype
    N = data.draw(st.sampled_from([1, 2, 7, 8, 33]))
    B = ints(data.draw, (A.n, N), dt)
    v, ro, ci = csr_dev(A)
    ri = S.sort_rows_by_nnz(ro, A.n)
    C = S.spmm(v, ro, ri, ci, dev(B, dt), A.m)
    assert np.array_equal(host_f64(C),
                          oracle.spmm(A.m, A.row_offsets, A.col_idx, A.values, dt, B, dt))


@SETTINGS
@given(data=st.data())
def test_sddmm_both_backends(data):
    A = data.draw(small_csr())
    dt = A.val_dtype
    K = data.draw(st.sampled_from([1, 5, 8, 16, 40, 64]))
    Ad, BT = ints(data.draw, (A.m, K), dt), ints(data.draw, (A.n, K), dt)
    _, ro, ci = csr_dev(A)
    ri = S.sort_rows_by_nnz(ro, A.n)
    ref = oracle.sddmm(A.row_offsets, A.col_idx, Ad, BT, dt)
    for backend, tau in (("general", None), ("structure_aware", None),
                         ("structure_aware", 0.05)):
        out = S.sddmm(ro, ri, ci, dev(Ad, dt), dev(BT, dt), backend=backend, tau=tau)
        assert np.array_equal(host_f64(out), ref), (backend, tau)


@SETTINGS
@given(data=st.data())
def test_csr_add(data):
    A = data.draw(small_csr())
    dt = A.val_dtype
    W = ints(data.draw, (A.m, A.n), dt)
    v, ro, ci = csr_dev(A)
    Wd = dev(W, dt)
    S.csr_add(v, ro, None, ci, Wd)
    ref = oracle.csr_add(A.row_offsets, A.col_idx, A.values, dt, W, dt)
    assert np.array_equal(host(Wd).view(np.uint8), np.asarray(ref).view(np.uint8))


@SETTINGS
@given(data=st.data())
def test_transpose_permutation_and_row_order(data):
    A = data.draw(small_csr())
    v, ro, ci = csr_dev(A)
    vT, roT, ciT = S.csr_transpose(v, ro, ci, A.m, A.n)
    ev, ero, eci = oracle.csr_transpose(A.m, A.n, A.row_offsets, A.col_idx, A.values)
    assert np.array_equal(host(roT), ero) and np.array_equal(host(ciT), eci)
    assert np.array_equal(host(vT).view(np.uint8), ev.view(np.uint8))
    src, roP, ciP = S.csr_transpose_permutation(ro, ci, A.m, A.n)
    esrc, _, _ = oracle.csr_transpose(A.m, A.n, A.row_offsets, A.col_idx,
                                      np.arange(A.nnz, dtype=np.int32))
    assert np.array_equal(host(src), esrc)
    assert np.array_equal(host(roP), ero) and np.array_equal(host(ciP), eci)
    if A.nnz:
        assert torch.equal(S.permute_values(v, src).view(torch.uint8), vT.view(torch.uint8))
    ri = S.sort_rows_by_nnz(ro, A.n)
    assert np.array_equal(host(ri).astype(np.int64),
                          oracle.row_idx(A.row_offsets).astype(np.int64))


@settings(max_examples=15, deadline=None,
          suppress_health_check=[HealthCheck.function_scoped_fixture])
@given(data=st.data())
def test_spmv_entry_ranges(data):
    # balanced rows of 0..L entries over thousands of rows: the planned SpMV
    # cuts the entries into ranges whose boundaries fall inside rows at
    # random; every row is written once, by the range it starts in
    m = data.draw(st.integers(1, 6000))
    n = data.draw(st.integers(1, 3000))
    L = data.draw(st.integers(1, 40))
    rng = np.random.default_rng(data.draw(st.integers(0, 2 ** 31)))
    lengths = rng.integers(0, min(L, n) + 1, m)
    rows = [np.sort(rng.choice(n, int(c), replace=False)) for c in lengths]
    A = gen.csr_from_row_lists(m, n, rows)
    if A.nnz == 0:
        return
    dt = data.draw(st.sampled_from(DTYPES))
    A = A.with_values(gen.f32_to_storage(rng.integers(-8, 9, A.nnz).astype(np.float32), dt), dt)
    x = ints(data.draw, (n, 1), dt)
    v, ro, ci = csr_dev(A)
    ri = S.sort_rows_by_nnz(ro, n)
    p = S.SpmmPlan(ro, ri, ci, n)
    y = S.spmm(v, ro, ri, ci, dev(x, dt), m, plan=p)
    assert np.array_equal(host_f64(y),
                          oracle.spmm(m, A.row_offsets, A.col_idx, A.values, dt, x, dt))
