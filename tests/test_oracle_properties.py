"""Randomized pins for the float64 CPU oracle (no GPU): small CSR matrices
drawn by hypothesis -- empty rows, empty matrices, columns in any order
inside a row, 16- and 32-bit indices, every value format -- with
integer-valued data, so every result is exact and is compared for equality
with a dense numpy computation of the same definition (spops README,
sections "Sparse Matrix Multiplication (SpMM)", "Sampled Dense-Dense Matrix
Multiplication (SDDMM)", "Sparse Addition", "CSR Transpose", and the row
order of section "Usage")."""
import numpy as np
from hypothesis import given, settings, strategies as st

from unstructured_sparse_linear_amd import gen

SETTINGS = settings(max_examples=60, deadline=None)
DTYPES = ["f32", "f16", "bf16"]


@st.composite
def small_csr(draw):
    m = draw(st.integers(0, 9))
    n = draw(st.integers(1, 11))
    rows = []
    for _ in range(m):
        cols = draw(st.lists(st.integers(0, n - 1), unique=True, max_size=n))
        rows.append(cols)                       # any order inside the row
    A = gen.csr_from_row_lists(m, n, rows)
    if draw(st.booleans()):
        A = gen.CSR(A.m, A.n, A.row_offsets, A.col_idx.astype(np.int32))
    dt = draw(st.sampled_from(DTYPES))
    vals = np.array(draw(st.lists(st.integers(-8, 8), min_size=A.nnz, max_size=A.nnz)),
                    dtype=np.float32)
    return A.with_values(gen.f32_to_storage(vals, dt), dt)


def ints(draw, shape, dt, lo=-8, hi=8):
    size = int(np.prod(shape))
    x = np.array(draw(st.lists(st.integers(lo, hi), min_size=size, max_size=size)),
                 dtype=np.float32).reshape(shape)
    return gen.f32_to_storage(x, dt)


@SETTINGS
@given(data=st.data())
def test_spmm_equals_dense_product(orc, data):
    A = data.draw(small_csr())
    N = data.draw(st.integers(1, 5))
    B = ints(data.draw, (A.n, N), A.val_dtype)
    C = orc.spmm(A.m, A.row_offsets, A.col_idx, A.values, A.val_dtype, B, A.val_dtype)
    ref = A.to_dense_f64() @ gen.storage_to_f64(B, A.val_dtype)
    assert np.array_equal(C, ref)


@SETTINGS
@given(data=st.data())
def test_sddmm_equals_masked_dense_product(orc, data):
    A = data.draw(small_csr())
    K = data.draw(st.integers(1, 6))
    Ad = ints(data.draw, (A.m, K), A.val_dtype)
    BT = ints(data.draw, (A.n, K), A.val_dtype)
    out = orc.sddmm(A.row_offsets, A.col_idx, Ad, BT, A.val_dtype)
    D = gen.storage_to_f64(Ad, A.val_dtype) @ gen.storage_to_f64(BT, A.val_dtype).T
    rows = np.repeat(np.arange(A.m), A.row_counts())
    assert np.array_equal(out, D[rows, A.col_idx.astype(np.int64)])


@SETTINGS
@given(data=st.data())
def test_csr_add_equals_dense_sum(orc, data):
    A = data.draw(small_csr())
    dt = A.val_dtype
    W = ints(data.draw, (A.m, A.n), dt)
    out = orc.csr_add(A.row_offsets, A.col_idx, A.values, dt, W, dt)
    ref = gen.storage_to_f64(W, dt) + A.to_dense_f64()   # small integers: exact in every format
    assert np.array_equal(gen.storage_to_f64(out, dt), ref)


@SETTINGS
@given(data=st.data())
def test_transpose_is_the_stable_column_sort(orc, data):
    A = data.draw(small_csr())
    vT, roT, ciT = orc.csr_transpose(A.m, A.n, A.row_offsets, A.col_idx, A.values)
    assert np.array_equal(np.diff(roT), np.bincount(A.col_idx.astype(np.int64),
                                                    minlength=A.n))
    rows = np.repeat(np.arange(A.m), A.row_counts())
    cols = A.col_idx.astype(np.int64)
    order = np.lexsort((np.arange(A.nnz), cols))   # by column, then source position
    assert np.array_equal(ciT.astype(np.int64), rows[order])
    assert np.array_equal(vT.view(np.uint8), A.values[order].view(np.uint8))
    # the same matrix, transposed
    DT = np.zeros((A.n, A.m))
    DT[np.repeat(np.arange(A.n), np.diff(roT)), ciT.astype(np.int64)] = \
        gen.storage_to_f64(vT, A.val_dtype)
    assert np.array_equal(DT, A.to_dense_f64().T)


@SETTINGS
@given(data=st.data())
def test_row_order_is_the_stable_descending_count_sort(orc, data):
    A = data.draw(small_csr())
    ri = orc.row_idx(A.row_offsets)
    assert np.array_equal(ri.astype(np.int64), np.argsort(-A.row_counts(), kind="stable"))
