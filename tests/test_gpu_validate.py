"""The CSR validator (spops_validate_csr) on valid matrices and on in-range
corruptions of each kind it checks: a repeated column inside a row, a
row_idx that is not a permutation, decreasing row offsets, a last offset
that is not nnz, a column outside [0, cols).  Every corruption keeps the
arrays' lengths, so the validator's reads stay in bounds by construction."""
import numpy as np
import pytest
import torch

import unstructured_sparse_linear_amd as S
from unstructured_sparse_linear_amd import gen
from unstructured_sparse_linear_amd import spops as SP
from helpers import dev

pytestmark = pytest.mark.gpu

CASES = [
    (41, 300, 200, 0.05, {}),
    (42, 1000, 40000, 0.001, {"empty_row_frac": 0.3}),
    (43, 40000, 50, 0.05, {"shuffle_within_rows": True}),
    (44, 5, 7, 0.0, {}),
]


def parts(A):
    ro, ci = dev(A.row_offsets), dev(A.col_idx)
    ri = S.sort_rows_by_nnz(ro, A.n)
    return ro, ci, ri


def findings(ro, ci, m, n, ri=None):
    try:
        S.validate_csr(ro, ci, m, n, ri)
        return 0
    except S.InvalidCSR as e:
        return e.findings


@pytest.mark.parametrize("seed,m,n,density,kw", CASES)
def test_valid_matrices_pass(seed, m, n, density, kw):
    A = gen.random_csr(seed, m, n, density, None, **kw)
    ro, ci, ri = parts(A)
    assert findings(ro, ci, m, n, ri) == 0
    assert findings(ro, ci, m, n, dev(gen.permutation(seed, m, "random"))) == 0


@pytest.mark.parametrize("seed,m,n,density,kw", CASES[:3])
def test_corruptions_are_found(seed, m, n, density, kw):
    A = gen.random_csr(seed, m, n, density, None, **kw)
    counts = np.diff(A.row_offsets)
    r = int(np.argmax(counts >= 2))
    p = int(A.row_offsets[r])
    # a column repeated inside row r
    ro, ci, ri = parts(A)
    ci[p + 1] = ci[p]
    assert findings(ro, ci, m, n, ri) == 8
    # row_idx with one row twice (another one missing)
    ro, ci, ri = parts(A)
    ri[1] = ri[0]
    assert findings(ro, ci, m, n, ri) == 4
    # decreasing offsets (all still inside [0, nnz])
    ro, ci, ri = parts(A)
    ro[r + 1] = int(A.row_offsets[r]) - 1 if A.row_offsets[r] > 0 else 0
    if int(ro[r + 1]) < int(A.row_offsets[r]):
        assert findings(ro, ci, m, n, ri) & 1
    ro, ci, ri = parts(A)
    ro[m] = A.nnz - 1
    assert findings(ro, ci, m, n, ri) & 1
    # a column outside [0, n)
    ro, ci, ri = parts(A)
    ci[p] = n if n <= 32767 or ci.dtype == torch.int32 else -1
    assert findings(ro, ci, m, n, ri) == 2
    ci[p] = -1
    assert findings(ro, ci, m, n, ri) == 2


def test_binding_switch_validates_operands():
    A = gen.random_csr(45, 200, 300, 0.05, "f32")
    ro, ci, ri = parts(A)
    v = dev(A.values)
    B = torch.ones((300, 8), device="cuda")
    r = int(np.argmax(np.diff(A.row_offsets) >= 2))
    ci[int(A.row_offsets[r]) + 1] = ci[int(A.row_offsets[r])]
    old = SP.VALIDATE
    SP.VALIDATE = True
    try:
        with pytest.raises(S.InvalidCSR):
            S.spmm(v, ro, ri, ci, B, 200)
        with pytest.raises(S.InvalidCSR):
            S.csr_transpose(v, ro, ci, 200, 300)
    finally:
        SP.VALIDATE = old
