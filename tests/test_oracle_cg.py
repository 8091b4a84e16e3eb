"""Pins of the oracle's conjugate-gradient solver against facts that do not
come from the oracle itself: the sparse product against dense algebra,
closed forms (a scaled identity converges in one step to b / c; a matrix with
d distinct eigenvalues in d steps), the method's invariants (conjugate search
directions, orthogonal residuals, a monotonically falling energy-norm error),
agreement with scipy's independent CG, and the stopping rules.  A dropped
beta term (steepest descent), a wrong sign or a transposed step breaks the
finite-termination and conjugacy pins."""
import numpy as np
import pytest
import scipy.sparse
import scipy.sparse.linalg

import oracle
from unstructured_sparse_linear_amd import gen


def _spd(seed, n, band=3, draws=2):
    rng = np.random.default_rng(seed)
    return gen.banded_spd(rng, np.random.default_rng(seed + 1), n, band=band,
                          offband_draws=draws)


def _dense(A):
    D = np.zeros((A.m, A.n))
    r = np.repeat(np.arange(A.m), np.diff(A.row_offsets))
    np.add.at(D, (r, A.col_idx.astype(np.int64)), A.values.astype(np.float64))
    return D


def _diag_csr(d):
    n = len(d)
    return gen.CSR(n, n, np.arange(n + 1, dtype=np.int32), np.arange(n, dtype=np.int16),
                   np.asarray(d, np.float32), "f32")


def _solve(A, b, **kw):
    return oracle.cg(A.m, A.row_offsets, A.col_idx, A.values, "f32", b, **kw)


def test_matvec_matches_dense_product():
    A = gen.random_csr(3, 70, 90, 0.1, "f32", empty_row_frac=0.2)
    x = np.random.default_rng(4).standard_normal(90)
    y = oracle.csr_matvec(A.m, A.row_offsets, A.col_idx, A.values.astype(np.float64), x)
    assert np.allclose(y, _dense(A) @ x, rtol=1e-13, atol=1e-13)


def test_scaled_identity_converges_in_one_step_exactly():
    b = np.random.default_rng(5).standard_normal(40)
    x, k, rel = _solve(_diag_csr(np.full(40, 4.0)), b, rtol=1e-12)
    assert k == 1 and rel == 0.0
    assert np.array_equal(x, b / 4.0)


def test_distinct_eigenvalues_bound_the_iterations():
    # CG on a matrix with d distinct eigenvalues ends (in exact arithmetic)
    # after at most d steps; steepest descent would need many more
    d = np.tile([1.0, 2.0, 3.0, 5.0], 25)
    b = np.random.default_rng(6).standard_normal(100)
    x, k, rel = _solve(_diag_csr(d), b, rtol=1e-12)
    assert k == 4 and rel <= 1e-12
    assert np.allclose(x, b / d, rtol=1e-12)


def test_small_spd_finite_termination():
    A = _spd(7, 30)
    b = np.random.default_rng(8).standard_normal(30)
    x, k, rel = _solve(A, b, rtol=1e-13, max_iter=30)
    assert k <= 30 and rel <= 1e-13
    assert np.allclose(x, np.linalg.solve(_dense(A), b), rtol=1e-10, atol=1e-12)


def test_directions_conjugate_and_residuals_orthogonal():
    A = _spd(9, 200)
    D = _dense(A)
    b = np.random.default_rng(10).standard_normal(200)
    _, k, _, ps, rs = _solve(A, b, rtol=1e-10, history=True)
    n = min(k, 8)
    for i in range(n):
        for j in range(i):
            pAp = ps[i] @ D @ ps[j]
            assert abs(pAp) <= 1e-9 * np.sqrt((ps[i] @ D @ ps[i]) * (ps[j] @ D @ ps[j]))
            assert abs(rs[i] @ rs[j]) <= 1e-9 * np.linalg.norm(rs[i]) * np.linalg.norm(rs[j])


def test_energy_norm_error_falls_monotonically():
    A = _spd(11, 300)
    D = _dense(A)
    b = np.random.default_rng(12).standard_normal(300)
    xs = np.linalg.solve(D, b)
    errs = []
    for it in range(0, 12):
        x, k, _ = _solve(A, b, rtol=0.0, max_iter=it)
        assert k == it
        e = x - xs
        errs.append(float(e @ D @ e))
    assert all(b_ < a_ for a_, b_ in zip(errs, errs[1:]))


@pytest.mark.parametrize("seed,n", [(13, 500), (14, 2000)])
def test_agrees_with_scipy_cg(seed, n):
    A = _spd(seed, n, band=8, draws=4)
    b = np.random.default_rng(seed + 100).standard_normal(n)
    x, k, rel = _solve(A, b, rtol=1e-8, max_iter=500)
    S = scipy.sparse.csr_matrix((A.values.astype(np.float64), A.col_idx.astype(np.int64),
                                 A.row_offsets.astype(np.int64)), shape=(n, n))
    its = []
    xs, info = scipy.sparse.linalg.cg(S, b, rtol=1e-8, atol=0.0, maxiter=500,
                                      callback=lambda _: its.append(1))
    assert info == 0 and rel <= 1e-8
    assert abs(len(its) - k) <= 1
    assert np.linalg.norm(x - xs) <= 1e-7 * np.linalg.norm(xs)
    # the true residual, not just the recursive one
    assert np.linalg.norm(b - S @ x) <= 2e-8 * np.linalg.norm(b)


def test_stopping_rules():
    A = _spd(15, 400)
    b = np.random.default_rng(16).standard_normal(400)
    # max_iter caps the work
    _, k, rel = _solve(A, b, rtol=1e-12, max_iter=3)
    assert k == 3 and rel > 1e-12
    # b = 0 from x0 = 0: nothing to do
    x, k, rel = _solve(A, np.zeros(400), rtol=1e-6)
    assert k == 0 and rel == 0.0 and not x.any()
    # a start that already solves the system exactly (integer diagonal system)
    d = np.arange(1, 51, dtype=np.float64)
    x0 = np.arange(50, dtype=np.float64) - 20
    x, k, rel = _solve(_diag_csr(d), d * x0, x0=x0, rtol=1e-6)
    assert k == 0 and rel == 0.0 and np.array_equal(x, x0)
