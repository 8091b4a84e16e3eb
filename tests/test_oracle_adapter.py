"""Pins of the oracle's sparse linear layer (forward S . X^T and its
gradients) against facts that do not come from the oracle itself: the
hand-derived gradients of the torchsparsegradutils README's Quick Start
example, finite differences (the loss is linear in each argument, so
integer-valued data make them exact), and float64 dense autograd in torch."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from unstructured_sparse_linear_amd import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_examples.json")


def _example():
    with open(GOLDEN) as f:
        return [e for e in json.load(f)["examples"] if e["name"] == "coo_2x3"][0]


def test_quick_start_example_gradients():
    ex = _example()
    sl = ex["sparse_linear"]
    ro = np.array(ex["row_offsets"], np.int32)
    ci = np.array(ex["col_idx"], np.int16)
    v = np.array(ex["values"], np.float32)
    xt = np.array(sl["xt"], np.float32)
    dyt = np.array(sl["dyt"], np.float32)
    yt = oracle.sparse_linear_forward(ex["m"], ro, ci, v, "f32", xt, "f32")
    assert np.array_equal(yt, np.array(sl["yt"], np.float64))
    dv, dxt = oracle.sparse_linear_backward(ex["m"], ex["n"], ro, ci, v, "f32", xt, dyt, "f32")
    assert np.array_equal(dv, np.array(sl["dvalues"], np.float64))
    assert np.array_equal(dxt, np.array(sl["dxt"], np.float64))


def _int_case(seed, m, n, T, density):
    A = gen.random_csr(seed, m, n, density, "f32", empty_row_frac=0.2)
    rng = np.random.default_rng(seed)
    v = rng.integers(-3, 4, A.nnz).astype(np.float32)
    xt = rng.integers(-3, 4, (n, T)).astype(np.float32)
    g = rng.integers(-3, 4, (m, T)).astype(np.float32)
    return A, v, xt, g


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_finite_differences_are_exact(seed):
    m, n, T = 9, 7, 4
    A, v, xt, g = _int_case(seed, m, n, T, 0.4)

    def loss(vv, xx):
        return float((g.astype(np.float64) *
                      oracle.sparse_linear_forward(m, A.row_offsets, A.col_idx, vv, "f32",
                                                   xx, "f32")).sum())

    dv, dxt = oracle.sparse_linear_backward(m, n, A.row_offsets, A.col_idx, v, "f32", xt, g,
                                            "f32")
    base = loss(v, xt)
    for p in range(A.nnz):
        e = v.copy()
        e[p] += 1.0
        assert loss(e, xt) - base == dv[p]
    for c in range(n):
        for j in range(T):
            x2 = xt.copy()
            x2[c, j] += 1.0
            assert loss(v, x2) - base == dxt[c, j]


@pytest.mark.parametrize("seed,m,n,T,density", [(4, 30, 20, 5, 0.2), (5, 1, 9, 3, 0.5),
                                                 (6, 40, 3, 8, 0.6)])
def test_matches_dense_autograd(seed, m, n, T, density):
    A = gen.random_csr(seed, m, n, density, "f32", shuffle_within_rows=True)
    rng = np.random.default_rng(seed)
    xt = rng.standard_normal((n, T)).astype(np.float32)
    g = rng.standard_normal((m, T)).astype(np.float32)
    rows = np.repeat(np.arange(m), np.diff(A.row_offsets))
    cols = A.col_idx.astype(np.int64)
    S = torch.zeros((m, n), dtype=torch.float64)
    S[rows, cols] = torch.from_numpy(A.values.astype(np.float64))
    S.requires_grad_(True)
    X = torch.from_numpy(xt.astype(np.float64)).requires_grad_(True)
    Y = S @ X
    (torch.from_numpy(g.astype(np.float64)) * Y).sum().backward()
    yt = oracle.sparse_linear_forward(m, A.row_offsets, A.col_idx, A.values, "f32", xt, "f32")
    dv, dxt = oracle.sparse_linear_backward(m, n, A.row_offsets, A.col_idx, A.values, "f32", xt,
                                            g, "f32")
    np.testing.assert_allclose(yt, Y.detach().numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dv, S.grad[rows, cols].numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dxt, X.grad.numpy(), rtol=1e-12, atol=1e-12)
