"""The sparse linear layer (SparseAdapter / sparse_linear) on the GPU against
the oracle: forward S . X^T, the autograd gradients with respect to the
stored values and to X^T, and the merge W += S."""
import numpy as np
import pytest
import torch

import oracle
import unstructured_sparse_linear_amd as S
from unstructured_sparse_linear_amd import gen
from helpers import TORCH_DT, csr_dev, dev, host, host_f64, rel_err

pytestmark = pytest.mark.gpu

# one rounding of an fp32 result to the output format, on top of the bar
ROUND = {"f32": 0.0, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}
BAR = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}

CASES = [
    # seed, out_features, in_features, tokens, density, dt, kw
    (1, 37, 53, 16, 0.2, "f32", {}),
    (2, 300, 200, 64, 0.05, "f16", {"empty_row_frac": 0.2}),
    (3, 200, 300, 256, 0.03, "bf16", {"shuffle_within_rows": True}),
    (4, 64, 40000, 8, 0.0005, "f16", {"col_index_dtype": np.int32}),
    (5, 513, 257, 128, 0.02, "bf16", {}),
]


def _setup(seed, m, n, T, density, dt, kw):
    A = gen.random_csr(seed, m, n, density, dt, **kw)
    xt = gen.dense(seed, 100, gen.S_B, (n, T), dt)
    g = gen.dense(seed, 100, gen.S_A, (m, T), dt)
    _, ro, ci = csr_dev(A)
    pattern = S.SparsePattern(ro, ci, m, n)
    return A, xt, g, pattern


@pytest.mark.parametrize("seed,m,n,T,density,dt,kw", CASES)
def test_forward_and_gradients(seed, m, n, T, density, dt, kw):
    A, xt, g, pattern = _setup(seed, m, n, T, density, dt, kw)
    layer = S.SparseAdapter(pattern, dev(A.values, dt).clone())
    X = dev(xt, dt).clone().requires_grad_(True)
    Y = layer(X)
    Y.backward(dev(g, dt))
    yt_ref = oracle.sparse_linear_forward(m, A.row_offsets, A.col_idx, A.values, dt, xt, dt)
    dv_ref, dxt_ref = oracle.sparse_linear_backward(m, n, A.row_offsets, A.col_idx, A.values,
                                                    dt, xt, g, dt)
    bound = BAR[dt] + ROUND[dt]
    assert Y.dtype == TORCH_DT[dt] and tuple(Y.shape) == (m, T)
    assert rel_err(host_f64(Y.detach()), yt_ref) <= bound, "forward"
    assert layer.values.grad is not None and layer.values.grad.dtype == TORCH_DT[dt]
    assert rel_err(host_f64(layer.values.grad), dv_ref) <= bound, "dvalues"
    assert rel_err(host_f64(X.grad), dxt_ref) <= bound, "dX^T"


def test_integer_values_bitexact():
    m, n, T = 300, 260, 64
    A = gen.random_csr(7, m, n, 0.05, "f32")
    rng = np.random.default_rng(7)
    v = rng.integers(-3, 4, A.nnz).astype(np.float32)
    xt = rng.integers(-3, 4, (n, T)).astype(np.float32)
    g = rng.integers(-3, 4, (m, T)).astype(np.float32)
    _, ro, ci = csr_dev(A)
    pattern = S.SparsePattern(ro, ci, m, n)
    vals = torch.from_numpy(v).cuda().requires_grad_(True)
    X = torch.from_numpy(xt).cuda().requires_grad_(True)
    Y = S.sparse_linear(vals, X, pattern)
    Y.backward(torch.from_numpy(g).cuda())
    yt_ref = oracle.sparse_linear_forward(m, A.row_offsets, A.col_idx, v, "f32", xt, "f32")
    dv_ref, dxt_ref = oracle.sparse_linear_backward(m, n, A.row_offsets, A.col_idx, v, "f32",
                                                    xt, g, "f32")
    assert np.array_equal(host_f64(Y.detach()), yt_ref)
    assert np.array_equal(host_f64(vals.grad), dv_ref)
    assert np.array_equal(host_f64(X.grad), dxt_ref)


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_merge_into_dense_weight(dt):
    A, xt, g, pattern = _setup(8, 120, 90, 4, 0.1, dt, {})
    layer = S.SparseAdapter(pattern, dev(A.values, dt).clone())
    W = gen.dense(8, 100, gen.S_W, (120, 90), dt)
    Wd = dev(W, dt).clone()
    layer.merge_into(Wd)
    ref = oracle.csr_add(A.row_offsets, A.col_idx, A.values, dt, W, dt)
    assert np.array_equal(host(Wd), ref)


def test_only_values_need_grad():
    A, xt, g, pattern = _setup(9, 50, 60, 8, 0.1, "f16", {})
    layer = S.SparseAdapter(pattern, dev(A.values, "f16").clone())
    Y = layer(dev(xt, "f16"))
    Y.backward(dev(g, "f16"))
    dv_ref = oracle.sparse_linear_backward(50, 60, A.row_offsets, A.col_idx, A.values, "f16",
                                           xt, g, "f16")[0]
    assert rel_err(host_f64(layer.values.grad), dv_ref) <= BAR["f16"] + ROUND["f16"]


def test_rejects_mismatched_inputs():
    A, xt, g, pattern = _setup(10, 20, 30, 4, 0.2, "f16", {})
    with pytest.raises(ValueError):
        S.sparse_linear(dev(A.values, "f16"), dev(xt, "f16").float(), pattern)
    with pytest.raises(ValueError):
        S.sparse_linear(dev(A.values, "f16"), dev(xt, "f16")[:5], pattern)


@pytest.mark.parametrize("cfg,dt", [(3, "f16"), (2, "f16")])
def test_full_size_layer_on_sampled_outputs(cfg, dt):
    # the layer at the size the benchmark times it (the workload's mask as S,
    # its dense B as X^T, its A operand as dY^T, 2048 tokens): forward and
    # both gradients on the GPU, checked on sampled rows of Y^T, the stored
    # entries of those rows (dvalues) and sampled rows of dX^T, each computed
    # by the oracle on the matching slab of S (or of S^T)
    w = gen.make_config(cfg, dt=dt)
    A = w.get("A")
    xt, g = w.get("B"), w.get("Ad")
    m, n = A.m, A.n
    _, ro, ci = csr_dev(A)
    pattern = S.SparsePattern(ro, ci, m, n)
    layer = S.SparseAdapter(pattern, dev(A.values, dt).clone())
    X = dev(xt, dt).clone().requires_grad_(True)
    Y = layer(X)
    Y.backward(dev(g, dt))
    torch.cuda.synchronize()
    bound = BAR[dt] + ROUND[dt]
    rng = np.random.default_rng(cfg)
    rows = np.sort(rng.choice(m, 48, replace=False))
    Yh, dvh = host_f64(Y.detach()), host_f64(layer.values.grad)
    for r in rows:
        slab = gen.csr_row_slab(A, int(r), int(r) + 1)
        yt = oracle.sparse_linear_forward(1, slab.row_offsets, slab.col_idx, slab.values, dt,
                                          xt, dt)
        dv, _ = oracle.sparse_linear_backward(1, n, slab.row_offsets, slab.col_idx,
                                              slab.values, dt, xt, g[r:r + 1], dt)
        assert rel_err(Yh[r], yt[0]) <= bound, ("forward row", r)
        p0, p1 = int(A.row_offsets[r]), int(A.row_offsets[r + 1])
        if p1 > p0:
            assert rel_err(dvh[p0:p1], dv) <= bound, ("dvalues row", r)
    # dX^T = S^T dY^T: rows of S^T are columns of S
    vT, roT, ciT = oracle.csr_transpose(m, n, A.row_offsets, A.col_idx, A.values)
    AT = gen.CSR(n, m, roT, ciT, vT, dt)
    dxh = host_f64(X.grad)
    for c in np.sort(rng.choice(n, 48, replace=False)):
        slab = gen.csr_row_slab(AT, int(c), int(c) + 1)
        dx = oracle.sparse_linear_forward(1, slab.row_offsets, slab.col_idx, slab.values, dt,
                                          g, dt)
        assert rel_err(dxh[c], dx[0]) <= bound, ("dX^T row", c)
