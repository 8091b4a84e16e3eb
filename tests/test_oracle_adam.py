"""Pins of the oracle's masked Adam step against facts that do not come from
the oracle: torch's own SparseAdam (the optimizer the SparseAdam page
documents, an independent implementation) on float64 CPU tensors, torch's
dense Adam where the two formulas coincide (every position materialized,
eps = 0), the closed form of the first step (with eps = 0 every materialized
value moves by exactly lr in the direction against its gradient), and the
mask: positions without a gradient keep their value and moments bit for
bit, a materialized zero gradient still decays the moments."""
import numpy as np
import pytest
import torch

import oracle


def _state(seed, n):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(n), np.abs(rng.standard_normal(n)) * 0.1,
            np.abs(rng.standard_normal(n)) * 0.01)


@pytest.mark.parametrize("maximize", [False, True])
def test_matches_torch_sparse_adam(maximize):
    n, steps = 300, 5
    rng = np.random.default_rng(1)
    theta = rng.standard_normal(n)
    p = torch.tensor(theta, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.SparseAdam([p], lr=1e-2, betas=(0.8, 0.95), eps=1e-6, maximize=maximize)
    m, v = np.zeros(n), np.zeros(n)
    for t in range(1, steps + 1):
        pos = np.sort(rng.choice(n, 90, replace=False))
        g = rng.standard_normal(90)
        p.grad = torch.sparse_coo_tensor(torch.tensor(pos)[None], torch.tensor(g), (n,))
        opt.step()
        theta, m, v = oracle.masked_adam(theta, "f64", g, "f64", m, v, t, 1e-2, 0.8, 0.95, 1e-6,
                                         maximize=maximize, positions=pos)
        st = opt.state[p]
        assert np.allclose(p.detach().numpy(), theta, rtol=1e-13, atol=1e-15)
        assert np.allclose(st["exp_avg"].numpy(), m, rtol=1e-13, atol=1e-15)
        assert np.allclose(st["exp_avg_sq"].numpy(), v, rtol=1e-13, atol=1e-15)


def test_matches_dense_adam_without_eps():
    n = 200
    rng = np.random.default_rng(2)
    theta = rng.standard_normal(n)
    p = torch.tensor(theta, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.Adam([p], lr=3e-3, betas=(0.9, 0.999), eps=0.0)
    m, v = np.zeros(n), np.zeros(n)
    for t in range(1, 6):
        g = rng.standard_normal(n)
        p.grad = torch.tensor(g)
        opt.step()
        theta, m, v = oracle.masked_adam(theta, "f64", g, "f64", m, v, t, 3e-3, 0.9, 0.999, 0.0)
        assert np.allclose(p.detach().numpy(), theta, rtol=1e-12, atol=1e-14)


def test_first_step_closed_form():
    theta, _, _ = _state(3, 100)
    g = np.random.default_rng(4).standard_normal(100)
    new, m, v = oracle.masked_adam(theta, "f64", g, "f64", np.zeros(100), np.zeros(100), 1,
                                   0.05, 0.9, 0.999, 0.0)
    assert np.allclose(new, theta - 0.05 * np.sign(g), rtol=0, atol=1e-15)
    assert np.allclose(m, 0.1 * g) and np.allclose(v, 0.001 * g * g)


def test_mask_semantics():
    theta, m0, v0 = _state(5, 50)
    pos = np.array([3, 7, 20, 41])
    g = np.array([0.5, 0.0, -2.0, 0.0])        # materialized zeros included
    new, m, v = oracle.masked_adam(theta, "f64", g, "f64", m0, v0, 7, 1e-3, 0.9, 0.99, 1e-8,
                                   positions=pos)
    rest = np.setdiff1d(np.arange(50), pos)
    assert np.array_equal(new[rest], theta[rest])
    assert np.array_equal(m[rest], m0[rest]) and np.array_equal(v[rest], v0[rest])
    # a materialized zero still decays both moments and moves the value
    assert m[7] == 0.9 * m0[7] and v[7] == 0.99 * v0[7] and new[7] != theta[7]
