"""GPU masked Adam against the float64 oracle, one step at a time: each step
starts the oracle from the GPU's own state before that step (values in
their storage format, f32 moments), so a comparison covers exactly one
step.  Values must agree to the value format's tolerance, moments to the
f32 one; positions without a gradient must keep their bits."""
import numpy as np
import pytest
import torch

import oracle
import unstructured_sparse_linear_amd as S
from unstructured_sparse_linear_amd import gen
from helpers import TORCH_DT, assert_close, dev, host, host_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    S.lib()
    yield
    torch.cuda.synchronize()


# The new value is one rounding of an fp32 result to the value format: it
# lies within half a unit in the last place of the exact value (relative
# 2^-p for p stored bits after the leading one: 2^-24 f32, 2^-11 f16, 2^-8
# bf16; near zero, half the smallest f16 subnormal spacing), plus the fp32
# arithmetic's own error: a few units of 2^-24 of the magnitudes that enter
# it -- the old value and the step computed from |beta1 m| + |(1 - beta1) g|
# (the two terms of the new first moment may cancel).
VALUE_REL = {"f32": 2.0 ** -24, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}
VALUE_ABS = {"f32": 0.0, "f16": 2.0 ** -25, "bf16": 0.0}


def assert_values_close(y, r, dt, scale):
    bound = VALUE_REL[dt] * np.abs(r) + VALUE_ABS[dt] + 1e-6 * scale
    bad = np.flatnonzero(np.abs(y - r) > bound)
    assert bad.size == 0, f"values: {bad.size} outside one rounding, e.g. {y[bad[:3]]} vs {r[bad[:3]]}"


def step_scale(old, m_old, g, v_new, step, lr, beta1, beta2, eps, positions=None):
    """|old value| + the step's size computed from absolute terms, per value."""
    scale = np.abs(np.asarray(old, np.float64)).copy()
    idx = np.arange(len(scale)) if positions is None else np.asarray(positions)
    a_t = lr * np.sqrt(1 - beta2 ** step) / (1 - beta1 ** step)
    mag = beta1 * np.abs(m_old[idx]) + (1 - beta1) * np.abs(np.asarray(g, np.float64))
    scale[idx] += a_t * mag / (np.sqrt(v_new[idx]) + eps)
    return scale


def _grad(rng, n, dt):
    return gen.normal(rng, n, dt, 0.1)


def _check_step(vals, m, v, g, dt, step, hp, positions=None):
    before = (host(vals), host_f64(m), host_f64(v))
    S.masked_adam(vals, dev(g, dt), m, v, step, lr=hp["lr"], betas=hp["betas"], eps=hp["eps"],
                  maximize=hp.get("maximize", False),
                  positions=None if positions is None else dev(positions.astype(np.int32)))
    ref_v, ref_m, ref_s = oracle.masked_adam(before[0], dt, g, dt, before[1], before[2], step,
                                             hp["lr"], hp["betas"][0], hp["betas"][1],
                                             hp["eps"], hp.get("maximize", False), positions)
    sc = step_scale(oracle.to_f64(before[0], dt), before[1], oracle.to_f64(g, dt), ref_s, step,
                    hp["lr"], hp["betas"][0], hp["betas"][1], hp["eps"], positions)
    assert_values_close(host_f64(vals), ref_v, dt, sc)
    assert_close(host_f64(m), ref_m, "f32", "exp_avg")
    assert_close(host_f64(v), ref_s, "f32", "exp_avg_sq")
    return before


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("maximize", [False, True])
def test_dense_gradient_steps(dt, maximize):
    n = 100_003
    rng = np.random.default_rng(1)
    vals = dev(gen.normal(rng, n, dt, 0.02), dt)
    m = torch.zeros(n, dtype=torch.float32, device="cuda")
    v = torch.zeros_like(m)
    hp = {"lr": 1e-3, "betas": (0.9, 0.999), "eps": 1e-8, "maximize": maximize}
    for step in range(1, 5):
        _check_step(vals, m, v, _grad(rng, n, dt), dt, step, hp)


def test_positions_update_only_listed_values():
    n, k = 50_000, 7_001
    rng = np.random.default_rng(2)
    vals = dev(gen.normal(rng, n, "f32"), "f32")
    m = dev(np.abs(gen.normal(rng, n, "f32", 0.01)))
    v = dev(np.abs(gen.normal(rng, n, "f32", 0.001)))
    hp = {"lr": 1e-2, "betas": (0.8, 0.99), "eps": 1e-6}
    for step in (3, 4):
        pos = np.sort(rng.choice(n, k, replace=False))
        g = _grad(rng, k, "f32")
        g[::10] = 0.0                      # materialized zeros still count
        before = _check_step(vals, m, v, g, "f32", step, hp, positions=pos)
        rest = np.setdiff1d(np.arange(n), pos)
        assert np.array_equal(host(vals)[rest], before[0][rest])
        assert np.array_equal(host_f64(m)[rest], before[1][rest])
        assert np.array_equal(host_f64(v)[rest], before[2][rest])


def test_positions_out_of_range_are_skipped():
    n = 1000
    vals = torch.ones(n, device="cuda")
    m = torch.zeros(n, device="cuda")
    v = torch.zeros(n, device="cuda")
    pos = torch.tensor([-1, 5, n, n + 7], dtype=torch.int32, device="cuda")
    g = torch.full((4,), 0.5, device="cuda")
    S.masked_adam(vals, g, m, v, 1, lr=0.1, eps=0.0, positions=pos)
    h = host(vals)
    # first step with eps = 0 moves a value by lr against its gradient's sign
    assert abs(h[5] - 0.9) < 1e-6 and np.count_nonzero(h != 1.0) == 1


def test_optimizer_trains_adapter_values():
    # the layer's dense value gradient, then a sparse COO gradient
    m_, n_, T = 300, 400, 64
    A = gen.random_csr(3, m_, n_, 0.05, "f32")
    P = S.SparsePattern(dev(A.row_offsets), dev(A.col_idx), m_, n_)
    layer = S.SparseAdapter(P, dev(A.values, "f32").clone())
    opt = S.MaskedAdam(layer.parameters(), lr=1e-2, betas=(0.9, 0.99), eps=1e-8)
    xt = dev(gen.normal(np.random.default_rng(4), (n_, T), "f32"))
    hp = {"lr": 1e-2, "betas": (0.9, 0.99), "eps": 1e-8}
    for step in (1, 2):
        opt.zero_grad()
        layer(xt).square().sum().backward()
        st = opt.state.get(layer.values, {})
        before = (host(layer.values.detach()),
                  host_f64(st["exp_avg"]) if st else np.zeros(A.nnz),
                  host_f64(st["exp_avg_sq"]) if st else np.zeros(A.nnz))
        g = host(layer.values.grad)
        opt.step()
        ref_v, ref_m, ref_s = oracle.masked_adam(before[0], "f32", g, "f32", before[1],
                                                 before[2], step, **_flat(hp))
        sc = step_scale(before[0], before[1], g, ref_s, step, 1e-2, 0.9, 0.99, 1e-8)
        assert_values_close(host_f64(layer.values.detach()), ref_v, "f32", sc)
        assert_close(host_f64(opt.state[layer.values]["exp_avg"]), ref_m, "f32", "m")
    # sparse gradient: only the named values move
    pos = np.array([0, 17, 99, A.nnz - 1])
    gv = np.array([0.3, -0.1, 0.0, 2.0], np.float32)
    layer.values.grad = torch.sparse_coo_tensor(torch.tensor(pos)[None].cuda(),
                                                torch.tensor(gv).cuda(), (A.nnz,)).coalesce()
    before = host(layer.values.detach())
    opt.step()
    after = host(layer.values.detach())
    moved = np.flatnonzero(after != before)
    assert set(moved.tolist()) <= set(pos.tolist()) and 0 in moved and A.nnz - 1 in moved


def _flat(hp):
    return {"lr": hp["lr"], "beta1": hp["betas"][0], "beta2": hp["betas"][1], "eps": hp["eps"]}


def test_masked_adam_rejects_bad_arguments():
    vals = torch.zeros(10, device="cuda")
    m, v = torch.zeros_like(vals), torch.zeros_like(vals)
    g = torch.ones(10, device="cuda")
    with pytest.raises(S.SpopsError):
        S.masked_adam(vals, g, m, v, 0)                    # step counts from 1
    with pytest.raises(S.SpopsError):
        S.masked_adam(vals, g, m, v, 1, betas=(1.0, 0.9))
    with pytest.raises(ValueError):
        S.masked_adam(vals, g[:5], m, v, 1)                # grad must cover every value
    with pytest.raises(ValueError):
        S.masked_adam(vals, g.half(), m, v, 1)             # grad in the values' dtype
