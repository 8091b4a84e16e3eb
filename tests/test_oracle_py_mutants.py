"""The pins of the oracle's Python-level functions (sparse linear layer, CG,
masked Adam, delta-coded rows) are sharp enough: plant a plausible mistake
in a copy of oracle/__init__.py, load the copy as a separate module (on the
CPU), put its function in place of the real one for the duration of the
test, and require that at least one pin fails."""
import importlib.util
import os
import types

import pytest

import oracle
import test_oracle_adam as TA
import test_oracle_adapter as TL
import test_oracle_cg as TC
import test_oracle_delta as TD

# (name, function replaced, old text, new text, pins that must catch it)
MUTANTS = [
    ("cg_steepest_descent", "cg", "p = r + (rr_new / rr) * p", "p = r.copy()",
     [TC.test_distinct_eigenvalues_bound_the_iterations]),
    ("cg_step_sign", "cg", "x += alpha * p", "x -= alpha * p",
     [lambda: TC.test_small_spd_finite_termination()]),
    ("cg_residual_from_p", "cg", "r -= alpha * q", "r -= alpha * p",
     [TC.test_distinct_eigenvalues_bound_the_iterations]),
    ("cg_stop_on_first_check", "cg", "while k < max_iter and rr > thr:",
     "while k < max_iter and rr > thr * 1e6:",
     [lambda: TC.test_agrees_with_scipy_cg(13, 500)]),
    ("adam_eps_inside_sqrt", "masked_adam", "np.sqrt(v[i]) + eps", "np.sqrt(v[i] + eps)",
     [lambda: TA.test_matches_torch_sparse_adam(False)]),
    ("adam_no_bias_correction", "masked_adam",
     "a_t = lr * np.sqrt(1.0 - beta2 ** step) / (1.0 - beta1 ** step)", "a_t = lr",
     [TA.test_first_step_closed_form]),
    ("adam_betas_swapped", "masked_adam", "m[i] = beta1 * m[i] + (1.0 - beta1) * g[j]",
     "m[i] = beta2 * m[i] + (1.0 - beta2) * g[j]",
     [TA.test_first_step_closed_form]),
    ("adam_no_maximize", "masked_adam", "    if maximize:\n        g = -g\n", "",
     [lambda: TA.test_matches_torch_sparse_adam(True)]),
    ("delta_code_off_by_one", "delta_encode", "code[pos] = (gap - 1 - 4 * pad).astype(np.uint32)",
     "code[pos] = (gap - 4 * pad).astype(np.uint32) & 3", [TD.test_hand_encoded_example]),
    ("delta_padding_threshold", "delta_encode", "pad = (gap - 1) // 4", "pad = gap // 5",
     [TD.test_hand_encoded_example,
      lambda: TD.test_round_trip_and_padding_count(1, 50, 70, 0.05, {})]),
    ("delta_decode_from_zero", "delta_decode", "cols = run - before - 1", "cols = run - before",
     [TD.test_hand_encoded_example]),
    ("linear_backward_wrong_input_row", "sparse_linear_backward",
     "dv[p] = float(np.dot(g[r[p]], x[c[p]]))", "dv[p] = float(np.dot(g[r[p]], x[r[p] % len(x)]))",
     [TL.test_quick_start_example_gradients, lambda: TL.test_finite_differences_are_exact(1)]),
    ("linear_backward_not_transposed", "sparse_linear_backward",
     "dxt[c[p]] += v[p] * g[r[p]]", "dxt[c[p]] += v[p] * g[c[p] % len(g)]",
     [TL.test_quick_start_example_gradients, lambda: TL.test_finite_differences_are_exact(1),
      lambda: TL.test_matches_dense_autograd(4, 30, 20, 5, 0.2)]),
]


def _mutant_module(old, new, tmp_path):
    src = open(oracle.__file__).read()
    assert src.count(old) == 1, "mutation site not unique"
    path = tmp_path / "oracle_py_mutant.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("oracle_py_mutant", path)
    mod = importlib.util.module_from_spec(spec)
    # the copy must find the real package's compiled C oracle and helpers
    mod.__dict__["__file__"] = oracle.__file__
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name,fn,old,new,checks", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_python_mutant_is_caught(tmp_path, monkeypatch, name, fn, old, new, checks):
    mod = _mutant_module(old, new, tmp_path)
    monkeypatch.setattr(oracle, fn, getattr(mod, fn))
    # functions the mutant calls internally must be its own (already are)
    caught = 0
    for check in checks:
        try:
            check()
        except AssertionError:
            caught += 1
    assert caught > 0, f"no pin caught mutant {name}"
