"""The oracle's pins are sharp enough: plant a plausible mistake in a copy of
oracle.c (on the CPU), rebuild it, and require that at least one pin fails.

Each mutant below is a single textual change of the kind a careless rewrite
would make: a dropped term, a wrong sign, a wrong index, a lost tie rule, a
lost stability guarantee.  Every mutant keeps all memory accesses in bounds.
"""
import shutil

import numpy as np
import pytest

import test_oracle as T

MUTANTS = [
    ("spmm_sign", "crow[j] += a * load_val", "crow[j] -= a * load_val",
     [lambda o: T.test_spmm_matches_dense_bruteforce(o, *T.CASES[0], 5)]),
    ("spmm_drop_first_term", "double a = load_val(val, vt, p);",
     "double a = (p == ro[r]) ? 0.0 : load_val(val, vt, p);",
     [lambda o: T.test_spmm_matches_dense_bruteforce(o, *T.CASES[0], 5)]),
    ("spmm_wrong_B_row", "load_val(B, bt, c * ldb + j)", "load_val(B, bt, (c > 0 ? c - 1 : c) * ldb + j)",
     [lambda o: T.test_spmm_identity_and_permutation_exact(o)]),
    ("sddmm_drop_k0", "for (int64_t kk = 0; kk < K; ++kk)", "for (int64_t kk = 1; kk < K; ++kk)",
     [lambda o: T.test_sddmm_matches_masked_dense(o, *T.CASES[0], 3)]),
    ("sddmm_wrong_BT_row", "load_val(BT, it, c * ldbt + kk)",
     "load_val(BT, it, (c > 0 ? c - 1 : c) * ldbt + kk)",
     [lambda o: T.test_sddmm_full_mask_is_dense_product(o)]),
    ("csr_add_sign", "load_val(W, wt, i) + load_val(val, vt, p)",
     "load_val(W, wt, i) - load_val(val, vt, p)",
     [lambda o: T.test_csr_add_equals_dense_sum(o, "f32", False)]),
    ("encode_ties_away", "double r = rint(a / q) * q;", "double r = floor(a / q + 0.5) * q;",
     [lambda o: T.test_encode_f16_matches_numpy(o),
      lambda o: T.test_csr_add_rounding_ties_to_even(o)]),
    ("decode_f16_subnormal_scale", "v = ldexp((double)f, -24);", "v = ldexp((double)f, -25);",
     [lambda o: T.test_decode_f16_all_patterns(o)]),
    ("decode_bf16_bias", "v = ldexp(128.0 + f, e - 134);", "v = ldexp(128.0 + f, e - 135);",
     [lambda o: T.test_decode_bf16_all_patterns(o)]),
    ("transpose_rows_reversed",
     "  for (int64_t r = 0; r < m; ++r) {\n    for (int64_t p = ro[r]; p < ro[r + 1]; ++p) {\n"
     "      int64_t c = load_idx(col, ct, p);\n      int64_t q = next[c]++;",
     "  for (int64_t r = m - 1; r >= 0; --r) {\n    for (int64_t p = ro[r]; p < ro[r + 1]; ++p) {\n"
     "      int64_t c = load_idx(col, ct, p);\n      int64_t q = next[c]++;",
     [lambda o: T.test_transpose_matches_scipy(o, *T.CASES[0])]),
    ("row_idx_ties_reversed",
     "  for (int64_t r = 0; r < m; ++r) {\n    int64_t b = maxc - (ro[r + 1] - ro[r]);",
     "  for (int64_t r = m - 1; r >= 0; --r) {\n    int64_t b = maxc - (ro[r + 1] - ro[r]);",
     [lambda o: T.test_row_idx_is_stable_descending_sort(o, *T.CASES[1])]),
]


@pytest.mark.parametrize("name,old,new,checks", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, orc, name, old, new, checks):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = open(orc._SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    mpath = tmp_path / "oracle_mutant.c"
    mpath.write_text(src.replace(old, new))
    lib = orc.load(orc.compile_source(str(mpath), str(tmp_path / "libmutant.so")))
    saved = orc._lib
    orc._lib = lib
    caught = False
    try:
        for chk in checks:
            try:
                chk(orc)
            except AssertionError:
                caught = True
    finally:
        orc._lib = saved
    assert caught, f"mutant {name} survived the pins"


def test_unmutated_oracle_passes_the_same_checks(orc):
    for _, _, _, checks in MUTANTS:
        for chk in checks:
            chk(orc)
    assert np.isfinite(1.0)
