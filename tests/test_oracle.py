"""Pins for the float64 CPU oracle (no GPU).

Each check ties the oracle to something other than itself: all bit patterns
of the 16-bit formats against numpy/torch casts, dense brute force with numpy
matmul, scipy's sparse routines, exact integer arithmetic, closed forms
(identity / permutation / all-ones operands) and the tiny matrices printed on
the pages (tests/golden/page_examples.json).
"""
import json
import os

import numpy as np
import pytest
import scipy.sparse as sp

from unstructured_sparse_linear_amd import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_examples.json")
NP = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}


def f64(x, dt):
    return gen.storage_to_f64(x, dt)


# ------------------------------------------------------------- codecs ----

def test_decode_f16_all_patterns(orc):
    b = np.arange(65536, dtype=np.uint16)
    assert np.array_equal(orc.decode(b, "f16"), b.view(np.float16).astype(np.float64),
                          equal_nan=True)


def test_decode_bf16_all_patterns(orc):
    import torch
    b = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(orc.decode(b, "bf16"), ref, equal_nan=True)


def test_encode_f16_matches_numpy(orc):
    rng = np.random.default_rng(7)
    x = rng.standard_normal(400_000) * 2.0 ** rng.integers(-30, 18, 400_000)
    # exact ties: midpoints between neighbouring f16 values, incl. subnormals
    h = rng.integers(0, 0x7BFF, 50_000).astype(np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    x = np.concatenate([x, 0.5 * (lo + hi), -0.5 * (lo + hi), [0.0, -0.0, 65504.0, 65519.99,
                                                               65520.0, 1e9, 2.0 ** -25,
                                                               3 * 2.0 ** -26]])
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(orc.encode(x, "f16"), ref)


def test_encode_bf16_matches_torch_and_hand_ties(orc):
    import torch
    rng = np.random.default_rng(8)
    # f32-representable inputs: torch's float32 -> bfloat16 cast is a single RNE
    x32 = (rng.standard_normal(400_000) * 2.0 ** rng.integers(-140, 120, 400_000)).astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(orc.encode(x32.astype(np.float64), "bf16"), ref)
    # hand-made ties: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 -> even (1.0)
    cases = {1.0 + 2.0 ** -8: 0x3F80, 1.0 + 3 * 2.0 ** -8: 0x3F82, -(1.0 + 2.0 ** -8): 0xBF80,
             1.0 + 2.0 ** -8 + 2.0 ** -40: 0x3F81, 2.0 ** -133: 0x0001, 2.0 ** -134: 0x0000,
             3 * 2.0 ** -135: 0x0001, float(2 ** 128): 0x7F80, (2 - 2.0 ** -8) * 2.0 ** 127: 0x7F80,
             (2 - 2.0 ** -7) * 2.0 ** 127: 0x7F7F}
    xs = np.array(list(cases.keys()))
    assert [int(v) for v in orc.encode(xs, "bf16")] == list(cases.values())


# ------------------------------------------------------------ helpers ----

def rand_case(seed, m, n, density, dt, **kw):
    return gen.random_csr(seed, m, n, density, dt, **kw)


CASES = [
    # seed, m, n, density, dt, kwargs
    (1, 37, 53, 0.2, "f32", {}),
    (2, 64, 17, 0.5, "f16", {"empty_row_frac": 0.3}),
    (3, 19, 200, 0.1, "bf16", {"shuffle_within_rows": True}),
    (4, 50, 40, 0.15, "f32", {"col_index_dtype": np.int32}),
    (5, 1, 9, 0.9, "f16", {}),
    (6, 9, 1, 0.7, "bf16", {}),
    (7, 33, 33, 0.0, "f32", {}),
]


# --------------------------------------------------------------- SpMM ----

@pytest.mark.parametrize("seed,m,n,density,dt,kw", CASES)
@pytest.mark.parametrize("N", [1, 5, 64])
def test_spmm_matches_dense_bruteforce(orc, seed, m, n, density, dt, kw, N):
    A = rand_case(seed, m, n, density, dt, **kw)
    B = gen.dense(seed, 100, gen.S_B, (n, N), dt)
    C = orc.spmm(m, A.row_offsets, A.col_idx, A.values, dt, B, dt)
    ref = A.to_dense_f64() @ f64(B, dt)
    np.testing.assert_allclose(C, ref, rtol=1e-12, atol=1e-12)


def test_spmm_matches_scipy_on_config1(orc):
    w = gen.make_config(1)
    A, B = w.get("A"), w.get("B")
    S = sp.csr_matrix((A.values.astype(np.float64), A.col_idx, A.row_offsets), shape=(A.m, A.n))
    C = orc.spmm(A.m, A.row_offsets, A.col_idx, A.values, "f32", B, "f32")
    np.testing.assert_allclose(C, S @ B.astype(np.float64), rtol=1e-12, atol=1e-12)


def test_spmm_identity_and_permutation_exact(orc):
    n, N = 300, 7
    B = gen.dense(0, 100, gen.S_B, (n, N), "f16")
    ident = gen.CSR(n, n, np.arange(n + 1, dtype=np.int32), np.arange(n, dtype=np.int16),
                    gen.f32_to_storage(np.ones(n, np.float32), "f16"), "f16")
    assert np.array_equal(orc.spmm(n, ident.row_offsets, ident.col_idx, ident.values, "f16",
                                   B, "f16"), f64(B, "f16"))
    perm = np.random.default_rng(3).permutation(n)
    P = gen.CSR(n, n, np.arange(n + 1, dtype=np.int32), perm.astype(np.int16),
                gen.f32_to_storage(np.ones(n, np.float32), "f16"), "f16")
    assert np.array_equal(orc.spmm(n, P.row_offsets, P.col_idx, P.values, "f16", B, "f16"),
                          f64(B, "f16")[perm])


def test_spmm_linear_in_disjoint_patterns(orc):
    A = rand_case(11, 40, 60, 0.3, "f32")
    # split the entries of each row alternately into two disjoint matrices
    keep = np.arange(A.nnz) % 2 == 0
    parts = []
    for mask in (keep, ~keep):
        rows = np.repeat(np.arange(A.m), A.row_counts())[mask]
        parts.append(gen.csr_from_coo(A.m, A.n, rows, A.col_idx[mask], A.values[mask], "f32"))
    B = gen.dense(11, 100, gen.S_B, (60, 9), "f32")
    full = orc.spmm(A.m, A.row_offsets, A.col_idx, A.values, "f32", B, "f32")
    s = sum(orc.spmm(P.m, P.row_offsets, P.col_idx, P.values, "f32", B, "f32") for P in parts)
    np.testing.assert_allclose(full, s, rtol=1e-13, atol=1e-13)


def test_spmm_integer_values_exact(orc):
    A = rand_case(12, 70, 90, 0.3, "bf16", integer_values=True)
    B = gen.dense(12, 100, gen.S_B, (90, 13), "bf16", integer_values=True)
    C = orc.spmm(A.m, A.row_offsets, A.col_idx, A.values, "bf16", B, "bf16")
    Ai = A.to_dense_f64().astype(np.int64)
    assert np.array_equal(C, (Ai @ f64(B, "bf16").astype(np.int64)).astype(np.float64))


def test_spmm_empty_matrix(orc):
    A = rand_case(13, 10, 10, 0.0, "f32")
    assert A.nnz == 0
    B = gen.dense(13, 100, gen.S_B, (10, 3), "f32")
    assert np.array_equal(orc.spmm(10, A.row_offsets, A.col_idx, A.values, "f32", B, "f32"),
                          np.zeros((10, 3)))


# -------------------------------------------------------------- SDDMM ----

@pytest.mark.parametrize("seed,m,n,density,dt,kw", CASES)
@pytest.mark.parametrize("K", [1, 3, 40])
def test_sddmm_matches_masked_dense(orc, seed, m, n, density, dt, kw, K):
    M = rand_case(seed, m, n, density, None, **kw)
    Ad = gen.dense(seed, 100, gen.S_A, (m, K), dt)
    BT = gen.dense(seed, 100, gen.S_BT, (n, K), dt)
    out = orc.sddmm(M.row_offsets, M.col_idx, Ad, BT, dt)
    full = f64(Ad, dt) @ f64(BT, dt).T
    rows = np.repeat(np.arange(m), M.row_counts())
    np.testing.assert_allclose(out, full[rows, M.col_idx.astype(np.int64)], rtol=1e-12,
                               atol=1e-12)


def test_sddmm_full_mask_is_dense_product(orc):
    m, n, K = 23, 31, 17
    M = gen.csr_from_row_lists(m, n, [np.arange(n)] * m)
    Ad = gen.dense(1, 100, gen.S_A, (m, K), "f32")
    BT = gen.dense(1, 100, gen.S_BT, (n, K), "f32")
    out = orc.sddmm(M.row_offsets, M.col_idx, Ad, BT, "f32").reshape(m, n)
    np.testing.assert_allclose(out, Ad.astype(np.float64) @ BT.astype(np.float64).T,
                               rtol=1e-12, atol=1e-12)


def test_sddmm_k1_is_exact_product(orc):
    M = rand_case(2, 30, 30, 0.3, None)
    Ad = gen.dense(2, 100, gen.S_A, (30, 1), "f32")
    BT = gen.dense(2, 100, gen.S_BT, (30, 1), "f32")
    out = orc.sddmm(M.row_offsets, M.col_idx, Ad, BT, "f32")
    rows = np.repeat(np.arange(30), M.row_counts())
    ref = Ad[rows, 0].astype(np.float64) * BT[M.col_idx.astype(np.int64), 0].astype(np.float64)
    assert np.array_equal(out, ref)


def test_sddmm_integer_values_exact(orc):
    M = rand_case(3, 45, 60, 0.2, None)
    Ad = gen.dense(3, 100, gen.S_A, (45, 33), "f16", integer_values=True)
    BT = gen.dense(3, 100, gen.S_BT, (60, 33), "f16", integer_values=True)
    out = orc.sddmm(M.row_offsets, M.col_idx, Ad, BT, "f16")
    full = Ad.astype(np.int64) @ BT.astype(np.int64).T
    rows = np.repeat(np.arange(45), M.row_counts())
    assert np.array_equal(out, full[rows, M.col_idx.astype(np.int64)].astype(np.float64))


# ------------------------------------------------------------ csr_add ----

def _round_to(x64, dt):
    import torch
    if dt == "f32":
        return x64.astype(np.float32)
    if dt == "f16":
        return x64.astype(np.float16)
    # sums of two bf16 numbers of similar magnitude are exact in f32, so the
    # f32 -> bf16 cast below rounds once
    return torch.from_numpy(x64.astype(np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("shuffle", [False, True])
def test_csr_add_equals_dense_sum(orc, dt, shuffle):
    m, n = 57, 83
    A = rand_case(21, m, n, 0.25, dt, shuffle_within_rows=shuffle, empty_row_frac=0.1)
    W = gen.dense(21, 100, gen.S_W, (m, n), dt, std=1.0)
    out = orc.csr_add(A.row_offsets, A.col_idx, A.values, dt, W, dt)
    ref = _round_to(f64(W, dt) + A.to_dense_f64(), dt)
    if dt == "f32":
        assert np.array_equal(out, ref)
    else:
        assert np.array_equal(out.view(np.uint16), np.asarray(ref).view(np.uint16))
    # untouched elements keep their bits
    untouched = A.to_dense_f64() == 0
    assert np.array_equal(out.view(np.uint8).reshape(m, -1)[:, :].reshape(m, n, -1)[untouched],
                          W.view(np.uint8).reshape(m, n, -1)[untouched])


def test_csr_add_rounding_ties_to_even(orc):
    # W = 1.0 and a = 2^-11: exact sum 1 + 2^-11 is halfway between two f16
    # neighbours (spacing 2^-10 above 1) -> rounds to 1.0 (even)
    A = gen.CSR(1, 2, np.array([0, 2], np.int32), np.array([0, 1], np.int16),
                np.array([2.0 ** -11, 3 * 2.0 ** -11], np.float16), "f16")
    W = np.array([[1.0, 1.0]], np.float16)
    out = orc.csr_add(A.row_offsets, A.col_idx, A.values, "f16", W, "f16")
    assert out[0, 0] == np.float16(1.0) and out[0, 1] == np.float16(1.0 + 2.0 ** -9)


# ----------------------------------------------------------- transpose ---

@pytest.mark.parametrize("seed,m,n,density,dt,kw", CASES)
def test_transpose_matches_scipy(orc, seed, m, n, density, dt, kw):
    A = rand_case(seed, m, n, density, dt, **kw)
    vT, roT, ciT = orc.csr_transpose(m, n, A.row_offsets, A.col_idx, A.values)
    S = sp.csr_matrix((np.arange(A.nnz), A.col_idx.astype(np.int64), A.row_offsets),
                      shape=(m, n))
    T = S.T.tocsr()   # data holds the source position of each entry
    assert np.array_equal(roT, T.indptr.astype(np.int32))
    assert np.array_equal(ciT.astype(np.int64), T.indices)
    assert np.array_equal(vT.view(np.uint8), A.values[T.data].view(np.uint8))
    assert np.array_equal(np.diff(roT), np.bincount(A.col_idx.astype(np.int64), minlength=n))


def test_transpose_twice_is_identity_for_sorted_rows(orc):
    A = rand_case(31, 120, 77, 0.1, "f32")
    vT, roT, ciT = orc.csr_transpose(120, 77, A.row_offsets, A.col_idx, A.values)
    v2, ro2, ci2 = orc.csr_transpose(77, 120, roT, ciT, vT, out_index_dtype=A.col_idx.dtype)
    assert np.array_equal(ro2, A.row_offsets) and np.array_equal(ci2, A.col_idx)
    assert np.array_equal(v2, A.values)


def test_transpose_wide_index_output(orc):
    # more than 32767 rows: the transposed column indices need int32
    m = 40000
    A = rand_case(32, m, 5, 0.0005, "f32")
    vT, roT, ciT = orc.csr_transpose(m, 5, A.row_offsets, A.col_idx, A.values)
    assert ciT.dtype == np.int32
    S = sp.csr_matrix((A.values, A.col_idx.astype(np.int64), A.row_offsets), shape=(m, 5))
    T = S.T.tocsr()
    assert np.array_equal(ciT, T.indices) and np.array_equal(vT, T.data)


# ------------------------------------------------------------- row_idx ---

@pytest.mark.parametrize("seed,m,n,density,dt,kw", CASES)
def test_row_idx_is_stable_descending_sort(orc, seed, m, n, density, dt, kw):
    A = rand_case(seed, m, n, density, None, **kw)
    ri = orc.row_idx(A.row_offsets)
    assert np.array_equal(ri.astype(np.int64), np.argsort(-A.row_counts(), kind="stable"))
    assert np.array_equal(np.sort(ri.astype(np.int64)), np.arange(m))


def test_row_idx_config5(orc):
    A = gen.make_config(5).get("mask")
    ri = orc.row_idx(A.row_offsets)
    assert np.array_equal(ri.astype(np.int64), np.argsort(-A.row_counts(), kind="stable"))


# ------------------------------------------------------- page examples ---

def _examples():
    with open(GOLDEN) as f:
        return json.load(f)["examples"]


@pytest.mark.parametrize("ex", _examples(), ids=lambda e: e["name"])
def test_page_examples(orc, ex):
    m, n = ex["m"], ex["n"]
    ro = np.array(ex["row_offsets"], np.int32)
    ci = np.array(ex["col_idx"], np.int16)
    v = np.array(ex["values"], np.float32)
    vT, roT, ciT = orc.csr_transpose(m, n, ro, ci, v)
    assert roT.tolist() == ex["transpose"]["row_offsets"]
    assert ciT.tolist() == ex["transpose"]["col_idx"]
    assert vT.tolist() == ex["transpose"]["values"]
    assert orc.row_idx(ro).tolist() == ex["row_idx"]
    B = np.array(ex["spmm"]["B"], np.float32)
    assert orc.spmm(m, ro, ci, v, "f32", B, "f32").tolist() == ex["spmm"]["C"]
    if "sddmm" in ex:
        out = orc.sddmm(ro, ci, np.array(ex["sddmm"]["A"], np.float32),
                        np.array(ex["sddmm"]["BT"], np.float32), "f32")
        assert out.tolist() == ex["sddmm"]["out"]
    if "csr_add" in ex:
        W = np.array(ex["csr_add"]["W"], np.float32)
        assert orc.csr_add(ro, ci, v, "f32", W, "f32").tolist() == ex["csr_add"]["result"]


def test_check_csr(orc):
    A = rand_case(41, 10, 10, 0.3, None)
    assert orc.check_csr(10, 10, A.row_offsets, A.col_idx) == 0
    bad = A.col_idx.copy()
    bad[0] = 10
    assert orc.check_csr(10, 10, A.row_offsets, bad) == 3
