"""GPU delta-coded rows against the oracle: the encoding bit for bit (row
offsets, 2-bit codes, values including the zero padding), the SpMV within
the value format's tolerance and bit-exact on integer data, column-order
errors, and the 8192 x 8192 half-dense size of the page's experiment on
sampled rows."""
import numpy as np
import pytest
import torch

import oracle
import unstructured_sparse_linear_amd as S
from unstructured_sparse_linear_amd import gen
from helpers import TORCH_DT, assert_close, csr_dev, dev, host, host_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    S.lib()
    yield
    torch.cuda.synchronize()


def encode(A):
    v, ro, ci = csr_dev(A)
    return S.delta_encode(v, ro, ci, A.m, A.n)


def codes_of(words_u32, e0, e1):
    e = np.arange(e0, e1)
    return (words_u32[e // 16] >> (2 * (e % 16)).astype(np.uint32)) & np.uint32(3)


CASES = [
    (1, 300, 500, 0.05, "f32", {}),                       # much padding
    (2, 257, 1000, 0.5, "f16", {"empty_row_frac": 0.2}),
    (3, 100, 3000, 0.9, "bf16", {}),
    (4, 64, 40000, 0.002, "f32", {"col_index_dtype": np.int32}),
    (5, 40, 1, 0.5, "f16", {}),
    (6, 33, 70, 0.0, "f32", {}),                          # no entries at all
]


@pytest.mark.parametrize("seed,m,n,density,dt,kw", CASES)
def test_encoding_bitexact(seed, m, n, density, dt, kw):
    A = gen.random_csr(seed, m, n, density, dt, **kw)
    D = encode(A)
    eo, words, ev = oracle.delta_encode(m, n, A.row_offsets, A.col_idx, A.values, dt)
    E = int(eo[-1])
    assert D.entries == E
    assert np.array_equal(host(D.enc_offsets), eo)
    gw = host(D.codes).view(np.uint32)
    assert np.array_equal(gw[:len(words)], words)
    gv = host(D.values)
    assert np.array_equal(gv[:E].view(np.uint8), np.asarray(ev).view(np.uint8))
    assert not gv[E:len(words) * 16].view(np.uint8).any()      # zero tail


@pytest.mark.parametrize("seed,m,n,density,dt,kw", CASES)
def test_spmv_parity(seed, m, n, density, dt, kw):
    A = gen.random_csr(seed, m, n, density, dt, **kw)
    x = gen.dense(seed, 100, gen.S_B, (n, 1), dt)
    D = encode(A)
    y = S.delta_spmv(D, dev(x, dt).reshape(-1))
    ref = oracle.spmm(m, A.row_offsets, A.col_idx, A.values, dt, x, dt)[:, 0]
    assert_close(host_f64(y), ref, dt, "delta spmv")


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_spmv_integer_bitexact_and_low_precision_output(dt):
    A = gen.random_csr(7, 500, 2000, 0.6, dt, integer_values=True)
    x = gen.dense(7, 100, gen.S_B, (2000, 1), dt, integer_values=True)
    D = encode(A)
    ref = oracle.spmm(A.m, A.row_offsets, A.col_idx, A.values, dt, x, dt)[:, 0]
    y = S.delta_spmv(D, dev(x, dt).reshape(-1))
    assert np.array_equal(host_f64(y), ref)
    if dt != "f32":
        # one rounding of the (exact) fp32 sum to the value format
        y16 = S.delta_spmv(D, dev(x, dt).reshape(-1), out_dtype=TORCH_DT[dt])
        assert rel_ok(host_f64(y16), ref, dt)


def rel_ok(y, r, dt):
    u = 2.0 ** -11 if dt == "f16" else 2.0 ** -8
    return np.all(np.abs(y - r) <= u * np.abs(r) + 1e-30)


def test_unsorted_or_out_of_range_columns_are_rejected():
    A = gen.random_csr(8, 50, 80, 0.3, "f32", shuffle_within_rows=True)
    with pytest.raises(S.SpopsError):
        encode(A)
    B = gen.random_csr(9, 20, 30, 0.3, "f32")
    v, ro, ci = csr_dev(B)
    ci[-1] = 30                      # one column past the end
    with pytest.raises(S.SpopsError):
        S.delta_encode(v, ro, ci, B.m, B.n)


def test_half_dense_8192_sampled_rows():
    # the page's MACKO experiment size: 8192 x 8192 at 50% density, f16
    A = gen.random_csr(10, 8192, 8192, 0.5, "f16")
    D = encode(A)
    x = gen.dense(10, 100, gen.S_B, (8192, 1), "f16")
    y = host_f64(S.delta_spmv(D, dev(x, "f16").reshape(-1)))
    eo = host(D.enc_offsets)
    words = host(D.codes).view(np.uint32)
    vals = host(D.values)
    rows = np.random.default_rng(11).choice(8192, 64, replace=False)
    for r in rows:
        a, b = A.row_offsets[r], A.row_offsets[r + 1]
        ro1 = np.array([0, b - a], np.int32)
        e_o, w_o, v_o = oracle.delta_encode(1, 8192, ro1, A.col_idx[a:b], A.values[a:b], "f16")
        assert eo[r + 1] - eo[r] == e_o[1]
        assert np.array_equal(codes_of(words, eo[r], eo[r + 1]), codes_of(w_o, 0, e_o[1]))
        assert np.array_equal(vals[eo[r]:eo[r + 1]].view(np.uint16), v_o.view(np.uint16))
        yr = oracle.spmm(1, ro1, A.col_idx[a:b], A.values[a:b], "f16", x, "f16")[0, 0]
        rms = np.sqrt(np.mean(y ** 2))
        assert abs(y[r] - yr) <= 2e-3 * max(abs(yr), rms)
