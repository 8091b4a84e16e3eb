"""Pins of the oracle's 2-bit delta-compressed row format (encode, decode,
SpMV) against facts that do not come from the oracle: a small matrix encoded
by hand, the round trip back to the same matrix (dense comparison), closed
forms for the padding count, and SpMV against the C oracle's CSR product
(exactly equal on integer data, since padding adds zero products)."""
import numpy as np
import pytest

import oracle
from unstructured_sparse_linear_amd import gen


def test_hand_encoded_example():
    # row 0: columns 0, 1, 5, 13 -> gaps 1, 1, 4, 8 -> codes 0, 0, 3, then a
    #        padding entry at column 9 (code 3) and column 13 (code 3)
    # row 1: empty
    # row 2: columns 7, 2 (stored unsorted) -> sorted 2, 7 -> gaps 3, 5 ->
    #        code 2, a padding entry at column 6 (code 3), column 7 (code 0)
    ro = np.array([0, 4, 4, 6], np.int32)
    ci = np.array([0, 1, 5, 13, 7, 2], np.int16)
    v = np.array([1, 2, 3, 4, 5, 6], np.float32)
    eo, words, ev = oracle.delta_encode(3, 16, ro, ci, v, "f32")
    assert eo.tolist() == [0, 5, 5, 8]
    codes = [0, 0, 3, 3, 3, 2, 3, 0]
    assert words.tolist() == [sum(c << (2 * e) for e, c in enumerate(codes))]
    assert ev.tolist() == [1, 2, 3, 0, 4, 6, 0, 5]
    _, cols, _ = oracle.delta_decode(3, eo, words, ev)
    assert cols.tolist() == [0, 1, 5, 9, 13, 2, 6, 7]


def _dense(m, n, ro, ci, v):
    D = np.zeros((m, n))
    r = np.repeat(np.arange(m), np.diff(np.asarray(ro, np.int64)))
    np.add.at(D, (r, np.asarray(ci, np.int64)), np.asarray(v, np.float64))
    return D


@pytest.mark.parametrize("seed,m,n,density,kw", [
    (1, 50, 70, 0.05, {}), (2, 40, 300, 0.5, {"shuffle_within_rows": True}),
    (3, 33, 200, 0.9, {"empty_row_frac": 0.2}), (4, 10, 1, 0.5, {}),
    (5, 20, 40000, 0.001, {"col_index_dtype": np.int32}),
])
def test_round_trip_and_padding_count(seed, m, n, density, kw):
    A = gen.random_csr(seed, m, n, density, "f32", **kw)
    eo, words, ev = oracle.delta_encode(m, n, A.row_offsets, A.col_idx, A.values, "f32")
    ro2, cols, v2 = oracle.delta_decode(m, eo, words, ev)
    assert np.array_equal(_dense(m, n, ro2, cols, v2),
                          _dense(m, n, A.row_offsets, A.col_idx, A.values))
    assert cols.min(initial=0) >= 0 and cols.max(initial=0) < n
    # padding: (gap - 1) // 4 entries before each stored entry
    for r in range(m):
        c = np.sort(A.col_idx[A.row_offsets[r]:A.row_offsets[r + 1]].astype(np.int64))
        gaps = np.diff(np.concatenate([[-1], c]))
        assert eo[r + 1] - eo[r] == len(c) + int(np.sum((gaps - 1) // 4))
        # every decoded column of the row is increasing, padding values are zero
        rc = cols[eo[r]:eo[r + 1]]
        assert np.all(np.diff(rc) >= 1) and np.all(np.diff(rc) <= 4)
        assert set(c.tolist()) <= set(rc.tolist())
        assert np.all(v2[eo[r]:eo[r + 1]][~np.isin(rc, c)] == 0)


def test_dense_row_and_single_entry_closed_forms():
    n = 37
    ro = np.array([0, n, n + 1], np.int32)
    ci = np.concatenate([np.arange(n), [n - 1]]).astype(np.int16)
    v = np.ones(n + 1, np.float32)
    eo, words, _ = oracle.delta_encode(2, n, ro, ci, v, "f32")
    # a full row needs no padding and all codes 0; a lone entry at column c
    # needs c // 4 padding entries
    assert eo.tolist() == [0, n, n + 1 + (n - 1) // 4]
    e = np.arange(n)
    assert np.all((words[e // 16] >> (2 * (e % 16)).astype(np.uint32)) & 3 == 0)


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_spmv_matches_csr_product(dt):
    A = gen.random_csr(6, 120, 500, 0.6, dt, shuffle_within_rows=True, empty_row_frac=0.1)
    x = gen.dense(6, 100, gen.S_B, (500, 1), dt)
    eo, words, ev = oracle.delta_encode(A.m, A.n, A.row_offsets, A.col_idx, A.values, dt)
    y = oracle.delta_spmv(A.m, eo, words, ev, dt, x, dt)
    ref = oracle.spmm(A.m, A.row_offsets, A.col_idx, A.values, dt, x, dt)[:, 0]
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)
    Ai = gen.random_csr(7, 80, 300, 0.7, dt, integer_values=True)
    xi = gen.dense(7, 100, gen.S_B, (300, 1), dt, integer_values=True)
    eo, words, ev = oracle.delta_encode(Ai.m, Ai.n, Ai.row_offsets, Ai.col_idx, Ai.values, dt)
    assert np.array_equal(oracle.delta_spmv(Ai.m, eo, words, ev, dt, xi, dt),
                          oracle.spmm(Ai.m, Ai.row_offsets, Ai.col_idx, Ai.values, dt, xi, dt)[:, 0])
