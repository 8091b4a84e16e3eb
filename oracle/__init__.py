"""CPU float64 oracle for the CSR sparse-dense operations (ctypes over oracle.c).

TEST INFRASTRUCTURE ONLY.  The GPU library never imports, links or calls this
package; only the tests, the smoke check and the benchmark's CPU-baseline leg
do.  Definitions and their sources are documented in oracle.c (spops README,
sections "Usage", "Sparse Addition", "Sparse Matrix Multiplication (SpMM)",
"Sampled Dense-Dense Matrix Multiplication (SDDMM)", "CSR Transpose").

Host arrays use the storage conventions of the input generators: 'f32' ->
float32, 'f16' -> float16, 'bf16' -> uint16 bit patterns; int16/int32 indices.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_DT = {"f32": 0, "f16": 1, "bf16": 2}
_NP = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}


def compile_source(src: str, out: str) -> str:
    """gcc -O2 with OpenMP and no fast-math; atomic replace of `out`."""
    tmp = out + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                           "-Wall", "-o", tmp, src, "-lm"])
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so next to it."""
    if force or not os.path.exists(_LIB):
        compile_source(_SRC, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = load(_LIB)
    return _lib


def load(path: str):
    """Load a compiled oracle library and declare its signatures."""
    L = ctypes.CDLL(path)
    i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    L.oracle_spmm.argtypes = [i64, i64, i64, vp, vp, i32, vp, i32, vp, i32, i64, vp]
    L.oracle_sddmm.argtypes = [i64, i64, i64, vp, vp, i32, vp, i64, vp, i64, i32, vp]
    L.oracle_csr_add.argtypes = [i64, i64, vp, vp, i32, vp, i32, vp, i32, i64]
    L.oracle_csr_transpose.argtypes = [i64, i64, vp, vp, i32, vp, i64, vp, vp, vp, i32]
    L.oracle_row_idx.argtypes = [i64, vp, vp, i32]
    L.oracle_check_csr.argtypes = [i64, i64, vp, vp, i32]
    L.oracle_decode_array.argtypes = [vp, i32, i64, vp]
    L.oracle_encode_array.argtypes = [vp, i32, i64, vp]
    L.oracle_num_threads.restype = i32
    for f in ("oracle_spmm", "oracle_sddmm", "oracle_csr_add", "oracle_csr_transpose",
              "oracle_row_idx", "oracle_check_csr"):
        getattr(L, f).restype = i32
    return L


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _itype(a: np.ndarray) -> int:
    if a.dtype == np.int16:
        return 0
    if a.dtype == np.int32:
        return 1
    raise TypeError(f"index arrays must be int16 or int32, got {a.dtype}")


def _c(a, dtype=None):
    a = np.ascontiguousarray(a if dtype is None else np.asarray(a, dtype=dtype))
    return a


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def check_csr(m, n, row_offsets, col_idx) -> int:
    ro, ci = _c(row_offsets, np.int32), _c(col_idx)
    return int(lib().oracle_check_csr(m, n, _p(ro), _p(ci), _itype(ci)))


def spmm(m: int, row_offsets, col_idx, values, val_dt: str, B, b_dt: str) -> np.ndarray:
    """C = A @ B in float64, A given by (row_offsets, col_idx, values)."""
    ro, ci, v = _c(row_offsets, np.int32), _c(col_idx), _c(values, _NP[val_dt])
    B = _c(B, _NP[b_dt])
    k, N = B.shape
    C = np.empty((m, N), dtype=np.float64)
    rc = lib().oracle_spmm(m, k, N, _p(ro), _p(ci), _itype(ci), _p(v), _DT[val_dt],
                           _p(B), _DT[b_dt], N, _p(C))
    assert rc == 0
    return C


def sddmm(row_offsets, col_idx, A, BT, in_dt: str) -> np.ndarray:
    """out[p] = <A[r(p), :], BT[col(p), :]> in float64 at every mask position."""
    ro, ci = _c(row_offsets, np.int32), _c(col_idx)
    A, BT = _c(A, _NP[in_dt]), _c(BT, _NP[in_dt])
    m, K = A.shape
    n = BT.shape[0]
    assert BT.shape[1] == K and len(ro) == m + 1
    out = np.empty(int(ro[-1]), dtype=np.float64)
    rc = lib().oracle_sddmm(m, n, K, _p(ro), _p(ci), _itype(ci), _p(A), K, _p(BT), K,
                            _DT[in_dt], _p(out))
    assert rc == 0
    return out


def csr_add(row_offsets, col_idx, values, val_dt: str, W, w_dt: str) -> np.ndarray:
    """Returns a copy of W with the sparse matrix added at its positions."""
    ro, ci, v = _c(row_offsets, np.int32), _c(col_idx), _c(values, _NP[val_dt])
    Wc = np.array(W, dtype=_NP[w_dt], copy=True, order="C")
    m, n = Wc.shape
    assert len(ro) == m + 1
    rc = lib().oracle_csr_add(m, n, _p(ro), _p(ci), _itype(ci), _p(v), _DT[val_dt],
                              _p(Wc), _DT[w_dt], n)
    assert rc == 0
    return Wc


def csr_transpose(m: int, n: int, row_offsets, col_idx, values=None, out_index_dtype=None):
    """A^T as (values_T, row_offsets_T[n+1], col_idx_T); values moved bitwise."""
    ro, ci = _c(row_offsets, np.int32), _c(col_idx)
    nnz = int(ro[-1])
    odt = out_index_dtype or (np.int16 if m <= 32767 else np.int32)
    out_ro = np.empty(n + 1, dtype=np.int32)
    out_ci = np.empty(nnz, dtype=odt)
    if values is not None:
        v = _c(values)
        out_v = np.empty_like(v)
        vb = v.dtype.itemsize
    else:
        v = out_v = np.empty(0, dtype=np.uint8)
        vb = 0
    rc = lib().oracle_csr_transpose(m, n, _p(ro), _p(ci), _itype(ci), _p(v), vb, _p(out_v),
                                    _p(out_ro), _p(out_ci), _itype(out_ci))
    assert rc == 0
    return (out_v if values is not None else None), out_ro, out_ci


def row_idx(row_offsets, index_dtype=None) -> np.ndarray:
    """Rows ordered by stored-entry count, most first, ties by ascending row."""
    ro = _c(row_offsets, np.int32)
    m = len(ro) - 1
    out = np.empty(m, dtype=index_dtype or (np.int16 if m <= 32767 else np.int32))
    rc = lib().oracle_row_idx(m, _p(ro), _p(out), _itype(out))
    assert rc == 0
    return out


def decode(bits: np.ndarray, dt: str) -> np.ndarray:
    b = _c(bits).view(np.uint16)
    out = np.empty(b.shape, dtype=np.float64)
    lib().oracle_decode_array(_p(b), _DT[dt], b.size, _p(out))
    return out


def encode(x: np.ndarray, dt: str) -> np.ndarray:
    xd = _c(x, np.float64)
    out = np.empty(xd.shape, dtype=np.uint16)
    lib().oracle_encode_array(_p(xd), _DT[dt], xd.size, _p(out))
    return out


def to_f64(x: np.ndarray, dt: str) -> np.ndarray:
    """Exact float64 view of stored values (own decoders for 16-bit formats)."""
    if dt in ("f32", "f64"):
        return np.asarray(x, dtype=np.float64)
    return decode(x, dt)


# --------------------------------------------------- sparse linear layer --
#
# The layer S · X^T (S sparse out x in, X^T dense in x tokens) and its
# gradients, the pairing the spops README's operations serve for sparse
# adaptation (csr_add "is used in the RoSA paper"; SDDMM handles RoSA's
# masks) and that the torchsparsegradutils README describes for sparse_mm
# (section "Key Features": gradients keep the sparsity of the matrix; its
# Quick Start multiplies a sparse 2 x 3 matrix into a dense one and calls
# backward).  Written directly from the stored entries in float64: a loss
# L = <G, S · X^T> has dL/dS[r][c] = <G[r], X^T[c]> at every stored (r, c)
# and dL/dX^T = S^T · G.

def _rows_of(row_offsets) -> np.ndarray:
    ro = np.asarray(row_offsets, dtype=np.int64)
    return np.repeat(np.arange(len(ro) - 1), np.diff(ro))


def sparse_linear_forward(m: int, row_offsets, col_idx, values, val_dt: str, xt,
                          x_dt: str) -> np.ndarray:
    """Y^T = S · X^T in float64, one stored entry at a time."""
    v, x = to_f64(values, val_dt), to_f64(xt, x_dt)
    r, c = _rows_of(row_offsets), np.asarray(col_idx, dtype=np.int64)
    yt = np.zeros((m, x.shape[1]), dtype=np.float64)
    for p in range(len(c)):
        yt[r[p]] += v[p] * x[c[p]]
    return yt


def sparse_linear_backward(m: int, n: int, row_offsets, col_idx, values, val_dt: str, xt,
                           dyt, x_dt: str):
    """(dvalues, dX^T) of L = <dY^T, S · X^T>: dvalues[p] = <dY^T[r], X^T[c]>
    for stored entry p = (r, c); dX^T[c] = sum over entries (r, c) of
    v * dY^T[r] (that is S^T · dY^T)."""
    v, x, g = to_f64(values, val_dt), to_f64(xt, x_dt), to_f64(dyt, x_dt)
    r, c = _rows_of(row_offsets), np.asarray(col_idx, dtype=np.int64)
    dv = np.empty(len(c), dtype=np.float64)
    dxt = np.zeros((n, x.shape[1]), dtype=np.float64)
    for p in range(len(c)):
        dv[p] = float(np.dot(g[r[p]], x[c[p]]))
        dxt[c[p]] += v[p] * g[r[p]]
    return dv, dxt


# ------------------------------------------------- conjugate gradients --
# The torchsparsegradutils README lists a CG solver among its built-in
# iterative solvers ("Built-in Iterative Solvers") and calls a generic sparse
# solve with it and a tolerance in its usage example ("Generic solve").  The
# page gives no steps, so this is the method of Hestenes and Stiefel ("Methods
# of Conjugate Gradients for Solving Linear Systems", J. Res. NBS 49, 1952) in
# its usual form: residual r = b - A x, search direction p, step
# alpha = (r.r) / (p.A p), new direction r + beta p with
# beta = (r_new.r_new) / (r.r).  It stops once the recursively updated
# residual satisfies ||r|| <= rtol * ||b|| (compared squared) or after
# max_iter iterations.  Everything is float64; A p is summed entry by entry in
# stored order.

def csr_matvec(m: int, row_offsets, col_idx, values_f64, x) -> np.ndarray:
    """y = A x in float64 (one stored entry at a time, stored order)."""
    r, c = _rows_of(row_offsets), np.asarray(col_idx, dtype=np.int64)
    return np.bincount(r, weights=np.asarray(values_f64) * np.asarray(x)[c], minlength=m)


def cg(m: int, row_offsets, col_idx, values, val_dt: str, b, x0=None, rtol: float = 1e-6,
       max_iter: int = 1000, history: bool = False):
    """Solve A x = b for symmetric positive definite A.  Returns
    (x, iterations, ||r|| / ||b||) and, with history=True, the lists of
    search directions and residuals of every iteration (for the pins)."""
    v = to_f64(values, val_dt)
    b = np.asarray(b, dtype=np.float64).reshape(-1)
    x = np.zeros(m) if x0 is None else np.asarray(x0, dtype=np.float64).reshape(-1).copy()
    r = b - csr_matvec(m, row_offsets, col_idx, v, x)
    p = r.copy()
    rr, bb = float(r @ r), float(b @ b)
    thr = rtol * rtol * bb
    k = 0
    ps, rs = [p.copy()], [r.copy()]
    while k < max_iter and rr > thr:
        q = csr_matvec(m, row_offsets, col_idx, v, p)
        alpha = rr / float(p @ q)
        x += alpha * p
        r -= alpha * q
        rr_new = float(r @ r)
        p = r + (rr_new / rr) * p
        rr = rr_new
        k += 1
        if history:
            ps.append(p.copy())
            rs.append(r.copy())
    rel = float(np.sqrt(rr / bb)) if bb > 0 else 0.0
    if history:
        return x, k, rel, ps, rs
    return x, k, rel


# ------------------------------------------------------------ masked Adam --
# The SparseAdam page (tensorplay.optim.sparse_adam) describes a masked Adam:
# only the positions where the gradient is materialized have their first and
# second moments and their parameter updated; every other position keeps its
# moments and value, and a materialized gradient of zero still counts.  The
# page names Adam and its arguments (lr, betas, eps, maximize) but not the
# update itself, so the step is Adam's (Kingma and Ba, "Adam: A Method for
# Stochastic Optimization", 2015, Algorithm 1) in the form that paper gives
# for efficiency at the end of its Section 2, with one step counter t for the
# whole parameter:
#   m <- beta1 m + (1 - beta1) g,  v <- beta2 v + (1 - beta2) g^2,
#   alpha_t = lr sqrt(1 - beta2^t) / (1 - beta1^t),
#   theta <- theta - alpha_t m / (sqrt(v) + eps)
# at the materialized positions (g negated when maximizing).  float64
# throughout; the new parameter is returned in float64 (rounded to the
# parameter's format by the caller when comparing).

def masked_adam(values, val_dt: str, grad, grad_dt: str, exp_avg, exp_avg_sq, step: int,
                lr: float, beta1: float, beta2: float, eps: float, maximize: bool = False,
                positions=None):
    """One masked Adam step on the CSR value vector.  `grad` holds the
    gradient of every position (positions=None) or of the listed positions
    only (unique indices into values).  Returns (values, exp_avg,
    exp_avg_sq) as new float64 arrays; unlisted positions are copied."""
    theta = to_f64(values, val_dt).copy()
    m = np.asarray(exp_avg, dtype=np.float64).copy()
    v = np.asarray(exp_avg_sq, dtype=np.float64).copy()
    g = to_f64(grad, grad_dt)
    idx = np.arange(len(theta)) if positions is None else np.asarray(positions, np.int64)
    if maximize:
        g = -g
    a_t = lr * np.sqrt(1.0 - beta2 ** step) / (1.0 - beta1 ** step)
    for j, i in enumerate(idx):
        m[i] = beta1 * m[i] + (1.0 - beta1) * g[j]
        v[i] = beta2 * v[i] + (1.0 - beta2) * g[j] * g[j]
        theta[i] = theta[i] - a_t * m[i] / (np.sqrt(v[i]) + eps)
    return theta, m, v


# ------------------------------------------------- delta-compressed rows --
# The UST news page (section "Formatos menos comuns") converts a matrix to a
# 2-bit delta-compressed format: rows stay a dense level, and inside a row
# the column coordinates are stored as differences (2 bits each) instead of
# indices; its MACKO experiment (section "Performance") runs SpMV on that
# format for low sparsity, with padding that stops at the end of each row.
# The page shows no layout, so this is the reading taken:
#   * each stored entry carries a 2-bit code d: its column is the previous
#     entry's column + d + 1 (the first entry of a row counts from column -1);
#   * a gap larger than 4 is bridged by zero-valued padding entries, each 4
#     columns after the previous entry, until the rest of the gap is <= 4;
#   * nothing is padded after a row's last entry (empty rows stay empty);
#   * enc_offsets[m+1] (int32) delimit the rows in the encoded stream; codes
#     are packed 16 per uint32, entry e in bits 2(e mod 16)..2(e mod 16)+1 of
#     word e // 16; values keep the matrix's format.
# Columns inside a row must be distinct; they are taken in ascending order.

def delta_encode(m: int, n: int, row_offsets, col_idx, values, val_dt: str):
    """CSR -> (enc_offsets[m+1] int32, codes uint32[ceil(E/16)], enc_values[E])
    with values in the storage convention of val_dt (padding = +0).

    Per row, with columns sorted and c_{-1} = -1, entry k has the gap
    g = c_k - c_{k-1} >= 1; it is preceded by p = (g - 1) // 4 padding
    entries (code 3, four columns each) and carries code g - 1 - 4p."""
    ro = np.asarray(row_offsets, np.int64)
    ci = np.asarray(col_idx, np.int64)
    vals = np.asarray(values)
    rows = _rows_of(ro)
    order = np.lexsort((ci, rows))            # by row, then column
    c, v, r = ci[order], vals[order], rows[order]
    prev = np.empty_like(c)
    prev[1:] = c[:-1]
    first = np.ones(len(c), bool)
    first[1:] = r[1:] != r[:-1]
    prev[first] = -1
    gap = c - prev
    pad = (gap - 1) // 4
    # position of each entry in the encoded stream: its paddings come first
    pos = np.cumsum(pad + 1) - 1
    E = int(pos[-1]) + 1 if len(pos) else 0
    code = np.full(E, 3, np.uint32)
    code[pos] = (gap - 1 - 4 * pad).astype(np.uint32)
    ev = np.zeros(E, dtype=vals.dtype)
    ev[pos] = v
    per_row = np.bincount(r, weights=pad + 1, minlength=m).astype(np.int64)
    enc_off = np.concatenate([[0], np.cumsum(per_row)]).astype(np.int32)
    words = np.zeros((E + 15) // 16, np.uint32)
    shifts = (2 * (np.arange(E) % 16)).astype(np.uint32)
    np.bitwise_or.at(words, np.arange(E) // 16, code << shifts)
    return enc_off, words, ev


def delta_decode(m: int, enc_offsets, codes, enc_values):
    """Encoded rows -> CSR (row_offsets, col_idx int64, values) holding every
    encoded entry, padding zeros included: a column is the running sum of
    (code + 1) along its row, starting from -1."""
    eo = np.asarray(enc_offsets, np.int64)
    words = np.asarray(codes, np.uint32)
    E = int(eo[-1])
    e = np.arange(E)
    code = (words[e // 16] >> (2 * (e % 16)).astype(np.uint32)) & np.uint32(3)
    run = np.cumsum(code.astype(np.int64) + 1)
    row_start = np.repeat(eo[:-1], np.diff(eo))
    before = np.concatenate([[0], run])[row_start]     # steps taken before the row
    cols = run - before - 1
    return eo.astype(np.int32), cols, np.asarray(enc_values)


def delta_spmv(m: int, enc_offsets, codes, enc_values, val_dt: str, x, x_dt: str) -> np.ndarray:
    """y = A x in float64 for A in the delta format, from the decoded entries."""
    eo, cols, ev = delta_decode(m, enc_offsets, codes, enc_values)
    return csr_matvec(m, eo, cols, to_f64(ev, val_dt), to_f64(np.asarray(x).reshape(-1), x_dt))
