"""The allocation-free csr_transpose (spops_csr_transpose_noalloc, scratch in
a fixed device array inside the library) against the workspace entry point
(spops_csr_transpose), bit for bit, on calls in a row whose second input is
smaller than the first, and the same input again after it."""
import ctypes

import numpy as np
import pytest
import torch

import unstructured_sparse_linear_amd as S
from unstructured_sparse_linear_amd import gen
from unstructured_sparse_linear_amd import spops as SP
from helpers import csr_dev

pytestmark = pytest.mark.gpu


def transpose(A, noalloc):
    v, ro, ci = csr_dev(A)
    m, n = A.m, A.n
    d = SP.csr_desc(v, ro, None, ci, m, n)
    oit = torch.int16 if m <= 32767 else torch.int32
    out_v = torch.full((A.nnz,), 7, dtype=v.dtype, device="cuda")
    out_ro = torch.full((n + 1,), -1, dtype=torch.int32, device="cuda")
    out_ci = torch.full((A.nnz,), -1, dtype=oit, device="cuda")
    L = SP.lib()
    if noalloc:
        st = L.spops_csr_transpose_noalloc(ctypes.byref(d), out_v.data_ptr(), out_ro.data_ptr(),
                                           out_ci.data_ptr(), SP._IT[oit], SP._stream(ro))
    else:
        ws = S.csr_transpose_workspace(m, n, A.nnz, "cuda")
        st = L.spops_csr_transpose(ctypes.byref(d), out_v.data_ptr(), out_ro.data_ptr(),
                                   out_ci.data_ptr(), SP._IT[oit], ws.data_ptr(), ws.numel(),
                                   SP._stream(ro))
    assert st == 0, st
    torch.cuda.synchronize()
    return [t.cpu().view(torch.int16 if t.dtype == torch.bfloat16 else t.dtype).numpy()
            for t in (out_v, out_ro, out_ci)]


def test_noalloc_transpose_matches_workspace_entry_point():
    big = gen.random_csr(31, 3000, 6000, 0.04, "bf16", shuffle_within_rows=True)
    small = gen.random_csr(32, 700, 40000, 0.003, "f32", empty_row_frac=0.2)
    for A in (big, small, big):
        got = transpose(A, True)
        ref = transpose(A, False)
        for g, r in zip(got, ref):
            assert g.dtype == r.dtype and np.array_equal(g, r)
