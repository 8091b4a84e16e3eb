"""C ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects invalid arguments before touching the device.

Pointers below are never dereferenced: every call here fails host-side
validation, so nothing is launched.
"""
import ctypes
import os
import re
import subprocess

import pytest

from unstructured_sparse_linear_amd import spops as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spops.h")
FAKE = 0x10000  # placeholder address; validation fails before any use


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(S.LIB_PATH):
        from unstructured_sparse_linear_amd import build
        build.build()
    return S.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spops_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_four_operations():
    names = declared_functions()
    for f in ("spops_spmm", "spops_sddmm", "spops_csr_add", "spops_csr_transpose",
              "spops_sort_rows_by_nnz"):
        assert f in names


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), f"{name} declared in spops.h but not exported"
    out = subprocess.run(["nm", "-D", "--defined-only", S.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = set(re.findall(r"\bT (spops_\w+)", out))
    assert set(declared_functions()) <= exported


def test_version_and_status_strings(L):
    assert L.spops_abi_version() == 1
    for code in range(12):
        assert L.spops_status_string(code) != b"unknown status"
    assert L.spops_status_string(0) == b"ok"


def desc(rows=4, cols=4, nnz=4, val_type=0, col_type=0, ri_type=0, values=FAKE, ro=FAKE,
         ri=FAKE, col=FAKE):
    d = S.CSRDesc()
    d.rows, d.cols, d.nnz = rows, cols, nnz
    d.val_type, d.col_type, d.row_idx_type = val_type, col_type, ri_type
    d.values, d.row_offsets, d.row_idx, d.col_idx = values, ro, ri, col
    return d


def spmm(L, d, b_type=0, N=8, ldb=8, C=FAKE, c_type=0, ldc=8, plan=None, ws=None, wsb=0):
    return L.spops_spmm(ctypes.byref(d), FAKE, b_type, N, ldb, C, c_type, ldc, plan, ws, wsb,
                        None)


def test_spmm_rejects_bad_arguments(L):
    assert L.spops_spmm(None, FAKE, 0, 8, 8, FAKE, 0, 8, None, None, 0, None) == 1
    assert spmm(L, desc(cols=40000, col_type=0)) == 4        # int16 cannot address 40000
    assert spmm(L, desc(rows=40000, ri_type=0)) == 4
    assert spmm(L, desc(), b_type=1) == 3                     # B dtype != values dtype
    assert spmm(L, desc(val_type=1), b_type=1, c_type=2) == 3  # C must be f32 or B's dtype
    assert spmm(L, desc(val_type=7), b_type=7) == 3
    assert spmm(L, desc(), ldb=4) == 2                        # ldb < N
    assert spmm(L, desc(), ldc=4) == 2
    assert spmm(L, desc(rows=-1)) == 2
    assert spmm(L, desc(rows=0, nnz=3)) == 2                  # entries without rows
    assert spmm(L, desc(ro=None)) == 1
    assert spmm(L, desc(ri=None)) == 1
    assert spmm(L, desc(values=None)) == 1
    assert spmm(L, desc(), C=None) == 1
    assert spmm(L, desc(), N=0) == 0                          # nothing to do


def test_sddmm_rejects_bad_arguments(L):
    d = desc(values=None)

    def f(dd, A, K, lda, BT, ldbt, it, out, ot, backend):
        return L.spops_sddmm(ctypes.byref(dd), A, K, lda, BT, ldbt, it, out, ot, backend, None,
                             None, 0, None)
    assert f(d, FAKE, 8, 8, FAKE, 8, 1, FAKE, 2, 0) == 3  # out bf16, in f16
    assert f(d, FAKE, 8, 4, FAKE, 8, 1, FAKE, 0, 0) == 2  # lda < K
    assert f(d, FAKE, 8, 8, FAKE, 8, 1, FAKE, 0, 9) == 6  # backend
    assert f(d, None, 8, 8, FAKE, 8, 1, FAKE, 0, 1) == 1
    assert f(d, FAKE, 8, 8, FAKE, 8, 1, None, 0, 1) == 1
    assert f(desc(cols=70000, col_type=0), FAKE, 8, 8, FAKE, 8, 1, FAKE, 0, 1) == 4
    assert f(desc(nnz=0, col=None), FAKE, 8, 8, FAKE, 8, 1, None, 0, 1) == 0


def test_sddmm_workspace_size_contract(L):
    b = ctypes.c_size_t()

    def ws(d, K, it, backend, plan=None):
        assert L.spops_sddmm_workspace_size(ctypes.byref(d), K, it, backend, plan,
                                            ctypes.byref(b)) == 0
        return b.value
    big = desc(rows=4096, cols=11008, nnz=450000, values=None)
    assert ws(big, 2048, 1, 1) == 0                      # general backend: none
    assert ws(big, 2048, 0, 0) == 0                      # f32: no dense tiles, none
    assert ws(big, 2044, 1, 0) == 0                      # K not a multiple of 8: none
    assert ws(big, 0, 1, 0) == 0
    assert ws(desc(nnz=0, col=None, values=None), 64, 1, 0) == 0
    # without a plan the structure-aware call builds one in the workspace: at
    # least the entry arrays (position, in-tile coordinates, sort keys)
    need = ws(big, 2048, 1, 0)
    assert need >= 4 * 450000 * 4
    assert ws(big, 2048, 2, 0) == need                   # same for bf16 and any K
    assert ws(big, 64, 1, 0) == need
    assert L.spops_sddmm_workspace_size(ctypes.byref(big), 2048, 1, 7, None,
                                        ctypes.byref(b)) == 6
    assert L.spops_sddmm_workspace_size(ctypes.byref(big), -1, 1, 0, None,
                                        ctypes.byref(b)) == 2
    # an execute call without a plan and with too little workspace is refused
    # before anything is launched
    f = L.spops_sddmm
    args = (FAKE, 2048, 2048, FAKE, 2048, 1, FAKE, 0, 0, None)
    assert f(ctypes.byref(big), *args, None, 0, None) == 5
    assert f(ctypes.byref(big), *args, FAKE, need - 1, None) == 5
    assert f(ctypes.byref(big), *args, FAKE + 16, need, None) == 5   # not 256-byte aligned


def test_options_round_trip(L):
    v = ctypes.c_int64()
    for opt in range(6):
        assert L.spops_get_option(opt, ctypes.byref(v)) == 0 and v.value == 0
        assert L.spops_set_option(opt, 3) == 0
        assert L.spops_get_option(opt, ctypes.byref(v)) == 0 and v.value == 3
        assert L.spops_set_option(opt, 0) == 0
    assert L.spops_set_option(6, 1) == 6 and L.spops_set_option(-1, 1) == 6
    assert L.spops_set_option(0, -1) == 9
    assert L.spops_get_option(0, None) == 1
    assert S.set_option("sddmm_splits", 4) == 0
    with S.option("sddmm_splits", 2):
        assert L.spops_get_option(4, ctypes.byref(v)) == 0 and v.value == 2
    assert S.set_option("sddmm_splits", 0) == 4


def test_csr_add_rejects_bad_arguments(L):
    f = L.spops_csr_add
    assert f(ctypes.byref(desc()), FAKE, 1, 4, None) == 3     # W dtype != values dtype
    assert f(ctypes.byref(desc()), FAKE, 0, 3, None) == 2     # ldw < cols
    assert f(ctypes.byref(desc()), None, 0, 4, None) == 1
    # row_idx is not used by csr_add: its absence is not an error
    assert f(ctypes.byref(desc(ri=None, ri_type=9)), None, 0, 4, None) == 1
    assert f(ctypes.byref(desc(ri=None, nnz=0, col=None, values=None)), None, 0, 4, None) == 0


def test_validate_rejects_bad_arguments(L):
    b = ctypes.c_size_t()
    assert L.spops_validate_csr_workspace_size(100, 50, 400, ctypes.byref(b)) == 0
    assert b.value > 0
    assert L.spops_validate_csr_workspace_size(-1, 50, 400, ctypes.byref(b)) == 2
    f = L.spops_validate_csr
    fd = ctypes.c_uint32(7)
    assert f(ctypes.byref(desc()), 1, None, 0, ctypes.byref(fd), None) == 5
    assert fd.value == 0
    assert f(ctypes.byref(desc()), 1, FAKE, 1, None, None) == 5
    assert f(ctypes.byref(desc(cols=40000)), 1, FAKE, 1 << 30, None, None) == 4
    assert f(ctypes.byref(desc(ro=None)), 1, FAKE, 1 << 30, None, None) == 1


def test_transpose_noalloc_limit(L):
    b = ctypes.c_size_t()
    assert L.spops_csr_transpose_noalloc_limit(ctypes.byref(b)) == 0
    assert b.value == 32 << 20
    assert L.spops_csr_transpose_noalloc_limit(None) == 1
    need = ctypes.c_size_t()
    f = L.spops_csr_transpose_noalloc
    # an input whose transpose needs more scratch than the array holds is
    # refused before anything is launched
    big = desc(rows=123440, cols=123440, nnz=3085894, ri_type=1, col_type=1)
    assert L.spops_csr_transpose_workspace_size(123440, 123440, 3085894,
                                                ctypes.byref(need)) == 0
    assert need.value > b.value
    assert f(ctypes.byref(big), FAKE, FAKE, FAKE, 1, None) == 5
    assert f(ctypes.byref(desc(rows=40000, ri_type=1)), FAKE, FAKE, FAKE, 0, None) == 4
    assert f(ctypes.byref(desc()), FAKE, None, FAKE, 0, None) == 1


def test_transpose_and_sort_reject_bad_arguments(L):
    b = ctypes.c_size_t()
    assert L.spops_csr_transpose_workspace_size(4, 4, 4, ctypes.byref(b)) == 0 and b.value > 0
    f = L.spops_csr_transpose
    assert f(ctypes.byref(desc()), FAKE, FAKE, FAKE, 0, FAKE, b.value - 1, None) == 5
    assert f(ctypes.byref(desc()), FAKE, FAKE, FAKE, 0, None, b.value, None) == 5
    assert f(ctypes.byref(desc(rows=40000, ri_type=1)), FAKE, FAKE, FAKE, 0, FAKE, 1 << 30,
             None) == 4                                       # transposed indices need int32
    assert f(ctypes.byref(desc()), FAKE, None, FAKE, 0, FAKE, b.value, None) == 1
    assert L.spops_sort_rows_by_nnz_workspace_size(100, 50, ctypes.byref(b)) == 0
    g = L.spops_sort_rows_by_nnz
    assert g(FAKE, 100, 50, FAKE, 0, FAKE, b.value - 1, None) == 5
    assert g(FAKE, 40000, 50, FAKE, 0, FAKE, 1 << 30, None) == 4
    assert g(None, 100, 50, FAKE, 0, FAKE, b.value, None) == 1
    assert g(FAKE, 0, 50, None, 0, None, 0, None) == 0


def test_transpose_permutation_and_permute_reject_bad_arguments(L):
    b = ctypes.c_size_t()
    assert L.spops_csr_transpose_permutation_workspace_size(4, 4, 4, ctypes.byref(b)) == 0
    t = ctypes.c_size_t()
    assert L.spops_csr_transpose_workspace_size(4, 4, 4, ctypes.byref(t)) == 0
    assert b.value >= t.value + 4 * 4                      # the transpose's, plus the indices
    assert L.spops_csr_transpose_permutation_workspace_size(4, 4, -1, ctypes.byref(b)) == 2
    assert L.spops_csr_transpose_permutation_workspace_size(4, 4, 4, None) == 1
    assert L.spops_csr_transpose_permutation_workspace_size(4, 4, 4, ctypes.byref(b)) == 0
    f = L.spops_csr_transpose_permutation
    big = 1 << 20
    assert f(ctypes.byref(desc()), FAKE, FAKE, FAKE, 0, FAKE, b.value - 1, None) == 5
    assert f(ctypes.byref(desc()), FAKE, FAKE, FAKE, 0, FAKE + 16, big, None) == 5  # alignment
    assert f(ctypes.byref(desc()), None, FAKE, FAKE, 0, FAKE, big, None) == 1
    assert f(ctypes.byref(desc()), FAKE, None, FAKE, 0, FAKE, big, None) == 1
    assert f(ctypes.byref(desc()), FAKE, FAKE, FAKE, 7, FAKE, big, None) == 3
    assert f(ctypes.byref(desc(rows=40000, ri_type=1)), FAKE, FAKE, FAKE, 0, FAKE, 1 << 30,
             None) == 4                                       # transposed indices need int32
    g = L.spops_permute_values
    assert g(FAKE, 10, 7, FAKE, 10, FAKE, None) == 3          # unknown dtype
    assert g(FAKE, 10, 1, FAKE, -1, FAKE, None) == 2
    assert g(FAKE, -1, 1, FAKE, 10, FAKE, None) == 2
    assert g(FAKE, 10, 1, None, 10, FAKE, None) == 1
    assert g(FAKE, 10, 1, FAKE, 10, None, None) == 1
    assert g(None, 0, 1, None, 0, None, None) == 0            # nothing to do


def test_python_binding_validates_before_the_library():
    import torch
    cpu = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(ValueError):
        S.sort_rows_by_nnz(cpu, 4)                            # not a GPU tensor
    with pytest.raises(ValueError):
        S.csr_desc(None, torch.zeros(8, dtype=torch.int32)[::2], None,
                   torch.zeros(3, dtype=torch.int16), 3, 3)   # non-contiguous


def test_product_path_does_not_reference_the_oracle():
    pkg = os.path.join(ROOT, "unstructured_sparse_linear_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), f
                assert "liboracle" not in text and "oracle.c" not in text, f
