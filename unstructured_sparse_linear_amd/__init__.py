"""Unstructured CSR sparse-dense products on AMD Instinct MI355X (gfx950).

SpMM, SDDMM (general and structure-aware), csr_add and csr_transpose over the
CSR layout of the spops README (values, int32 row_offsets, int16/int32
col_idx, nnz-sorted row_idx).  The work runs in hand-written HIP kernels
behind the C ABI in include/spops.h (libspops.so); this package only
marshals torch tensors into that ABI.  Nothing here falls back to another
implementation: calls raise if libspops.so is missing.
"""
from .adapter import MaskedAdam, SparseAdapter, SparsePattern, sparse_linear  # noqa: F401
from .spops import (  # noqa: F401
    SddmmPlan,
    SpmmPlan,
    DeltaMatrix,
    InvalidCSR,
    SpopsError,
    cg,
    delta_encode,
    delta_spmv,
    clear_plan_caches,
    csr_add,
    csr_transpose,
    csr_transpose_permutation,
    csr_transpose_workspace,
    lib,
    masked_adam,
    option,
    permute_values,
    sddmm,
    set_option,
    sort_rows_by_nnz,
    sort_rows_workspace,
    spmm,
    validate_csr,
)

__all__ = ["spmm", "sddmm", "csr_add", "csr_transpose", "sort_rows_by_nnz", "SpmmPlan",
           "SddmmPlan", "SpopsError", "lib", "clear_plan_caches", "csr_transpose_workspace",
           "sort_rows_workspace", "SparsePattern", "SparseAdapter", "sparse_linear", "cg",
           "masked_adam", "MaskedAdam", "DeltaMatrix", "delta_encode", "delta_spmv",
           "option", "set_option", "validate_csr", "InvalidCSR", "csr_transpose_permutation",
           "permute_values"]
