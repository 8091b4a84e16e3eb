"""Python binding of libspops (ctypes).  Argument marshalling only: every step
of every operation runs in the HIP kernels behind the C ABI in
include/spops.h; PyTorch provides device memory and the current stream.

The signatures follow the spops README (IST-DASLab), sections "Sparse
Addition", "Sparse Matrix Multiplication (SpMM)", "Sampled Dense-Dense Matrix
Multiplication (SDDMM)" and "CSR Transpose"; section "Important Notes" asks
for contiguous inputs, int32 row offsets and int16 for the other index lists
(int32 is accepted where 16 bits cannot address the extent).
"""
from __future__ import annotations

import ctypes
import os
from collections import OrderedDict
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspops.so")

F32, F16, BF16 = 0, 1, 2
I16, I32 = 0, 1
STRUCTURE_AWARE, GENERAL = 0, 1
_DT = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}
_IT = {torch.int16: I16, torch.int32: I32}
_BACKENDS = {"structure_aware": STRUCTURE_AWARE, "sputnik": GENERAL, "general": GENERAL}

STATUS = {0: "ok", 1: "null pointer", 2: "shape", 3: "dtype", 4: "index width",
          5: "workspace", 6: "unsupported", 7: "plan mismatch", 8: "HIP error",
          9: "argument out of range", 10: "column order", 11: "invalid index data"}
INVALID_FLAGS = {1: "offsets", 2: "column", 4: "row_idx", 8: "duplicate"}
# Set SPOPS_VALIDATE=1 in the environment (read once, when this module is
# imported) to run validate_csr on the sparse operands of every spmm, sddmm,
# csr_add and csr_transpose call of this binding before the operation
# (slow: it synchronizes; for debugging).
VALIDATE = os.environ.get("SPOPS_VALIDATE", "") == "1"


class SpopsError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed with status {code} ({msg})")
        self.code = code


class CSRDesc(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("nnz", ctypes.c_int64),
                ("val_type", ctypes.c_int), ("col_type", ctypes.c_int),
                ("row_idx_type", ctypes.c_int), ("values", ctypes.c_void_p),
                ("row_offsets", ctypes.c_void_p), ("row_idx", ctypes.c_void_p),
                ("col_idx", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libspops.so; raises if it was not built (no fallback exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libspops.so not found at {LIB_PATH}; build it with "
                               "`python -m unstructured_sparse_linear_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
        P = ctypes.POINTER
        cp = P(CSRDesc)
        sigs = {
            "spops_abi_version": ([], i32),
            "spops_status_string": ([i32], ctypes.c_char_p),
            "spops_spmm": ([cp, vp, i32, i64, i64, vp, i32, i64, vp, vp, sz, vp], i32),
            "spops_spmm_plan_create": ([cp, vp, P(vp)], i32),
            "spops_spmm_plan_destroy": ([vp], i32),
            "spops_spmm_workspace_size": ([vp, i64, P(sz)], i32),
            "spops_spmm_plan_info": ([vp, P(i64), P(i64), P(i64)], i32),
            "spops_sddmm": ([cp, vp, i64, i64, vp, i64, i32, vp, i32, i32, vp, vp, sz, vp],
                            i32),
            "spops_sddmm_workspace_size": ([cp, i64, i32, i32, vp, P(sz)], i32),
            "spops_set_option": ([i32, i64], i32),
            "spops_get_option": ([i32, P(i64)], i32),
            "spops_sddmm_plan_create": ([cp, ctypes.c_double, vp, P(vp)], i32),
            "spops_sddmm_plan_destroy": ([vp], i32),
            "spops_sddmm_plan_info": ([vp, P(i64), P(i64), P(i64), P(i64), P(i64)], i32),
            "spops_csr_add": ([cp, vp, i32, i64, vp], i32),
            "spops_csr_transpose_workspace_size": ([i64, i64, i64, P(sz)], i32),
            "spops_csr_transpose": ([cp, vp, vp, vp, i32, vp, sz, vp], i32),
            "spops_csr_transpose_noalloc": ([cp, vp, vp, vp, i32, vp], i32),
            "spops_csr_transpose_permutation_workspace_size": ([i64, i64, i64, P(sz)], i32),
            "spops_csr_transpose_permutation": ([cp, vp, vp, vp, i32, vp, sz, vp], i32),
            "spops_permute_values": ([vp, i64, i32, vp, i64, vp, vp], i32),
            "spops_validate_csr_workspace_size": ([i64, i64, i64, P(sz)], i32),
            "spops_validate_csr": ([cp, i32, vp, sz, P(ctypes.c_uint32), vp], i32),
            "spops_csr_transpose_noalloc_limit": ([P(sz)], i32),
            "spops_sort_rows_by_nnz_workspace_size": ([i64, i64, P(sz)], i32),
            "spops_sort_rows_by_nnz": ([vp, i64, i64, vp, i32, vp, sz, vp], i32),
            "spops_cg_workspace_size": ([cp, vp, P(sz)], i32),
            "spops_delta_size_workspace": ([i64, P(sz)], i32),
            "spops_delta_size": ([cp, vp, P(i64), vp, sz, vp], i32),
            "spops_delta_encode": ([cp, vp, i64, vp, vp, vp], i32),
            "spops_delta_spmv": ([i64, i64, vp, i64, vp, vp, i32, vp, vp, i32, vp], i32),
            "spops_masked_adam": ([vp, i32, i64, vp, vp, i64, vp, vp, i64, ctypes.c_double,
                                   ctypes.c_double, ctypes.c_double, ctypes.c_double, i32, vp],
                                  i32),
            "spops_cg": ([cp, vp, vp, ctypes.c_double, i64, i64, vp, vp, sz, P(i64),
                          P(ctypes.c_double), vp], i32),
        }
        for name, (args, res) in sigs.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _check(fn: str, code: int):
    if code != 0:
        msg = lib().spops_status_string(code)
        raise SpopsError(fn, code, msg.decode() if msg else STATUS.get(code, "?"))


def _stream(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None or t.numel() == 0 else t.data_ptr()


def _require(t: torch.Tensor, name: str, dtypes=None):
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor, got device {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name} must have dtype in {dtypes}, got {t.dtype}")


def _index_type(t: torch.Tensor, name: str, extent: int) -> int:
    _require(t, name, (torch.int16, torch.int32))
    if t.dtype == torch.int16 and extent > 32767:
        raise ValueError(f"{name} is int16 but must address {extent} entries; use int32")
    return _IT[t.dtype]


def csr_desc(values, row_offsets, row_idx, col_idx, m: int, n: int) -> CSRDesc:
    """Marshal a CSR given as tensors into the C descriptor."""
    _require(row_offsets, "row_offsets", (torch.int32,))
    if row_offsets.numel() != m + 1:
        raise ValueError(f"row_offsets must have m+1 = {m + 1} entries")
    nnz = col_idx.numel()
    d = CSRDesc()
    d.rows, d.cols, d.nnz = m, n, nnz
    d.col_type = _index_type(col_idx, "col_idx", n)
    d.row_offsets = row_offsets.data_ptr()
    d.col_idx = _ptr(col_idx)
    if values is not None:
        _require(values, "values", tuple(_DT))
        if values.numel() != nnz:
            raise ValueError("values and col_idx must have the same length")
        d.val_type = _DT[values.dtype]
        d.values = _ptr(values)
    if row_idx is not None:
        d.row_idx_type = _index_type(row_idx, "row_idx", m)
        if row_idx.numel() != m:
            raise ValueError(f"row_idx must have m = {m} entries")
        d.row_idx = _ptr(row_idx)
    return d


# ------------------------------------------------------------- plans -----

class SpmmPlan:
    """Row-splitting schedule of one CSR pattern (row_offsets + row_idx)."""

    def __init__(self, row_offsets: torch.Tensor, row_idx: torch.Tensor,
                 col_idx: torch.Tensor, n: int):
        m = row_offsets.numel() - 1
        self._keep = (row_offsets, row_idx)
        d = csr_desc(None, row_offsets, row_idx, col_idx, m, n)
        h = ctypes.c_void_p()
        _check("spops_spmm_plan_create", lib().spops_spmm_plan_create(
            ctypes.byref(d), _stream(row_offsets), ctypes.byref(h)))
        self.handle = h
        self._ws = {}

    def info(self):
        s, c, mx = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        _check("spops_spmm_plan_info", lib().spops_spmm_plan_info(
            self.handle, ctypes.byref(s), ctypes.byref(c), ctypes.byref(mx)))
        return {"split_rows": s.value, "chunks": c.value, "max_row_nnz": mx.value}

    def workspace(self, N: int, device) -> Optional[torch.Tensor]:
        # asked every call (cheap), the buffer kept per N and grown when a
        # call needs more
        b = ctypes.c_size_t()
        _check("spops_spmm_workspace_size",
               lib().spops_spmm_workspace_size(self.handle, N, ctypes.byref(b)))
        if b.value == 0:
            return None
        ws = self._ws.get(N)
        if ws is None or ws.numel() < b.value:
            ws = torch.empty(b.value, dtype=torch.uint8, device=device)
            self._ws[N] = ws
        return ws

    def __del__(self):
        h = getattr(self, "handle", None)
        if h and _lib is not None:
            _lib.spops_spmm_plan_destroy(h)
            self.handle = None


class SddmmPlan:
    """Dense-row / dense-column detection and entry partition of one mask."""

    def __init__(self, row_offsets: torch.Tensor, col_idx: torch.Tensor, m: int, n: int,
                 tau: Optional[float] = None):
        self._keep = (row_offsets, col_idx)
        d = csr_desc(None, row_offsets, None, col_idx, m, n)
        h = ctypes.c_void_p()
        if tau is None:
            tau = 0.0  # the library's default density threshold
        _check("spops_sddmm_plan_create", lib().spops_sddmm_plan_create(
            ctypes.byref(d), ctypes.c_double(tau), _stream(row_offsets), ctypes.byref(h)))
        self.handle = h

    def info(self):
        v = [ctypes.c_int64() for _ in range(5)]
        _check("spops_sddmm_plan_info",
               lib().spops_sddmm_plan_info(self.handle, *[ctypes.byref(x) for x in v]))
        keys = ("dense_rows", "dense_cols", "tiled_nnz", "rest_nnz", "tiles")
        return dict(zip(keys, (x.value for x in v)))

    def __del__(self):
        h = getattr(self, "handle", None)
        if h and _lib is not None:
            _lib.spops_sddmm_plan_destroy(h)
            self.handle = None


class _PlanCache:
    def __init__(self, cap: int = 16):
        self.cap = cap
        self.d: "OrderedDict[tuple, object]" = OrderedDict()

    def get(self, key, make, keep=()):
        """The plan cached under key, or a new one from make().  The tensors
        the key was made from (keep) are held with the plan: while they live
        no other tensor can take their address, so a key built from data
        pointers (and version counters) never matches a different tensor."""
        if key in self.d:
            self.d.move_to_end(key)
            return self.d[key][0]
        v = make()
        self.d[key] = (v, tuple(keep))
        if len(self.d) > self.cap:
            self.d.popitem(last=False)
        return v

    def clear(self):
        self.d.clear()


_spmm_plans = _PlanCache()
_sddmm_plans = _PlanCache()


_ws_pool = {}


def _workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    """Scratch device memory reused across calls of the same size on the same
    stream (calls on one stream run in order, so they never overlap)."""
    if nbytes == 0:
        return None
    key = (str(device), nbytes, torch.cuda.current_stream(device).cuda_stream)
    if key not in _ws_pool:
        _ws_pool[key] = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return _ws_pool[key]


def _tkey(t: torch.Tensor):
    return (t.data_ptr(), t.numel(), t.dtype, t._version)


def clear_plan_caches():
    _spmm_plans.clear()
    _sddmm_plans.clear()
    _ws_pool.clear()


# ------------------------------------------------------------ validation --

class InvalidCSR(ValueError):
    def __init__(self, findings: int):
        names = [v for k, v in INVALID_FLAGS.items() if findings & k]
        super().__init__(f"invalid CSR index data: {', '.join(names)}")
        self.findings = findings


def validate_csr(row_offsets: torch.Tensor, col_indices: torch.Tensor, m: int, n: int,
                 row_indices: Optional[torch.Tensor] = None,
                 check_duplicates: bool = True) -> int:
    """Checks the CSR's index data on the device (include/spops.h,
    spops_validate_csr); returns 0 or raises InvalidCSR with the failed
    checks.  Synchronizes."""
    d = csr_desc(None, row_offsets, row_indices, col_indices, m, n)
    wb = ctypes.c_size_t()
    _check("spops_validate_csr_workspace_size", lib().spops_validate_csr_workspace_size(
        m, n, d.nnz, ctypes.byref(wb)))
    ws = torch.empty(wb.value, dtype=torch.uint8, device=row_offsets.device)
    f = ctypes.c_uint32()
    st = lib().spops_validate_csr(ctypes.byref(d), int(bool(check_duplicates)), ws.data_ptr(),
                                  ws.numel(), ctypes.byref(f), _stream(row_offsets))
    if st == 11:
        raise InvalidCSR(int(f.value))
    _check("spops_validate_csr", st)
    return 0


def _maybe_validate(row_offsets, col_indices, m, n, row_indices=None):
    if VALIDATE:
        validate_csr(row_offsets, col_indices, m, n, row_indices)


# --------------------------------------------------------------- options --

OPTIONS = {"spmm_pointer_loads": 0, "transpose_force_scan": 1, "transpose_wide_records": 2,
           "sddmm_buckets": 3, "sddmm_splits": 4, "sddmm_rest_split": 5}


def set_option(name: str, value: int) -> int:
    """Sets a process-wide switch of the library (include/spops.h,
    spops_set_option) and returns its previous value."""
    o = OPTIONS[name]
    old = ctypes.c_int64()
    _check("spops_get_option", lib().spops_get_option(o, ctypes.byref(old)))
    _check("spops_set_option", lib().spops_set_option(o, int(value)))
    return old.value


class option:
    """Context manager: `with option("sddmm_splits", 4): ...`."""

    def __init__(self, name: str, value: int):
        self.name, self.value = name, value

    def __enter__(self):
        self.old = set_option(self.name, self.value)
        return self

    def __exit__(self, *exc):
        set_option(self.name, self.old)
        return False


# ------------------------------------------------------------ operations --

def spmm(A_val: torch.Tensor, A_row_offsets: torch.Tensor, A_row_indices: torch.Tensor,
         A_col_indices: torch.Tensor, B: torch.Tensor, m: int,
         out_dtype: torch.dtype = torch.float32, plan: Optional[SpmmPlan] = None,
         use_plan: bool = True, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C[m x N] = A[m x k] @ B[k x N] (fp32 accumulation)."""
    _require(B, "B", tuple(_DT))
    if B.dim() != 2:
        raise ValueError("B must be 2-D")
    k, N = B.shape
    if A_val.dtype != B.dtype:
        raise ValueError("A_val and B must share a dtype")
    d = csr_desc(A_val, A_row_offsets, A_row_indices, A_col_indices, m, k)
    _maybe_validate(A_row_offsets, A_col_indices, m, k, A_row_indices)
    if out is None:
        out = torch.empty((m, N), dtype=out_dtype, device=B.device)
    else:
        _require(out, "out", (out_dtype,))
        if tuple(out.shape) != (m, N):
            raise ValueError("out has the wrong shape")
    if plan is None and use_plan:
        plan = _spmm_plans.get(("spmm", _tkey(A_row_offsets), _tkey(A_row_indices), d.nnz, k),
                               lambda: SpmmPlan(A_row_offsets, A_row_indices, A_col_indices, k),
                               (A_row_offsets, A_row_indices))
    ws = plan.workspace(N, B.device) if plan is not None else None
    _check("spops_spmm", lib().spops_spmm(
        ctypes.byref(d), _ptr(B), _DT[B.dtype], N, N, _ptr(out), _DT[out_dtype], N,
        plan.handle if plan is not None else None, _ptr(ws),
        ws.numel() if ws is not None else 0, _stream(B)))
    return out


def sddmm(out_row_offsets: torch.Tensor, out_row_indices: torch.Tensor,
          out_col_indices: torch.Tensor, A: torch.Tensor, BT: torch.Tensor,
          backend: str = "structure_aware", out_dtype: torch.dtype = torch.float32,
          plan: Optional[SddmmPlan] = None, tau: Optional[float] = None,
          out: Optional[torch.Tensor] = None,
          workspace: Optional[torch.Tensor] = None, use_plan: bool = True) -> torch.Tensor:
    """values[p] = A[r(p)] . BT[c(p)] at every position of the CSR mask.
    The structure-aware backend uses `plan`, else a cached plan for this
    mask; with use_plan=False and no plan the library partitions the mask
    inside the call (in the workspace, no allocation or synchronization)."""
    if backend not in _BACKENDS:
        raise ValueError(f"backend must be one of {sorted(_BACKENDS)}")
    _require(A, "A", tuple(_DT))
    _require(BT, "BT", tuple(_DT))
    if A.dim() != 2 or BT.dim() != 2 or A.shape[1] != BT.shape[1] or A.dtype != BT.dtype:
        raise ValueError("A (m x K) and BT (n x K) must be 2-D with the same K and dtype")
    m, K = A.shape
    n = BT.shape[0]
    d = csr_desc(None, out_row_offsets, out_row_indices, out_col_indices, m, n)
    _maybe_validate(out_row_offsets, out_col_indices, m, n, out_row_indices)
    nnz = d.nnz
    if out is None:
        out = torch.empty(nnz, dtype=out_dtype, device=A.device)
    b = _BACKENDS[backend]
    if b == STRUCTURE_AWARE and plan is None and use_plan and nnz > 0:
        plan = _sddmm_plans.get(("sddmm", _tkey(out_row_offsets), _tkey(out_col_indices), m, n,
                                 tau), lambda: SddmmPlan(out_row_offsets, out_col_indices, m, n,
                                                         tau),
                                (out_row_offsets, out_col_indices))
    ph = plan.handle if (plan is not None and b == STRUCTURE_AWARE) else None
    if workspace is None:
        wb = ctypes.c_size_t()
        _check("spops_sddmm_workspace_size", lib().spops_sddmm_workspace_size(
            ctypes.byref(d), K, _DT[A.dtype], b, ph, ctypes.byref(wb)))
        workspace = _workspace(wb.value, A.device)
    _check("spops_sddmm", lib().spops_sddmm(
        ctypes.byref(d), _ptr(A), K, max(K, 1), _ptr(BT), max(K, 1), _DT[A.dtype], _ptr(out),
        _DT[out_dtype], b, ph, _ptr(workspace), workspace.numel() if workspace is not None else 0,
        _stream(A)))
    return out


def csr_add(A_val: torch.Tensor, A_row_offsets: torch.Tensor, A_row_indices: torch.Tensor,
            A_col_indices: torch.Tensor, B: torch.Tensor) -> torch.Tensor:
    """B += A in place (one rounding to B's dtype per entry); returns B."""
    _require(B, "B", tuple(_DT))
    if B.dim() != 2:
        raise ValueError("B must be 2-D")
    m, n = B.shape
    if A_val.dtype != B.dtype:
        raise ValueError("A_val and B must share a dtype")
    d = csr_desc(A_val, A_row_offsets, A_row_indices, A_col_indices, m, n)
    _maybe_validate(A_row_offsets, A_col_indices, m, n, A_row_indices)
    _check("spops_csr_add", lib().spops_csr_add(ctypes.byref(d), _ptr(B), _DT[B.dtype], n,
                                                _stream(B)))
    return B


def csr_transpose_workspace(m: int, n: int, nnz: int, device) -> torch.Tensor:
    b = ctypes.c_size_t()
    _check("spops_csr_transpose_workspace_size",
           lib().spops_csr_transpose_workspace_size(m, n, nnz, ctypes.byref(b)))
    return torch.empty(max(b.value, 1), dtype=torch.uint8, device=device)


def csr_transpose(A_val: Optional[torch.Tensor], A_row_offsets: torch.Tensor,
                  A_col_indices: torch.Tensor, m: int, n: int,
                  workspace: Optional[torch.Tensor] = None,
                  out: Optional[Tuple[Optional[torch.Tensor], torch.Tensor,
                                      torch.Tensor]] = None
                  ) -> Tuple[Optional[torch.Tensor], torch.Tensor, torch.Tensor]:
    """A^T as (values_T, row_offsets_T [n+1] int32, col_idx_T [nnz]); `out`
    gives preallocated (values_T or None, row_offsets_T, col_idx_T)."""
    d = csr_desc(A_val, A_row_offsets, None, A_col_indices, m, n)
    _maybe_validate(A_row_offsets, A_col_indices, m, n)
    dev = A_row_offsets.device
    nnz = d.nnz
    oit = torch.int16 if m <= 32767 else torch.int32
    if out is None:
        out_ro = torch.empty(n + 1, dtype=torch.int32, device=dev)
        out_ci = torch.empty(nnz, dtype=oit, device=dev)
        out_v = torch.empty_like(A_val) if A_val is not None else None
    else:
        out_v, out_ro, out_ci = out
        _require(out_ro, "out row_offsets", (torch.int32,))
        _require(out_ci, "out col_idx", (torch.int16, torch.int32))
        if out_ro.numel() != n + 1 or out_ci.numel() != nnz or out_ci.dtype != oit:
            raise ValueError("out arrays have the wrong size or index type")
        if A_val is not None:
            if out_v is None:
                raise ValueError("out values missing")
            _require(out_v, "out values", (A_val.dtype,))
            if out_v.numel() != nnz:
                raise ValueError("out values have the wrong size")
    if workspace is None:
        workspace = csr_transpose_workspace(m, n, nnz, dev)
    _check("spops_csr_transpose", lib().spops_csr_transpose(
        ctypes.byref(d), _ptr(out_v), out_ro.data_ptr(), _ptr(out_ci), _IT[oit],
        workspace.data_ptr(), workspace.numel(), _stream(A_row_offsets)))
    return out_v, out_ro, out_ci


def csr_transpose_permutation(A_row_offsets: torch.Tensor, A_col_indices: torch.Tensor,
                              m: int, n: int) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """The permutation csr_transpose applies to the values of this pattern:
    (src [nnz] int32, row_offsets_T [n+1] int32, col_idx_T [nnz]), with
    values_T = permute_values(values, src)."""
    d = csr_desc(None, A_row_offsets, None, A_col_indices, m, n)
    _maybe_validate(A_row_offsets, A_col_indices, m, n)
    dev = A_row_offsets.device
    nnz = d.nnz
    oit = torch.int16 if m <= 32767 else torch.int32
    src = torch.empty(nnz, dtype=torch.int32, device=dev)
    out_ro = torch.empty(n + 1, dtype=torch.int32, device=dev)
    out_ci = torch.empty(nnz, dtype=oit, device=dev)
    b = ctypes.c_size_t()
    _check("spops_csr_transpose_permutation_workspace_size",
           lib().spops_csr_transpose_permutation_workspace_size(m, n, nnz, ctypes.byref(b)))
    ws = _workspace(b.value, dev)
    _check("spops_csr_transpose_permutation", lib().spops_csr_transpose_permutation(
        ctypes.byref(d), _ptr(src), out_ro.data_ptr(), _ptr(out_ci), _IT[oit], _ptr(ws),
        ws.numel() if ws is not None else 0, _stream(A_row_offsets)))
    return src, out_ro, out_ci


def permute_values(values: torch.Tensor, src: torch.Tensor,
                   out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out[j] = values[src[j]] (bit for bit); e.g. A^T's values from A's with
    src from csr_transpose_permutation."""
    _require(values, "values", (torch.float32, torch.float16, torch.bfloat16))
    _require(src, "src", (torch.int32,))
    if out is None:
        out = torch.empty(src.numel(), dtype=values.dtype, device=values.device)
    else:
        _require(out, "out", (values.dtype,))
        if out.numel() != src.numel():
            raise ValueError("out has the wrong size")
    _check("spops_permute_values", lib().spops_permute_values(
        _ptr(values), values.numel(), _DT[values.dtype], _ptr(src), src.numel(), _ptr(out),
        _stream(values)))
    return out


def sort_rows_workspace(m: int, n: int, device) -> torch.Tensor:
    b = ctypes.c_size_t()
    _check("spops_sort_rows_by_nnz_workspace_size",
           lib().spops_sort_rows_by_nnz_workspace_size(m, n, ctypes.byref(b)))
    return torch.empty(max(b.value, 1), dtype=torch.uint8, device=device)


def sort_rows_by_nnz(row_offsets: torch.Tensor, n: int,
                     index_dtype: Optional[torch.dtype] = None,
                     workspace: Optional[torch.Tensor] = None,
                     out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """row_idx: rows by entry count, most first, ties by ascending row."""
    _require(row_offsets, "row_offsets", (torch.int32,))
    m = row_offsets.numel() - 1
    dt = index_dtype or (torch.int16 if m <= 32767 else torch.int32)
    if out is None:
        out = torch.empty(m, dtype=dt, device=row_offsets.device)
    if workspace is None:
        workspace = sort_rows_workspace(m, n, row_offsets.device)
    _check("spops_sort_rows_by_nnz", lib().spops_sort_rows_by_nnz(
        row_offsets.data_ptr(), m, n, _ptr(out), _IT[out.dtype], workspace.data_ptr(),
        workspace.numel(), _stream(row_offsets)))
    return out


def cg(A_val: torch.Tensor, A_row_offsets: torch.Tensor, A_row_indices: torch.Tensor,
       A_col_indices: torch.Tensor, b: torch.Tensor, x: Optional[torch.Tensor] = None,
       rtol: float = 1e-6, max_iter: int = 1000, check_every: int = 8,
       plan: Optional[SpmmPlan] = None, use_plan: bool = True):
    """Conjugate gradients for A x = b (A square, symmetric positive definite,
    f32 values).  `x` (optional) is the initial guess and is overwritten with
    the solution; without it the solve starts from zero.  Returns
    (x, iterations, ||r|| / ||b||).  Blocks: the solver reads its state back
    every `check_every` iterations."""
    _require(b, "b", (torch.float32,))
    m = b.numel()
    if b.dim() != 1:
        raise ValueError("b must be 1-D")
    if A_val.dtype != torch.float32:
        raise ValueError("cg needs f32 values")
    d = csr_desc(A_val, A_row_offsets, A_row_indices, A_col_indices, m, m)
    if x is None:
        x = torch.zeros_like(b)
    else:
        _require(x, "x", (torch.float32,))
        if x.shape != b.shape:
            raise ValueError("x must have b's shape")
    if plan is None and use_plan:
        plan = _spmm_plans.get(("spmm", _tkey(A_row_offsets), _tkey(A_row_indices), d.nnz, m),
                               lambda: SpmmPlan(A_row_offsets, A_row_indices, A_col_indices, m),
                               (A_row_offsets, A_row_indices))
    ph = plan.handle if plan is not None else None
    wb = ctypes.c_size_t()
    _check("spops_cg_workspace_size", lib().spops_cg_workspace_size(
        ctypes.byref(d), ph, ctypes.byref(wb)))
    ws = _workspace(wb.value, b.device)
    its, rel = ctypes.c_int64(), ctypes.c_double()
    _check("spops_cg", lib().spops_cg(
        ctypes.byref(d), _ptr(b), _ptr(x), float(rtol), int(max_iter), int(check_every), ph,
        _ptr(ws), ws.numel() if ws is not None else 0, ctypes.byref(its), ctypes.byref(rel),
        _stream(b)))
    return x, int(its.value), float(rel.value)


def masked_adam(values: torch.Tensor, grad: torch.Tensor, exp_avg: torch.Tensor,
                exp_avg_sq: torch.Tensor, step: int, lr: float = 1e-3, betas=(0.9, 0.999),
                eps: float = 1e-8, maximize: bool = False,
                positions: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One masked Adam step, in place on `values`, `exp_avg` and `exp_avg_sq`
    (f32 moments).  `grad` covers every value (positions=None) or the
    distinct int32 `positions` only.  Returns `values`."""
    _require(values, "values", tuple(_DT))
    _require(grad, "grad", (values.dtype,))
    _require(exp_avg, "exp_avg", (torch.float32,))
    _require(exp_avg_sq, "exp_avg_sq", (torch.float32,))
    n = values.numel()
    if exp_avg.numel() != n or exp_avg_sq.numel() != n:
        raise ValueError("moments must match values")
    if positions is None:
        if grad.numel() != n:
            raise ValueError("grad must cover every value when positions is None")
    else:
        _require(positions, "positions", (torch.int32,))
        if positions.numel() != grad.numel():
            raise ValueError("positions and grad must have the same length")
    _check("spops_masked_adam", lib().spops_masked_adam(
        _ptr(values), _DT[values.dtype], n, _ptr(grad), _ptr(positions), grad.numel(),
        _ptr(exp_avg), _ptr(exp_avg_sq), int(step), float(lr), float(betas[0]),
        float(betas[1]), float(eps), int(bool(maximize)), _stream(values)))
    return values


class DeltaMatrix:
    """A matrix in the 2-bit delta-coded row format (see include/spops.h):
    enc_offsets[m+1] int32, codes[ceil(E/16)] (int32 storage of the uint32
    words), values[16 ceil(E/16)] in the matrix dtype."""

    def __init__(self, m: int, n: int, enc_offsets: torch.Tensor, codes: torch.Tensor,
                 values: torch.Tensor, entries: int):
        self.m, self.n = m, n
        self.enc_offsets, self.codes, self.values, self.entries = (enc_offsets, codes, values,
                                                                   entries)


def delta_encode(A_val: torch.Tensor, A_row_offsets: torch.Tensor, A_col_indices: torch.Tensor,
                 m: int, n: int) -> DeltaMatrix:
    """CSR (columns strictly ascending in each row) -> DeltaMatrix.  Two
    library calls: the encoded size (synchronizes), then the encoding."""
    _require(A_val, "A_val", tuple(_DT))
    d = csr_desc(A_val, A_row_offsets, None, A_col_indices, m, n)
    dev = A_row_offsets.device
    wb = ctypes.c_size_t()
    _check("spops_delta_size_workspace", lib().spops_delta_size_workspace(m, ctypes.byref(wb)))
    ws = _workspace(wb.value, dev)
    eo = torch.empty(m + 1, dtype=torch.int32, device=dev)
    E = ctypes.c_int64()
    _check("spops_delta_size", lib().spops_delta_size(
        ctypes.byref(d), _ptr(eo), ctypes.byref(E), _ptr(ws), wb.value, _stream(A_row_offsets)))
    words = (E.value + 15) // 16
    codes = torch.empty(max(words, 1), dtype=torch.int32, device=dev)
    vals = torch.empty(max(words, 1) * 16, dtype=A_val.dtype, device=dev)
    _check("spops_delta_encode", lib().spops_delta_encode(
        ctypes.byref(d), _ptr(eo), E.value, _ptr(codes), _ptr(vals), _stream(A_row_offsets)))
    return DeltaMatrix(m, n, eo, codes, vals, E.value)


def delta_spmv(D: DeltaMatrix, x: torch.Tensor, out_dtype: torch.dtype = torch.float32,
               out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = A x for A in the delta format (fp32 accumulation)."""
    _require(x, "x", (D.values.dtype,))
    if x.numel() != D.n:
        raise ValueError("x must have n entries")
    if out is None:
        out = torch.empty(D.m, dtype=out_dtype, device=x.device)
    else:
        _require(out, "out", (out_dtype,))
        if out.numel() != D.m:
            raise ValueError("out must have m entries")
    _check("spops_delta_spmv", lib().spops_delta_spmv(
        D.m, D.n, _ptr(D.enc_offsets), D.entries, _ptr(D.codes), _ptr(D.values),
        _DT[D.values.dtype], _ptr(x), _ptr(out), _DT[out_dtype], _stream(x)))
    return out
