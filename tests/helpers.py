"""Test helpers: host <-> device conversion and the parity error measures."""
import numpy as np
import torch

TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
NP_DT = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}

# Parity bars: max relative error against the float64 oracle, with the
# relative measure guarded by the RMS of the whole output (see rel_err).
TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}


def dev(x: np.ndarray, dt: str = None, device="cuda") -> torch.Tensor:
    """Host array (generator storage convention) -> device tensor."""
    if dt == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(device)


def host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> host array in the generator storage convention."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def host_f64(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        t = t.to(torch.float32)
    return t.numpy().astype(np.float64)


def csr_dev(A, device="cuda"):
    """(values, row_offsets, col_idx) of a generator CSR on the device."""
    v = dev(A.values, A.val_dtype, device) if A.values is not None else None
    return v, dev(A.row_offsets, None, device), dev(A.col_idx, None, device)


def rel_err(y: np.ndarray, r: np.ndarray) -> float:
    """max_i |y_i - r_i| / max(|r_i|, rms(r)); inf on any NaN/Inf mismatch."""
    y = np.asarray(y, dtype=np.float64).ravel()
    r = np.asarray(r, dtype=np.float64).ravel()
    if y.size == 0:
        return 0.0
    if not np.array_equal(np.isfinite(y), np.isfinite(r)):
        return float("inf")
    fin = np.isfinite(r)
    y, r = y[fin], r[fin]
    if y.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(r * r)))
    den = np.maximum(np.abs(r), rms if rms > 0 else 1.0)
    return float(np.max(np.abs(y - r) / den))


def assert_close(y, r, dt, what=""):
    e = rel_err(y, r)
    assert e <= TOL[dt], f"{what}: rel err {e:.3e} > {TOL[dt]:.1e}"
    return e
