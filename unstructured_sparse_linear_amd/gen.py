"""Seeded synthetic inputs for the CSR sparse-dense products.

This module only builds inputs: sparsity patterns in the CSR layout the spops
page fixes (spops README, "Usage": values / row_offsets[m+1] / col_idx), and
dense operands drawn from normal distributions.  It holds none of the
arithmetic of the operations themselves, so both the GPU path and the CPU
oracle can consume its arrays without sharing any computation.

Storage conventions (host, numpy):
  * value dtypes are named 'f32', 'f16', 'bf16'; f32 -> np.float32,
    f16 -> np.float16, bf16 -> np.uint16 holding the bfloat16 bit pattern;
  * row_offsets is int32 (spops README, "Important Notes");
  * col_idx is int16 when n <= 32767 and int32 otherwise (the 16-bit index
    rule of the same notes, widened where 16 bits cannot address n).

Every array comes from its own numpy PCG64 stream
``default_rng([seed, config_id, stream_id])`` so that arrays are independent
of the order in which they are requested.

The five workloads (sizes, densities, distributions) follow the configurations
the benchmark is quoted on; each builder's docstring states how an
under-specified phrase of that description is read.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, Dict, Optional

import numpy as np

VALUE_DTYPES = ("f32", "f16", "bf16")
ELEM_SIZE = {"f32": 4, "f16": 2, "bf16": 2}

# stream ids (fixed, so a given seed always gives the same arrays)
S_MASK, S_VALUES, S_B, S_A, S_BT, S_W, S_B1, S_PERM, S_EXTRA = range(9)


def rng_for(seed: int, cfg: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(cfg), int(stream)])


def index_dtype_for(extent: int):
    """int16 when every index in [0, extent) fits a signed 16-bit value."""
    return np.int16 if extent <= 32767 else np.int32


# ---------------------------------------------------------------- values --

def f32_to_storage(x32: np.ndarray, dt: str) -> np.ndarray:
    """Round float32 samples to the storage dtype (round to nearest even)."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    if dt == "f32":
        return x32
    if dt == "f16":
        return x32.astype(np.float16)
    if dt == "bf16":
        import torch  # the bf16 cast is torch's RNE conversion
        t = torch.from_numpy(x32).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    raise ValueError(f"unknown dtype {dt!r}")


def storage_to_f64(x: np.ndarray, dt: str) -> np.ndarray:
    """Exact widening of stored values to float64 (for statistics only)."""
    if dt == "bf16":
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def normal(rng: np.random.Generator, shape, dt: str, std: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return f32_to_storage(x, dt)


# ------------------------------------------------------------------ CSR ----

@dataclass
class CSR:
    m: int
    n: int
    row_offsets: np.ndarray            # int32 [m+1]
    col_idx: np.ndarray                # int16 / int32 [nnz]
    values: Optional[np.ndarray] = None
    val_dtype: Optional[str] = None

    @property
    def nnz(self) -> int:
        return int(self.row_offsets[-1])

    def row_counts(self) -> np.ndarray:
        return np.diff(self.row_offsets.astype(np.int64))

    def with_values(self, values: np.ndarray, dt: str) -> "CSR":
        assert values.shape == (self.nnz,)
        return CSR(self.m, self.n, self.row_offsets, self.col_idx, values, dt)

    def to_dense_f64(self) -> np.ndarray:
        """Dense float64 copy (tiny matrices; used by test brute force)."""
        d = np.zeros((self.m, self.n))
        v = storage_to_f64(self.values, self.val_dtype) if self.values is not None \
            else np.ones(self.nnz)
        rows = np.repeat(np.arange(self.m), self.row_counts())
        np.add.at(d, (rows, self.col_idx.astype(np.int64)), v)
        return d


def csr_from_row_lists(m: int, n: int, cols_per_row) -> CSR:
    counts = np.fromiter((len(c) for c in cols_per_row), dtype=np.int64, count=m)
    ro = np.zeros(m + 1, dtype=np.int64)
    np.cumsum(counts, out=ro[1:])
    if ro[-1] > np.iinfo(np.int32).max:
        raise ValueError("nnz exceeds int32 row_offsets")
    col = np.concatenate([np.asarray(c, dtype=np.int64) for c in cols_per_row]) \
        if m and ro[-1] else np.zeros(0, dtype=np.int64)
    return CSR(m, n, ro.astype(np.int32), col.astype(index_dtype_for(n)))


def csr_from_coo(m: int, n: int, rows: np.ndarray, cols: np.ndarray,
                 vals: Optional[np.ndarray] = None, dt: Optional[str] = None) -> CSR:
    """COO triples (unique positions) to CSR with columns ascending in a row."""
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    order = np.lexsort((cols, rows))
    rows, cols = rows[order], cols[order]
    ro = np.zeros(m + 1, dtype=np.int64)
    np.cumsum(np.bincount(rows, minlength=m), out=ro[1:])
    v = None if vals is None else np.asarray(vals)[order]
    return CSR(m, n, ro.astype(np.int32), cols.astype(index_dtype_for(n)), v, dt)


def _sample_wo_replacement(rng: np.random.Generator, pop: int, k: int) -> np.ndarray:
    if k > pop:
        raise ValueError("sample larger than population")
    if pop <= 64_000_000 and k > pop // 64:
        return rng.permutation(pop)[:k]
    return rng.choice(pop, size=k, replace=False)


def bernoulli_mask(rng: np.random.Generator, m: int, n: int, p: float) -> CSR:
    """Each cell present independently with probability p.

    Drawn row by row: nnz_r ~ Binomial(n, p), then nnz_r distinct columns
    uniformly without replacement, stored ascending.
    """
    counts = rng.binomial(n, p, size=m)
    rows = [np.sort(_sample_wo_replacement(rng, n, int(c))) for c in counts]
    return csr_from_row_lists(m, n, rows)


def cross_mask(rng: np.random.Generator, m: int, n: int, density: float,
               hot_row_frac: float, hot_col_frac: float, hot_share: float) -> CSR:
    """Mask whose nonzeros cluster in a few rows and columns.

    Reading: round(density*m*n) nonzeros; a random set R of round(hot_row_frac*m)
    rows and C of round(hot_col_frac*n) columns; round(hot_share*nnz) positions
    are drawn uniformly without replacement from the cross (R x all) U (all x C)
    and the rest from its complement.  (The literal reading, 90% of the nonzeros
    inside R x C, does not fit: R x C holds fewer cells than that.)
    """
    nnz = int(round(density * m * n))
    nr = int(round(hot_row_frac * m))
    nc = int(round(hot_col_frac * n))
    hot_rows = np.sort(rng.choice(m, size=nr, replace=False))
    hot_cols = np.sort(rng.choice(n, size=nc, replace=False))
    cold_rows = np.setdiff1d(np.arange(m), hot_rows)
    cold_cols = np.setdiff1d(np.arange(n), hot_cols)
    n_hot = int(round(hot_share * nnz))
    n_cold = nnz - n_hot
    # cross index space: [0, nr*n) -> hot row x any col;
    # [nr*n, nr*n + (m-nr)*nc) -> cold row x hot col
    size_a = nr * n
    size_h = size_a + len(cold_rows) * nc
    h = _sample_wo_replacement(rng, size_h, n_hot)
    in_a = h < size_a
    ha, hb = h[in_a], h[~in_a] - size_a
    r1, c1 = hot_rows[ha // n], ha % n
    r2, c2 = cold_rows[hb // nc], hot_cols[hb % nc]
    q = _sample_wo_replacement(rng, len(cold_rows) * len(cold_cols), n_cold)
    r3, c3 = cold_rows[q // len(cold_cols)], cold_cols[q % len(cold_cols)]
    rows = np.concatenate([r1, r2, r3])
    cols = np.concatenate([c1, c2, c3])
    out = csr_from_coo(m, n, rows, cols)
    out.hot_rows, out.hot_cols = hot_rows, hot_cols  # type: ignore[attr-defined]
    return out


def banded_spd(rng_pattern: np.random.Generator, rng_values: np.random.Generator,
               n: int, band: int = 8, offband_draws: int = 4) -> CSR:
    """Symmetric, strictly diagonally dominant f32 matrix.

    Pattern: every |i-j| <= band, plus for each row i `offband_draws` columns
    drawn uniformly from {j : |i-j| > band}, mirrored to (j, i), duplicates
    merged.  Off-diagonal a_ij = a_ji ~ N(0,1) rounded to f32; the diagonal is
    1 + sum_j |a_ij| (rounded to f32), which makes the matrix SPD.
    """
    i = np.arange(n, dtype=np.int64)
    lo = np.maximum(i - band, 0)
    hi = np.minimum(i + band, n - 1)
    width = hi - lo + 1
    # off-band draws: t uniform in [0, n - width), skip the band
    t = (rng_pattern.random((n, offband_draws)) * (n - width)[:, None]).astype(np.int64)
    j = np.where(t < lo[:, None], t, t + width[:, None])
    ii = np.repeat(i, offband_draws)
    jj = j.reshape(-1)
    # unordered pairs (a < b): band pairs and off-band pairs
    band_a = np.concatenate([i[: n - d] for d in range(1, band + 1)])
    band_b = np.concatenate([i[d:] for d in range(1, band + 1)])
    pa = np.concatenate([band_a, np.minimum(ii, jj)])
    pb = np.concatenate([band_b, np.maximum(ii, jj)])
    key = np.unique(pa * n + pb)
    pa, pb = key // n, key % n
    v = rng_values.standard_normal(size=len(key), dtype=np.float32)
    rows = np.concatenate([pa, pb, i])
    cols = np.concatenate([pb, pa, i])
    absum = np.zeros(n)
    np.add.at(absum, pa, np.abs(v.astype(np.float64)))
    np.add.at(absum, pb, np.abs(v.astype(np.float64)))
    diag = (1.0 + absum).astype(np.float32)
    vals = np.concatenate([v, v, diag])
    return csr_from_coo(n, n, rows, cols, vals, "f32")


def zipf_row_counts(rng: np.random.Generator, m: int, s: float, mean: float,
                    cap: int) -> np.ndarray:
    """Row lengths from a Zipf(s) law, scaled so the mean is `mean`.

    z_r ~ Zipf(s) i.i.d.; nnz_r = clip(rint(c * z_r), 1, cap), with the scale c
    found by bisection on the drawn z so that sum(nnz_r) is as close as
    possible to mean*m.  (An unscaled capped Zipf(1.5) has a mean near 97, not
    64, so some scale is needed to meet both the law and the stated mean.)
    """
    z = rng.zipf(s, size=m).astype(np.float64)
    target = mean * m

    def total(c):
        return int(np.clip(np.rint(c * z), 1, cap).sum())

    lo, hi = 0.0, float(cap)
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if total(mid) < target:
            lo = mid
        else:
            hi = mid
    c = lo if abs(total(lo) - target) <= abs(total(hi) - target) else hi
    return np.clip(np.rint(c * z), 1, cap).astype(np.int64)


def rows_with_counts(rng: np.random.Generator, n: int, counts: np.ndarray) -> list:
    return [np.sort(_sample_wo_replacement(rng, n, int(c))) for c in counts]


# ---------------------------------------------------------- test inputs ---

def random_csr(seed: int, m: int, n: int, density: float, dt: Optional[str] = "f32",
               empty_row_frac: float = 0.0, shuffle_within_rows: bool = False,
               col_index_dtype=None, integer_values: bool = False,
               std: float = 1.0) -> CSR:
    """Small random CSR for tests: Bernoulli pattern, optional empty rows,
    optional unsorted columns inside rows, optional small-integer values."""
    rng = rng_for(seed, 100, S_MASK)
    csr = bernoulli_mask(rng, m, n, density)
    if empty_row_frac > 0 and m > 0:
        kill = rng.random(m) < empty_row_frac
        rows = [csr.col_idx[csr.row_offsets[r]:csr.row_offsets[r + 1]] if not kill[r]
                else np.zeros(0, dtype=np.int64) for r in range(m)]
        csr = csr_from_row_lists(m, n, rows)
    if shuffle_within_rows:
        col = csr.col_idx.copy()
        for r in range(m):
            a, b = csr.row_offsets[r], csr.row_offsets[r + 1]
            col[a:b] = rng.permutation(col[a:b])
        csr.col_idx = col
    if col_index_dtype is not None:
        csr.col_idx = csr.col_idx.astype(col_index_dtype)
    if dt is not None:
        vr = rng_for(seed, 100, S_VALUES)
        if integer_values:
            vals = f32_to_storage(vr.integers(-3, 4, size=csr.nnz).astype(np.float32), dt)
        else:
            vals = normal(vr, csr.nnz, dt, std)
        csr = csr.with_values(vals, dt)
    return csr


def dense(seed: int, cfg: int, stream: int, shape, dt: str, std: float = 1.0,
          integer_values: bool = False) -> np.ndarray:
    rng = rng_for(seed, cfg, stream)
    if integer_values:
        return f32_to_storage(rng.integers(-3, 4, size=shape).astype(np.float32), dt)
    return normal(rng, shape, dt, std)


def permutation(seed: int, m: int, kind: str, index_dtype=None) -> np.ndarray:
    """Row permutations used as row_idx in tests: identity, reversed, random."""
    if kind == "identity":
        p = np.arange(m)
    elif kind == "reversed":
        p = np.arange(m)[::-1].copy()
    elif kind == "random":
        p = rng_for(seed, 101, S_PERM).permutation(m)
    else:
        raise ValueError(kind)
    return p.astype(index_dtype or index_dtype_for(m))


# -------------------------------------------------------- the workloads ---

@dataclass
class Workload:
    """One configuration; arrays are built on first use and cached."""
    cfg: int
    name: str
    seed: int
    dt: str
    m: int
    n: int
    N: tuple                  # SpMM widths
    K: int                    # SDDMM inner size
    _builders: Dict[str, Callable[[], object]] = field(default_factory=dict, repr=False)
    _cache: Dict[str, object] = field(default_factory=dict, repr=False)

    def get(self, key: str):
        if key not in self._cache:
            self._cache[key] = self._builders[key]()
        return self._cache[key]

    def keys(self):
        return list(self._builders)

    def drop(self, key: str):
        self._cache.pop(key, None)


CONFIG_NAMES = {
    1: "tiny-uniform-512-f32",
    2: "llm-adapter-4096-f16",
    3: "cross-4096x11008",
    4: "banded-spd-123440-f32",
    5: "zipf-rows-16384-bf16",
}


def make_config(cfg: int, seed: int = 0, dt: Optional[str] = None) -> Workload:
    """The five workloads.  Keys: 'A' (CSR with values), 'mask' (same pattern),
    'B' (SpMM dense operand, k x N), 'Ad' and 'BT' (SDDMM operands, m x K and
    n x K), 'W' (dense m x n target of csr_add; for config 4 a slab of rows)."""
    r = lambda s: rng_for(seed, cfg, s)  # noqa: E731
    if cfg == 1:
        dt = dt or "f32"
        w = Workload(cfg, CONFIG_NAMES[cfg], seed, dt, 512, 512, (64,), 64)
        w._builders["mask"] = lambda: bernoulli_mask(r(S_MASK), 512, 512, 0.02)
        w._builders["A"] = lambda: w.get("mask").with_values(
            normal(r(S_VALUES), w.get("mask").nnz, dt, 1.0), dt)
        w._builders["B"] = lambda: normal(r(S_B), (512, 64), dt)
        w._builders["Ad"] = lambda: normal(r(S_A), (512, 64), dt)
        w._builders["BT"] = lambda: normal(r(S_BT), (512, 64), dt)
        w._builders["W"] = lambda: normal(r(S_W), (512, 512), dt)
        return w
    if cfg == 2:
        dt = dt or "f16"
        w = Workload(cfg, CONFIG_NAMES[cfg], seed, dt, 4096, 4096, (2048,), 2048)
        w._builders["mask"] = lambda: bernoulli_mask(r(S_MASK), 4096, 4096, 0.01)
        w._builders["A"] = lambda: w.get("mask").with_values(
            normal(r(S_VALUES), w.get("mask").nnz, dt, 0.02), dt)
        w._builders["B"] = lambda: normal(r(S_B), (4096, 2048), dt)
        w._builders["Ad"] = lambda: normal(r(S_A), (4096, 2048), dt)
        w._builders["BT"] = lambda: normal(r(S_BT), (4096, 2048), dt)
        w._builders["W"] = lambda: normal(r(S_W), (4096, 4096), dt, 0.02)
        return w
    if cfg == 3:
        dt = dt or "f16"
        m, n = 4096, 11008
        w = Workload(cfg, CONFIG_NAMES[cfg] + "-" + dt, seed, dt, m, n, (2048,), 2048)
        w._builders["mask"] = lambda: cross_mask(r(S_MASK), m, n, 0.01, 0.05, 0.05, 0.9)
        w._builders["A"] = lambda: w.get("mask").with_values(
            normal(r(S_VALUES), w.get("mask").nnz, dt, 1.0), dt)
        w._builders["B"] = lambda: normal(r(S_B), (n, 2048), dt)
        w._builders["Ad"] = lambda: normal(r(S_A), (m, 2048), dt)
        w._builders["BT"] = lambda: normal(r(S_BT), (n, 2048), dt)
        w._builders["W"] = lambda: normal(r(S_W), (m, n), dt, 0.02)
        return w
    if cfg == 4:
        dt = "f32"
        n = 123_440
        w = Workload(cfg, CONFIG_NAMES[cfg], seed, dt, n, n, (1, 32), 32)
        w._builders["A"] = lambda: banded_spd(r(S_MASK), r(S_VALUES), n)
        w._builders["mask"] = lambda: w.get("A")
        w._builders["B1"] = lambda: normal(r(S_B1), (n, 1), dt)
        w._builders["B"] = lambda: normal(r(S_B), (n, 32), dt)
        w._builders["Ad"] = lambda: normal(r(S_A), (n, 32), dt)
        w._builders["BT"] = lambda: normal(r(S_BT), (n, 32), dt)
        # csr_add target: the dense 123440^2 f32 matrix (61 GB) is replaced by
        # slabs of 8192 rows; 'W' is the first slab
        w._builders["W"] = lambda: normal(r(S_W), (8192, n), dt)
        return w
    if cfg == 5:
        dt = dt or "bf16"
        n = 16384

        def mask5():
            counts = zipf_row_counts(r(S_MASK), n, 1.5, 64.0, 4096)
            return csr_from_row_lists(n, n, rows_with_counts(r(S_EXTRA), n, counts))

        w = Workload(cfg, CONFIG_NAMES[cfg], seed, dt, n, n, (256,), 256)
        w._builders["mask"] = mask5
        w._builders["A"] = lambda: w.get("mask").with_values(
            normal(r(S_VALUES), w.get("mask").nnz, dt, 1.0), dt)
        w._builders["B"] = lambda: normal(r(S_B), (n, 256), dt)
        w._builders["Ad"] = lambda: normal(r(S_A), (n, 256), dt)
        w._builders["BT"] = lambda: normal(r(S_BT), (n, 256), dt)
        w._builders["W"] = lambda: normal(r(S_W), (n, n), dt)
        return w
    raise ValueError(f"unknown config {cfg}")


def csr_row_slab(csr: CSR, r0: int, r1: int) -> CSR:
    """Rows [r0, r1) of a CSR as a CSR of its own (offsets rebased to 0)."""
    a, b = int(csr.row_offsets[r0]), int(csr.row_offsets[r1])
    ro = (csr.row_offsets[r0:r1 + 1].astype(np.int64) - a).astype(np.int32)
    v = None if csr.values is None else csr.values[a:b]
    return CSR(r1 - r0, csr.n, ro, csr.col_idx[a:b], v, csr.val_dtype)
