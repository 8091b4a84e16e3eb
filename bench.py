#!/usr/bin/env python3
"""Benchmark of the CSR sparse-dense hot path on one MI355X.

Headline: the structure-aware SDDMM on the cross-clustered 4096 x 11008 mask
with f16 operands (K = 2048), the largest workload in the metric's units.
`value` is that operation's algorithmic bytes over its cold-cache time (GB/s);
`roofline` describes its kernels against the HBM peak.

A step is one pass of the whole hot path over the headline workload, every
operation on the GPU through libspops:
  1. SpMM          C = A @ B                     (row order from row_idx)
  2. SDDMM         A_d @ BT^T sampled at A's mask (structure-aware backend)
  3. csr_add       W += A in place
  4. csr_transpose A^T in CSR
  5. row order     row_idx of A^T (rows by entry count)
captured once as a HIP graph and replayed K times (ms_per_step).  Plans
(SpMM row splitting, SDDMM dense-row/column partition) depend only on the
sparsity pattern; they are built once before timing (plan once, execute
many) and their build time is reported separately.

`per_config` times every gated case of the other workloads the same way
(SpMM on the LLM-adapter mask, SDDMM f16 and bf16 on the cross mask, SpMV
and 32-column SpMM on the banded SPD matrix, SpMM and SDDMM on the Zipf-row
matrix): cold median / p10 / p90, algorithmic bytes, fraction of the HBM
peak, counter traffic where committed, the on-chip gather rate against the
measured ceiling, and the float64 oracle's time on the host for the same
operation.

Timing.  Every working set here fits in the 256 MB Infinity Cache, so each
timed call starts after an untimed read of a 512 MiB scratch buffer that
evicts L2 and the Infinity Cache (inputs resident in HBM, caches cold; a
write of the buffer would leave dirty lines whose write-back then runs
during the timed call: --flush write), and is bracketed by HIP events on the
stream the library launches on.

Algorithmic bytes per operation (each input read once, each output written
once; k' / n' = distinct columns touched, m' = rows with entries):
  SpMM      nnz*(s_v+s_ci) + 4(m+1) + m*s_ri + k'*N*s_B + m*N*s_C
  SDDMM     nnz*s_ci + 4(m+1) + m*s_ri + m'*K*s_A + n'*K*s_BT + nnz*s_out
  csr_add   nnz*(s_v+s_ci) + 4(m+1) + m*s_ri + 2*nnz*s_W
  transpose nnz*(s_v+s_ci) + 4(m+1) + nnz*(s_v+s_ri') + 4(n+1)
  row order 4(n+1) + n*s_ri'
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FLUSH_BYTES = 512 << 20        # > 256 MB Infinity Cache + 8 x 4 MB L2
DEFAULT_CONFIG = 3             # headline: the largest workload in the metric's units
DEFAULT_DTYPE = "f16"
# the operations each workload names (the others are run as derived cases)
NAMED_OPS = {1: ("spmm", "sddmm"), 2: ("spmm",), 3: ("sddmm",), 4: ("spmv", "spmm"),
             5: ("spmm", "sddmm")}
# gated cases of every workload: (config, value dtype, operation)
GATED = [(2, "f16", "spmm"), (3, "f16", "sddmm"), (3, "bf16", "sddmm"), (4, "f32", "spmv"),
         (4, "f32", "spmm"), (5, "bf16", "spmm"), (5, "bf16", "sddmm")]
ESZ = {"f32": 4, "f16": 2, "bf16": 2}
COUNTERS = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--settle-ms", type=float, default=50.0,
                   help="untimed flush + call traffic before each timed loop (0: none)")
    p.add_argument("--config", type=int, default=DEFAULT_CONFIG,
                   help="workload 1-5 (3, the cross-clustered SDDMM, is the headline)")
    p.add_argument("--dtype", default=None,
                   help="value dtype of config 3 (f16, the default, or bf16)")
    p.add_argument("--no-flush", action="store_true", help="warm caches (not the metric)")
    p.add_argument("--flush", default="read", choices=("read", "write"),
                   help="how the caches are emptied before each timed call")
    p.add_argument("--no-graph", action="store_true", help="time the step eagerly")
    p.add_argument("--serial-step", action="store_true",
                   help="capture the step on one stream (no overlap of independent operations)")
    p.add_argument("--streams", type=int, default=2, choices=(1, 2, 3),
                   help="streams the step graph spreads independent operations over")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--ops", default="spmm,sddmm,csr_add,transpose,row_order")
    p.add_argument("--no-adapter", action="store_true",
                   help="skip the sparse-layer training step (forward, both gradients, Adam, merge)")
    p.add_argument("--records", default=None,
                   help="also write one JSON record per operation to this file (JSONL)")
    p.add_argument("--no-ceilings", action="store_true",
                   help="skip the copy and gather rate measurements")
    p.add_argument("--no-per-config", action="store_true",
                   help="skip the per-workload table of the gated cases")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run plain 256 MiB device copies (reference for HBM counters)")
    return p.parse_args()


class Flush:
    """Empties the L2s and the Infinity Cache before a timed call by reading a
    512 MiB buffer (default) or by writing it (--flush write).  Either way the
    timed call's inputs then come from HBM.  A write leaves the Infinity Cache
    full of dirty lines, and their write-back to HBM then runs during the
    timed call and takes part of its bandwidth (a 27 MB streaming read: 9.2 us
    after a read, 13.9 us after a write); a read leaves clean lines."""

    def __init__(self, dev, mode="read"):
        import torch
        self.buf = torch.ones(FLUSH_BYTES // 8, dtype=torch.int64, device=dev)
        self.mode = mode
        self.sink = None

    def __call__(self):
        if self.mode == "write":
            self.buf.fill_(1)
        else:
            self.sink = self.buf.sum()


def settle(fn, ms):
    """Runs fn (an untimed cache flush + call) back to back for about `ms`
    milliseconds of host time.  After an idle spell the first cold calls
    run slower until the GPU has carried this traffic for some tens of
    milliseconds: on the cross-clustered SDDMM the first ~100 cold calls
    after idle measured 72 -> 66.5 us, and a GPU-side delay before each call
    kept them at ~72 us.  Timing from the sustained state matches a
    continuously loaded GPU and makes the figures independent of what ran
    before."""
    import torch
    if ms <= 0:
        return
    t_end = time.perf_counter() + ms / 1e3
    while time.perf_counter() < t_end:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()


def copy_calibration(steps):
    """Plain device-to-device copies of a known size: what the HBM byte
    counters read for them calibrates the counters of the real kernels.  A
    second check with the access shape of the gathers: after a 512 MiB read
    that evicts the caches, each XCD gathers 4 KiB rows at random from its
    own 2 MiB slice of a 16 MiB source (the measurement library's sliced
    gather, 16 row reads per wave, every row of every slice touched with
    near certainty), so the memory reads are the source once plus the index
    list."""
    import ctypes

    import torch
    n = 256 << 20
    a = torch.ones(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(steps):
        b.copy_(a)
    torch.cuda.synchronize()
    del a, b
    path = os.path.join(ROOT, "unstructured_sparse_linear_amd", "libspops_ceilings.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not built; run __graft_entry__.build()")
    L = ctypes.CDLL(path)
    f = L.spops_ceil_gather
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                  ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int
    src = torch.full((16 << 20,), 3, dtype=torch.uint8, device="cuda")
    blocks, per_wave, rows = 2048, 16, (2 << 20) // 4096
    sink = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
    idx_np = np.random.default_rng(0).integers(0, rows, blocks * 4 * per_wave).astype(np.int32)
    idx = torch.from_numpy(idx_np).to("cuda")
    flush_buf = torch.ones(64 << 20, dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(steps):
        flush_buf.sum()
        assert f(src.data_ptr(), rows, 4096, 1, idx.data_ptr(), per_wave, blocks,
                 sink.data_ptr(), ctypes.c_void_p(stream.cuda_stream)) == 0
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "copies": steps,
                      "gather_source_bytes": 16 << 20, "gather_index_bytes": int(idx_np.nbytes),
                      "gathers": steps}))


def alg_bytes(A, N, K, dt):
    m, n, nnz = A.m, A.n, A.nnz
    s_v, s_ci = ESZ[dt], A.col_idx.dtype.itemsize
    s_ri = 2 if m <= 32767 else 4
    s_riT = 2 if n <= 32767 else 4
    col = A.col_idx.astype(np.int64)
    kp = len(np.unique(col))
    mp = int(np.count_nonzero(A.row_counts()))
    return {
        "spmm": nnz * (s_v + s_ci) + 4 * (m + 1) + m * s_ri + kp * N * s_v + m * N * 4,
        "spmv": nnz * (s_v + s_ci) + 4 * (m + 1) + m * s_ri + kp * s_v + m * 4,
        "sddmm": nnz * s_ci + 4 * (m + 1) + m * s_ri + mp * K * s_v + kp * K * s_v + nnz * 4,
        "csr_add": nnz * (s_v + s_ci) + 4 * (m + 1) + m * s_ri + 2 * nnz * s_v,
        "transpose": nnz * (s_v + s_ci) + 4 * (m + 1) + nnz * (s_v + s_riT) + 4 * (n + 1),
        "row_order": 4 * (n + 1) + n * s_riT,
    }


def flops(A, N, K):
    return {"spmm": 2 * A.nnz * N, "spmv": 2 * A.nnz, "sddmm": 2 * A.nnz * K}


def kernel_sources_sha(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "unstructured_sparse_linear_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


KERNEL_FILES = {"spmm": ["spmm.hip", "common.h"], "spmv": ["spmm.hip", "common.h"],
                "sddmm": ["sddmm.hip", "sddmm_dense.hip", "common.h"],
                "csr_add": ["csr_add.hip", "common.h"], "transpose": ["radix.hip", "common.h"],
                "row_order": ["radix.hip", "common.h"]}


MFMA_COUNTERS = os.path.join(ROOT, "profiles", "mfma_busy.json")


def mfma_busy_for(op, config, dt):
    """MFMA busy fraction of the structure-aware SDDMM's tile kernel from the
    committed counter run (profiles/mfma_busy.json, keyed "config3_f16"),
    while the kernel sources still match the ones it was taken on; else None."""
    if op != "sddmm" or not os.path.exists(MFMA_COUNTERS):
        return None
    ent = json.load(open(MFMA_COUNTERS)).get(f"config{config}_{dt}")
    if not ent or ent.get("source_sha") != kernel_sources_sha(KERNEL_FILES[op]):
        return None
    return ent.get("mfma_busy_frac")


def transpose_kernels(n, nnz):
    """Kernels of one csr_transpose (up to 2^17 columns: count with row
    expansion, a scan of the count table above 128 tiles of 2048 entries,
    scatter, bucket finish; wider: full LSD passes)."""
    if n > 1 << 17:
        return ["expand_rows_kernel", "radix_count_kernel", "scan_*", "radix_scatter_kernel",
                "transpose_finish_kernel"]
    tiles = -(-nnz // 2048)
    scan = ([] if tiles <= 128 else ["scan_single_kernel"] if tiles * 256 <= 65536
            else ["scan_local_kernel", "scan_add_kernel"])
    return ["transpose_count_kernel"] + scan + ["radix_scatter_kernel", "transpose_bucket_kernel"]


def op_kernels(spmm_info, sddmm_info, m, n, nnz, K=0, esz=2):
    """Kernels one call of each operation launches (names as in rocprofv3).
    The structure-aware SDDMM adds its remainder's K pieces with a third
    kernel when BT (n x K, 16-bit) exceeds 32 MiB."""
    spmm = ["spmm_kernel"] + (["spmm_fixup_kernel"] if spmm_info.get("chunks", 0) else [])
    # N == 1: entry-range blocks through LDS when the plan finds the rows
    # balanced (longest row <= 2 * mean + 32) and short (<= 128 entries),
    # else a group of lanes per row
    mr = spmm_info.get("max_row_nnz", 0)
    balanced = m > 0 and 0 < mr <= min(128, 2 * (nnz // m) + 32)
    spmv = (["spmv_flat_kernel"] if balanced and not spmm_info.get("chunks", 0)
            else ["spmv_kernel"] + (["spmm_fixup_kernel"] if spmm_info.get("chunks", 0) else []))
    pieces = (sddmm_info.get("tiles", 0) and sddmm_info.get("rest_nnz", 0) and esz == 2
              and n * K * 2 > (32 << 20))
    sddmm = ((["sddmm_tile_kernel"] if sddmm_info.get("tiles", 0) else [])
             + (["sddmm_list_kernel"] if sddmm_info.get("rest_nnz", 0) else [])
             + (["sddmm_piece_sum_kernel"] if pieces else []))
    return {"spmm": spmm, "spmv": spmv, "sddmm": sddmm or ["sddmm_list_kernel"],
            "csr_add": ["csr_add_kernel"],
            "transpose": transpose_kernels(n, nnz),
            # the row order of A^T (n rows, keys up to m)
            "row_order": (["sort_rows_block_kernel"] if n <= 16384 and m <= 65535
                          else ["transpose_count_kernel", "radix_scatter_kernel",
                                "store_perm_kernel"] if -(-n // 2048) <= 128
                          else ["radix_count_kernel", "scan_*", "radix_scatter_kernel",
                                "store_perm_kernel"])}


def traffic_for(op, config, dt=None):
    """HBM bytes per call (all the operation's kernels) from committed
    rocprofv3 counter runs, if they were taken on the current kernel source;
    else None.  Keyed by workload ("config3_f16") or config ("config3")."""
    try:
        with open(COUNTERS) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = (rec.get(f"config{config}_{dt}", {}) if dt else {}).get(op) or \
        rec.get(f"config{config}", {}).get(op)
    if not ent or ent.get("source_sha") != kernel_sources_sha(KERNEL_FILES[op]):
        return None
    return ent.get("hbm_bytes_per_launch")


def cpu_baseline(w, A, dt, N, K, ops, oracle):
    """The float64 oracle on the host cores, same workload, one warm-up then
    the median of 3 runs per operation."""
    B, Ad, BT, W = w.get("B"), w.get("Ad"), w.get("BT"), w.get("W")
    B1 = w.get("B1") if "spmv" in ops else None
    ab = alg_bytes(A, N, K, dt)
    fns = {
        "spmm": lambda: oracle.spmm(A.m, A.row_offsets, A.col_idx, A.values, dt, B, dt),
        "spmv": lambda: oracle.spmm(A.m, A.row_offsets, A.col_idx, A.values, dt, B1, dt),
        "sddmm": lambda: oracle.sddmm(A.row_offsets, A.col_idx, Ad, BT, dt),
        "csr_add": lambda: oracle.csr_add(A.row_offsets, A.col_idx, A.values, dt, W, dt),
        "transpose": lambda: oracle.csr_transpose(A.m, A.n, A.row_offsets, A.col_idx, A.values),
        "row_order": lambda: oracle.row_idx(tro),
    }
    _, tro, _ = oracle.csr_transpose(A.m, A.n, A.row_offsets, A.col_idx, None)
    per, total_s, total_b = {}, 0.0, 0
    for op in ops:
        fns[op]()
        ts = []
        for _ in range(3):
            t0 = time.perf_counter()
            fns[op]()
            ts.append(time.perf_counter() - t0)
        t = float(np.median(ts))
        per[op] = round(t * 1e3, 3)
        total_s += t
        total_b += ab[op]
    return {"value": round(total_b / total_s / 1e9, 3), "unit": "GB/s",
            "cores": oracle.num_threads(), "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"the full workload (all {len(ops)} operations, one pass each), "
                      "median of 3 after 1 warm-up",
            "ms_per_op": per, "ms_per_step": round(total_s * 1e3, 3)}


def adapter_step(S, w, A, dt, N, dev, flush, args):
    """One training step of the sparse layer Y^T = S . X^T with S = A (values
    A.values, pattern A) and X^T = the workload's dense B (k x N): forward,
    the gradients of the stored values (SDDMM of dY^T and X^T) and of X^T
    (S^T's values by the pattern's transpose permutation, then S^T . dY^T),
    a masked Adam step on the values, and the merge W += S;
    outputs in the input dtype, as the autograd layer produces them.
    Captured as a HIP graph, cold caches."""
    import torch
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dt]

    def to(x, d=None):
        if d == "bf16":
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(
                torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    m, n = A.m, A.n
    v, ro, ci = to(A.values, dt), to(A.row_offsets), to(A.col_idx)
    P = S.SparsePattern(ro, ci, m, n)
    xt = to(w.get("B"), dt)                   # X^T: in_features x tokens
    if w.get("Ad").shape != (m, N):
        return None
    dyt = to(w.get("Ad"), dt)                 # dY^T: out_features x tokens (synthetic)
    W = to(w.get("W"), dt) if w.get("W").shape == (m, n) else None
    yt = torch.empty((m, N), dtype=tdt, device=dev)
    dv = torch.empty_like(v)
    vT = torch.empty_like(v)
    dxt = torch.empty((n, N), dtype=tdt, device=dev)

    m1 = torch.zeros(A.nnz, dtype=torch.float32, device=dev)
    m2 = torch.zeros_like(m1)

    def run():
        S.spmm(v, P.ro, P.ri, P.ci, xt, m, out_dtype=tdt, plan=P.spmm_plan, out=yt)
        S.sddmm(P.ro, P.ri, P.ci, dyt, xt, plan=P.sddmm_plan, out_dtype=tdt, out=dv)
        P.transposed_values(v, out=vT)
        S.spmm(vT, P.roT, P.riT, P.ciT, dyt, n, out_dtype=tdt, plan=P.spmmT_plan, out=dxt)
        # optimizer step on the values (the step number is fixed in the graph)
        S.masked_adam(v, dv, m1, m2, 1, lr=1e-4)
        if W is not None:
            S.csr_add(v, P.ro, P.ri, P.ci, W)

    for _ in range(2):
        run()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()

    def untimed_step():
        if not args.no_flush:
            flush()
        graph.replay()
    settle(untimed_step, args.settle_ms)
    stream = torch.cuda.current_stream(dev)
    ts = []
    for _ in range(max(args.steps, 5)):
        if not args.no_flush:
            flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    t = float(np.mean(ts))
    s_v, s_ci = ESZ[dt], A.col_idx.dtype.itemsize
    s_ri, s_riT = (2 if m <= 32767 else 4), (2 if n <= 32767 else 4)
    kp = len(np.unique(A.col_idx))
    mp = int(np.count_nonzero(A.row_counts()))
    nnz = A.nnz
    parts = {
        "forward_spmm": nnz * (s_v + s_ci) + 4 * (m + 1) + m * s_ri + kp * N * s_v + m * N * s_v,
        "grad_values_sddmm": nnz * s_ci + 4 * (m + 1) + m * s_ri + mp * N * s_v + kp * N * s_v
        + nnz * s_v,
        # S^T's values: S's values through the transpose's permutation (found
        # once with the pattern): read the permutation and the values, write
        "transposed_values": nnz * (4 + 2 * s_v),
        "grad_input_spmm": nnz * (s_v + s_riT) + 4 * (n + 1) + n * s_riT + mp * N * s_v
        + n * N * s_v,
    }
    parts["masked_adam"] = nnz * (3 * s_v + 16)
    if W is not None:
        parts["merge_csr_add"] = nnz * (s_v + s_ci) + 4 * (m + 1) + m * s_ri + 2 * nnz * s_v
    total = sum(parts.values())
    return {"ms": round(t, 4), "alg_bytes": int(total), "gbps": round(total / t / 1e6, 1),
            "frac_hbm": round(total / t / 1e6 / HBM_PEAK_GBS, 4),
            "steps": list(parts), "tokens": N,
            "layout": "feature-major (X^T in_features x tokens), outputs in the input dtype",
            "step": "hip graph replay, cold caches"}


def cg_solve(S, w, A, dev, args):
    """Conjugate gradients on the workload's SPD matrix (A, f32) with b = the
    SpMV vector, rtol 1e-6, convergence checked every 16 iterations.  Per
    iteration: one SpMV and three vector kernels (p.q; x and r; p).  The
    matrix stays in the caches between iterations, as in any solve, so only
    the first iteration starts cold."""
    import torch

    if w.dt != "f32" or A.m != A.n or "B1" not in w._builders:
        return None
    m = A.m
    v = torch.from_numpy(A.values).to(dev)
    ro = torch.from_numpy(A.row_offsets).to(dev)
    ci = torch.from_numpy(A.col_idx).to(dev)
    ri = S.sort_rows_by_nnz(ro, A.n)
    plan = S.SpmmPlan(ro, ri, ci, m)
    b = torch.from_numpy(np.ascontiguousarray(w.get("B1")[:, 0])).to(dev)
    x = torch.zeros_like(b)
    S.cg(v, ro, ri, ci, b, x=x.zero_(), rtol=1e-6, max_iter=1000, check_every=16, plan=plan)
    torch.cuda.synchronize()
    ts, iters, rel = [], 0, 0.0
    for _ in range(max(3, min(args.steps, 10))):
        x.zero_()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        _, iters, rel = S.cg(v, ro, ri, ci, b, x=x, rtol=1e-6, max_iter=1000, check_every=16,
                             plan=plan)
        torch.cuda.synchronize()
        ts.append(time.perf_counter() - t0)
    t = float(np.median(ts))
    s_ci = A.col_idx.dtype.itemsize
    kp = len(np.unique(A.col_idx))
    spmv = A.nnz * (4 + s_ci) + 4 * (m + 1) + kp * 4 + m * 4
    per_iter = spmv + 11 * 4 * m          # p.q: 2 reads; x, r: 4 reads 2 writes; p: 2 + 1
    return {"iterations": iters, "rel_residual": rel, "rtol": 1e-6, "ms": round(t * 1e3, 3),
            "us_per_iteration": round(t * 1e6 / max(iters, 1), 2),
            "alg_bytes_per_iteration": int(per_iter),
            "gbps": round(per_iter * iters / t / 1e9, 1),
            "frac_hbm": round(per_iter * iters / t / 1e9 / HBM_PEAK_GBS, 4),
            "timing": "host wall clock around the call (it synchronizes at its checks)"}


def delta_spmv_bench(S, dev, flush, args):
    """SpMV on the 2-bit delta-coded rows against CSR SpMV, same matrix: the
    8192 x 8192 size of the UST page's MACKO experiment at 50% and 90%
    density, f16 values, cold caches, HIP events around each call."""
    import torch
    from unstructured_sparse_linear_amd import gen

    out = {}
    for density in (0.5, 0.9):
        A = gen.random_csr(20, 8192, 8192, density, "f16")
        v = torch.from_numpy(A.values).to(dev)
        ro = torch.from_numpy(A.row_offsets).to(dev)
        ci = torch.from_numpy(A.col_idx).to(dev)
        x = torch.from_numpy(gen.dense(20, 100, gen.S_B, (8192,), "f16")).to(dev)
        D = S.delta_encode(v, ro, ci, A.m, A.n)
        ri = S.sort_rows_by_nnz(ro, A.n)
        plan = S.SpmmPlan(ro, ri, ci, A.n)
        y = torch.empty(A.m, dtype=torch.float32, device=dev)
        y2 = torch.empty((A.m, 1), dtype=torch.float32, device=dev)
        x2 = x.reshape(-1, 1)
        runs = {"delta": lambda: S.delta_spmv(D, x, out=y),
                "csr": lambda: S.spmm(v, ro, ri, ci, x2, A.m, plan=plan, out=y2)}
        words = (D.entries + 15) // 16
        byts = {"delta": D.entries * 2 + 4 * words + 4 * (A.m + 1) + 2 * A.n + 4 * A.m,
                "csr": A.nnz * 4 + 4 * (A.m + 1) + 2 * A.m + 2 * A.n + 4 * A.m}
        res = {}
        for name, fn in runs.items():
            fn()
            torch.cuda.synchronize()
            ts = []
            for _ in range(max(args.steps, 5)):
                if not args.no_flush:
                    flush()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                fn()
                e1.record()
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
            t = float(np.mean(ts))
            res[name] = {"ms": round(t, 4), "alg_bytes": int(byts[name]),
                         "gbps": round(byts[name] / t / 1e6, 1),
                         "frac_hbm": round(byts[name] / t / 1e6 / HBM_PEAK_GBS, 4)}
        res["nnz"] = A.nnz
        res["encoded_entries"] = D.entries
        out[f"density_{density}"] = res
        del D, v, ro, ci
    return out


def measure_ceilings(dev, flush):
    """Rates that bound the gather-shaped kernels, measured with the
    measurement library (libspops_ceilings.so): a plain 256 MiB device copy
    after a cache flush, and row gathers (16-byte lanes, a wave per row and
    half a wave per 512-byte row, 8 rows in flight per lane) of 512 B, 1 KiB
    and 4 KiB rows at random indices, from
    a 2 MiB slice per XCD (L2-resident) and from one 16 MiB source shared by
    all XCDs (Infinity Cache), warm, 5 back-to-back launches; and the on-chip
    rates of the kernels' inner loops, from the same library: 16-byte LDS
    reads without bank conflicts, v_fma_f32 and v_dot2_f32_f16 (eight
    independent chains per lane; 2 and 4 flops per instruction), 2048
    workgroups of 256 threads, 5 back-to-back launches after one."""
    import ctypes

    import torch

    path = os.path.join(ROOT, "unstructured_sparse_linear_amd", "libspops_ceilings.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not built; run __graft_entry__.build()")
    L = ctypes.CDLL(path)
    f = L.spops_ceil_gather
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                  ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int
    stream = torch.cuda.current_stream(dev)
    out = {}
    a = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    ts = []
    for _ in range(5):
        flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        b.copy_(a)
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    out["copy_gbps"] = round(2 * (256 << 20) / float(np.median(ts)) / 1e6, 1)
    del a, b
    src = torch.empty(16 << 20, dtype=torch.uint8, device=dev)
    src.fill_(3)
    blocks = 2048
    sink = torch.empty(blocks * 256, dtype=torch.int32, device=dev)
    rng = np.random.default_rng(0)
    for rb in (512, 1024, 4096):
        per_wave = {512: 128, 1024: 64, 4096: 16}[rb]
        waves = blocks * 4
        for sliced, label in ((1, "l2"), (0, "ic")):
            rows = (2 << 20) // rb if sliced else (16 << 20) // rb
            idx = torch.from_numpy(rng.integers(0, rows, waves * per_wave).astype(np.int32)).to(dev)
            args = (src.data_ptr(), rows, rb, sliced, idx.data_ptr(), per_wave, blocks,
                    sink.data_ptr(), ctypes.c_void_p(stream.cuda_stream))
            assert f(*args) == 0
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(5):
                f(*args)
            e1.record(stream)
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) / 5
            name = f"{rb // 1024}kib" if rb >= 1024 else f"{rb}b"
            out[f"gather_{label}_{name}_gbps"] = round(waves * per_wave * rb / t / 1e6, 1)

    def rate(launch, work):
        assert launch() == 0
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(5):
            assert launch() == 0
        e1.record(stream)
        torch.cuda.synchronize()
        return work * 5 / (e0.elapsed_time(e1) * 1e-3)

    st = ctypes.c_void_p(stream.cuda_stream)
    L.spops_ceil_lds.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    L.spops_ceil_valu.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p,
                                  ctypes.c_void_p]
    threads, iters = blocks * 256, 400
    out["lds_read_gbps"] = round(rate(lambda: L.spops_ceil_lds(blocks, iters, sink.data_ptr(), st),
                                      threads * iters * 128) / 1e9, 1)
    out["valu_fma_f32_tflops"] = round(rate(
        lambda: L.spops_ceil_valu(0, blocks, iters, sink.data_ptr(), st),
        threads * iters * 32 * 2) / 1e12, 1)
    out["valu_dot2_f16_tflops"] = round(rate(
        lambda: L.spops_ceil_valu(1, blocks, iters, sink.data_ptr(), st),
        threads * iters * 32 * 4) / 1e12, 1)
    return out


def gathered_bytes(op, A, N, K, dt, tiles=0):
    """Bytes the operation gathers on chip (one operand row segment per
    stored entry) and the size of one gathered segment.  A structure-aware
    SDDMM with dense tiles does not gather per entry (its figure is the
    tile kernel's MFMA busy): none."""
    s = ESZ[dt]
    if op in ("spmm", "spmv"):
        n_ = N if op == "spmm" else 1
        return A.nnz * n_ * s, min(n_ * s, 1024)
    if op == "sddmm" and not tiles:
        return A.nnz * K * s, K * s
    return 0, 0


def measure_case(S, cfg, dt, op, dev, flush, reps, args, ceil=None, oracle=None):
    """One gated case alone: plan built untimed, then `reps` cold calls (each
    after the cache flush) bracketed by HIP events on the current stream.
    With `oracle`, the float64 oracle of the same operation on the host
    (one warm-up, median of 3)."""
    import torch
    from unstructured_sparse_linear_amd import gen

    w = gen.make_config(cfg, dt=dt if cfg == 3 else None)
    A = w.get("A")
    dt = w.dt

    def to(x, d=None):
        if d == "bf16":
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(
                torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    ro, ci = to(A.row_offsets), to(A.col_idx)
    ri = S.sort_rows_by_nnz(ro, A.n)
    N, K = 1, w.K
    t0 = time.perf_counter()
    if op in ("spmm", "spmv"):
        v = to(A.values, dt)
        Bh = w.get("B1") if op == "spmv" else w.get("B")
        B = to(Bh, dt)
        N = B.shape[1]
        plan = S.SpmmPlan(ro, ri, ci, A.n)
        out = torch.empty((A.m, N), dtype=torch.float32, device=dev)
        ws = plan.workspace(N, dev)
        fn = lambda: S.spmm(v, ro, ri, ci, B, A.m, plan=plan, out=out)  # noqa: E731
        info = plan.info()
    else:
        Ad, BT = to(w.get("Ad"), dt), to(w.get("BT"), dt)
        plan = S.SddmmPlan(ro, ci, A.m, A.n)
        out = torch.empty(A.nnz, dtype=torch.float32, device=dev)
        fn = lambda: S.sddmm(ro, ri, ci, Ad, BT, plan=plan, out=out)  # noqa: E731
        info = plan.info()
    torch.cuda.synchronize()
    plan_ms = (time.perf_counter() - t0) * 1e3
    fn()
    torch.cuda.synchronize()

    def flushed_call():
        if not args.no_flush:
            flush()
        fn()
    settle(flushed_call, args.settle_ms)
    stream = torch.cuda.current_stream(dev)
    evs = []
    for _ in range(reps):
        if not args.no_flush:
            flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) for a, b in evs)
    t = float(np.median(ts))
    wevs = []
    for _ in range(5):  # back to back, no flush
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        wevs.append((e0, e1))
    torch.cuda.synchronize()
    warm = [a.elapsed_time(b) for a, b in wevs]
    ab = alg_bytes(A, N, K, dt)[op if op != "spmv" else "spmv"]
    fl = flops(A, N, K)[op]
    traffic = traffic_for(op, cfg, dt)
    ent = {"workload": w.name if cfg == 3 else gen.CONFIG_NAMES[cfg], "op": op, "dtype": dt,
           "out_dtype": "f32", "backend": "structure_aware" if op == "sddmm" else None,
           "m": A.m, "n": A.n, "nnz": A.nnz, "N_or_K": N if op in ("spmm", "spmv") else K,
           "kernels": op_kernels(info if op != "sddmm" else {}, info if op == "sddmm" else {},
                                 A.m, A.n, A.nnz, K, ESZ[dt])[op],
           "plan": info, "plan_ms": round(plan_ms, 2),
           "us_median": round(t * 1e3, 2), "us_p10": round(ts[len(ts) // 10] * 1e3, 2),
           "us_p90": round(ts[(9 * len(ts)) // 10] * 1e3, 2),
           "us_warm_median": round(float(np.median(warm)) * 1e3, 2),
           "alg_bytes": int(ab), "flops": int(fl), "gbps": round(ab / t / 1e6, 1),
           "frac_hbm": round(ab / t / 1e6 / HBM_PEAK_GBS, 4),
           "frac_hbm_copy": (round(ab / t / 1e6 / ceil["copy_gbps"], 4)
                             if ceil and ceil.get("copy_gbps") else None),
           "gflops": round(fl / t / 1e6, 1),
           "hbm_bytes_counters": traffic,
           "traffic_ratio": round(traffic / ab, 2) if traffic else None,
           "hbm_gbps_counters": round(traffic / t / 1e6, 1) if traffic else None,
           "mfma_busy": mfma_busy_for(op, cfg, dt)}
    gb, seg = gathered_bytes(op, A, N, K, dt, info.get("tiles", 0) if op == "sddmm" else 0)
    if ceil and gb:
        key = ("gather_l2_4kib_gbps" if seg > 2048 else "gather_l2_1kib_gbps" if seg > 512
               else "gather_l2_512b_gbps")
        rate = gb / t / 1e6
        ent["gather_rate_gbps"] = round(rate, 1)
        ent["frac_of_gather_ceiling"] = round(rate / ceil[key], 4)
        ent["gather_ceiling"] = key
    if oracle is not None:
        if op in ("spmm", "spmv"):
            f = lambda: oracle.spmm(A.m, A.row_offsets, A.col_idx, A.values, dt, Bh, dt)  # noqa
        else:
            Adh, BTh = w.get("Ad"), w.get("BT")
            f = lambda: oracle.sddmm(A.row_offsets, A.col_idx, Adh, BTh, dt)  # noqa
        f()
        cts = []
        for _ in range(3):
            c0 = time.perf_counter()
            f()
            cts.append(time.perf_counter() - c0)
        ct = float(np.median(cts))
        ent["oracle_ms"] = round(ct * 1e3, 2)
        ent["oracle_gbps"] = round(ab / ct / 1e9, 3)
        ent["oracle_threads"] = oracle.num_threads()
        ent["gpu_over_oracle"] = round(ct * 1e3 / t, 1)
    return ent


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def write_records(path, result, args, A, dt, N, K, ab, fl):
    """One record per operation with the fields of the measurement plan:
    times (cold median / p10 / p90, warm), rates against the nominal HBM
    peak and the measured copy rate, counter traffic where committed for
    these kernel sources, the plan time and the CPU oracle's time.  Accuracy
    fields stay null here: parity is checked by the tests, not the bench."""
    copy = (result.get("ceilings") or {}).get("copy_gbps")
    cpu = result.get("cpu_baseline") or {}
    plans = result["plans"]
    with open(path, "a") as f:
        for op, b in result["ops_breakdown"].items():
            t = b["ms"]
            traffic = traffic_for(op, args.config, dt) if op in KERNEL_FILES else None
            rec = {
                "config": args.config, "workload": result["config"]["workload"], "op": op,
                "dtype": dt, "out_dtype": "f32" if op in ("spmm", "spmv", "sddmm") else dt,
                "backend": "structure_aware" if op == "sddmm" else None,
                "tau": None if op != "sddmm" else "default",
                "m": A.m, "n": A.n,
                "N_or_K": {"spmm": N, "spmv": 1, "sddmm": K}.get(op),
                "nnz": A.nnz, "alg_bytes": b["alg_bytes"], "flops": fl.get(op),
                "t_med_us": round(t * 1e3, 2), "t_p10_us": round(b["ms_p10"] * 1e3, 2),
                "t_p90_us": round(b["ms_p90"] * 1e3, 2),
                "t_warm_med_us": round(b["ms_warm"] * 1e3, 2),
                "plan_us": (round(result["plan_ms"]["sddmm_partition"] * 1e3, 1) if op == "sddmm"
                            else round(result["plan_ms"]["spmm_schedule_and_row_order"] * 1e3, 1)
                            if op in ("spmm", "spmv") else None),
                "gbps_alg": b["gbps"], "gflops": b.get("gflops"),
                "frac_hbm_nominal": b["frac_hbm"],
                "frac_hbm_copy": round(b["gbps"] / copy, 4) if copy else None,
                "hbm_bytes_counters": traffic,
                "refetch": round(traffic / b["alg_bytes"], 2) if traffic else None,
                "mfma_busy": mfma_busy_for(op, args.config, dt),
                "oracle_s": (cpu.get("ms_per_op", {}).get(op, 0) / 1e3) if cpu else None,
                "oracle_threads": cpu.get("cores"), "cpu_model": cpu_model() if cpu else None,
                "max_rel_err": None, "normwise_err": None, "bitexact_idx": None,
                "seed": 0,
                "kernel_sources_sha": kernel_sources_sha(KERNEL_FILES.get(op, ["common.h"])),
                "plan": plans["sddmm"] if op == "sddmm" else plans["spmm"],
            }
            f.write(json.dumps(rec) + "\n")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards without collectives; see the design notes)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.steps)
        return
    import torch

    import unstructured_sparse_linear_amd as S
    from unstructured_sparse_linear_amd import gen

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    S.lib()
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    ops = [o for o in args.ops.split(",") if o]
    if args.config == 4 and "spmm" in ops and "spmv" not in ops:
        ops.insert(ops.index("spmm") + 1, "spmv")  # config 4 names both N = 1 and N = 32

    w = gen.make_config(args.config,
                        dt=args.dtype or (DEFAULT_DTYPE if args.config == 3 else None))
    A = w.get("A")
    dt = w.dt
    N = w.N[-1]
    K = w.K
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dt]

    def to(x, d=None):
        if d == "bf16":
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(
                torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    v, ro, ci = to(A.values, dt), to(A.row_offsets), to(A.col_idx)
    B = to(w.get("B"), dt)
    B1 = to(w.get("B1"), dt) if "spmv" in ops else None
    Ad, BT = to(w.get("Ad"), dt), to(w.get("BT"), dt)
    Wd = to(w.get("W"), dt) if "csr_add" in ops else None
    if args.config == 4 and Wd is not None:
        A_add = gen.csr_row_slab(A, 0, Wd.shape[0])
        va, roa, cia = to(A_add.values, dt), to(A_add.row_offsets), to(A_add.col_idx)
    else:
        A_add, va, roa, cia = A, v, ro, ci
    m, n = A.m, A.n

    # plans and row order, once per pattern (not timed)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ri = S.sort_rows_by_nnz(ro, n)
    spmm_plan = S.SpmmPlan(ro, ri, ci, n)
    torch.cuda.synchronize()
    t_spmm_plan = time.perf_counter() - t0
    t0 = time.perf_counter()
    sddmm_plan = S.SddmmPlan(ro, ci, m, n)
    torch.cuda.synchronize()
    t_sddmm_plan = time.perf_counter() - t0
    ri_add = ri if A_add is A else S.sort_rows_by_nnz(roa, n)
    C = torch.empty((m, N), dtype=torch.float32, device=dev)
    C1 = torch.empty((m, 1), dtype=torch.float32, device=dev)
    out = torch.empty(A.nnz, dtype=torch.float32, device=dev)
    tws = S.csr_transpose_workspace(m, n, A.nnz, dev)
    sws = S.sort_rows_workspace(n, m, dev)
    vT = torch.empty_like(v)
    roT = torch.empty(n + 1, dtype=torch.int32, device=dev)
    ciT = torch.empty(A.nnz, dtype=torch.int16 if m <= 32767 else torch.int32, device=dev)
    riT = torch.empty(n, dtype=torch.int16 if n <= 32767 else torch.int32, device=dev)
    flush = Flush(dev, args.flush)
    ws = spmm_plan.workspace(N, dev)
    from unstructured_sparse_linear_amd import spops as SP

    def run_op(op):
        if op == "spmm":
            S.spmm(v, ro, ri, ci, B, m, plan=spmm_plan, out=C)
        elif op == "spmv":
            S.spmm(v, ro, ri, ci, B1, m, plan=spmm_plan, out=C1)
        elif op == "sddmm":
            S.sddmm(ro, ri, ci, Ad, BT, plan=sddmm_plan, out=out)
        elif op == "csr_add":
            S.csr_add(va, roa, ri_add, cia, Wd)
        elif op == "transpose":
            import ctypes
            d = SP.csr_desc(v, ro, None, ci, m, n)
            SP._check("spops_csr_transpose", SP.lib().spops_csr_transpose(
                ctypes.byref(d), vT.data_ptr(), roT.data_ptr(), ciT.data_ptr(),
                SP._IT[ciT.dtype], tws.data_ptr(), tws.numel(), SP._stream(ro)))
        elif op == "row_order":
            S.sort_rows_by_nnz(roT, m, workspace=sws, out=riT)
    del ws

    stream = torch.cuda.current_stream(dev)

    def cold():
        if not args.no_flush:
            flush()

    def ev():
        return torch.cuda.Event(enable_timing=True)

    for _ in range(args.warmup):
        cold()
        for op in ops:
            run_op(op)
    torch.cuda.synchronize()

    def warm_step():
        cold()
        for op in ops:
            run_op(op)
    settle(warm_step, args.settle_ms)

    # per-operation cold timing (eager)
    per_op = {op: [] for op in ops}
    for _ in range(args.steps):
        for op in ops:
            cold()
            e0, e1 = ev(), ev()
            e0.record(stream)
            run_op(op)
            e1.record(stream)
            per_op[op].append((e0, e1))
    torch.cuda.synchronize()
    per_op = {op: [a.elapsed_time(b) for a, b in v] for op, v in per_op.items()}

    # per-operation warm timing: 10 back-to-back calls between two events
    # (no flush, so the working set sits in the Infinity Cache), 3 times
    warm = {}
    for op in ops:
        reps = []
        for _ in range(3):
            e0, e1 = ev(), ev()
            e0.record(stream)
            for _ in range(10):
                run_op(op)
            e1.record(stream)
            torch.cuda.synchronize()
            reps.append(e0.elapsed_time(e1) / 10)
        warm[op] = float(np.median(reps))

    # the whole step, captured once and replayed
    # Independent operations run on separate streams inside the graph (fork
    # from the capturing stream, join at the end of the step): with two
    # streams the two gather-bound products share one, longest (by the cold
    # times just measured) first, and the short launch-bound operations
    # (csr_add, transpose, then the row order of A^T, which needs the
    # transpose) take the other; with three, SpMM and SDDMM get one each.
    # Default stream priorities.
    graph = None
    side_ops = [o for o in ops if o in ("csr_add", "transpose", "row_order")]
    main_ops = sorted([o for o in ops if o not in side_ops],
                      key=lambda o: -float(np.median(per_op[o])))
    nstreams = 1 if args.serial_step or not side_ops or not main_ops else args.streams
    lanes = ([ops] if nstreams == 1 else [main_ops, side_ops] if nstreams == 2
             else [[o] for o in main_ops] + [side_ops])
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        extra = [torch.cuda.Stream(device=dev) for _ in lanes[1:]]
        with torch.cuda.graph(graph):
            cur = torch.cuda.current_stream(dev)
            for st in extra:
                st.wait_stream(cur)
            for st, lane_ops in zip(extra, lanes[1:]):
                with torch.cuda.stream(st):
                    for op in lane_ops:
                        run_op(op)
            for op in lanes[0]:
                run_op(op)
            for st in extra:
                cur.wait_stream(st)
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream(dev)

    def step():
        cold()
        e0, e1 = ev(), ev()
        e0.record(stream)
        if graph is not None:
            graph.replay()
        else:
            for op in ops:
                run_op(op)
        e1.record(stream)
        return e0, e1

    step()
    torch.cuda.synchronize()

    def untimed_step():
        cold()
        if graph is not None:
            graph.replay()
        else:
            for op in ops:
                run_op(op)
    settle(untimed_step, args.settle_ms)
    events = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        events.append(step())
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = [a.elapsed_time(b) for a, b in events]
    ab = alg_bytes(A, N, K, dt)
    if args.config == 4:
        ab["csr_add"] = alg_bytes(A_add, N, K, dt)["csr_add"]
    fl = flops(A, N, K)
    mean_step = float(np.mean(step_ms))
    total_bytes = sum(ab[o] for o in ops)
    total_flops = sum(fl.get(o, 0) for o in ops)
    breakdown = {}
    for op in ops:
        t = float(np.median(per_op[op]))
        breakdown[op] = {"ms": round(t, 4), "ms_p10": round(float(np.percentile(per_op[op], 10)), 4),
                         "ms_p90": round(float(np.percentile(per_op[op], 90)), 4),
                         "alg_bytes": int(ab[op]), "gbps": round(ab[op] / t / 1e6, 1),
                         "frac_hbm": round(ab[op] / t / 1e6 / HBM_PEAK_GBS, 4)}
        if op in fl:
            breakdown[op]["gflops"] = round(fl[op] / t / 1e6, 1)
        breakdown[op]["ms_warm"] = round(warm[op], 4)
    # the headline operation: the longer of the operations the workload names
    # (its kernels listed together: long rows split, dense tiles plus the
    # remainder)
    kernels = op_kernels(spmm_plan.info(), sddmm_plan.info(), m, A.n, A.nnz, K, ESZ[dt])
    gated = [o for o in ops if o in NAMED_OPS[args.config]]
    dom = max(gated or ops, key=lambda o: breakdown[o]["ms"])
    achieved = ab[dom] / breakdown[dom]["ms"] / 1e6
    traffic = traffic_for(dom, args.config, dt)
    result = {
        "metric": "SpMM/SDDMM effective HBM GB/s and GFLOP/s (2*nnz*N), % of HBM roofline",
        "value": round(achieved, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(mean_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "f16": "f16-in/f32-acc", "bf16": "bf16-in/f32-acc"}[dt],
        "data": "synthetic (seeded generators, seed 0)",
        "config": {"workload": w.name, "config_id": args.config, "m": m, "n": n, "nnz": A.nnz,
                   "N": N, "K": K, "value_dtype": dt, "ops": ops,
                   "caches": "warm" if args.no_flush else
                   f"cold (512 MiB {args.flush} before each timed call)",
                   "settle_ms": args.settle_ms,
                   "step": "eager" if args.no_graph else
                   "hip graph replay, streams: " + " | ".join("+".join(x) for x in lanes)},
        "value_op": {"op": dom, "us": round(breakdown[dom]["ms"] * 1e3, 2),
                     "alg_bytes": int(ab[dom]), "gflops": breakdown[dom].get("gflops"),
                     "frac_hbm": round(achieved / HBM_PEAK_GBS, 4),
                     "timing": "cold median over the steps, HIP events on the library's stream"},
        "eager_sum_of_ops_ms": round(sum(float(np.mean(v)) for v in per_op.values()), 4),
        "step_gbps_all_ops": round(total_bytes / mean_step / 1e6, 2),
        "step_gflops": round(total_flops / mean_step / 1e6, 1),
        "wall_ms_per_step_incl_flush": round(wall / args.steps * 1e3, 4),
        "ms_per_step_p10_p90": [round(float(np.percentile(step_ms, 10)), 4),
                                round(float(np.percentile(step_ms, 90)), 4)],
        "ops_breakdown": breakdown,
        "plan_ms": {"spmm_schedule_and_row_order": round(t_spmm_plan * 1e3, 2),
                    "sddmm_partition": round(t_sddmm_plan * 1e3, 2)},
        "plans": {"spmm": spmm_plan.info(), "sddmm": sddmm_plan.info()},
        "roofline": {"bound": "hbm", "kernel": "+".join(kernels[dom]), "op": dom,
                     "launch_us": round(breakdown[dom]["ms"] * 1e3, 2),
                     "alg_bytes_per_launch": int(ab[dom]),
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "traffic_ratio": round(traffic / ab[dom], 2) if traffic else None,
                     # the bandwidth the HBM byte counters imply (traffic over the
                     # same cold time) and its fraction of the peak
                     "traffic_gbps": (round(traffic / breakdown[dom]["ms"] / 1e6, 1)
                                      if traffic else None),
                     "traffic_frac": (round(traffic / breakdown[dom]["ms"] / 1e6 / HBM_PEAK_GBS,
                                            4) if traffic else None),
                     "mfma_busy": mfma_busy_for(dom, args.config, dt)},
    }
    if not args.no_ceilings:
        ceil = measure_ceilings(dev, flush)
        result["ceilings"] = ceil
        gb, seg = gathered_bytes(dom, A, N if dom != "spmv" else 1, K, dt,
                                 sddmm_plan.info().get("tiles", 0) if dom == "sddmm" else 0)
        if gb:
            key = ("gather_l2_4kib_gbps" if seg > 2048 else "gather_l2_1kib_gbps" if seg > 512
                   else "gather_l2_512b_gbps")
            rate = gb / breakdown[dom]["ms"] / 1e6
            result["roofline"]["gathered_bytes_per_launch"] = int(gb)
            result["roofline"]["gather_rate_gbps"] = round(rate, 1)
            result["roofline"]["gather_ceiling"] = key
            result["roofline"]["frac_of_gather_ceiling"] = round(rate / ceil[key], 4)
    if not args.no_adapter:
        result["next_adapter_step"] = adapter_step(S, w, A, dt, N, dev, flush, args)
    oracle = None
    if not args.no_cpu_baseline:
        import oracle
        result["cpu_baseline"] = cpu_baseline(w, A, dt, N, K, [dom], oracle)
        result["cpu_baseline"]["sample"] = (
            f"the headline operation ({dom}) on the full workload, one warm-up then the "
            "median of 3; the float64 oracle as it stands")
    if not args.no_per_config:
        ceil = result.get("ceilings")
        per = {}
        for cfg, cdt, op in GATED:
            ent = measure_case(S, cfg, cdt, op, dev, flush, max(args.steps, 10), args, ceil,
                               oracle)
            per[f"{ent['workload']}:{op}"] = ent
            torch.cuda.empty_cache()
        result["per_config"] = per
    if not args.no_adapter:
        w4 = gen.make_config(4)
        result["next_cg"] = cg_solve(S, w4, w4.get("A"), dev, args)
        if args.config == DEFAULT_CONFIG:
            result["next_delta_spmv"] = delta_spmv_bench(S, dev, flush, args)
    if args.records:
        write_records(args.records, result, args, A, dt, N, K, ab, fl)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
