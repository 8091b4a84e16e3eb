"""The hot path captured in a HIP graph (through torch.cuda.CUDAGraph) gives,
on every replay, exactly the results of the same calls run eagerly.  Replays
are separated by eager work and synchronizations, and each is checked."""
import numpy as np
import pytest
import torch

import oracle
import unstructured_sparse_linear_amd as S
from unstructured_sparse_linear_amd import gen
from helpers import csr_dev, dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dt,heavy", [("f16", False), ("bf16", True)])
def test_graph_replays_match_eager(dt, heavy):
    if heavy:
        rng = np.random.default_rng(3)
        counts = np.concatenate([[1500, 700, 300], rng.integers(0, 40, 997)])
        A = gen.csr_from_row_lists(1000, 3000, [np.sort(rng.choice(3000, int(c), replace=False))
                                                for c in counts])
        A = A.with_values(gen.normal(rng, A.nnz, dt), dt)
    else:
        A = gen.random_csr(5, 1200, 2600, 0.02, dt)
    m, n, N, K = A.m, A.n, 256, 128
    v, ro, ci = csr_dev(A)
    ri = S.sort_rows_by_nnz(ro, n)
    B = dev(gen.dense(5, 100, gen.S_B, (n, N), dt), dt)
    Ad = dev(gen.dense(5, 100, gen.S_A, (m, K), dt), dt)
    BT = dev(gen.dense(5, 100, gen.S_BT, (n, K), dt), dt)
    W0 = dev(gen.dense(5, 100, gen.S_W, (m, n), dt), dt)
    plan = S.SpmmPlan(ro, ri, ci, n)
    splan = S.SddmmPlan(ro, ci, m, n, tau=0.02)
    C = torch.empty((m, N), dtype=torch.float32, device="cuda")
    out = torch.empty(A.nnz, dtype=torch.float32, device="cuda")
    W = W0.clone()
    tws = S.csr_transpose_workspace(m, n, A.nnz, "cuda")
    sws = S.sort_rows_workspace(n, m, "cuda")
    roT = torch.empty(n + 1, dtype=torch.int32, device="cuda")
    riT = torch.empty(n, dtype=torch.int16, device="cuda")

    def step():
        S.spmm(v, ro, ri, ci, B, m, plan=plan, out=C)
        S.sddmm(ro, ri, ci, Ad, BT, plan=splan, out=out)
        S.csr_add(v, ro, ri, ci, W)
        _, roT2, _ = S.csr_transpose(v, ro, ci, m, n, workspace=tws)
        roT.copy_(roT2)
        S.sort_rows_by_nnz(roT, m, workspace=sws, out=riT)

    step()
    torch.cuda.synchronize()
    ref = [C.clone(), out.clone(), W.clone(), roT.clone(), riT.clone()]
    W.copy_(W0)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        W.copy_(W0)
        C.zero_()
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [C, out, W, roT, riT]
        for a, b in zip(got, ref):
            assert torch.equal(a, b), f"replay {rep} differs"
        # unrelated eager work between replays
        _ = (B.float() @ B.float().T).sum().item()


@pytest.mark.parametrize("m,n,density", [
    (300, 40000, 0.01),    # row order of 40000 rows: radix passes, no scan
    (3000, 3000, 0.04),    # transpose of ~360 K entries: scan between count and scatter
    (50, 300000, 0.002),   # > 2^17 columns: full LSD transpose; row order with scans
])
def test_graph_replays_of_radix_paths(m, n, density):
    A = gen.random_csr(7, m, n, density, "f32")
    v, ro, ci = csr_dev(A)
    tws = S.csr_transpose_workspace(m, n, A.nnz, "cuda")
    sws = S.sort_rows_workspace(n, m, "cuda")
    it = torch.int16 if m <= 32767 else torch.int32
    vT = torch.empty(A.nnz, dtype=torch.float32, device="cuda")
    roT = torch.empty(n + 1, dtype=torch.int32, device="cuda")
    ciT = torch.empty(A.nnz, dtype=it, device="cuda")
    riT = torch.empty(n, dtype=torch.int16 if n <= 32767 else torch.int32, device="cuda")

    def step():
        S.csr_transpose(v, ro, ci, m, n, workspace=tws, out=(vT, roT, ciT))
        S.sort_rows_by_nnz(roT, m, workspace=sws, out=riT)

    step()
    torch.cuda.synchronize()
    ref = [vT.clone(), roT.clone(), ciT.clone(), riT.clone()]
    ev, ero, eci = oracle.csr_transpose(m, n, A.row_offsets, A.col_idx, A.values)
    assert np.array_equal(ref[1].cpu().numpy(), ero)
    assert np.array_equal(ref[2].cpu().numpy(), eci)
    assert np.array_equal(ref[0].cpu().numpy().view(np.uint8), ev.view(np.uint8))
    assert np.array_equal(ref[3].cpu().numpy(), oracle.row_idx(ero))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for x in (vT, roT, ciT, riT):
            x.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip([vT, roT, ciT, riT], ref):
            assert torch.equal(a, b), f"replay {rep} differs"
        _ = (v.float() * 2).sum().item()


def test_graph_replays_of_the_next_rows_match_eager():
    # delta-coded SpMV, a masked Adam step and the sparse layer's training
    # step (forward, both gradients, merge) on two streams, captured once and
    # replayed; each replay is compared with the same sequence run eagerly
    # from the same state
    dt = "f16"
    A = gen.random_csr(7, 700, 900, 0.3, dt)
    m, n, T = A.m, A.n, 64
    v, ro, ci = csr_dev(A)
    D = S.delta_encode(v, ro, ci, m, n)
    x = dev(gen.dense(7, 100, gen.S_B1, (n,), dt), dt)
    y = torch.empty(m, dtype=torch.float32, device="cuda")
    P = S.SparsePattern(ro, ci, m, n)
    xt = dev(gen.dense(7, 100, gen.S_B, (n, T), dt), dt)
    dyt = dev(gen.dense(7, 100, gen.S_A, (m, T), dt), dt)
    W0 = dev(gen.dense(7, 100, gen.S_W, (m, n), dt), dt)
    th0 = v.clone()
    yt = torch.empty((m, T), dtype=torch.float16, device="cuda")
    dv = torch.empty_like(v)
    vT = torch.empty_like(v)
    dxt = torch.empty((n, T), dtype=torch.float16, device="cuda")
    th, W = th0.clone(), W0.clone()
    m1 = torch.zeros(A.nnz, dtype=torch.float32, device="cuda")
    m2 = torch.zeros_like(m1)
    side = torch.cuda.Stream()

    def step():
        cur = torch.cuda.current_stream()
        side.wait_stream(cur)
        with torch.cuda.stream(side):
            S.delta_spmv(D, x, out=y)
        S.spmm(th, P.ro, P.ri, P.ci, xt, m, out_dtype=torch.float16, plan=P.spmm_plan, out=yt)
        S.sddmm(P.ro, P.ri, P.ci, dyt, xt, plan=P.sddmm_plan, out_dtype=torch.float16, out=dv)
        P.transposed_values(th, out=vT)
        S.spmm(vT, P.roT, P.riT, P.ciT, dyt, n, out_dtype=torch.float16, plan=P.spmmT_plan,
               out=dxt)
        S.masked_adam(th, dv, m1, m2, 3, lr=1e-3)
        S.csr_add(th, P.ro, P.ri, P.ci, W)
        cur.wait_stream(side)

    def reset():
        th.copy_(th0)
        W.copy_(W0)
        m1.zero_()
        m2.zero_()
        for t in (y, yt, dv, vT, dxt):
            t.zero_()

    reset()
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (y, yt, dv, vT, dxt, th, W, m1, m2)]
    reset()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((y, yt, dv, vT, dxt, th, W, m1, m2), ref):
            assert torch.equal(a, b), f"replay {rep} differs"
        _ = (xt.float() @ xt.float().T).sum().item()


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_graph_replays_sddmm_without_plan(dt):
    # structure-aware SDDMM with no plan: the partition is built inside the
    # call on the stream, in the caller's workspace, so the whole call can be
    # captured; each replay must give the oracle's values (integer data:
    # exact) and the eager result
    m, n, K = 2100, 900, 136
    M = gen.cross_mask(gen.rng_for(12, 102, 0), m, n, 0.05, 264 / m, 290 / n, 0.9)
    _, ro, ci = csr_dev(M)
    ri = S.sort_rows_by_nnz(ro, n)
    Ad = dev(gen.dense(12, 100, gen.S_A, (m, K), dt, integer_values=True), dt)
    BT = dev(gen.dense(12, 100, gen.S_BT, (n, K), dt, integer_values=True), dt)
    ref = oracle.sddmm(M.row_offsets, M.col_idx, host_bits(Ad, dt), host_bits(BT, dt), dt)
    out = torch.empty(M.nnz, dtype=torch.float32, device="cuda")
    import ctypes
    from unstructured_sparse_linear_amd import spops as SP
    d = SP.csr_desc(None, ro, ri, ci, m, n)
    b = ctypes.c_size_t()
    assert SP.lib().spops_sddmm_workspace_size(ctypes.byref(d), K, SP._DT[Ad.dtype], 0, None,
                                               ctypes.byref(b)) == 0
    assert b.value > 0
    ws = torch.empty(b.value, dtype=torch.uint8, device="cuda")
    S.sddmm(ro, ri, ci, Ad, BT, use_plan=False, workspace=ws, out=out)
    torch.cuda.synchronize()
    eager = out.clone()
    assert np.array_equal(eager.double().cpu().numpy(), ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        S.sddmm(ro, ri, ci, Ad, BT, use_plan=False, workspace=ws, out=out)
    torch.cuda.synchronize()
    for rep in range(3):
        out.zero_()
        ws.fill_(0xAB)  # the plan must not depend on what the workspace held
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs"
        _ = (Ad.float() @ BT.float().T).sum().item()


def host_bits(t, dt):
    """Device tensor -> host array in the generators' storage convention."""
    t = t.cpu()
    if dt == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
