"""Sparse linear layer with autograd, built from the four CSR operations.

This is the sparse-adaptation pattern the spops README's SDDMM and csr_add
serve (robust sparse adaptation of a dense weight W by a sparse S): a layer
computes S·x, training needs the gradients with respect to S's stored values
and to the input, and the trained S is finally merged into W.  Activations
are kept feature-major (X^T is in_features x tokens, row-major), which makes
every step one call into libspops and needs no dense transpose:

    forward    Y^T  = S · X^T                         spmm
    backward   dS   = dY^T · (X^T)^T sampled at S     sddmm (A = dY^T, BT = X^T)
               dX^T = S^T · dY^T                      values of S^T (the
                                                      transpose's permutation,
                                                      found once) + spmm
    merge      W   += S                               csr_add
    optimizer  values -= Adam step (masked)           masked_adam (MaskedAdam)

The module only marshals tensors: outputs are allocated here and every value
is computed by the library's kernels (it raises if libspops.so is missing).
"""
from __future__ import annotations

from typing import Optional

import torch

from .spops import (SddmmPlan, SpmmPlan, csr_add, csr_transpose_permutation, masked_adam,
                    permute_values, sddmm, sort_rows_by_nnz, spmm)


class SparsePattern:
    """A CSR sparsity pattern of S (out_features x in_features) and what is
    derived from it once: the row order, the SpMM / SDDMM plans, the pattern
    of S^T with its own row order and plan, and the permutation that takes
    S's values to S^T's."""

    def __init__(self, row_offsets: torch.Tensor, col_idx: torch.Tensor,
                 out_features: int, in_features: int):
        self.ro, self.ci = row_offsets, col_idx
        self.m, self.n = out_features, in_features
        self.nnz = col_idx.numel()
        self.ri = sort_rows_by_nnz(row_offsets, in_features)
        self.spmm_plan = SpmmPlan(row_offsets, self.ri, col_idx, in_features)
        self.sddmm_plan = SddmmPlan(row_offsets, col_idx, out_features, in_features)
        self.srcT, self.roT, self.ciT = csr_transpose_permutation(row_offsets, col_idx,
                                                                  out_features, in_features)
        self.riT = sort_rows_by_nnz(self.roT, out_features)
        self.spmmT_plan = SpmmPlan(self.roT, self.riT, self.ciT, out_features)

    def transposed_values(self, values: torch.Tensor,
                          out: Optional[torch.Tensor] = None) -> torch.Tensor:
        """Values of S^T in the order of the transposed pattern (what
        csr_transpose gives, bit for bit)."""
        return permute_values(values, self.srcT, out=out)


class _SparseLinearFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, values: torch.Tensor, xt: torch.Tensor, pattern: SparsePattern):
        P = pattern
        yt = spmm(values, P.ro, P.ri, P.ci, xt, P.m, out_dtype=xt.dtype, plan=P.spmm_plan)
        ctx.save_for_backward(values, xt)
        ctx.pattern = P
        return yt

    @staticmethod
    def backward(ctx, dyt: torch.Tensor):
        values, xt = ctx.saved_tensors
        P = ctx.pattern
        dyt = dyt.contiguous()
        dv = dxt = None
        if ctx.needs_input_grad[0]:
            dv = sddmm(P.ro, P.ri, P.ci, dyt, xt, plan=P.sddmm_plan, out_dtype=values.dtype)
        if ctx.needs_input_grad[1]:
            vt = P.transposed_values(values)
            dxt = spmm(vt, P.roT, P.riT, P.ciT, dyt, P.n, out_dtype=xt.dtype,
                       plan=P.spmmT_plan)
        return dv, dxt, None


def sparse_linear(values: torch.Tensor, xt: torch.Tensor, pattern: SparsePattern) -> torch.Tensor:
    """Y^T = S · X^T with S = (pattern, values); differentiable in values and X^T.
    values and X^T share a dtype (f32, f16 or bf16); Y^T has that dtype too
    (fp32 accumulation, one rounding)."""
    if values.dtype != xt.dtype:
        raise ValueError("values and X^T must share a dtype")
    if xt.dim() != 2 or xt.shape[0] != pattern.n:
        raise ValueError("X^T must be in_features x tokens")
    return _SparseLinearFn.apply(values, xt, pattern)


class SparseAdapter(torch.nn.Module):
    """A trainable sparse matrix S on a fixed pattern: forward(X^T) = S · X^T;
    merge_into(W) adds S into a dense out_features x in_features weight."""

    def __init__(self, pattern: SparsePattern, values: torch.Tensor):
        super().__init__()
        if values.numel() != pattern.nnz:
            raise ValueError("one value per stored entry of the pattern")
        self.pattern = pattern
        self.values = torch.nn.Parameter(values)

    def forward(self, xt: torch.Tensor) -> torch.Tensor:
        return sparse_linear(self.values, xt, self.pattern)

    @torch.no_grad()
    def merge_into(self, W: torch.Tensor) -> torch.Tensor:
        P = self.pattern
        return csr_add(self.values.detach(), P.ro, P.ri, P.ci, W)


class MaskedAdam(torch.optim.Optimizer):
    """The masked Adam of the SparseAdam page (tensorplay.optim.sparse_adam)
    for value vectors, each step one launch of the library's kernel
    (spops_masked_adam).  A dense gradient updates every value; a 1-D sparse
    COO gradient (coalesced) updates only the values it names, leaving the
    others and their moments untouched.  Moments are kept in f32."""

    def __init__(self, params, lr: float = 1e-3, betas=(0.9, 0.999), eps: float = 1e-8,
                 maximize: bool = False):
        if not (lr >= 0.0 and eps >= 0.0 and 0.0 <= betas[0] < 1.0 and 0.0 <= betas[1] < 1.0):
            raise ValueError("need lr >= 0, eps >= 0 and betas in [0, 1)")
        super().__init__(params, dict(lr=lr, betas=tuple(betas), eps=eps, maximize=maximize))

    @torch.no_grad()
    def step(self, closure=None):
        loss = None
        if closure is not None:
            with torch.enable_grad():
                loss = closure()
        for group in self.param_groups:
            for p in group["params"]:
                if p.grad is None:
                    continue
                if p.dim() != 1 or not p.is_contiguous():
                    raise ValueError("MaskedAdam trains contiguous 1-D value vectors")
                st = self.state[p]
                if not st:
                    st["step"] = 0
                    st["exp_avg"] = torch.zeros(p.shape, dtype=torch.float32, device=p.device)
                    st["exp_avg_sq"] = torch.zeros(p.shape, dtype=torch.float32,
                                                   device=p.device)
                st["step"] += 1
                g = p.grad
                kw = dict(lr=group["lr"], betas=group["betas"], eps=group["eps"],
                          maximize=group["maximize"])
                if g.is_sparse:
                    if not g.is_coalesced():
                        raise ValueError("sparse gradients must be coalesced")
                    pos = g.indices()[0].to(torch.int32)
                    masked_adam(p.data, g.values().contiguous(), st["exp_avg"],
                                st["exp_avg_sq"], st["step"], positions=pos, **kw)
                else:
                    masked_adam(p.data, g.contiguous(), st["exp_avg"], st["exp_avg_sq"],
                                st["step"], **kw)
        return loss
