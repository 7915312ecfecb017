"""Calls of the HIP entry points for the GPU tests, with every buffer the
kernels write prefilled with NaN (outputs, the split-KV workspace and the
backward's row-statistics workspace).  An element a kernel fails to write then
stays NaN and fails the comparison with the oracle, whatever the allocator
happened to leave in that memory."""

from __future__ import annotations

import math

import io_aware_tiled_fa_amd as fa


def nan_fwd(q, k, v, *, causal=False, scale=None, splits=None, general=False, stream=None):
    """fa.fwd into NaN-filled o and lse (and a NaN-filled workspace for splits)."""
    import torch

    B, H, M, D = q.shape
    out = torch.full_like(q, math.nan)
    lse = torch.full((B, H, M), math.nan, dtype=torch.float32, device=q.device)
    ws = None
    if splits is not None:
        need = max(fa.fa_splitkv_workspace_bytes(B, H, M, D, splits), 16)
        ws = torch.full((need // 4 + 1,), math.nan, dtype=torch.float32, device=q.device)
    return fa.fwd(q, k, v, causal=causal, scale=scale, out=out, lse=lse, splits=splits,
                  workspace=ws, general=general, stream=stream)


def nan_bwd(q, k, v, o, lse, dout, *, causal=False, scale=None, stream=None):
    """fa.bwd into NaN-filled dq, dk, dv and a NaN-filled delta workspace."""
    import torch

    B, H, M, _ = q.shape
    dq = torch.full_like(q, math.nan)
    dk = torch.full_like(k, math.nan)
    dv = torch.full_like(v, math.nan)
    delta = torch.full((2, B, H, M), math.nan, dtype=torch.float32, device=q.device)
    return fa.bwd(q, k, v, o, lse, dout, causal=causal, scale=scale, dq=dq, dk=dk, dv=dv,
                  delta=delta, stream=stream)
