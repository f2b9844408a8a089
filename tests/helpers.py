"""Shared test plumbing: build pools from a workload, run the HIP path through
the C ABI, and compare against the fp64 oracle on the same tensors."""
from __future__ import annotations

import numpy as np
import torch

from oracle import BF16, F32, oracle_rows, lora_scale
from rank_adapter_gemm_amd import lora as L

# Tolerances (element-wise, relative to 1 + |ref|):
#   fp32 inputs: 1e-5; bf16 inputs with fp32 accumulation: 2e-2.
TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}
# Delta-sensitive check of the low-rank term alone (shrink + expand into a
# zero output): max |err| <= DELTA_TOL * max |delta_ref|.  bf16 output
# rounding alone is 2^-9 relative.
DELTA_TOL = {torch.float32: 1e-5, torch.bfloat16: 1e-2}


def to_oracle(t: torch.Tensor) -> np.ndarray:
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    raise TypeError(t.dtype)


def oracle_code(dtype: torch.dtype) -> int:
    return F32 if dtype == torch.float32 else BF16


def build_pool(wl, proj, stream=None) -> L.AdapterPool:
    pool = L.AdapterPool(wl.n_slots, proj.d_in, proj.d_out, wl.max_rank, wl.dtype)
    for s in range(wl.n_slots):
        r = int(wl.ranks[s])
        if r > 0:
            pool.upload(s, proj.A[s], proj.B[s], r, float(wl.alphas[s]), lda=wl.max_rank,
                        ldb=proj.d_out, stream=stream)
    return pool


def oracle_for(wl, proj, rows, want_u=False, want_delta=False, ids=None, n_threads=None):
    """fp64 oracle rows for one projection (only the slots the rows use are copied)."""
    ids = wl.ids if ids is None else ids
    used = sorted({int(ids[r]) for r in rows if 0 <= int(ids[r]) < wl.n_slots})
    A = [None] * wl.n_slots
    B = [None] * wl.n_slots
    for s in used:
        r = int(wl.ranks[s])
        A[s] = to_oracle(proj.A[s, :, :r])
        B[s] = to_oracle(proj.B[s, :r, :])
    scales = [lora_scale(float(wl.alphas[s]), int(wl.ranks[s])) for s in range(wl.n_slots)]
    return oracle_rows(oracle_code(wl.dtype), to_oracle(wl.x_for(proj)), to_oracle(proj.W), ids,
                       A, B, [int(r) for r in wl.ranks], scales, rows=rows, want_u=want_u,
                       u_stride=wl.max_rank, want_delta=want_delta, n_threads=n_threads)


def rel_err(y_gpu: torch.Tensor, y_ref: np.ndarray) -> float:
    y = y_gpu.detach().float().cpu().double().numpy()
    return float(np.max(np.abs(y - y_ref) / (1.0 + np.abs(y_ref)))) if y.size else 0.0


def assert_parity(y_gpu: torch.Tensor, y_ref: np.ndarray, dtype: torch.dtype, what: str = ""):
    e = rel_err(y_gpu, y_ref)
    assert e <= TOL[dtype], "%s: max |y - ref| / (1 + |ref|) = %.3e > %.1e" % (what, e, TOL[dtype])
    return e


def forward(wl, proj, pool, ids_dev, mode, flags=0, ws=None, y=None):
    x = wl.x_for(proj)
    if ws is None:
        ws = L.Workspace(wl.T, wl.n_slots, wl.max_rank, max(p.d_out for p in wl.projections))
    if y is None:
        y = torch.empty(wl.T, proj.d_out, dtype=wl.dtype, device=x.device)
    L.lora_linear_forward(x, proj.W, y, wl.T, pool.pool, ids_dev, mode, flags, ws.buf)
    return y, ws
