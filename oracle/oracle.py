"""fp64 CPU oracle for the mixed-adapter LoRA linear layer (test infrastructure).

TEST INFRASTRUCTURE ONLY: only the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP library under ``rank_adapter_gemm_amd/`` and never imports it.

Contents
--------
``lora_scale(alpha, r)``
    s = alpha / r, one fp32 value per adapter ("LoRAX, in depth", section "Computing a batch that mixes
    adapters"; the value 2.0 = alpha / r in the example of "Serving multiple
    LoRAs ...", section "Not merging the weights, computing in batches").
``adapter_param_count(d_in, d_out, r)``
    r * (d_in + d_out): the parameter count of one adapted matrix
    ("Multi-LoRA Serving: Architecture for Thousands of Adapters", sections
    "Context and Background" and "A worked memory example").
``oracle_segments(ids, n_slots)``
    the integer segment metadata: a sequential counting sort of token rows by
    adapter id, stable in the original row order, with the "no adapter"
    rows (-1) first ("Serving multiple LoRAs ...", the ``sgmv`` routine of
    the example: stable argsort by adapter, then consecutive-unique counts;
    "Multi-LoRA Serving 与 Adapter 隔离", section on adapter ownership in one
    continuous batch: grouping by adapter, then scatter back by offsets).
``oracle_rows(...)``
    the fp64 per-row output (C code in ``lora_oracle.c``), optionally with
    the rank-width shrink result u and the unscaled low-rank term delta.
``oracle_segmented(...)``
    a second route: the segment-by-segment structure of ``lora_mixed_batch``
    ("LoRAX, in depth", section "Computing a batch that mixes adapters") run
    over the segment metadata and scattered back to the original row order.

Readings of the pages used here (each also listed in the design notes):
  * row-vector orientation y = xW + s (xA) B with A [d_in, r], B [r, d_out];
  * the "no adapter" marker is -1; an id outside [-1, n_slots) or naming an
    empty slot (rank 0) contributes nothing (base row only);
  * s = alpha / r with the adapter's true rank, applied to (xA)B.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import sys
from typing import Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lora_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F32 = 0
BF16 = 1

_lib = None


def build_oracle(force: bool = False) -> str:
    """Compile ``lora_oracle.c`` with gcc into ``liboracle.so`` (in-tree)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-o", tmp, _SRC]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build_oracle()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.oracle_lora_rows.restype = ctypes.c_int
        lib.oracle_lora_rows.argtypes = [
            ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int,
        ]
        _lib = lib
    return _lib


def affinity_cores() -> int:
    """Cores in this process's affinity mask."""
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def default_threads() -> int:
    """Worker threads: every core of the affinity mask, but no more than the
    host's declared CPU share (OMP_NUM_THREADS) where one is set."""
    n = affinity_cores()
    share = os.environ.get("OMP_NUM_THREADS", "")
    if share.isdigit() and int(share) > 0:
        n = min(n, int(share))
    return n


def lora_scale(alpha: float, r: int) -> float:
    """s = alpha / r with the adapter's true rank ("LoRAX, in depth", section
    "Computing a batch that mixes adapters"), held as one fp32 value per
    adapter: alpha as an fp32 number divided by r in IEEE fp32 (one correctly
    rounded quotient), then widened exactly to double.  The pages fix no
    precision for s; a per-slot fp32 scale is the reading used for the whole
    layer.  For alpha = 2r (and every scale the workloads use) s is a power
    of two and exact in any precision."""
    if r <= 0:
        return 0.0
    return float(np.float32(alpha) / np.float32(r))


def adapter_param_count(d_in: int, d_out: int, r: int) -> int:
    """Parameters of one adapted matrix: A is d_in x r, B is r x d_out."""
    return int(r) * (int(d_in) + int(d_out))


# --------------------------------------------------------------------------
# Segment metadata
# --------------------------------------------------------------------------
def oracle_segments(ids: Sequence[int], n_slots: int) -> dict:
    """Sequential counting sort of rows by adapter id (stable), as plain loops.

    Bucket k = id + 1, so the "no adapter" rows (-1) form bucket 0 and come
    first.  Ids outside [-1, n_slots) are treated as "no adapter" (bucket 0).

    Returns int32 arrays:
      offsets   [n_slots + 2]  exclusive prefix sum of the bucket counts
                               (offsets[-1] == T)
      perm      [T]            row indices in (bucket, original row) order
      seg_id    [n_seg]        slot of each non-empty adapter segment, ascending
      seg_start [n_seg + 1]    first sorted position of each segment, then T
      n_seg                    number of non-empty adapter segments
    The "no adapter" block is counted in offsets but is not a segment.
    """
    ids = [int(v) for v in np.asarray(ids).reshape(-1).tolist()]
    T = len(ids)
    n_buckets = n_slots + 1
    keys = [(v + 1) if (-1 <= v < n_slots) else 0 for v in ids]
    counts = [0] * n_buckets
    for k in keys:
        counts[k] += 1
    offsets = [0] * (n_buckets + 1)
    for b in range(n_buckets):
        offsets[b + 1] = offsets[b] + counts[b]
    cursor = offsets[:n_buckets]
    cursor = list(cursor)
    perm = [0] * T
    for t, k in enumerate(keys):
        perm[cursor[k]] = t
        cursor[k] += 1
    seg_id, seg_start = [], []
    for b in range(1, n_buckets):
        if counts[b] > 0:
            seg_id.append(b - 1)
            seg_start.append(offsets[b])
    seg_start.append(T)
    return {
        "offsets": np.asarray(offsets, dtype=np.int32),
        "perm": np.asarray(perm, dtype=np.int32),
        "seg_id": np.asarray(seg_id, dtype=np.int32),
        "seg_start": np.asarray(seg_start, dtype=np.int32),
        "n_seg": len(seg_id),
    }


# --------------------------------------------------------------------------
# Row outputs
# --------------------------------------------------------------------------
def _as_storage(a: np.ndarray, dtype: int) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if dtype == F32:
        if a.dtype != np.float32:
            raise TypeError("fp32 oracle input must be float32, got %s" % a.dtype)
    else:
        if a.dtype != np.uint16:
            raise TypeError("bf16 oracle input must be the raw uint16 bit pattern, got %s" % a.dtype)
    return a


def oracle_rows(dtype: int, x: np.ndarray, W: np.ndarray, ids: np.ndarray,
                A: Sequence, B: Sequence, ranks: Sequence[int], scales: Sequence[float],
                rows: Sequence[int] | None = None, want_u: bool = False, u_stride: int | None = None,
                want_delta: bool = False, n_threads: int | None = None) -> dict:
    """fp64 outputs for the listed rows (all rows when ``rows`` is None).

    x [T, d_in], W [d_in, d_out]; A[s] [d_in, ranks[s]] and B[s] [ranks[s], d_out]
    per slot s (None for an empty slot); storage dtype float32 (F32) or the raw
    bf16 bit pattern as uint16 (BF16).  Returns {"y": [n, d_out] float64,
    optionally "u": [n, u_stride], "delta": [n, d_out]}.
    """
    x = _as_storage(x, dtype)
    W = _as_storage(W, dtype)
    T, d_in = x.shape
    d_in_w, d_out = W.shape
    if d_in_w != d_in:
        raise ValueError("x and W disagree on d_in")
    ids = np.ascontiguousarray(np.asarray(ids, dtype=np.int32).reshape(-1))
    if ids.shape[0] != T:
        raise ValueError("ids must have one entry per row of x")
    rows = np.arange(T, dtype=np.int64) if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    if rows.size and (rows.min() < 0 or rows.max() >= T):
        raise ValueError("row index out of range")
    n_slots = len(A)
    if len(B) != n_slots or len(ranks) != n_slots or len(scales) != n_slots:
        raise ValueError("per-slot lists must have equal length")
    keep = []
    a_ptrs = (ctypes.c_void_p * max(n_slots, 1))()
    b_ptrs = (ctypes.c_void_p * max(n_slots, 1))()
    ranks_arr = np.zeros(max(n_slots, 1), dtype=np.int32)
    scales_arr = np.zeros(max(n_slots, 1), dtype=np.float64)
    for s in range(n_slots):
        r = int(ranks[s])
        ranks_arr[s] = r
        scales_arr[s] = float(scales[s])
        if r > 0 and A[s] is not None and B[s] is not None:
            a = _as_storage(A[s], dtype)
            b = _as_storage(B[s], dtype)
            if a.shape != (d_in, r) or b.shape != (r, d_out):
                raise ValueError("slot %d: A must be [d_in, r] and B [r, d_out]" % s)
            keep += [a, b]
            a_ptrs[s] = a.ctypes.data
            b_ptrs[s] = b.ctypes.data
        else:
            ranks_arr[s] = 0
    n = rows.shape[0]
    y = np.zeros((n, d_out), dtype=np.float64)
    max_r = int(max([int(r) for r in ranks] + [1]))
    us = int(u_stride) if u_stride is not None else max_r
    u = np.zeros((n, us), dtype=np.float64) if want_u else None
    delta = np.zeros((n, d_out), dtype=np.float64) if want_delta else None
    rc = _load().oracle_lora_rows(
        dtype, x.ctypes.data, d_in, d_out, W.ctypes.data, ids.ctypes.data, rows.ctypes.data, n,
        ctypes.cast(a_ptrs, ctypes.c_void_p), ctypes.cast(b_ptrs, ctypes.c_void_p),
        ranks_arr.ctypes.data, scales_arr.ctypes.data, n_slots,
        y.ctypes.data, u.ctypes.data if u is not None else None, us,
        delta.ctypes.data if delta is not None else None,
        int(n_threads or default_threads()))
    if rc != 0:
        raise ValueError("oracle_lora_rows rejected its arguments")
    out = {"y": y}
    if want_u:
        out["u"] = u
    if want_delta:
        out["delta"] = delta
    return out


def oracle_segmented(dtype: int, x: np.ndarray, W: np.ndarray, ids: np.ndarray,
                     A: Sequence, B: Sequence, ranks: Sequence[int], scales: Sequence[float],
                     n_threads: int | None = None) -> np.ndarray:
    """Second route: base rows, then one adapter segment at a time.

    Rows are grouped by the segment metadata, each segment is evaluated with
    its single adapter, and the results are scattered back through ``perm``
    (the ``lora_mixed_batch`` structure, with the per-row arithmetic of
    ``oracle_rows``).  Must equal ``oracle_rows`` exactly.
    """
    ids = np.asarray(ids, dtype=np.int32).reshape(-1)
    T = ids.shape[0]
    n_slots = len(A)
    seg = oracle_segments(ids, n_slots)
    d_out = W.shape[1]
    y = np.empty((T, d_out), dtype=np.float64)
    perm = seg["perm"]
    # no-adapter block (bucket 0): base product only
    base_rows = perm[: seg["offsets"][1]]
    if base_rows.size:
        none_ids = np.full(T, -1, dtype=np.int32)
        y[base_rows] = oracle_rows(dtype, x, W, none_ids, A, B, ranks, scales,
                                   rows=base_rows, n_threads=n_threads)["y"]
    for k in range(seg["n_seg"]):
        lo, hi = int(seg["seg_start"][k]), int(seg["seg_start"][k + 1])
        rows = perm[lo:hi]
        one = np.full(T, int(seg["seg_id"][k]), dtype=np.int32)
        y[rows] = oracle_rows(dtype, x, W, one, A, B, ranks, scales,
                              rows=rows, n_threads=n_threads)["y"]
    return y


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even) and
    return the bit patterns as uint16.  NaN is not expected in these inputs."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


if __name__ == "__main__":  # build step: python oracle/oracle.py
    print(build_oracle(force="--force" in sys.argv))
