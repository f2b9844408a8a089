"""Seeded synthetic workloads for the mixed-adapter LoRA layer.

Random draws only: this module holds none of the layer's arithmetic, and
serves both the GPU path (tests, benchmark) and the CPU oracle, which get the
very same tensors.  All values are drawn as fp32 normals from a seeded
torch.Generator on the target device and cast (round to nearest even) to the
workload's dtype; integer draws (request lengths, adapter ids, ranks, request
order) come from a seeded numpy Generator, so they do not depend on the
device.

Five workloads, named by what they are:
  tiny_fp32        T=64, 256->256, r=8, 4 slots, fp32, ids uniform over {-1,0..3}
  decode_bgmv      T=256 single-token requests, 4096->4096, r=16, 128 slots,
                   ids Zipf(1.1) with 10% base-only rows, values N(0, 0.02), alpha 32
  prefill_sgmv     64 requests of UniformInt[64,1024] tokens, adapter-contiguous,
                   32 slots each used by 2 requests, 4096->14336, r=32, alpha 64
  layer_8b         192 decode + 4 prefill chunks of 512 = 2240 rows, request order
                   shuffled, Zipf(1.0) over 1000 slots, 7 projections of an 8B model
  stress_70b       512 decode + 2 prefill chunks of 2048 = 4608 rows, 514 requests
                   shuffled, ids uniform over 256 slots, ranks from {8,16,32,64}
                   padded to 64, alpha = 2r, 5 projections of a 70B model
  decode_70b       the decode rows alone: 512 single-token requests on the 70B
                   q projection with the same adapter mix (measures the
                   per-row shrink's true-rank reads in BGMV mode and sets
                   AUTO's segment threshold; not one of the five parity
                   configurations)

The adapter orientation is the pages' row-vector form: A [d_in, r], B [r, d_out].
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

WORKLOADS = ("tiny_fp32", "decode_bgmv", "prefill_sgmv", "layer_8b", "stress_70b", "decode_70b")


@dataclass
class Projection:
    name: str
    d_in: int
    d_out: int
    x_group: str                     # which input tensor feeds it
    W: torch.Tensor = None           # [d_in, d_out]
    A: torch.Tensor = None           # [n_slots, d_in, max_rank] (columns >= rank unused)
    B: torch.Tensor = None           # [n_slots, max_rank, d_out] (rows >= rank unused)


@dataclass
class Workload:
    name: str
    dtype: torch.dtype
    T: int
    n_slots: int
    max_rank: int
    ids: np.ndarray                  # int32 [T], -1 = no adapter
    ranks: np.ndarray                # int32 [n_slots]
    alphas: np.ndarray               # float64 [n_slots]
    request_lengths: list
    request_ids: list
    xs: dict = field(default_factory=dict)      # x_group -> [T, d_in]
    projections: list = field(default_factory=list)

    def x_for(self, proj: Projection) -> torch.Tensor:
        return self.xs[proj.x_group]

    def slot_A(self, proj: Projection, slot: int) -> torch.Tensor:
        return proj.A[slot, :, : int(self.ranks[slot])]

    def slot_B(self, proj: Projection, slot: int) -> torch.Tensor:
        return proj.B[slot, : int(self.ranks[slot]), :]


def zipf_ids(rng: np.random.Generator, n: int, s: float, size: int) -> np.ndarray:
    """Finite Zipf(s) over n slots: P(k) proportional to k^-s, k = 1..n, slot k-1."""
    p = np.arange(1, n + 1, dtype=np.float64) ** (-s)
    p /= p.sum()
    return rng.choice(n, size=size, p=p).astype(np.int32)


def _normal(gen, shape, std, dtype, device):
    t = torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def _spec(name: str):
    if name == "tiny_fp32":
        return dict(seed=1, dtype=torch.float32, n_slots=4, max_rank=8,
                    projs=[("proj", 256, 256, "x")])
    if name == "decode_bgmv":
        return dict(seed=2, dtype=torch.bfloat16, n_slots=128, max_rank=16,
                    projs=[("q", 4096, 4096, "attn_in")])
    if name == "prefill_sgmv":
        return dict(seed=3, dtype=torch.bfloat16, n_slots=32, max_rank=32,
                    projs=[("gate", 4096, 14336, "mlp_in")])
    if name == "layer_8b":
        return dict(seed=4, dtype=torch.bfloat16, n_slots=1000, max_rank=16,
                    projs=[("q", 4096, 4096, "attn_in"), ("k", 4096, 1024, "attn_in"),
                           ("v", 4096, 1024, "attn_in"), ("o", 4096, 4096, "attn_out"),
                           ("gate", 4096, 14336, "mlp_in"), ("up", 4096, 14336, "mlp_in"),
                           ("down", 14336, 4096, "mlp_mid")])
    if name == "stress_70b":
        return dict(seed=5, dtype=torch.bfloat16, n_slots=256, max_rank=64,
                    projs=[("q", 8192, 8192, "attn_in"), ("o", 8192, 8192, "attn_out"),
                           ("gate", 8192, 28672, "mlp_in"), ("up", 8192, 28672, "mlp_in"),
                           ("down", 28672, 8192, "mlp_mid")])
    if name == "decode_70b":
        return dict(seed=6, dtype=torch.bfloat16, n_slots=256, max_rank=64,
                    projs=[("q", 8192, 8192, "attn_in")])
    raise ValueError("unknown workload %r (one of %s)" % (name, ", ".join(WORKLOADS)))


def _rows(name: str, rng: np.random.Generator, n_slots: int):
    """Request lengths and per-request ids, expanded to per-token ids in
    request order (each request's tokens contiguous)."""
    if name == "tiny_fp32":
        T = 64
        ids = rng.integers(-1, n_slots, size=T).astype(np.int32)
        return [1] * T, ids.tolist(), ids
    if name == "decode_bgmv":
        T = 256
        ids = zipf_ids(rng, n_slots, 1.1, T)
        ids[rng.random(T) < 0.10] = -1
        return [1] * T, ids.tolist(), ids
    if name == "prefill_sgmv":
        lengths = rng.integers(64, 1025, size=64).tolist()
        owners = rng.permutation(np.repeat(np.arange(32, dtype=np.int32), 2)).tolist()
        order = sorted(range(64), key=lambda i: owners[i])        # adapter-contiguous
        lengths = [lengths[i] for i in order]
        owners = [owners[i] for i in order]
    elif name == "layer_8b":
        lengths = [1] * 192 + [512] * 4
        owners = zipf_ids(rng, n_slots, 1.0, len(lengths)).tolist()
        perm = rng.permutation(len(lengths))
        lengths = [lengths[i] for i in perm]
        owners = [owners[i] for i in perm]
    elif name == "decode_70b":
        lengths = [1] * 512
        owners = rng.integers(0, n_slots, size=len(lengths)).tolist()
    elif name == "stress_70b":
        lengths = [1] * 512 + [2048] * 2
        owners = rng.integers(0, n_slots, size=len(lengths)).tolist()
        perm = rng.permutation(len(lengths))
        lengths = [lengths[i] for i in perm]
        owners = [owners[i] for i in perm]
    else:
        raise ValueError(name)
    ids = np.repeat(np.asarray(owners, dtype=np.int32), lengths).astype(np.int32)
    return lengths, owners, ids


def make_workload(name: str, device: str | torch.device = "cpu", seed: int | None = None,
                  projections: list | None = None) -> Workload:
    """Draw one workload.  `projections` restricts which projections are drawn."""
    sp = _spec(name)
    seed = sp["seed"] if seed is None else seed
    rng = np.random.default_rng(seed)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    dtype, n_slots, R = sp["dtype"], sp["n_slots"], sp["max_rank"]
    lengths, owners, ids = _rows(name, rng, n_slots)
    T = int(ids.shape[0])

    if name in ("stress_70b", "decode_70b"):
        ranks = rng.choice(np.array([8, 16, 32, 64], dtype=np.int32), size=n_slots).astype(np.int32)
        alphas = 2.0 * ranks.astype(np.float64)
    else:
        ranks = np.full(n_slots, R, dtype=np.int32)
        alphas = np.full(n_slots, {"tiny_fp32": 16.0, "decode_bgmv": 32.0, "prefill_sgmv": 64.0,
                                   "layer_8b": 32.0}[name], dtype=np.float64)

    wl = Workload(name=name, dtype=dtype, T=T, n_slots=n_slots, max_rank=R, ids=ids, ranks=ranks,
                  alphas=alphas, request_lengths=lengths, request_ids=owners)
    projs = sp["projs"] if projections is None else [p for p in sp["projs"] if p[0] in projections]

    # value distributions
    if name == "tiny_fp32":
        d = 256
        sd_x, sd_w, sd_a, sd_b = 1.0, 1.0 / np.sqrt(d), 1.0 / np.sqrt(d), 1.0 / np.sqrt(R)
    elif name == "decode_bgmv":
        sd_x = sd_w = sd_a = sd_b = 0.02
    else:
        sd_x, sd_w, sd_a, sd_b = 1.0, 0.02, 0.02, 0.01

    for pname, d_in, d_out, group in projs:
        if group not in wl.xs:
            wl.xs[group] = _normal(gen, (T, d_in), sd_x, dtype, device)
    for pname, d_in, d_out, group in projs:
        pr = Projection(pname, d_in, d_out, group)
        pr.W = _normal(gen, (d_in, d_out), sd_w, dtype, device)
        pr.A = _normal(gen, (n_slots, d_in, R), sd_a, dtype, device)
        pr.B = _normal(gen, (n_slots, R, d_out), sd_b, dtype, device)
        wl.projections.append(pr)
    return wl


def sample_rows(wl: Workload, n_random: int = 32, seed: int = 0, max_rows: int | None = None,
                n_base: int = 64) -> np.ndarray:
    """A seeded, stratified row sample for oracle checks at full size.

    Strata, in priority order: the first row of every adapter segment (rows
    in stable sorted order, so one row per distinct adapter and rank class),
    the last row of every segment, up to two further rows per segment, up to
    n_base base-only rows, the first and last row of the batch, and n_random
    uniform rows.  Without max_rows every stratum is kept whole; with it the
    strata are taken in that order until max_rows rows are reached, so a
    truncated sample still holds one row of every adapter before anything
    else."""
    rng = np.random.default_rng(seed)
    ids = wl.ids
    T = wl.T
    order = np.argsort(ids, kind="stable")
    sid = ids[order]
    starts = np.flatnonzero(np.r_[True, sid[1:] != sid[:-1]])
    ends = np.r_[starts[1:], T] - 1
    firsts, lasts, inner = [], [], []
    base = np.flatnonzero(ids < 0)
    for s, e in zip(starts, ends):
        if sid[s] < 0:
            continue
        firsts.append(int(order[s]))
        lasts.append(int(order[e]))
        if e - s >= 2:
            inner.extend(int(order[i]) for i in rng.choice(np.arange(s + 1, e), size=min(2, e - s - 1),
                                                          replace=False))
    base_pick = [int(i) for i in rng.choice(base, size=min(n_base, base.size), replace=False)] if base.size else []
    strata = [firsts, lasts, inner, base_pick, [0, T - 1], [int(i) for i in rng.integers(0, T, size=n_random)]]
    rows: list = []
    seen = set()
    for stratum in strata:
        for r in stratum:
            if r in seen:
                continue
            if max_rows is not None and len(rows) >= max_rows:
                break
            seen.add(r)
            rows.append(r)
    return np.asarray(sorted(rows), dtype=np.int64)
