"""Seeded sweep over random valid shapes, through the C ABI, against the fp64
oracle on sampled rows.

Every case is drawn from its seed: T log-uniform in [1, 4096], d_in and d_out
log-uniform multiples of 8 (16 for the FP8 base's d_in) up to 4096 and 20000
columns (d_in * d_out at most 2^25), each half the time from the multi-tile
part of its range (T >= 256, d_in >= 512, d_out >= 1024); max_rank one of
the allowed multiples of 8, 1-63 slots with random ranks (some empty), and
an id mix drawn from uniform, skewed, one-adapter, all-base and sorted
batches, with a share of base rows and, in some cases, out-of-range ids; a
further set of forward cases uses packed pools (each slot's rank rounded up
to 8 rows, some with an octet to spare).  Each case runs every mode
(AUTO, BGMV, SGMV) with the fused and the separate expand and checks the
sampled rows (the first and last rows, rows at 64-, 128- and 256-row tile
edges and random rows) against the oracle, the device error word against
the first bad row, and that a repeat call is bitwise the same.  The sliced
and FP8-base entry points get the same treatment.  Adapter scales are
alpha / r = 2, so the low-rank term is as large as the base product and a
wrong or dropped term exceeds the tolerance."""
import numpy as np
import pytest
import torch

from oracle import BF16, F32, lora_scale, oracle_rows
from rank_adapter_gemm_amd import lora as L

from helpers import assert_parity, to_oracle
from helpers_fp8 import Fp8Case, assert_within

pytestmark = pytest.mark.gpu

RANKS = [8, 16, 24, 32, 48, 64, 96, 128]
MODES = (L.LORA_MODE_AUTO, L.LORA_MODE_BGMV, L.LORA_MODE_SGMV)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


def _log_int(rng, lo, hi):
    return int(np.clip(np.exp(rng.uniform(np.log(lo), np.log(hi + 1))), lo, hi))


def draw_case(seed, k_quant=8, max_slice_rank=128):
    """Shape, ranks and ids of one sweep case (host-side numbers only)."""
    rng = np.random.default_rng(10_000 + seed)
    big = rng.random(3) < 0.5                          # half the draws from the multi-tile range
    T = _log_int(rng, 256 if big[0] else 1, 4096)
    d_in = k_quant * _log_int(rng, 512 // k_quant if big[1] else 1, 4096 // k_quant)
    cap = min(20000, 2 ** 25 // d_in) // 8
    d_out = 8 * _log_int(rng, min(128, cap) if big[2] else 1, cap)
    R = int(rng.choice([r for r in RANKS if r <= max_slice_rank]))
    n_slots = _log_int(rng, 1, 63)
    ranks = rng.integers(1, R + 1, size=n_slots)
    ranks[rng.random(n_slots) < 0.1] = 0
    if not ranks.any():
        ranks[0] = R
    live = np.flatnonzero(ranks)
    kind = rng.choice(["uniform", "skewed", "one", "base", "sorted"])
    if kind == "skewed":
        p = 1.0 / np.arange(1, n_slots + 1) ** 1.2
        ids = rng.choice(n_slots, size=T, p=p / p.sum())
    elif kind == "one":
        ids = np.full(T, int(rng.choice(live)))
    elif kind == "base":
        ids = np.full(T, -1)
    else:
        ids = rng.integers(0, n_slots, size=T)
        if kind == "sorted":
            ids = np.sort(ids)
    ids = ids.astype(np.int32)
    if kind != "base":
        ids[rng.random(T) < rng.uniform(0, 0.5)] = -1
    if rng.random() < 0.3:
        ids[rng.integers(0, T)] = int(rng.choice([-7, -2, n_slots, n_slots + 5]))
    bad = [t for t, a in enumerate(ids) if a != -1 and not (0 <= a < n_slots and ranks[a] > 0)]
    edges = [e + d for e in range(64, T, 64) for d in (-1, 0)]
    rows = np.unique(np.concatenate([np.arange(min(T, 4)), np.arange(max(T - 4, 0), T),
                                     rng.choice(edges, size=min(len(edges), 12), replace=False)
                                     if edges else np.zeros(0, np.int64),
                                     rng.integers(0, T, size=16)])).astype(np.int64)
    return dict(T=T, d_in=d_in, d_out=d_out, R=R, ranks=[int(r) for r in ranks], ids=ids, kind=str(kind),
                first_bad=min(bad) if bad else -1, rows=rows, rng=rng)


def describe(c, extra=""):
    line = "case T=%d d_in=%d d_out=%s R=%d slots=%d ids=%s first_bad=%d%s" % (
        c["T"], c["d_in"], c["d_out"], c["R"], len(c["ranks"]), c["kind"], c["first_bad"], extra)
    print(line, flush=True)
    return line


class Layer:
    """x, W and one adapter pool on the GPU; A, B kept for the oracle."""

    def __init__(self, c, d_out, dtype, seed, x=None, packed=False):
        g = torch.Generator(device="cuda")
        g.manual_seed(seed)
        T, d_in, R = c["T"], c["d_in"], c["R"]
        self.dtype, self.d_out, self.ranks = dtype, d_out, c["ranks"]
        self.x = torch.randn(T, d_in, generator=g, device="cuda").to(dtype) if x is None else x
        self.W = (torch.randn(d_in, d_out, generator=g, device="cuda") / d_in ** 0.5).to(dtype)
        capacity = None
        if packed:   # each slot its rank rounded up to 8 rows, some an octet more
            extra = np.random.default_rng(seed).random(len(self.ranks)) < 0.3
            capacity = [min(R, max(8, -(-int(r) // 8) * 8 + 8 * int(e))) for r, e in zip(self.ranks, extra)]
        self.pool = L.AdapterPool(len(self.ranks), d_in, d_out, R, dtype, capacity=capacity)
        self.A, self.B, self.alphas = {}, {}, {}
        for s, r in enumerate(self.ranks):
            if r > 0:
                self.A[s] = (torch.randn(d_in, r, generator=g, device="cuda") / d_in ** 0.5).to(dtype)
                self.B[s] = (torch.randn(r, d_out, generator=g, device="cuda") / r ** 0.5).to(dtype)
                self.alphas[s] = 2.0 * r
                self.pool.upload(s, self.A[s], self.B[s], r, self.alphas[s])

    def oracle(self, ids, rows):
        used = {int(ids[t]) for t in rows} & set(self.A)
        n = len(self.ranks)
        A = [to_oracle(self.A[s]) if s in used else None for s in range(n)]
        B = [to_oracle(self.B[s]) if s in used else None for s in range(n)]
        sc = [lora_scale(self.alphas[s], self.ranks[s]) if s in self.alphas else 0.0 for s in range(n)]
        code = F32 if self.dtype == torch.float32 else BF16
        return oracle_rows(code, to_oracle(self.x), to_oracle(self.W), ids, A, B, self.ranks, sc,
                           rows=rows)["y"]


@pytest.mark.parametrize("seed,packed", [(s, False) for s in range(64)] + [(s, True) for s in range(64, 88)])
def test_sweep_forward(seed, packed):
    c = draw_case(seed)
    dtype = torch.float32 if c["rng"].random() < 0.25 else torch.bfloat16
    what = describe(c, " dtype=%s%s" % (str(dtype).split(".")[-1], " packed" if packed else ""))
    lay = Layer(c, c["d_out"], dtype, seed, packed=packed)
    ids_dev = torch.as_tensor(c["ids"], device="cuda")
    ref = lay.oracle(c["ids"], c["rows"])
    sel = torch.as_tensor(c["rows"], device="cuda")
    T = c["T"]
    for mode in MODES:
        for flags in (0, L.LORA_FLAG_SEPARATE_EXPAND):
            ws = L.Workspace(T, len(c["ranks"]), c["R"], c["d_out"])
            ys = []
            for _ in range(2):
                y = torch.full((T, c["d_out"]), 7.0, dtype=dtype, device="cuda")
                L.lora_linear_forward(lay.x, lay.W, y, T, lay.pool.pool, ids_dev, mode, flags, ws.buf)
                ys.append(y)
            torch.cuda.synchronize()
            w = "%s mode %d flags %d" % (what, mode, flags)
            assert_parity(ys[0][sel], ref, dtype, w)
            assert torch.equal(ys[0], ys[1]), w + " (repeat call)"
            assert L.lora_get_device_error(ws.buf) == c["first_bad"], w


@pytest.mark.parametrize("seed", range(20))
def test_sweep_sliced(seed):
    rng = np.random.default_rng(20_000 + seed)
    n = int(rng.integers(2, 5))
    c = draw_case(100 + seed, max_slice_rank=128 // n)
    d_outs = [8 * _log_int(rng, 1, min(20000, 2 ** 25 // c["d_in"]) // 8) for _ in range(n)]
    what = describe(c, " slices=%s" % d_outs)
    layers = [Layer(c, d_outs[0], torch.bfloat16, seed * 8)]
    layers += [Layer(c, d, torch.bfloat16, seed * 8 + i + 1, x=layers[0].x) for i, d in enumerate(d_outs[1:])]
    ids_dev = torch.as_tensor(c["ids"], device="cuda")
    refs = [lay.oracle(c["ids"], c["rows"]) for lay in layers]
    sel = torch.as_tensor(c["rows"], device="cuda")
    T, x = c["T"], layers[0].x
    for mode in MODES:
        for flags in (0, L.LORA_FLAG_SEPARATE_EXPAND):
            ws = L.Workspace(T, len(c["ranks"]), c["R"], sum(d_outs), n_slices=n)
            runs = []
            for _ in range(2):
                ys = [torch.full((T, d), 7.0, dtype=torch.bfloat16, device="cuda") for d in d_outs]
                L.lora_linear_forward_sliced(x, [lay.W for lay in layers], ys, T, [lay.pool.pool for lay in layers],
                                             ids_dev, mode, flags, ws.buf)
                runs.append(ys)
            torch.cuda.synchronize()
            for s in range(n):
                w = "%s slice %d mode %d flags %d" % (what, s, mode, flags)
                assert_parity(runs[0][s][sel], refs[s], torch.bfloat16, w)
                assert torch.equal(runs[0][s], runs[1][s]), w + " (repeat call)"
            assert L.lora_get_device_error(ws.buf) == c["first_bad"], what


@pytest.mark.parametrize("seed", range(20))
def test_sweep_fp8(seed):
    c = draw_case(200 + seed, k_quant=16)
    what = describe(c, " fp8")
    f = Fp8Case(c["T"], c["d_in"], c["d_out"], c["ranks"], c["R"], seed=seed, ids=c["ids"])
    ref, tol = f.reference(c["rows"])
    sel = torch.as_tensor(c["rows"], device="cuda")
    first = None
    for mode in MODES:
        for flags in (0, L.LORA_FLAG_SEPARATE_EXPAND):
            y, ws = f.run(mode, flags)
            w = "%s mode %d flags %d" % (what, mode, flags)
            assert_within(y[sel], ref, tol, w)
            assert L.lora_get_device_error(ws.buf) == c["first_bad"], w
            if first is None:
                first = y
    again, _ = f.run(MODES[0], 0)
    assert torch.equal(first, again), what + " (repeat call)"
