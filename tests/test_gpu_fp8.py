"""GPU parity of the FP8-base path (E4M3 base weight and activations, bf16
adapters) against the fp64 oracle in oracle/fp8.py.

* Quantizers: codes and scales bitwise equal to the oracle's (an integer
  result decided in fp32 on both sides), on rows and columns with ragged
  tails, zero rows, ties and a wide spread of magnitudes.
* Base GEMM and whole layer: element-wise within a bound derived from the
  arithmetic -- bf16 rounding of y (unit roundoff 2^-8 of |ref|; with the
  separate expand the base product is rounded once more, 2^-8 of |base|),
  the fp32 low-rank path (2^-10 of the magnitude of its terms,
  |s| sum_j |u_j| |B_jn|) and the matrix cores' accumulation of FP8
  products (below 2^-12 of each 64-product block's largest term, so 2^-11
  of S = s_x s_w sum_k |dq(xq) dq(wq)|).
  Shapes are chosen so every tile plan runs: 128x64 whole tiles, 128x128
  split-K (eight wavefronts), 256x128 whole tiles, 256x256 whole tiles plus a
  split tail.
* The low-rank term is really added (a delta-sensitive check), bad ids are
  flagged and computed as base rows, T = 0 is a no-op, and the decode-sized
  workload at full size matches on sampled rows in the benchmark's launch
  configuration.
"""
import numpy as np
import pytest
import torch

from oracle import BF16, lora_scale, oracle_rows
from oracle.fp8 import oracle_fp8_base, quantize_rows_e4m3, quantize_weight_e4m3
from rank_adapter_gemm_amd import lora as L
from rank_adapter_gemm_amd.workloads import make_workload, sample_rows

from helpers import to_oracle
from helpers_fp8 import Fp8Case, assert_within, f32, fp8_bound

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


def test_quantize_rows_bitwise():
    torch.manual_seed(0)
    T, K = 300, 1040                                   # K not a multiple of the 2048-value row sweep
    x = torch.randn(T, K, device="cuda")
    x *= torch.exp2(torch.randint(-30, 30, (T, 1), device="cuda").float())   # wide spread of row scales
    x[3] = 0.0
    x[4] = -0.0
    x[5, :] = 1e-3
    x[5, 7] = 448.0                                    # ties and exact grid values after scaling
    x[6] = torch.linspace(-1, 1, K, device="cuda")
    x = x.to(torch.bfloat16)
    xq = torch.full((T, K), 0xAB, dtype=torch.uint8, device="cuda")
    xs = torch.full((T,), float("nan"), device="cuda")
    L.lora_quantize_rows_fp8(x, T, K, xq, xs)
    torch.cuda.synchronize()
    rq, rs = quantize_rows_e4m3(f32(x))
    assert np.array_equal(xs.cpu().numpy(), rs)
    got = xq.cpu().numpy()
    bad = np.argwhere(got != rq)
    assert bad.size == 0, "first code mismatch at %s: gpu %#x oracle %#x" % (
        bad[0], got[tuple(bad[0])], rq[tuple(bad[0])])


@pytest.mark.parametrize("K,N", [(1040, 264), (4096, 4096), (16, 8)])
def test_quantize_weight_bitwise(K, N):
    g = torch.Generator(device="cuda")
    g.manual_seed(K + N)
    W = torch.randn(K, N, generator=g, device="cuda") * 0.02
    if N > 8:
        W[:, 5] = 0.0                                  # a zero column: scale 0, zero codes
        W[:, 9] *= 1e-20
    W = W.to(torch.bfloat16)
    wt = L.Fp8Weight(W)
    torch.cuda.synchronize()
    rq, rs = quantize_weight_e4m3(f32(W))
    assert np.array_equal(wt.scale.cpu().numpy(), rs)
    assert np.array_equal(wt.codes.cpu().numpy(), rq)


# (T, K, N): the tile plan each shape takes
GEMM_SHAPES = [
    (300, 208, 264),    # 128x64 whole tiles (K too short to split), ragged T and N
    (300, 1040, 264),   # 128x128 split-K, ragged K
    (37, 2048, 1024),   # 128x128 split-K (decode-sized, eight K ranges)
    (2048, 512, 3584),  # 256x128 whole tiles
    (4352, 1024, 4096), # 256x256 whole tiles plus a split-K tail round
    (300, 256, 16408),  # 256x128 in column bands (129 column tiles, the last band one tile wide)
    (520, 1024, 16384), # column bands with a split-K tail round
]


@pytest.mark.parametrize("T,K,N", GEMM_SHAPES)
def test_gemm_fp8_base(T, K, N):
    c = Fp8Case(T, K, N, ranks=[8], R=8, seed=T + K)
    ws = L.Workspace(T, 1, 8, N, fp8_d_in=K)
    xq = torch.empty(T, K, dtype=torch.uint8, device="cuda")
    xs = torch.empty(T, device="cuda")
    L.lora_quantize_rows_fp8(c.x, T, K, xq, xs)
    y = torch.full((T, N), 7.0, dtype=torch.bfloat16, device="cuda")
    L.lora_gemm_fp8(xq, xs, c.wt.codes, c.wt.scale, y, T, K, N, ws.buf)
    torch.cuda.synchronize()
    rows = np.arange(T) if T <= 512 else np.unique(np.concatenate([np.arange(0, T, 7), np.arange(T - 300, T)]))
    rq, rs = quantize_rows_e4m3(f32(c.x)[rows])
    wq, wsc = c.weight_codes()
    assert np.array_equal(xq.cpu().numpy()[rows], rq)
    ref = oracle_fp8_base(rq, rs, wq, wsc)
    tol = 2.0 ** -8 * np.abs(ref) + fp8_bound(rq, rs, wq, wsc) + 1e-30
    assert_within(y[torch.as_tensor(rows, device="cuda")], ref, tol, "gemm_fp8 %dx%dx%d" % (T, K, N))
    # without workspace: whole tiles only, same result up to fp32 summation order
    y2 = torch.full((T, N), 7.0, dtype=torch.bfloat16, device="cuda")
    L.lora_gemm_fp8(xq, xs, c.wt.codes, c.wt.scale, y2, T, K, N)
    torch.cuda.synchronize()
    assert_within(y2[torch.as_tensor(rows, device="cuda")], ref, tol, "gemm_fp8 no-split %dx%dx%d" % (T, K, N))


FWD_SHAPES = [
    (300, 208, 264, 16, [3, 16, 0, 9, 13]),     # 128x64 whole tiles, ragged everything
    (37, 2048, 1024, 16, [16, 16, 7, 0]),       # decode-sized split-K
    (200, 1024, 4096, 32, [32, 17, 8, 0, 32]),  # decode-sized, larger rank
    (1500, 512, 512, 16, [16, 4, 16, 12]),      # SGMV-sized (AUTO picks SGMV from LORA_AUTO_SGMV_MIN_ROWS rows)
    (2048, 512, 3584, 8, [8, 8, 3]),            # 256x128 whole tiles with the fused expand
    (1, 16, 8, 8, [8, 5]),                      # the smallest shape: one row, one K step, one column octet
    (1, 4096, 4096, 16, [16, 16, 16]),          # one decode row
    (5, 48, 24, 128, [128, 1, 77, 0]),          # max rank 128, ragged ranks, K and N far below a tile
    (520, 1024, 16384, 16, [16, 9, 0, 16]),     # column bands, split-K tail, expand fused and in the reduction
]


@pytest.mark.parametrize("T,K,N,R,ranks", FWD_SHAPES)
def test_forward_fp8_every_row(T, K, N, R, ranks):
    rng = np.random.default_rng(T)
    n = len(ranks)
    ids = rng.integers(-1, n, size=T).astype(np.int32)
    if T > 12:
        ids[[3, 7]] = [-3, n]                          # out of range: flagged, base rows
    empty = [s for s, r in enumerate(ranks) if r == 0]
    if empty and T > 12:
        ids[12] = empty[0]                             # an empty slot: flagged too
    if T <= 5:                                         # tiny batches: every row on a usable adapter, in turn
        usable = [a for a in range(n) if ranks[a] > 0]
        ids[:] = [usable[i % len(usable)] for i in range(T)]
    bad_rows = [t for t, a in enumerate(ids) if a != -1 and not (0 <= a < n and ranks[a] > 0)]
    c = Fp8Case(T, K, N, ranks, R, seed=T + 1, ids=ids)
    rows = None if T <= 512 else np.unique(np.concatenate([np.arange(0, T, 5), np.arange(T - 64, T)]))
    ref, tol = c.reference(rows)
    sel = slice(None) if rows is None else torch.as_tensor(rows, device="cuda")
    outs = []
    for mode in (L.LORA_MODE_AUTO, L.LORA_MODE_BGMV, L.LORA_MODE_SGMV):
        for flags in (0, L.LORA_FLAG_SEPARATE_EXPAND):
            y, ws = c.run(mode, flags)
            what = "fp8 T=%d K=%d N=%d mode %d flags %d" % (T, K, N, mode, flags)
            assert_within(y[sel], ref, tol, what)
            assert L.lora_get_device_error(ws.buf) == (min(bad_rows) if bad_rows else -1), what
            outs.append(y)
    y2, _ = c.run(L.LORA_MODE_BGMV, 0)
    assert torch.equal(outs[2], y2), "not deterministic"


def test_forward_fp8_delta_is_applied():
    """Values N(0, 0.02) as in the decode workload: the low-rank term is small
    next to the tolerance of y, so check it alone -- the FP8 layer with
    adapters minus the same layer with every row a base row, against the
    oracle's low-rank term."""
    T, K, N, R = 256, 1024, 4096, 16
    c = Fp8Case(T, K, N, [16, 16, 16], R, seed=5, base_frac=0.0, sd=(0.02, 0.02))
    for mode in (L.LORA_MODE_BGMV, L.LORA_MODE_SGMV):
        for flags in (0, L.LORA_FLAG_SEPARATE_EXPAND):
            y, _ = c.run(mode, flags)
            ids_save = c.ids_dev.clone()
            c.ids_dev.fill_(-1)
            y0, _ = c.run(mode, flags)
            c.ids_dev.copy_(ids_save)
            A = [to_oracle(a) for a in c.A]
            B = [to_oracle(b) for b in c.B]
            sc = [lora_scale(a, r) for a, r in zip(c.alphas, c.ranks)]
            zero_w = np.zeros((K, N), np.uint16)
            d_ref = oracle_rows(BF16, to_oracle(c.x), zero_w, c.ids, A, B, c.ranks, sc)["y"]
            d_gpu = y.float().cpu().double().numpy() - y0.float().cpu().double().numpy()
            # each of y, y0 is rounded to bf16 once: 2^-9 of |y| each, plus the fp32 paths
            bound = 2.0 ** -8 * np.abs(y.float().cpu().double().numpy()) + 2.0 ** -10 * np.abs(d_ref).max()
            assert np.abs(d_ref).max() > 10 * bound.max() / 4, "delta too small to be seen"
            assert np.all(np.abs(d_gpu - d_ref) <= bound + 1e-30), "mode %d flags %d" % (mode, flags)


@pytest.mark.parametrize("T,K,N,mode", [(256, 1024, 4096, L.LORA_MODE_BGMV), (37, 2048, 1024, L.LORA_MODE_BGMV),
                                         (300, 208, 264, L.LORA_MODE_AUTO), (1500, 512, 512, L.LORA_MODE_SGMV)])
def test_forward_fp8_codes_match_the_row_quantizer(T, K, N, mode):
    """The forward quantizes x itself (for BGMV rows inside the shrink's
    launch): with every row a base row its y depends on the codes and
    scales alone, so it must equal, bitwise, the standalone row quantizer
    followed by lora_gemm_fp8 on the same workspace size."""
    c = Fp8Case(T, K, N, [16, 8], 16, seed=T + N, ids=np.full(T, -1, np.int32))
    y, ws = c.run(mode, 0)
    xq = torch.empty(T, K, dtype=torch.uint8, device="cuda")
    xs = torch.empty(T, device="cuda")
    L.lora_quantize_rows_fp8(c.x, T, K, xq, xs)
    y_ref = torch.full((T, N), 7.0, dtype=torch.bfloat16, device="cuda")
    ws2 = L.Workspace(T, c.n_slots, c.R, N, fp8_d_in=K)
    L.lora_gemm_fp8(xq, xs, c.wt.codes, c.wt.scale, y_ref, T, K, N, ws2.buf)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)
    assert L.lora_get_device_error(ws.buf) == -1


def test_forward_fp8_empty_batch():
    c = Fp8Case(4, 64, 64, [8], 8, seed=9)
    y, ws = c.run(L.LORA_MODE_AUTO, 0, T=0)
    assert torch.all(y.float() == 7.0)


def test_decode_workload_full_size_sampled():
    """The decode workload (T = 256, 4096 -> 4096, r = 16, 128 slots) at full
    size through lora_linear_forward_fp8 as the benchmark runs it, every
    column of a bounded row sample against the oracle."""
    wl = make_workload("decode_bgmv", device="cuda")
    proj = wl.projections[0]
    x = wl.x_for(proj)
    pool = L.AdapterPool(wl.n_slots, proj.d_in, proj.d_out, wl.max_rank, wl.dtype)
    for s in range(wl.n_slots):
        r = int(wl.ranks[s])
        if r > 0:
            pool.upload(s, proj.A[s], proj.B[s], r, float(wl.alphas[s]), lda=wl.max_rank, ldb=proj.d_out)
    wt = L.Fp8Weight(proj.W)
    ids_dev = torch.as_tensor(wl.ids, device="cuda")
    ws = L.Workspace(wl.T, wl.n_slots, wl.max_rank, proj.d_out, fp8_d_in=proj.d_in)
    y = torch.empty(wl.T, proj.d_out, dtype=wl.dtype, device="cuda")
    L.lora_linear_forward_fp8(x, wt.codes, wt.scale, y, wl.T, pool.pool, ids_dev, L.LORA_MODE_AUTO, 0, ws.buf)
    torch.cuda.synchronize()
    assert L.lora_get_device_error(ws.buf) == -1
    rows = sample_rows(wl, max_rows=48)
    wq, wsc = quantize_weight_e4m3(f32(proj.W))
    assert np.array_equal(wt.codes.cpu().numpy(), wq) and np.array_equal(wt.scale.cpu().numpy(), wsc)
    xq, xs = quantize_rows_e4m3(f32(x)[rows])
    base = oracle_fp8_base(xq, xs, wq, wsc)
    used = sorted({int(wl.ids[r]) for r in rows if wl.ids[r] >= 0})
    A = [None] * wl.n_slots
    B = [None] * wl.n_slots
    for s in used:
        A[s] = to_oracle(wl.slot_A(proj, s))
        B[s] = to_oracle(wl.slot_B(proj, s))
    sc = [lora_scale(float(wl.alphas[s]), int(wl.ranks[s])) for s in range(wl.n_slots)]
    lo = oracle_rows(BF16, to_oracle(x), np.zeros((proj.d_in, proj.d_out), np.uint16), wl.ids, A, B,
                     [int(r) for r in wl.ranks], sc, rows=rows)["y"]
    ref = base + lo
    # fused expand: one rounding of y; |lo| stands in for the magnitude of
    # the low-rank terms (the decode values make them tiny next to |y|)
    tol = 2.0 ** -8 * np.abs(ref) + 2.0 ** -8 * np.abs(lo) + fp8_bound(xq, xs, wq, wsc) + 1e-30
    assert_within(y[torch.as_tensor(rows, device="cuda")], ref, tol, "decode workload fp8")


def test_prefill_workload_full_size_sampled():
    """The prefill workload (32 432 rows in 64 adapter segments, 4096 -> 14336,
    r = 32) at full size through lora_linear_forward_fp8 (SGMV), every column
    of a bounded row sample against the oracle."""
    wl = make_workload("prefill_sgmv", device="cuda")
    proj = wl.projections[0]
    x = wl.x_for(proj)
    pool = L.AdapterPool(wl.n_slots, proj.d_in, proj.d_out, wl.max_rank, wl.dtype)
    for s in range(wl.n_slots):
        r = int(wl.ranks[s])
        if r > 0:
            pool.upload(s, proj.A[s], proj.B[s], r, float(wl.alphas[s]), lda=wl.max_rank, ldb=proj.d_out)
    wt = L.Fp8Weight(proj.W)
    ids_dev = torch.as_tensor(wl.ids, device="cuda")
    ws = L.Workspace(wl.T, wl.n_slots, wl.max_rank, proj.d_out, fp8_d_in=proj.d_in)
    y = torch.empty(wl.T, proj.d_out, dtype=wl.dtype, device="cuda")
    L.lora_linear_forward_fp8(x, wt.codes, wt.scale, y, wl.T, pool.pool, ids_dev, L.LORA_MODE_AUTO, 0, ws.buf)
    torch.cuda.synchronize()
    assert L.lora_get_device_error(ws.buf) == -1
    rows = sample_rows(wl, max_rows=64)
    wq, wsc = quantize_weight_e4m3(f32(proj.W))
    xq, xs = quantize_rows_e4m3(f32(x)[rows])
    base = oracle_fp8_base(xq, xs, wq, wsc)
    used = sorted({int(wl.ids[r]) for r in rows if wl.ids[r] >= 0})
    A = [None] * wl.n_slots
    B = [None] * wl.n_slots
    for s in used:
        A[s] = to_oracle(wl.slot_A(proj, s))
        B[s] = to_oracle(wl.slot_B(proj, s))
    sc = [lora_scale(float(wl.alphas[s]), int(wl.ranks[s])) for s in range(wl.n_slots)]
    lo = oracle_rows(BF16, to_oracle(x), np.zeros((proj.d_in, proj.d_out), np.uint16), wl.ids, A, B,
                     [int(r) for r in wl.ranks], sc, rows=rows)["y"]
    ref = base + lo
    # fused expand: one rounding of y; |lo| stands in for the low-rank terms' magnitude
    tol = 2.0 ** -8 * np.abs(ref) + 2.0 ** -6 * np.abs(lo) + fp8_bound(xq, xs, wq, wsc) + 1e-30
    assert_within(y[torch.as_tensor(rows, device="cuda")], ref, tol, "prefill workload fp8")
