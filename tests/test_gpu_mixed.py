"""GPU checks of the per-segment mode choice in mixed batches ("Serving
multiple LoRAs: segmented matrix multiplies and adapter scheduling", section
"Not merging the weights, computing in batches": BGMV for decode rows, SGMV
for prefill segments, both in one forward).

In AUTO mode a batch of at least LORA_AUTO_SGMV_MIN_ROWS rows is split by segment length:
every segment takes the grouped shrink; segments of at least L rows take the
expand fused into the GEMM, shorter ones (decode rows) a per-row expand after
the GEMM, which visits their rows last.  The GEMM's row
order is checked bit for bit against the order derived from the oracle's
segment metadata; the outputs against the fp64 oracle for several L, every
expand path, packed pools, sliced calls and the FP8 base."""
import numpy as np
import pytest
import torch

from oracle import oracle_segments
from rank_adapter_gemm_amd import lora as L

from helpers import assert_parity
from test_gpu_packed import Batch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


def expected_gemm_order(ids, n_slots, short_len):
    """The stable partition of the sorted rows: the -1 block and segments of
    at least short_len rows first, then the shorter segments."""
    ref = oracle_segments(ids, n_slots)
    perm, off = ref["perm"], ref["offsets"]
    long_rows, short_rows = [], []
    for k in range(n_slots + 1):
        rows = perm[off[k]:off[k + 1]].tolist()
        if k >= 1 and 0 < len(rows) < short_len:
            short_rows += rows
        else:
            long_rows += rows
    return np.asarray(long_rows + short_rows, np.int32), len(long_rows)


@pytest.mark.parametrize("short_len", [1, 2, 16, 255])
def test_gemm_row_order_bit_exact(short_len):
    rng = np.random.default_rng(short_len)
    n_slots, T = 37, 3000
    lengths = [1] * 700 + [500, 800, 300] + list(rng.integers(2, 20, size=40))
    owners = rng.integers(-1, n_slots, size=len(lengths))
    order = rng.permutation(len(lengths))
    ids = np.repeat(owners[order], np.asarray(lengths)[order]).astype(np.int32)[:T]
    T = ids.size
    ids[[3, 900]] = [-7, n_slots + 2]                  # bad ids count as -1 (base rows)
    d = 64
    x = torch.zeros(T, d, dtype=torch.bfloat16, device="cuda")
    W = torch.zeros(d, d, dtype=torch.bfloat16, device="cuda")
    y = torch.empty(T, d, dtype=torch.bfloat16, device="cuda")
    pool = L.AdapterPool(n_slots, d, d, 8, torch.bfloat16)
    zA = torch.zeros(d, 8, dtype=torch.bfloat16, device="cuda")
    zB = torch.zeros(8, d, dtype=torch.bfloat16, device="cuda")
    for slot in range(n_slots):
        pool.upload(slot, zA, zB, 8, 16.0)
    ws = L.Workspace(T, n_slots, 8, d)
    ids_dev = torch.as_tensor(ids, device="cuda")
    L.lora_linear_forward(x, W, y, T, pool.pool, ids_dev, L.LORA_MODE_AUTO, L.LORA_FLAG_SHORT_SEGMENT(short_len),
                          ws.buf)
    torch.cuda.synchronize()
    seg = ws.segments(T)
    gp, nl = expected_gemm_order(ids, n_slots, short_len)
    assert int(seg["n_fused"].cpu()[0]) == nl
    assert np.array_equal(seg["gemm_perm"].cpu().numpy(), gp)
    ref = oracle_segments(ids, n_slots)
    assert np.array_equal(seg["perm"].cpu().numpy(), ref["perm"])
    assert L.lora_get_device_error(ws.buf) == 3
    # reading the error word leaves the segments in place
    assert int(seg["n_fused"].cpu()[0]) == nl
    # the public builder groups every segment: the GEMM order is perm itself
    L.lora_build_segments(ids_dev, T, n_slots, 8, ws.buf)
    torch.cuda.synchronize()
    assert int(seg["n_fused"].cpu()[0]) == T
    assert np.array_equal(seg["gemm_perm"].cpu().numpy(), ref["perm"])


@pytest.mark.parametrize("which", ["padded", "packed"])
def test_mixed_batch_every_threshold(which):
    """A mixed batch (decode rows and prefill chunks of heterogeneous-rank
    adapters, shuffled): AUTO at several thresholds, SGMV and BGMV, fused and
    separate expand, all against the oracle and within two bf16 roundings of
    each other."""
    ranks = [8, 16, 32, 64, 8, 24, 40, 64, 16, 56, 8, 32, 48, 16, 8, 64]
    b = Batch(200, [700, 400, 300, 9, 5, 17], 1024, 2048, ranks, 64, seed=11)
    assert b.T >= L.LORA_AUTO_SGMV_MIN_ROWS
    ref = b.oracle()
    outs = []
    runs = [(L.LORA_MODE_AUTO, L.LORA_FLAG_SHORT_SEGMENT(n)) for n in (0, 1, 4, 64, 255)]
    runs += [(L.LORA_MODE_SGMV, 0), (L.LORA_MODE_BGMV, 0)]
    for mode, fl in runs:
        for sep in (0, L.LORA_FLAG_SEPARATE_EXPAND):
            y = b.run(which, mode, fl | sep)
            assert_parity(y, ref, torch.bfloat16, "%s mode=%d flags=%#x" % (which, mode, fl | sep))
            outs.append(y.float())
    for y in outs[1:]:
        assert torch.max((y - outs[0]).abs() / (1 + outs[0].abs())).item() <= 2 ** -6


def test_mixed_batch_sliced_and_reused_segments():
    """Two slices sharing x in AUTO mode (segments built once, threshold 64:
    the decode rows, about 33 per adapter here, take the per-row path), then a
    third projection reusing the segments."""
    ranks = [8, 32, 16, 64, 24, 8, 40, 16]
    b = Batch(300, [600, 500, 200], 1024, 1536, ranks, 64, seed=12, n_slices=3)
    ws = L.Workspace(b.T, b.n_slots, 64, 2 * 1536, n_slices=2)
    ys = [torch.empty(b.T, 1536, dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    L.lora_linear_forward_sliced(b.x, [s["W"] for s in b.slices[:2]], ys[:2], b.T,
                                 [s["padded"].pool for s in b.slices[:2]], b.ids_dev, L.LORA_MODE_AUTO,
                                 L.LORA_FLAG_SHORT_SEGMENT(64), ws.buf)
    assert L.lora_get_device_error(ws.buf) == -1
    L.lora_linear_forward(b.x, b.slices[2]["W"], ys[2], b.T, b.slices[2]["packed"].pool, b.ids_dev,
                          L.LORA_MODE_AUTO, L.LORA_FLAG_SEGMENTS_READY, ws.buf)
    torch.cuda.synchronize()
    for k in range(3):
        assert_parity(ys[k], b.oracle(k), torch.bfloat16, "slice %d" % k)
    seg = ws.segments(b.T)
    _, nl = expected_gemm_order(b.ids, b.n_slots, 64)
    assert int(seg["n_fused"].cpu()[0]) == nl < b.T


def test_mixed_batch_fp8_thresholds_agree():
    """The FP8-base forward in AUTO mode with the per-row path (threshold 16)
    and without it (threshold 1): same codes, the low-rank term added
    differently, within two bf16 roundings."""
    ranks = [8, 16, 32, 64, 8, 24]
    b = Batch(150, [800, 200], 1024, 2048, ranks, 64, seed=13)
    sl = b.slices[0]
    w8 = L.Fp8Weight(sl["W"])
    outs = []
    for n in (1, 16):
        ws = L.Workspace(b.T, b.n_slots, 64, 2048, fp8_d_in=1024)
        y = torch.empty(b.T, 2048, dtype=torch.bfloat16, device="cuda")
        L.lora_linear_forward_fp8(b.x, w8.codes, w8.scale, y, b.T, sl["padded"].pool, b.ids_dev, L.LORA_MODE_AUTO,
                                  L.LORA_FLAG_SHORT_SEGMENT(n), ws.buf)
        torch.cuda.synchronize()
        assert L.lora_get_device_error(ws.buf) == -1
        outs.append(y.float())
    assert torch.max((outs[1] - outs[0]).abs() / (1 + outs[0].abs())).item() <= 2 ** -6


def test_overwritten_segment_tables_stay_in_bounds():
    """lora_gemm takes its split-K scratch from the first byte of the buffer it
    is given, so a forward workspace passed to it loses its segment tables.
    SGMV calls on such tables (here: overwritten by the plain GEMM's fp32
    partials, then by seeded random words over the whole workspace) give
    wrong rows but read and write only inside their buffers; building the
    segments again (after preparing the randomised workspace again) restores
    parity."""
    ranks = [8, 16, 32, 64, 8, 24, 40, 64]
    b = Batch(300, [700, 500, 300], 512, 1024, ranks, 64, seed=21)
    assert b.T >= L.LORA_AUTO_SGMV_MIN_ROWS
    sl = b.slices[0]
    pool = sl["padded"].pool
    ws = L.Workspace(b.T, b.n_slots, 64, 1024)
    y = torch.zeros(b.T, 1024, dtype=torch.bfloat16, device="cuda")
    v = torch.zeros(b.T, 64, dtype=torch.float32, device="cuda")
    sgmv, ready = L.LORA_MODE_SGMV, L.LORA_FLAG_SEGMENTS_READY

    def calls():
        L.lora_shrink(b.x, b.T, pool, b.ids_dev, sgmv, v, ws.buf)
        L.lora_gemm_expand(b.x, sl["W"], y, b.T, pool, b.ids_dev, v, sgmv, ws.buf)
        L.lora_expand(v, b.T, pool, b.ids_dev, sgmv, y, ws.buf)
        L.lora_linear_forward(b.x, sl["W"], y, b.T, pool, b.ids_dev, L.LORA_MODE_AUTO, ready, ws.buf)
        L.lora_linear_forward(b.x, sl["W"], y, b.T, pool, b.ids_dev, sgmv, ready | L.LORA_FLAG_SEPARATE_EXPAND,
                              ws.buf)
        torch.cuda.synchronize()

    L.lora_build_segments(b.ids_dev, b.T, b.n_slots, 64, ws.buf)
    L.lora_gemm(b.x, sl["W"], y, b.T, 512, 1024, L.LORA_BF16, ws=ws.buf)
    calls()
    g = torch.Generator(device="cuda")
    g.manual_seed(21)
    words = ws.buf.numel() // 4
    ws.buf[:4 * words].view(torch.int32).copy_(
        torch.randint(-2 ** 31, 2 ** 31 - 1, (words,), generator=g, device="cuda", dtype=torch.int64).to(torch.int32))
    calls()
    # the random words also replaced the error word and counters: a workspace
    # overwritten as a whole is prepared again, as after allocation
    L.lora_workspace_init(ws.buf)
    y.zero_()
    L.lora_linear_forward(b.x, sl["W"], y, b.T, pool, b.ids_dev, sgmv, 0, ws.buf)
    torch.cuda.synchronize()
    assert L.lora_get_device_error(ws.buf) == -1
    assert_parity(y, b.oracle(), torch.bfloat16, "after rebuilding the segments")


@pytest.mark.parametrize("dT", [-1, 0])
def test_auto_threshold_builds_segments_from_min_rows(dT):
    """AUTO takes the per-row path below LORA_AUTO_SGMV_MIN_ROWS rows (no
    segments are built in a fresh workspace) and builds segments from that
    many rows on; both agree with the oracle."""
    T_dec = L.LORA_AUTO_SGMV_MIN_ROWS + dT
    ranks = [8, 16, 32, 64, 8, 24, 40, 64, 16, 56, 8, 32]
    b = Batch(T_dec, [], 512, 1024, ranks, 64, seed=30 + dT)
    assert b.T == T_dec
    ws = L.Workspace(b.T, b.n_slots, 64, 1024)
    ws.segments(b.T)["n_seg"].fill_(-7)                 # a sentinel only a segment build overwrites
    y = torch.empty(b.T, 1024, dtype=torch.bfloat16, device="cuda")
    L.lora_linear_forward(b.x, b.slices[0]["W"], y, b.T, b.slices[0]["padded"].pool, b.ids_dev, L.LORA_MODE_AUTO, 0,
                          ws.buf)
    torch.cuda.synchronize()
    assert L.lora_get_device_error(ws.buf) == -1
    n_seg = int(ws.segments(b.T)["n_seg"].cpu()[0])
    if dT < 0:
        assert n_seg == -7
    else:
        assert n_seg == len(np.unique(b.ids[b.ids >= 0]))
    assert_parity(y, b.oracle(), torch.bfloat16, "T=%d" % b.T)
