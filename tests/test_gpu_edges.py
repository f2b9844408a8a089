"""GPU edge cases and invariants: ragged shapes (tails of every tile), T = 0
and 1, ranks below max_rank, empty and cleared slots, bad ids, base-only
batches, determinism, row permutation, mode independence, pool layout."""
import numpy as np
import pytest
import torch

from oracle import BF16, F32, lora_scale, oracle_rows
from rank_adapter_gemm_amd import lora as L

from helpers import TOL, assert_parity, to_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


class Case:
    """A small synthetic batch with explicit per-slot ranks."""

    def __init__(self, T, d_in, d_out, ranks, max_rank, dtype, seed=0, base_frac=0.2, ids=None,
                 alphas=None):
        g = torch.Generator(device="cuda")
        g.manual_seed(seed)
        rng = np.random.default_rng(seed)
        self.T, self.d_in, self.d_out, self.R, self.dtype = T, d_in, d_out, max_rank, dtype
        self.ranks = list(ranks)
        self.n_slots = len(ranks)
        self.alphas = list(alphas) if alphas is not None else [2.0 * r for r in ranks]
        self.x = (torch.randn(T, d_in, generator=g, device="cuda")).to(dtype)
        self.W = (torch.randn(d_in, d_out, generator=g, device="cuda") / d_in ** 0.5).to(dtype)
        self.A = [(torch.randn(d_in, max(r, 1), generator=g, device="cuda") / d_in ** 0.5).to(dtype)
                  for r in ranks]
        self.B = [(torch.randn(max(r, 1), d_out, generator=g, device="cuda") / max(r, 1) ** 0.5).to(dtype)
                  for r in ranks]
        if ids is None:
            ids = rng.integers(0, self.n_slots, size=T).astype(np.int32)
            ids[rng.random(T) < base_frac] = -1
        self.ids = np.asarray(ids, dtype=np.int32)
        self.pool = L.AdapterPool(self.n_slots, d_in, d_out, max_rank, dtype)
        for s, r in enumerate(ranks):
            if r > 0:
                self.pool.upload(s, self.A[s], self.B[s], r, self.alphas[s])
        self.ids_dev = torch.as_tensor(self.ids, device="cuda")

    def run(self, mode=L.LORA_MODE_AUTO, flags=0, T=None, split_scratch=True):
        T = self.T if T is None else T
        ws = L.Workspace(max(T, 1), self.n_slots, self.R, self.d_out if split_scratch else 0)
        y = torch.full((max(T, 1), self.d_out), 7.0, dtype=self.dtype, device="cuda")
        L.lora_linear_forward(self.x, self.W, y, T, self.pool.pool, self.ids_dev, mode, flags, ws.buf)
        torch.cuda.synchronize()
        return y, ws

    def oracle(self, ids=None):
        ids = self.ids if ids is None else ids
        code = F32 if self.dtype == torch.float32 else BF16
        A = [to_oracle(a) if r > 0 else None for a, r in zip(self.A, self.ranks)]
        B = [to_oracle(b) if r > 0 else None for b, r in zip(self.B, self.ranks)]
        sc = [lora_scale(a, r) for a, r in zip(self.alphas, self.ranks)]
        return oracle_rows(code, to_oracle(self.x), to_oracle(self.W), ids, A, B, self.ranks, sc)["y"]


MODES = [L.LORA_MODE_BGMV, L.LORA_MODE_SGMV]
FLAGS = [0, L.LORA_FLAG_SEPARATE_EXPAND]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_ragged_shapes_every_tile_tail(dtype):
    """T, d_in, d_out not multiples of any tile (K tails of 8, N tails of 8),
    ranks 1..max_rank not multiples of 8."""
    c = Case(T=300, d_in=200, d_out=264, ranks=[3, 16, 1, 9, 13], max_rank=16, dtype=dtype, seed=1)
    ref = c.oracle()
    for mode in MODES:
        for flags in FLAGS:
            y, ws = c.run(mode, flags)
            assert_parity(y, ref, dtype, "ragged mode=%d flags=%d" % (mode, flags))
            assert L.lora_get_device_error(ws.buf) == -1


def test_large_ragged_bf16():
    c = Case(T=1100, d_in=1032, d_out=2056, ranks=[64, 8, 40, 24], max_rank=64,
             dtype=torch.bfloat16, seed=2)
    ref = c.oracle()
    for mode in MODES + [L.LORA_MODE_AUTO]:
        y, _ = c.run(mode)
        assert_parity(y, ref, torch.bfloat16, "large ragged mode=%d" % mode)


def test_t_zero_is_noop_and_t_one():
    c = Case(T=1, d_in=64, d_out=64, ranks=[8], max_rank=8, dtype=torch.bfloat16, seed=3, ids=[0])
    y, _ = c.run(T=0)
    assert (y.float() == 7.0).all()
    y, _ = c.run()
    assert_parity(y, c.oracle(), torch.bfloat16, "T=1")


def test_all_base_rows_equal_plain_gemm_bitwise():
    c = Case(T=513, d_in=256, d_out=512, ranks=[8, 16], max_rank=16, dtype=torch.bfloat16, seed=4,
             ids=np.full(513, -1, np.int32))
    yg = torch.empty(513, 512, dtype=torch.bfloat16, device="cuda")
    L.lora_gemm(c.x, c.W, yg, 513, 256, 512, L.LORA_BF16)
    for mode in MODES:
        for flags in FLAGS:
            y, _ = c.run(mode, flags)
            assert torch.equal(y, yg)
    assert_parity(yg, c.oracle(), torch.bfloat16, "gemm")


def test_bad_ids_and_empty_slots_are_base_rows_and_flagged():
    T = 200
    rng = np.random.default_rng(5)
    ids = rng.integers(0, 3, size=T).astype(np.int32)
    ids[[7, 50, 120]] = [-5, 3, 1000]
    ids[[9, 60]] = 2                      # slot 2 is empty (rank 0)
    c = Case(T=T, d_in=128, d_out=96, ranks=[8, 5, 0], max_rank=8, dtype=torch.bfloat16, seed=5,
             ids=ids)
    yg = torch.empty(T, 96, dtype=torch.bfloat16, device="cuda")
    L.lora_gemm(c.x, c.W, yg, T, 128, 96, L.LORA_BF16)
    bad = [7, 50, 120, 9, 60] + [i for i in range(T) if ids[i] == 2]
    for mode in MODES:
        y, ws = c.run(mode)
        assert L.lora_get_device_error(ws.buf) == min(bad)
        assert L.lora_get_device_error(ws.buf) == -1          # cleared by the read
        assert torch.equal(y[bad], yg[bad])
        assert_parity(y, c.oracle(), torch.bfloat16, "bad ids mode=%d" % mode)


def test_clear_slot_then_upload_again():
    c = Case(T=64, d_in=64, d_out=64, ranks=[8, 8], max_rank=8, dtype=torch.bfloat16, seed=6,
             ids=np.zeros(64, np.int32))
    yg = torch.empty(64, 64, dtype=torch.bfloat16, device="cuda")
    L.lora_gemm(c.x, c.W, yg, 64, 64, 64, L.LORA_BF16)
    c.pool.clear(0)
    y, ws = c.run()
    assert torch.equal(y, yg)
    assert L.lora_get_device_error(ws.buf) == 0            # row 0 names an empty slot
    c.pool.upload(0, c.A[0], c.B[0], 8, c.alphas[0])
    y, _ = c.run()
    assert_parity(y, c.oracle(), torch.bfloat16, "re-upload")


def test_pool_layout_and_strided_upload():
    """Upload with lda > r reads the right columns; the pool holds A^T rank
    rows and B in rank octets, zero beyond the rank."""
    d_in, d_out, R, r = 40, 24, 16, 5
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    Abig = torch.randn(d_in, 11, generator=g, device="cuda").to(torch.bfloat16)
    B = torch.randn(r, d_out, generator=g, device="cuda").to(torch.bfloat16)
    pool = L.AdapterPool(3, d_in, d_out, R, torch.bfloat16)
    pool.upload(1, Abig, B, r, 10.0, lda=11)
    torch.cuda.synchronize()
    a = pool.a.view(torch.bfloat16).view(3, R, d_in)
    b = pool.b.view(torch.bfloat16).view(3, R // 8, d_out, 8)
    assert torch.equal(a[1, :r], Abig[:, :r].t())
    assert (a[1, r:].float() == 0).all() and (a[0].float() == 0).all()
    Bp = torch.zeros(R, d_out, dtype=torch.bfloat16, device="cuda")
    Bp[:r] = B
    assert torch.equal(b[1], Bp.view(R // 8, 8, d_out).permute(0, 2, 1))
    assert pool.rank.cpu().tolist() == [0, 5, 0]
    assert pool.scale.cpu().tolist()[1] == pytest.approx(2.0)


def test_deterministic_and_row_permutation():
    c = Case(T=700, d_in=512, d_out=384, ranks=[16, 8, 12, 16], max_rank=16,
             dtype=torch.bfloat16, seed=8)
    for mode in MODES:
        y1, _ = c.run(mode)
        y2, _ = c.run(mode)
        assert torch.equal(y1, y2)
    # permute the rows (and their ids): the output rows permute bitwise
    p = torch.as_tensor(np.random.default_rng(9).permutation(700), device="cuda")
    c2 = Case(T=700, d_in=512, d_out=384, ranks=[16, 8, 12, 16], max_rank=16,
              dtype=torch.bfloat16, seed=8)
    c2.x = c.x[p].contiguous()
    c2.ids_dev = c.ids_dev[p].contiguous()
    c2.ids = c.ids[p.cpu().numpy()]
    for mode in MODES:
        for flags in FLAGS:
            y1, _ = c.run(mode, flags)
            y2, _ = c2.run(mode, flags)
            assert torch.equal(y2, y1[p]), "mode %d flags %d" % (mode, flags)


def test_modes_agree():
    c = Case(T=2048, d_in=1024, d_out=1024, ranks=[32] * 6, max_rank=32, dtype=torch.bfloat16,
             seed=10)
    outs = [c.run(m, f)[0].float() for m in MODES for f in FLAGS]
    ref = c.oracle()
    for y in outs:
        assert_parity(y, ref, torch.bfloat16, "modes")
    # two roundings at most differ between the forms: 2 bf16 ulps of |y|
    for y in outs[1:]:
        assert torch.max((y - outs[0]).abs() / (1 + outs[0].abs())).item() <= 2 ** -6


def test_host_errors_enqueue_nothing():
    c = Case(T=16, d_in=64, d_out=64, ranks=[8], max_rank=8, dtype=torch.bfloat16, seed=11)
    ws = L.Workspace(16, 1, 8, 64)
    y = torch.empty(16, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(L.LoraError) as e:
        c.pool.upload(0, c.A[0], c.B[0], 9, 1.0)
    assert e.value.status == L.LORA_ERR_RANK_EXCEEDS_MAX
    with pytest.raises(L.LoraError) as e:
        c.pool.upload(1, c.A[0], c.B[0], 8, 1.0)
    assert e.value.status == L.LORA_ERR_SLOT_OUT_OF_RANGE
    small = torch.empty(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(L.LoraError) as e:
        L.lora_linear_forward(c.x, c.W, y, 16, c.pool.pool, c.ids_dev, 0, 0, small)
    assert e.value.status == L.LORA_ERR_WORKSPACE_TOO_SMALL
    with pytest.raises(L.LoraError) as e:
        L.lora_linear_forward(c.x[:, 1:], c.W, y, 16, c.pool.pool, c.ids_dev, 0, 0, ws.buf)
    assert e.value.status == L.LORA_ERR_INVALID_ARGUMENT      # misaligned x


@pytest.mark.parametrize("T,d_in,d_out", [(256, 4096, 4096), (64, 1032, 520), (2240, 4096, 1024),
                                          (300, 2048, 264), (4096, 512, 256), (2240, 1024, 4096),
                                          (520, 1024, 8192), (300, 256, 16408), (520, 1024, 16384),
                                          (3328, 256, 4096)])
def test_split_k_and_tile_configs(T, d_in, d_out):
    """Small batches split the GEMM over K when the workspace holds the fp32
    partials, and larger ones split only a mostly idle last round of tiles
    (2240 x 1024 x 4096: 288 tiles of 256 x 128, the last 32 split in two;
    520 x 1024 x 8192: 320 tiles of 128 x 128, the last 64 split in two); with
    and without that scratch the results agree with the oracle (and with each
    other to fp32 summation order), for every tile shape the planner picks.
    The last two are wide grids that the XCDs take in column bands:
    300 x 256 x 16408 is 2 x 129 tiles of 256 x 128 (the last band one tile
    wide, the last tile 24 columns), 520 x 1024 x 16384 is 3 x 128 tiles of
    256 x 128 whose last 128 are split in two, so the reduction walks the
    same order.  3328 x 256 x 4096 is 208 tiles of 256 x 256: one round,
    taken over 416 tiles of 256 x 128."""
    c = Case(T=T, d_in=d_in, d_out=d_out, ranks=[16, 8, 16, 4], max_rank=16, dtype=torch.bfloat16,
             seed=12)
    ref = c.oracle()
    outs = []
    for split_scratch in (True, False):
        for mode in MODES:
            for flags in FLAGS:
                y, ws = c.run(mode, flags, split_scratch=split_scratch)
                assert_parity(y, ref, torch.bfloat16, "T=%d split=%s mode=%d flags=%d"
                              % (T, split_scratch, mode, flags))
                outs.append(y.float())
    for y in outs[1:]:
        assert torch.max((y - outs[0]).abs() / (1 + outs[0].abs())).item() <= 2 ** -6
    # the plain GEMM entry point, with and without scratch
    ws = torch.empty(L.lora_workspace_bytes(T, 1, 8, d_out), dtype=torch.uint8, device="cuda")
    y1 = torch.empty(T, d_out, dtype=torch.bfloat16, device="cuda")
    y2 = torch.empty(T, d_out, dtype=torch.bfloat16, device="cuda")
    L.lora_gemm(c.x, c.W, y1, T, d_in, d_out, L.LORA_BF16, ws=ws)
    L.lora_gemm(c.x, c.W, y2, T, d_in, d_out, L.LORA_BF16)
    base = c.oracle(ids=np.full(T, -1, np.int32))
    assert_parity(y1, base, torch.bfloat16, "gemm split")
    assert_parity(y2, base, torch.bfloat16, "gemm")


@pytest.mark.parametrize("T", [300, 1500])
def test_padding_to_max_rank_does_not_change_results(T):
    """The same adapters (ranks 3..16) in pools padded to max_rank 16, 32 and
    64: kernels read only each slot's own rank rows, so the outputs agree to
    fp32 summation order (and with the oracle), in both modes."""
    ranks = [16, 3, 8, 13, 0, 9]
    outs = {}
    for R in (16, 32, 64):
        c = Case(T=T, d_in=512, d_out=768, ranks=ranks, max_rank=R, dtype=torch.bfloat16, seed=3)
        ref = c.oracle()
        for mode in MODES:
            y, _ = c.run(mode, 0)
            assert_parity(y, ref, torch.bfloat16, "R=%d mode=%d" % (R, mode))
            outs[(R, mode)] = y.float()
    base = outs[(16, L.LORA_MODE_BGMV)]
    for key, y in outs.items():
        assert torch.max((y - base).abs() / (1 + base.abs())).item() <= 2 ** -7, key


def test_fused_expand_carries_v_at_fp32():
    """The fused expand feeds s v to the matrix cores at its full fp32 value.
    Exact inputs: x = (1, 1, 1, 0, ...), A's three rank columns give
    v = (1 + 2^-9 + 2^-20, -1, -2^-9) exactly in fp32, B = 1 on those ranks,
    s = 1 and W = 0, so y = 2^-20 exactly (a bf16 value).  A bf16 high/low
    split of v (16 bits) would lose the 2^-20 and give 0.  Whole tiles
    (2048 x 4096 is 256 tiles of 256 x 128, no K split) and the separate
    expand both give 2^-20 on every element."""
    T, d_in, d_out = 2048, 64, 4096
    x = torch.zeros(T, d_in, dtype=torch.bfloat16, device="cuda")
    x[:, :3] = 1.0
    W = torch.zeros(d_in, d_out, dtype=torch.bfloat16, device="cuda")
    A = torch.zeros(d_in, 3, dtype=torch.float32)
    A[0, 0], A[1, 0], A[2, 0] = 1.0, 2.0 ** -9, 2.0 ** -20
    A[0, 1] = -1.0
    A[1, 2] = -(2.0 ** -9)
    A = A.to(torch.bfloat16).cuda()
    B = torch.ones(3, d_out, dtype=torch.bfloat16, device="cuda")
    pool = L.AdapterPool(1, d_in, d_out, 8, torch.bfloat16)
    pool.upload(0, A, B, 3, 3.0)                         # s = alpha / r = 1
    ids = torch.zeros(T, dtype=torch.int32, device="cuda")
    for mode in (L.LORA_MODE_AUTO, L.LORA_MODE_SGMV, L.LORA_MODE_BGMV):
        for flags in FLAGS:
            ws = L.Workspace(T, 1, 8, d_out)
            y = torch.empty(T, d_out, dtype=torch.bfloat16, device="cuda")
            L.lora_linear_forward(x, W, y, T, pool.pool, ids, mode, flags, ws.buf)
            torch.cuda.synchronize()
            assert (y.float() == 2.0 ** -20).all(), "mode %d flags %d" % (mode, flags)
