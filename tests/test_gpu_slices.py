"""GPU parity of the multi-slice entry points (projections sharing x: one
shrink for all slices).  The sliced shrink must give bitwise the v that one
lora_shrink per pool gives.  Each slice of lora_linear_forward_sliced must
match the fp64 oracle and agree with lora_linear_forward on its own pool:
bitwise with the separate expand (one GEMM per slice), else within one bf16
step (the slices share one GEMM launch, planned over all their tiles, so a
tile may be computed whole here and split over K there).  Covered: BGMV
and SGMV, fused and separate expand, the decode-sized fused path next to
grouped slices, repeat calls (deterministic) and reused segments."""
import numpy as np
import pytest
import torch

from oracle import BF16, F32, lora_scale, oracle_rows
from rank_adapter_gemm_amd import lora as L

from helpers import assert_parity, to_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


class Sliced:
    """n_slices pools over one x and one id vector; slot ranks differ by slice."""

    def __init__(self, T, d_in, d_outs, ranks, R, dtype=torch.bfloat16, seed=0):
        g = torch.Generator(device="cuda")
        g.manual_seed(seed)
        rng = np.random.default_rng(seed)
        self.T, self.d_in, self.d_outs, self.R, self.dtype = T, d_in, d_outs, R, dtype
        self.ranks = ranks                                   # [slice][slot]
        n_slots = len(ranks[0])
        self.n_slots = n_slots
        self.x = torch.randn(T, d_in, generator=g, device="cuda").to(dtype)
        ids = rng.integers(-1, n_slots, size=T).astype(np.int32)
        self.ids = ids
        self.ids_dev = torch.as_tensor(ids, device="cuda")
        self.W, self.A, self.B, self.pools, self.alphas = [], [], [], [], []
        for s, d_out in enumerate(d_outs):
            self.W.append((torch.randn(d_in, d_out, generator=g, device="cuda") / d_in ** 0.5).to(dtype))
            A = [(torch.randn(d_in, max(r, 1), generator=g, device="cuda") / d_in ** 0.5).to(dtype)
                 for r in ranks[s]]
            B = [(torch.randn(max(r, 1), d_out, generator=g, device="cuda") / max(r, 1) ** 0.5).to(dtype)
                 for r in ranks[s]]
            al = [2.0 * r + s for r in ranks[s]]
            pool = L.AdapterPool(n_slots, d_in, d_out, R, dtype)
            for slot, r in enumerate(ranks[s]):
                if r > 0:
                    pool.upload(slot, A[slot], B[slot], r, al[slot])
            self.A.append(A)
            self.B.append(B)
            self.alphas.append(al)
            self.pools.append(pool)

    def oracle(self, s):
        code = F32 if self.dtype == torch.float32 else BF16
        rk = self.ranks[s]
        A = [to_oracle(a) if r > 0 else None for a, r in zip(self.A[s], rk)]
        B = [to_oracle(b) if r > 0 else None for b, r in zip(self.B[s], rk)]
        sc = [lora_scale(a, r) for a, r in zip(self.alphas[s], rk)]
        return oracle_rows(code, to_oracle(self.x), to_oracle(self.W[s]), self.ids, A, B, rk, sc)["y"]


@pytest.mark.parametrize("T", [300, 1500])
@pytest.mark.parametrize("mode", [L.LORA_MODE_BGMV, L.LORA_MODE_SGMV])
def test_sliced_shrink_is_bitwise_per_pool(T, mode):
    c = Sliced(T, 512, [512, 128, 128], [[16, 8, 16, 0, 12], [16, 16, 4, 8, 12], [0, 16, 16, 8, 3]],
               R=16, seed=T)
    n = len(c.pools)
    ws = L.Workspace(T, c.n_slots, c.R, 0, n_slices=n)
    if mode == L.LORA_MODE_SGMV:
        L.lora_build_segments(c.ids_dev, T, c.n_slots, c.R, ws.buf)
    v = torch.full((T, n * c.R), float("nan"), dtype=torch.float32, device="cuda")
    L.lora_shrink_sliced(c.x, T, [p.pool for p in c.pools], c.ids_dev, mode, v, ws.buf)
    for s in range(n):
        ws1 = L.Workspace(T, c.n_slots, c.R, 0)
        if mode == L.LORA_MODE_SGMV:
            L.lora_build_segments(c.ids_dev, T, c.n_slots, c.R, ws1.buf)
        v1 = torch.full((T, c.R), float("nan"), dtype=torch.float32, device="cuda")
        L.lora_shrink(c.x, T, c.pools[s].pool, c.ids_dev, mode, v1, ws1.buf)
        torch.cuda.synchronize()
        assert torch.equal(v[:, s * c.R:(s + 1) * c.R], v1), "slice %d" % s


def assert_within_one_step(a, b, what):
    """Two bf16 roundings of nearly the same fp32 value: each element equal
    or one rounding step apart (2^-7 relative), plus an absolute allowance
    for what differs before the rounding.  A tile computed whole adds the
    low-rank term through the matrix cores with s*v split into two bf16
    parts (about 16 significant bits, an error near 2^-17 of |s v_j B_jn|
    summed over the ranks); a tile split over K sums it in fp32, and sums
    the base product in another order.  2^-14 of the largest output covers
    both (the observed gap is near 2^-19 of it) and stays far below what a
    wrong or dropped term would give."""
    a, b = a.float(), b.float()
    d = (a - b).abs()
    lim = 2.0 ** -7 * b.abs() + 2.0 ** -14 * b.abs().max()
    bad = d > lim
    assert not bad.any(), "%s: %d elements beyond one bf16 step, max diff %g" % (what, int(bad.sum()),
                                                                                   float(d.max()))


# (T, d_in, widths, bitwise): slices that alone fill the chip with whole
# 256 x 256 tiles (2048 rows x 7168 columns, K too short to split) run one
# GEMM each, bitwise as the per-pool call; the others share a grouped GEMM.
@pytest.mark.parametrize("T,d_in,d_outs,bitwise", [
    (300, 512, [512, 128, 128], False), (1500, 512, [256, 256], False),
    (256, 1024, [4096, 1024, 1024], False), (2240, 1024, [4096, 1024, 1024], False),
    (700, 512, [640, 200, 1000, 72], False), (2048, 512, [7168, 7168], True)])
def test_sliced_forward_matches_per_pool(T, d_in, d_outs, bitwise):
    n = len(d_outs)
    ranks = [[16, 8, 16, 0, 12], [16, 16, 4, 8, 12], [0, 16, 16, 8, 3], [8, 0, 16, 16, 1]][:n]
    c = Sliced(T, d_in, d_outs, ranks, R=16, seed=T + n)
    refs = [c.oracle(s) for s in range(n)]
    for mode in (L.LORA_MODE_AUTO, L.LORA_MODE_BGMV, L.LORA_MODE_SGMV):
        for flags in (0, L.LORA_FLAG_SEPARATE_EXPAND):
            ws = L.Workspace(T, c.n_slots, c.R, sum(d_outs), n_slices=n)
            ys = [torch.full((T, d), 7.0, dtype=c.dtype, device="cuda") for d in d_outs]
            L.lora_linear_forward_sliced(c.x, c.W, ys, T, [p.pool for p in c.pools], c.ids_dev, mode, flags,
                                         ws.buf)
            again = [torch.full((T, d), 7.0, dtype=c.dtype, device="cuda") for d in d_outs]
            L.lora_linear_forward_sliced(c.x, c.W, again, T, [p.pool for p in c.pools], c.ids_dev, mode, flags,
                                         ws.buf)
            for s in range(n):
                ws1 = L.Workspace(T, c.n_slots, c.R, d_outs[s])
                y1 = torch.full((T, d_outs[s]), 7.0, dtype=c.dtype, device="cuda")
                L.lora_linear_forward(c.x, c.W[s], y1, T, c.pools[s].pool, c.ids_dev, mode, flags, ws1.buf)
                torch.cuda.synchronize()
                what = "T=%d slice %d mode %d flags %d" % (T, s, mode, flags)
                assert torch.equal(again[s], ys[s]), what + " (repeat call)"
                if bitwise or flags & L.LORA_FLAG_SEPARATE_EXPAND:
                    assert torch.equal(ys[s], y1), what
                else:
                    assert_within_one_step(ys[s], y1, what)
                assert_parity(ys[s], refs[s], c.dtype, what)
            # slots empty in slice 0 or 2 are flagged, as each per-pool call would
            bad = [t for t, a in enumerate(c.ids) if a >= 0 and any(rk[a] == 0 for rk in ranks)]
            assert L.lora_get_device_error(ws.buf) == (min(bad) if bad else -1)


def test_sliced_forward_reuses_segments():
    T, n = 1500, 2
    c = Sliced(T, 512, [256, 256], [[16, 8, 16, 4, 12], [16, 16, 4, 8, 12]], R=16, seed=7)
    ws = L.Workspace(T, c.n_slots, c.R, 256, n_slices=n)
    L.lora_build_segments(c.ids_dev, T, c.n_slots, c.R, ws.buf)
    ys = [torch.empty(T, 256, dtype=c.dtype, device="cuda") for _ in range(n)]
    L.lora_linear_forward_sliced(c.x, c.W, ys, T, [p.pool for p in c.pools], c.ids_dev, L.LORA_MODE_SGMV,
                                 L.LORA_FLAG_SEGMENTS_READY, ws.buf)
    torch.cuda.synchronize()
    for s in range(n):
        assert_parity(ys[s], c.oracle(s), c.dtype, "slice %d" % s)
    assert L.lora_get_device_error(ws.buf) == -1
