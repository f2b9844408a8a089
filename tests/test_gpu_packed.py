"""GPU checks of packed adapter pools: each slot holds its own rank rows
(capacity a multiple of 8), back to back, with no padding to max_rank (the
heterogeneous-rank layout of "Multi-LoRA Serving: Architecture for Thousands
of Adapters", section "Heterogeneous batching and rank").

Every kernel reads only a slot's first r rank rows, so a packed pool and a
padded pool holding the same adapters give bitwise the same outputs, in
every mode and expand path; both agree with the fp64 oracle."""
import numpy as np
import pytest
import torch

from oracle import BF16, lora_scale, oracle_rows
from rank_adapter_gemm_amd import lora as L

from helpers import assert_parity, to_oracle

pytestmark = pytest.mark.gpu

MODES = [L.LORA_MODE_BGMV, L.LORA_MODE_SGMV, L.LORA_MODE_AUTO]
FLAGS = [0, L.LORA_FLAG_SEPARATE_EXPAND]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


class Batch:
    """A mixed batch (decode rows and prefill chunks, shuffled) over slots of
    heterogeneous ranks, with one padded and one packed pool of the same
    adapters (capacity = rank rounded up to 8)."""

    def __init__(self, T_dec, chunks, d_in, d_out, ranks, R, seed, n_slices=1):
        g = torch.Generator(device="cuda")
        g.manual_seed(seed)
        rng = np.random.default_rng(seed)
        n = len(ranks)
        self.ranks, self.R, self.n_slots, self.d_in = list(ranks), R, n, d_in
        lengths = [1] * T_dec + list(chunks)
        owners = rng.integers(-1, n, size=len(lengths))
        order = rng.permutation(len(lengths))
        self.ids = np.repeat(owners[order], np.asarray(lengths)[order]).astype(np.int32)
        self.T = int(self.ids.size)
        self.ids_dev = torch.as_tensor(self.ids, device="cuda")
        self.x = torch.randn(self.T, d_in, generator=g, device="cuda").to(torch.bfloat16)
        self.cap = [max(8, (r + 7) // 8 * 8) for r in ranks]
        self.slices = []
        for _ in range(n_slices):
            W = (torch.randn(d_in, d_out, generator=g, device="cuda") * 0.03).to(torch.bfloat16)
            A = [(torch.randn(d_in, r, generator=g, device="cuda") * 0.03).to(torch.bfloat16) for r in ranks]
            B = [(torch.randn(r, d_out, generator=g, device="cuda") * 0.05).to(torch.bfloat16) for r in ranks]
            pads = L.AdapterPool(n, d_in, d_out, R, torch.bfloat16)
            pack = L.AdapterPool(n, d_in, d_out, R, torch.bfloat16, capacity=self.cap)
            for s, r in enumerate(ranks):
                pads.upload(s, A[s], B[s], r, 2.0 * r)
                pack.upload(s, A[s], B[s], r, 2.0 * r)
            self.slices.append(dict(W=W, A=A, B=B, padded=pads, packed=pack, d_out=d_out))

    def oracle(self, k=0):
        sl = self.slices[k]
        return oracle_rows(BF16, to_oracle(self.x), to_oracle(sl["W"]), self.ids, [to_oracle(a) for a in sl["A"]],
                           [to_oracle(b) for b in sl["B"]], self.ranks,
                           [lora_scale(2.0 * r, r) for r in self.ranks])["y"]

    def run(self, which, mode, flags, k=0):
        sl = self.slices[k]
        ws = L.Workspace(self.T, self.n_slots, self.R, sl["d_out"])
        y = torch.full((self.T, sl["d_out"]), 3.0, dtype=torch.bfloat16, device="cuda")
        L.lora_linear_forward(self.x, sl["W"], y, self.T, sl[which].pool, self.ids_dev, mode, flags, ws.buf)
        torch.cuda.synchronize()
        assert L.lora_get_device_error(ws.buf) == -1
        return y


def test_packed_pool_layout():
    """Slot s's A^T rank rows start at rank row row0[s], its B octets at
    octet row row0[s] / 8; rows past the slot's rank are zero; an upload
    touches only its own slot; rank and scale as for a padded pool."""
    d_in, d_out, cap = 48, 40, [8, 24, 16]
    pool = L.AdapterPool(3, d_in, d_out, 24, torch.bfloat16, capacity=cap)
    assert pool.row0_host.tolist() == [0, 8, 32, 48]
    assert pool.row0.cpu().tolist() == [0, 8, 32, 48]
    assert pool.a.numel() == 48 * d_in * 2 and pool.b.numel() == 48 * d_out * 2
    g = torch.Generator(device="cuda")
    g.manual_seed(1)
    A = (torch.randn(d_in, 19, generator=g, device="cuda")).to(torch.bfloat16)
    B = (torch.randn(19, d_out, generator=g, device="cuda")).to(torch.bfloat16)
    pool.upload(1, A, B, 19, 38.0)
    torch.cuda.synchronize()
    a = pool.a.view(torch.bfloat16).view(48, d_in)
    b = pool.b.view(torch.bfloat16).view(6, d_out, 8)
    assert torch.equal(a[8:27], A.t())
    assert (a[27:32].float() == 0).all() and (a[:8].float() == 0).all() and (a[32:].float() == 0).all()
    Bp = torch.zeros(24, d_out, dtype=torch.bfloat16, device="cuda")
    Bp[:19] = B
    assert torch.equal(b[1:4], Bp.view(3, 8, d_out).permute(0, 2, 1))
    assert (b[0].float() == 0).all() and (b[4:].float() == 0).all()
    assert pool.rank.cpu().tolist() == [0, 19, 0]
    assert pool.scale.cpu().tolist()[1] == 2.0
    with pytest.raises(L.LoraError) as e:
        pool.upload(0, A, B, 9, 18.0, lda=19)
    assert e.value.status == L.LORA_ERR_RANK_EXCEEDS_MAX
    pool.upload(0, A, B, 8, 16.0, lda=19)
    pool.clear(1)
    torch.cuda.synchronize()
    assert (a[8:32].float() == 0).all() and torch.equal(a[:8], A[:, :8].t())
    assert pool.rank.cpu().tolist() == [8, 0, 0]


@pytest.mark.parametrize("T_dec,chunks,d_in,d_out,R", [
    (96, [300, 200], 1024, 1536, 64),     # mixed batch: SGMV in AUTO
    (160, [], 2048, 1024, 64),            # decode-sized BGMV batch at max rank 64
])
def test_packed_equals_padded(T_dec, chunks, d_in, d_out, R):
    ranks = [8, 16, 32, 64, 8, 24, 40, 64, 16, 56, 8, 32]
    b = Batch(T_dec, chunks, d_in, d_out, ranks, R, seed=T_dec)
    ref = b.oracle()
    for mode in MODES:
        for flags in FLAGS:
            y0 = b.run("padded", mode, flags)
            y1 = b.run("packed", mode, flags)
            assert torch.equal(y0, y1), "mode %d flags %d" % (mode, flags)
            assert_parity(y1, ref, torch.bfloat16, "packed mode=%d flags=%d" % (mode, flags))


def test_packed_decode_fused_shrink():
    """Decode-sized BGMV batch whose shrink runs inside the split-K GEMM
    (max rank 16, ranks 8 and 16): the GEMM's DMA takes only each slot's own
    rank rows, from its packed position."""
    b = Batch(256, [], 2048, 4096, [8, 16, 16, 8, 16, 8, 8], 16, seed=3)
    ref = b.oracle()
    for flags in FLAGS:
        y0 = b.run("padded", L.LORA_MODE_BGMV, flags)
        y1 = b.run("packed", L.LORA_MODE_BGMV, flags)
        assert torch.equal(y0, y1)
        assert_parity(y1, ref, torch.bfloat16, "packed decode flags=%d" % flags)


def test_packed_sliced_and_fp8():
    """Two packed slices sharing x through lora_linear_forward_sliced agree
    bitwise with the padded slices; the FP8-base forward reads packed slots
    too."""
    ranks = [8, 32, 16, 64, 24, 8]
    b = Batch(64, [700, 300], 1024, 2048, ranks, 64, seed=5, n_slices=2)
    for which in ("padded", "packed"):
        ws = L.Workspace(b.T, b.n_slots, 64, 4096, n_slices=2)
        ys = [torch.empty(b.T, 2048, dtype=torch.bfloat16, device="cuda") for _ in range(2)]
        L.lora_linear_forward_sliced(b.x, [s["W"] for s in b.slices], ys, b.T,
                                     [s[which].pool for s in b.slices], b.ids_dev, L.LORA_MODE_AUTO, 0, ws.buf)
        torch.cuda.synchronize()
        if which == "padded":
            ys_pad = ys
        else:
            for k in range(2):
                assert torch.equal(ys[k], ys_pad[k])
                assert_parity(ys[k], b.oracle(k), torch.bfloat16, "packed slice %d" % k)
    sl = b.slices[0]
    w8 = L.Fp8Weight(sl["W"])
    outs = []
    for which in ("padded", "packed"):
        ws = L.Workspace(b.T, b.n_slots, 64, 2048, fp8_d_in=1024)
        y = torch.empty(b.T, 2048, dtype=torch.bfloat16, device="cuda")
        L.lora_linear_forward_fp8(b.x, w8.codes, w8.scale, y, b.T, sl[which].pool, b.ids_dev, L.LORA_MODE_AUTO,
                                  0, ws.buf)
        torch.cuda.synchronize()
        outs.append(y)
    assert torch.equal(outs[0], outs[1])
