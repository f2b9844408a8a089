"""The forward without a caller workspace (lora_linear_forward_noalloc): its
workspace is the library's own device array.  Two calls in a row through the
C ABI, the second with a smaller batch, each checked against
lora_linear_forward with a caller workspace (and the fp64 oracle) to the
bf16 bar; the error output, and the size limit."""
import numpy as np
import pytest
import torch

from rank_adapter_gemm_amd import lora as L

from helpers import TOL, assert_parity
from test_gpu_packed import Batch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


def _compare(b, flags, err_expected):
    sl = b.slices[0]
    ref_y = b.run("padded", L.LORA_MODE_AUTO, flags) if err_expected == -1 else None
    y = torch.full((b.T, sl["d_out"]), 5.0, dtype=torch.bfloat16, device="cuda")
    err = torch.full((1,), 1234, dtype=torch.int32, device="cuda")
    L.lora_linear_forward_noalloc(b.x, sl["W"], y, b.T, sl["padded"].pool, b.ids_dev, L.LORA_MODE_AUTO, flags, err)
    torch.cuda.synchronize()
    assert int(err.cpu()[0]) == err_expected
    if ref_y is None:                     # a planted bad id: the caller-workspace forward, same ids
        ws = L.Workspace(b.T, b.n_slots, b.R, sl["d_out"])
        ref_y = torch.empty_like(y)
        L.lora_linear_forward(b.x, sl["W"], ref_y, b.T, sl["padded"].pool, b.ids_dev, L.LORA_MODE_AUTO, flags,
                              ws.buf)
        torch.cuda.synchronize()
        assert L.lora_get_device_error(ws.buf) == err_expected
    d = (y.float() - ref_y.float()).abs() / (1 + ref_y.float().abs())
    assert d.max().item() <= TOL[torch.bfloat16]
    return y


def test_noalloc_matches_workspace_forward_twice():
    ranks = [8, 16, 32, 64, 8, 24, 40, 64, 16, 56]
    big = Batch(200, [700, 400, 300, 9], 1024, 2048, ranks, 64, seed=21)
    assert big.T >= 1024
    y1 = _compare(big, 0, -1)
    assert_parity(y1, big.oracle(), torch.bfloat16, "noalloc, mixed batch")
    # second call, smaller batch (decode-sized: the shrink inside the split-K
    # GEMM), with a bad id planted in row 7
    small = Batch(160, [], 1024, 1024, [16, 8, 16, 16], 16, seed=22)
    small.ids[7] = 99
    small.ids_dev = torch.as_tensor(small.ids, device="cuda")
    y2 = _compare(small, 0, 7)
    ids_ok = small.ids.copy()
    ids_ok[7] = -1                        # the oracle computes a bad id as a base row
    small.ids = ids_ok
    assert_parity(y2, small.oracle(), torch.bfloat16, "noalloc, decode batch")


def test_noalloc_rejects_batches_beyond_its_scratch():
    pool = L.AdapterPool(4, 64, 64, 128, torch.bfloat16)
    t = torch.zeros(16, 64, dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros(16, dtype=torch.int32, device="cuda")
    # 16 K-split partials of v alone: 16 * 8192 * 128 * 4 bytes > 64 MiB
    assert L.lora_workspace_bytes(8192, 4, 128) > L.LORA_NOALLOC_SCRATCH_BYTES
    with pytest.raises(L.LoraError) as e:
        L.lora_linear_forward_noalloc(t, t, t, 8192, pool.pool, ids, L.LORA_MODE_AUTO, 0)
    assert e.value.status == L.LORA_ERR_WORKSPACE_TOO_SMALL
    assert L.lora_workspace_bytes(4096, 4, 128) <= L.LORA_NOALLOC_SCRATCH_BYTES
