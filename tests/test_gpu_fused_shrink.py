"""GPU parity of the decode-sized path where the shrink runs inside the
split-K base GEMM (batches of at most 256 rows in BGMV mode; 128 x 128
tiles, or one 256-row tile of 64-column tiles where the wider column tiles
are too few to cover the rows): every row against the fp64 oracle, for each supported max rank,
with ranks below the maximum, base rows, an empty slot and out-of-range ids
(which must be flagged and computed as base rows), plus bitwise determinism
and agreement with the unfused path (separate shrink kernel)."""
import numpy as np
import pytest
import torch

from rank_adapter_gemm_amd import lora as L

from helpers import TOL, assert_parity
from test_gpu_edges import Case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


# (T, d_in, d_out, max_rank, ranks): each shape gives a split-K plan whose
# column tiles, 64 / max_rank rows each, cover a row tile.
CASES = [
    (256, 1024, 4096, 16, [16, 16, 7, 16, 0, 12]),   # 128 x 128, two row tiles
    (200, 2048, 2048, 8, [8, 3, 0, 5]),              # 128 x 128, ragged second row tile
    (100, 1024, 4096, 32, [32, 17, 8, 0, 32]),       # 256 x 64 (32 wide tiles x 2 rows < 100)
    (37, 2048, 4096, 64, [64, 8, 33, 0]),            # 256 x 64
    (1, 512, 1024, 16, [16, 4]),                     # 128 x 128, one row
]


@pytest.mark.parametrize("T,d_in,d_out,R,ranks", CASES)
def test_fused_shrink_every_row(T, d_in, d_out, R, ranks):
    rng = np.random.default_rng(T)
    n = len(ranks)
    ids = rng.integers(-1, n, size=T).astype(np.int32)
    if T > 10:
        ids[[3, 7]] = [-3, n]                          # out of range: flagged, base rows
    empty = [s for s, r in enumerate(ranks) if r == 0]
    if empty and T > 12:
        ids[12] = empty[0]                             # names an empty slot: flagged too
    bad_rows = [t for t, a in enumerate(ids) if a != -1 and not (0 <= a < n and ranks[a] > 0)]
    c = Case(T=T, d_in=d_in, d_out=d_out, ranks=ranks, max_rank=R, dtype=torch.bfloat16,
             seed=T, ids=ids)
    # the oracle treats every unusable id as a base row
    ref = c.oracle()
    y, ws = c.run(L.LORA_MODE_BGMV, 0)
    assert_parity(y, ref, torch.bfloat16, "fused shrink T=%d R=%d" % (T, R))
    assert L.lora_get_device_error(ws.buf) == (min(bad_rows) if bad_rows else -1)
    y2, ws2 = c.run(L.LORA_MODE_BGMV, 0)
    assert torch.equal(y, y2), "not deterministic"
    ys, _ = c.run(L.LORA_MODE_BGMV, L.LORA_FLAG_SEPARATE_EXPAND)
    assert_parity(ys, ref, torch.bfloat16, "unfused T=%d R=%d" % (T, R))
    d = (y.float() - ys.float()).abs() / (1 + ys.float().abs())
    assert d.max().item() <= 2.0 ** -6


def test_fused_shrink_delta_is_applied():
    """All values N(0, 0.02) (the decode workload's scale): the low-rank term
    is far below the bf16 tolerance, so compare against the oracle with and
    without adapters to show the delta is really there."""
    T, d_in, d_out, R = 256, 1024, 4096, 16
    c = Case(T=T, d_in=d_in, d_out=d_out, ranks=[16, 16, 16], max_rank=R, dtype=torch.bfloat16,
             seed=5, base_frac=0.0)
    ref = c.oracle()
    base = c.oracle(ids=np.full(T, -1, np.int32))
    y, _ = c.run(L.LORA_MODE_BGMV, 0)
    delta_ref = ref - base
    delta_gpu = y.float().cpu().double().numpy() - base
    err = np.abs(delta_gpu - delta_ref).max()
    # bf16 rounding of y (2^-9 relative to |y|) dominates; the delta itself is O(1)
    bound = 2.0 ** -8 * (1 + np.abs(ref).max())
    assert np.abs(delta_ref).max() > 0.1
    assert err <= bound, "%.3e > %.3e" % (err, bound)
