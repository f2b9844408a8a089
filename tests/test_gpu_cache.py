"""GPU checks of the adapter residency cache: a host tier of 10 adapters
(packed in the slot layout) served through 4 HBM slots of two pools kept in
step.  Batches are mapped, computed and committed without any host
synchronisation between them, so evictions overlap earlier batches' kernels;
every batch's outputs are then checked against the fp64 oracle on the
adapters' original weights, and the counters against the batch contents.
The host tier is page-locked (copied by the gather kernel reading mapped
host memory), or every other adapter is in pageable memory (copied by the
runtime), so one map mixes both kinds of copy."""
import numpy as np
import pytest
import torch

from oracle import BF16, lora_scale, oracle_rows
from rank_adapter_gemm_amd import lora as L

from helpers import assert_parity, to_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


@pytest.mark.parametrize("host", ["pinned", "mixed"])
@pytest.mark.parametrize("mode", [L.LORA_MODE_BGMV, L.LORA_MODE_SGMV])
def test_cache_serves_batches_through_few_slots(mode, host):
    torch.manual_seed(0)
    rng = np.random.default_rng(1)
    n_slots, n_adapters, R, d_in, d_outs, T = 4, 10, 16, 512, [256, 384], 200
    dt = torch.bfloat16
    ranks = [int(r) for r in rng.choice([4, 8, 12, 16], size=n_adapters)]
    alphas = [2.0 * r + a for a, r in enumerate(ranks)]
    A = [[(torch.randn(d_in, r) / d_in ** 0.5).to(dt) for r in ranks] for _ in d_outs]   # [pool][adapter]
    B = [[(torch.randn(r, d) / r ** 0.5).to(dt) for r in ranks] for d in d_outs]
    W = [(torch.randn(d_in, d) / d_in ** 0.5).to(dt).cuda() for d in d_outs]
    pools = [L.AdapterPool(n_slots, d_in, d, R, dt) for d in d_outs]
    cache = L.AdapterCache(n_slots, [p.pool for p in pools], n_adapters)
    for a in range(n_adapters):
        ha, hb = [], []
        for p, d in enumerate(d_outs):
            pin = host == "pinned" or a % 2 == 0
            sa = torch.empty(R * d_in, dtype=dt)
            sb = torch.empty(R * d, dtype=dt)
            if pin:
                sa, sb = sa.pin_memory(), sb.pin_memory()
            L.lora_pack_host(d_in, d, R, L.LORA_BF16, A[p][a], B[p][a], ranks[a], sa, sb)
            ha.append(sa)
            hb.append(sb)
        cache.register(a, ha, hb, ranks[a], alphas[a])

    copy = torch.cuda.Stream()                 # default priority
    compute = torch.cuda.current_stream()
    ws = L.Workspace(T, n_slots, R, max(d_outs))
    batches = [[0, 1, 2], [2, 3], [4, 5, 6, 7], [0, 1], [8, 9, 2], [3, 4, 5, 6], [0, 9], [7]]
    runs = []
    n_distinct = 0
    for adapters in batches:
        row_ad = rng.choice(adapters + [-1], size=T).astype(np.int32)
        slots = cache.map(row_ad.tolist(), compute, copy)
        ids = torch.as_tensor(np.asarray(slots, np.int32)).cuda()
        x = torch.randn(T, d_in, device="cuda").to(dt)
        ys = [torch.empty(T, d, dtype=dt, device="cuda") for d in d_outs]
        for p in range(len(d_outs)):
            L.lora_linear_forward(x, W[p], ys[p], T, pools[p].pool, ids, mode, 0, ws.buf)
        cache.commit(compute)
        runs.append((row_ad, x, ys))
        n_distinct += len(set(int(a) for a in row_ad if a >= 0))
    torch.cuda.synchronize()
    assert L.lora_get_device_error(ws.buf) == -1
    for row_ad, x, ys in runs:
        for p in range(len(d_outs)):
            ref = oracle_rows(BF16, to_oracle(x), to_oracle(W[p]), row_ad, [to_oracle(a) for a in A[p]],
                              [to_oracle(b) for b in B[p]], ranks,
                              [lora_scale(al, r) for al, r in zip(alphas, ranks)])["y"]
            assert_parity(ys[p], ref, dt, "pool %d" % p)
    st = cache.stats()
    assert st["hits"] + st["misses"] == n_distinct
    assert st["bytes"] == st["misses"] * sum(R * (d_in + d) * 2 for d in d_outs)
    assert st["misses"] >= n_adapters and st["evictions"] == st["misses"] - n_slots
    cache.close()
