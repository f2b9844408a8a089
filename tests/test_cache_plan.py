"""CPU checks of the residency cache's policy (planning-only caches run the
same bookkeeping as GPU ones, with no device work) and of lora_pack_host
against an independent numpy construction of the slot layout."""
import numpy as np
import pytest
import torch

from rank_adapter_gemm_amd import lora as L


@pytest.fixture(scope="module", autouse=True)
def _lib():
    L.load()


def plan_cache(n_slots=3, n_adapters=10):
    c = L.AdapterCache(n_slots, [], n_adapters)
    for a in range(n_adapters):
        c.register(a, [], [], 8, 16.0)
    return c


def resident(c, n_adapters=10):
    return {a: c.slot_of(a) for a in range(n_adapters) if c.slot_of(a) >= 0}


def test_lru_order_and_empty_slots_first():
    c = plan_cache()
    s = c.map([0, 1, -1, 2, 1])
    assert s[2] == -1 and s[1] == s[4]
    assert sorted({s[0], s[1], s[3]}) == [0, 1, 2]                 # empty slots taken first
    assert c.stats() == dict(hits=0, misses=3, evictions=0, bytes=0)
    c.map([0, 1])                                                 # 2 is now least recently used
    s = c.map([3])
    assert c.slot_of(2) == -1 and s[0] == resident(c)[3]
    assert c.stats()["evictions"] == 1
    c.map([0])                                                    # LRU order now 1, 3, 0
    c.map([4, 0])                                                 # evicts 1
    assert set(resident(c)) == {0, 3, 4}
    st = c.stats()
    assert st["hits"] == 2 + 1 + 1 and st["misses"] == 3 + 1 + 1 and st["evictions"] == 2


def test_batch_never_evicts_its_own_adapters():
    c = plan_cache()
    c.map([0, 1, 2])
    c.map([5, 6, 7])                                              # all three replaced, none of the batch twice
    r = resident(c)
    assert set(r) == {5, 6, 7} and len(set(r.values())) == 3


def test_too_many_adapters_or_bad_ids_change_nothing():
    c = plan_cache()
    c.map([0, 1])
    before = (resident(c), c.stats())
    with pytest.raises(L.LoraError) as e:
        c.map([2, 3, 4, 5])
    assert e.value.status == L.LORA_ERR_UNSUPPORTED
    for bad in ([0, 10], [-2], [11]):
        with pytest.raises(L.LoraError) as e:
            c.map(bad)
        assert e.value.status == L.LORA_ERR_INVALID_ARGUMENT
    assert (resident(c), c.stats()) == before
    c2 = L.AdapterCache(2, [], 4)
    c2.register(0, [], [], 8, 1.0)
    with pytest.raises(L.LoraError):
        c2.map([1])                                               # not registered
    assert c2.map([]) == [] and c2.map([-1, -1]) == [-1, -1]


def test_reregister_drops_residency():
    c = plan_cache()
    c.map([0, 1])
    c.register(0, [], [], 8, 32.0)                                # a new version of adapter 0
    assert c.slot_of(0) == -1 and c.slot_of(1) >= 0
    c.map([0])
    assert c.stats()["misses"] == 3


def test_create_and_register_validation():
    with pytest.raises(L.LoraError):
        L.AdapterCache(0, [], 4)
    with pytest.raises(L.LoraError):
        L.AdapterCache(4, [], 0)
    c = L.AdapterCache(4, [], 4)
    with pytest.raises(L.LoraError):
        c.register(4, [], [], 8, 1.0)
    with pytest.raises(L.LoraError):
        c.register(0, [], [], 0, 1.0)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_pack_host_matches_slot_layout(dtype):
    rng = np.random.default_rng(0)
    d_in, d_out, R, r = 24, 40, 16, 11
    A = torch.as_tensor(rng.standard_normal((d_in, r + 3)), dtype=torch.float32).to(dtype)   # lda = r + 3
    B = torch.as_tensor(rng.standard_normal((r, d_out)), dtype=torch.float32).to(dtype)
    a_slot = torch.full((R * d_in,), 7.0, dtype=dtype)
    b_slot = torch.full((R * d_out,), 7.0, dtype=dtype)
    code = L.LORA_BF16 if dtype == torch.bfloat16 else L.LORA_F32
    L.lora_pack_host(d_in, d_out, R, code, A, B, r, a_slot, b_slot)
    # independent construction: A^T rows, then B octets [R/8][d_out][8]
    at = np.zeros((R, d_in))
    at[:r] = A.float().numpy()[:, :r].T
    bpad = np.zeros((R, d_out))
    bpad[:r] = B.float().numpy()
    oct_ = bpad.reshape(R // 8, 8, d_out).transpose(0, 2, 1)
    assert np.array_equal(a_slot.float().numpy().reshape(R, d_in), at)
    assert np.array_equal(b_slot.float().numpy().reshape(R // 8, d_out, 8), oct_)
    with pytest.raises(L.LoraError) as e:
        L.lora_pack_host(d_in, d_out, 8, code, A, B, r, a_slot, b_slot)
    assert e.value.status == L.LORA_ERR_RANK_EXCEEDS_MAX
