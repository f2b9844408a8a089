"""CPU checks of the C-ABI library: it loads, exports every function that
include/lora.h declares, and its host-side validation and size arithmetic
behave as documented.  No GPU work is launched here (every call below
returns before anything is enqueued)."""
import ctypes
import os
import re

import pytest

from rank_adapter_gemm_amd import lora as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "lora.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lora_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return L.load()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert len(names) >= 15
    assert sorted(L.EXPORTED) == names
    for n in names:
        assert hasattr(lib, n), n


def test_header_constants_match_the_binding():
    """The integer #defines of include/lora.h and the binding's copies agree."""
    src = open(os.path.join(ROOT, "include", "lora.h")).read()
    defs = dict(re.findall(r"#define\s+(LORA_[A-Z0-9_]+)\s+(0x[0-9a-fA-F]+|\d+)\b", src))
    assert int(defs["LORA_AUTO_SGMV_MIN_ROWS"], 0) == L.LORA_AUTO_SGMV_MIN_ROWS
    assert int(defs["LORA_FLAG_SEGMENTS_READY"], 0) == L.LORA_FLAG_SEGMENTS_READY
    assert int(defs["LORA_FLAG_SEPARATE_EXPAND"], 0) == L.LORA_FLAG_SEPARATE_EXPAND
    m = re.search(r"#define\s+LORA_NOALLOC_SCRATCH_BYTES\s+\(\(size_t\)(\d+) << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == L.LORA_NOALLOC_SCRATCH_BYTES


def test_version_and_status_strings(lib):
    assert "gfx950" in L.lora_version()
    for code in range(7):
        assert L.status_string(code) and L.status_string(code) != "unknown status"
    assert L.status_string(99) == "unknown status"


def test_pool_bytes():
    a, b = L.lora_pool_bytes(128, 4096, 4096, 16, L.LORA_BF16)
    assert a == 128 * 16 * 4096 * 2 and b == 128 * 16 * 4096 * 2
    a, b = L.lora_pool_bytes(4, 256, 256, 8, L.LORA_F32)
    assert a == b == 4 * 8 * 256 * 4
    for bad in [(0, 64, 64, 8), (4, 60, 64, 8), (4, 64, 60, 8), (4, 64, 64, 12), (4, 64, 64, 136),
                (4, 64, 64, 0)]:
        with pytest.raises(L.LoraError) as e:
            L.lora_pool_bytes(*bad, L.LORA_BF16)
        assert e.value.status == L.LORA_ERR_INVALID_ARGUMENT
    with pytest.raises(L.LoraError) as e:
        L.lora_pool_bytes(16001, 64, 64, 8, L.LORA_BF16)
    assert e.value.status == L.LORA_ERR_UNSUPPORTED
    with pytest.raises(L.LoraError):
        L.lora_pool_bytes(4, 64, 64, 8, 7)


def test_packed_pool_bytes_and_validation(lib):
    """A packed pool stores each slot's own rank rows: bytes are sum(capacity)
    rows of d_in (A) and of d_out (B) instead of n_slots * max_rank; the
    capacities must be multiples of 8 in [8, 128]; an upload above a slot's
    capacity is LORA_ERR_RANK_EXCEEDS_MAX before anything is enqueued."""
    import numpy as np
    cap = [8, 16, 32, 64, 8]
    a, b = L.lora_pool_bytes_packed(5, 8192, 28672, cap, L.LORA_BF16)
    assert a == sum(cap) * 8192 * 2 and b == sum(cap) * 28672 * 2
    pa, pb = L.lora_pool_bytes(5, 8192, 28672, 64, L.LORA_BF16)
    assert a * 320 == pa * 128 and b * 320 == pb * 128        # 128 of 320 padded rows
    for bad in ([8, 12], [8, 0], [8, 136], [4, 8]):
        with pytest.raises(L.LoraError) as e:
            L.lora_pool_bytes_packed(len(bad), 64, 64, bad, L.LORA_BF16)
        assert e.value.status == L.LORA_ERR_INVALID_ARGUMENT
    fake = 1 << 40
    row0 = np.array([0, 8, 24, 56], dtype=np.int32)            # capacities 8, 16, 32
    p = L.lora_pool_t(3, 64, 64, 32, L.LORA_BF16, fake, fake, fake, fake, fake, row0.ctypes.data)
    up = lib.lora_pool_upload
    assert up(ctypes.byref(p), 0, fake, 9, fake, 64, 9, 1.0, None) == L.LORA_ERR_RANK_EXCEEDS_MAX
    assert up(ctypes.byref(p), 1, fake, 17, fake, 64, 17, 1.0, None) == L.LORA_ERR_RANK_EXCEEDS_MAX
    assert up(ctypes.byref(p), 2, fake, 33, fake, 64, 33, 1.0, None) == L.LORA_ERR_RANK_EXCEEDS_MAX
    assert up(ctypes.byref(p), 3, fake, 8, fake, 64, 8, 1.0, None) == L.LORA_ERR_SLOT_OUT_OF_RANGE
    # a descriptor with only one of row0 / row0_host is not a valid pool
    half = L.lora_pool_t(3, 64, 64, 32, L.LORA_BF16, fake, fake, fake, fake, fake, None)
    assert up(ctypes.byref(half), 0, fake, 8, fake, 64, 8, 1.0, None) == L.LORA_ERR_INVALID_ARGUMENT
    # creation checks its capacities (and max_rank against them) before any GPU work
    cr = lib.lora_pool_create_packed
    out = L.lora_pool_t()
    r0 = np.zeros(4, dtype=np.int32)
    for caps, R in (([8, 16, 44], 64), ([8, 16, 64], 32), ([8, 16, 0], 32)):
        c = np.asarray(caps, dtype=np.int32)
        assert cr(ctypes.byref(out), 3, 64, 64, R, L.LORA_BF16, c.ctypes.data, r0.ctypes.data, fake, fake, fake,
                  fake, fake, None) == L.LORA_ERR_INVALID_ARGUMENT
    # packed pools cannot back a residency cache
    h = ctypes.c_void_p()
    assert lib.lora_cache_create(ctypes.byref(h), 3, ctypes.byref(p), 1, 8) == L.LORA_ERR_UNSUPPORTED


def test_workspace_bytes():
    assert L.lora_workspace_bytes(-1, 4, 8) == 0
    assert L.lora_workspace_bytes(10, 0, 8) == 0
    assert L.lora_workspace_bytes(10, 4, 7) == 0
    assert L.lora_workspace_bytes(10, 4, 8, 12) == 0
    n0 = L.lora_workspace_bytes(0, 4, 8)
    n1 = L.lora_workspace_bytes(1000, 4, 8)
    n2 = L.lora_workspace_bytes(100000, 4, 8)
    assert 0 < n0 < n1 < n2
    # holds at least v [T, max_rank] fp32, perm [T] and the k-split partials
    assert n2 >= 100000 * (8 * 4 + 4 + 16 * 8 * 4)
    assert n2 % 256 == 0
    # with d_out: room for 16 fp32 partial copies of a small batch's output,
    # and never more than 128 MiB of partial tiles
    assert L.lora_workspace_bytes(256, 4, 8, 4096) >= L.lora_workspace_bytes(256, 4, 8) + 16 * 256 * 4096 * 4
    assert L.lora_workspace_bytes(100000, 4, 8, 4096) == n2 + (128 << 20)
    assert L.lora_workspace_bytes(2240, 1000, 16, 14336) <= L.lora_workspace_bytes(2240, 1000, 16) + (128 << 20)


def test_validation_returns_before_launch(lib):
    pool = L.lora_pool_t()
    # a null pool descriptor / zeroed descriptor is rejected
    assert lib.lora_pool_upload(None, 0, None, 1, None, 1, 1, 1.0, None) == L.LORA_ERR_INVALID_ARGUMENT
    assert lib.lora_pool_upload(ctypes.byref(pool), 0, None, 1, None, 1, 1, 1.0, None) == L.LORA_ERR_INVALID_ARGUMENT
    assert lib.lora_pool_clear(ctypes.byref(pool), 0, None) == L.LORA_ERR_INVALID_ARGUMENT
    # fake, aligned, never-dereferenced device addresses: validation only
    fake = 1 << 40
    ok = L.lora_pool_t(4, 64, 64, 8, L.LORA_BF16, fake, fake, fake, fake)
    assert lib.lora_pool_upload(ctypes.byref(ok), 4, fake, 8, fake, 64, 8, 1.0, None) == L.LORA_ERR_SLOT_OUT_OF_RANGE
    assert lib.lora_pool_upload(ctypes.byref(ok), -1, fake, 8, fake, 64, 8, 1.0, None) == L.LORA_ERR_SLOT_OUT_OF_RANGE
    assert lib.lora_pool_upload(ctypes.byref(ok), 0, fake, 9, fake, 64, 9, 1.0, None) == L.LORA_ERR_RANK_EXCEEDS_MAX
    assert lib.lora_pool_upload(ctypes.byref(ok), 0, fake, 2, fake, 64, 0, 1.0, None) == L.LORA_ERR_INVALID_ARGUMENT
    assert lib.lora_pool_upload(ctypes.byref(ok), 0, fake, 2, fake, 63, 2, 1.0, None) == L.LORA_ERR_INVALID_ARGUMENT
    assert lib.lora_pool_upload(ctypes.byref(ok), 0, fake, 1, fake, 64, 2, 1.0, None) == L.LORA_ERR_INVALID_ARGUMENT
    assert lib.lora_pool_clear(ctypes.byref(ok), 4, None) == L.LORA_ERR_SLOT_OUT_OF_RANGE
    ws_need = L.lora_workspace_bytes(16, 4, 8)
    f = lib.lora_linear_forward
    assert f(fake, fake, fake, 16, ctypes.byref(ok), fake, 0, 0, fake, ws_need - 1, None) == L.LORA_ERR_WORKSPACE_TOO_SMALL
    assert f(fake, fake, fake, -1, ctypes.byref(ok), fake, 0, 0, fake, ws_need, None) == L.LORA_ERR_INVALID_ARGUMENT
    assert f(fake + 2, fake, fake, 16, ctypes.byref(ok), fake, 0, 0, fake, ws_need, None) == L.LORA_ERR_INVALID_ARGUMENT
    assert f(fake, fake, fake, 16, ctypes.byref(ok), None, 0, 0, fake, ws_need, None) == L.LORA_ERR_INVALID_ARGUMENT
    assert f(fake, fake, fake, 16, ctypes.byref(ok), fake, 3, 0, fake, ws_need, None) == L.LORA_ERR_INVALID_ARGUMENT
    assert f(fake, fake, fake, 16, ctypes.byref(ok), fake, 0, 4, fake, ws_need, None) == L.LORA_ERR_INVALID_ARGUMENT
    assert f(fake, fake, fake, 16, ctypes.byref(ok), fake, 0, 0x10000, fake, ws_need, None) == L.LORA_ERR_INVALID_ARGUMENT
    # the short-segment threshold bits are accepted (T == 0: nothing enqueued)
    assert f(None, None, None, 0, ctypes.byref(ok), None, 0, L.LORA_FLAG_SHORT_SEGMENT(200) | 3, fake, ws_need,
             None) == L.LORA_OK
    assert L.LORA_FLAG_SHORT_SEGMENT(16) == 0x1000
    # T == 0 is a no-op that returns OK without touching anything
    assert f(None, None, None, 0, ctypes.byref(ok), None, 0, 0, fake, ws_need, None) == L.LORA_OK
    assert lib.lora_shrink(None, 0, ctypes.byref(ok), None, 0, None, fake, ws_need, None) == L.LORA_OK
    assert lib.lora_expand(None, 0, ctypes.byref(ok), None, 0, None, fake, ws_need, None) == L.LORA_OK
    assert lib.lora_build_segments(None, 0, 4, 8, fake, ws_need, None) == L.LORA_OK
    assert lib.lora_build_segments(fake, 16, 16001, 8, fake, ws_need, None) == L.LORA_ERR_UNSUPPORTED
    g = lib.lora_gemm
    assert g(fake, fake, fake, 4, 60, 64, L.LORA_BF16, None, 0, None) == L.LORA_ERR_INVALID_ARGUMENT
    assert g(fake, fake, fake, 4, 64, 64, 5, None, 0, None) == L.LORA_ERR_INVALID_ARGUMENT
    assert g(None, None, None, 0, 64, 64, L.LORA_BF16, None, 0, None) == L.LORA_OK
    row = ctypes.c_int32()
    assert lib.lora_get_device_error(None, 256, None, ctypes.byref(row)) == L.LORA_ERR_INVALID_ARGUMENT


def test_segments_view_is_pointer_arithmetic(lib):
    fake = 1 << 40
    need = L.lora_workspace_bytes(100, 10, 8)
    seg = L.lora_segments_t()
    assert lib.lora_segments_view(fake, need, 100, 10, 8, ctypes.byref(seg)) == L.LORA_OK
    ptrs = [seg.offsets, seg.perm, seg.seg_id, seg.seg_start, seg.n_seg, seg.gemm_perm]
    assert all(fake <= p < fake + need for p in ptrs)
    assert len(set(ptrs)) == 6 and all(p % 16 == 0 for p in ptrs)
    assert fake <= seg.n_fused < fake + 256 and seg.n_fused % 4 == 0
    # segment regions do not depend on max_rank (reuse across pools)
    seg2 = L.lora_segments_t()
    assert lib.lora_segments_view(fake, L.lora_workspace_bytes(100, 10, 64), 100, 10, 64,
                                  ctypes.byref(seg2)) == L.LORA_OK
    assert seg2.perm == seg.perm and seg2.offsets == seg.offsets


def test_sliced_validation(lib):
    """Pools of one sliced call must agree on n_slots, d_in, max_rank and
    dtype; at most 4 slices and 128 summed ranks.  All checks run on the host
    before anything is enqueued (fake device addresses)."""
    fake = 1 << 40
    P = L.lora_pool_t
    q = P(8, 256, 512, 16, L.LORA_BF16, fake, fake, fake, fake)
    k = P(8, 256, 128, 16, L.LORA_BF16, fake, fake, fake, fake)
    assert L.lora_workspace_bytes_sliced(64, 8, 16, 3, 512) == L.lora_workspace_bytes(64, 8, 48, 512)
    assert L.lora_workspace_bytes_sliced(64, 8, 16, 1, 0) == L.lora_workspace_bytes(64, 8, 16, 0)
    assert L.lora_workspace_bytes_sliced(64, 8, 64, 3, 0) == 0        # 192 ranks
    assert L.lora_workspace_bytes_sliced(64, 8, 16, 5, 0) == 0
    need = L.lora_workspace_bytes_sliced(64, 8, 16, 3, 512)
    arr = L._pool_array([q, k, k])
    f = lib.lora_shrink_sliced
    bad = L._pool_array([q, P(8, 264, 128, 16, L.LORA_BF16, fake, fake, fake, fake)])
    assert f(fake, 64, bad, 2, fake, 0, fake, fake, need, None) == L.LORA_ERR_INVALID_ARGUMENT
    bad = L._pool_array([q, P(8, 256, 128, 32, L.LORA_BF16, fake, fake, fake, fake)])
    assert f(fake, 64, bad, 2, fake, 0, fake, fake, need, None) == L.LORA_ERR_INVALID_ARGUMENT
    bad = L._pool_array([q, P(9, 256, 128, 16, L.LORA_BF16, fake, fake, fake, fake)])
    assert f(fake, 64, bad, 2, fake, 0, fake, fake, need, None) == L.LORA_ERR_INVALID_ARGUMENT
    five = L._pool_array([q] * 5)
    assert f(fake, 64, five, 5, fake, 0, fake, fake, need, None) == L.LORA_ERR_UNSUPPORTED
    big = P(8, 256, 512, 128, L.LORA_BF16, fake, fake, fake, fake)
    assert f(fake, 64, L._pool_array([big, big]), 2, fake, 0, fake, fake, need, None) == L.LORA_ERR_UNSUPPORTED
    assert f(fake, 64, arr, 0, fake, 0, fake, fake, need, None) == L.LORA_ERR_INVALID_ARGUMENT
    need0 = L.lora_workspace_bytes_sliced(64, 8, 16, 3, 0)     # the check these entry points make
    assert f(fake, 64, arr, 3, fake, 0, fake, fake, need0 - 1, None) == L.LORA_ERR_WORKSPACE_TOO_SMALL
    assert f(fake, 64, L._pool_array([q]), 1, fake, 0, fake, fake, L.lora_workspace_bytes(64, 8, 16) - 1,
             None) == L.LORA_ERR_WORKSPACE_TOO_SMALL
    assert f(None, 0, arr, 3, None, 0, None, fake, need, None) == L.LORA_OK   # T == 0
    g = lib.lora_linear_forward_sliced
    W = (ctypes.c_void_p * 3)(fake, fake, fake)
    Y = (ctypes.c_void_p * 3)(fake, fake, None)
    assert g(fake, W, Y, 64, arr, 3, fake, 0, 0, fake, need, None) == L.LORA_ERR_INVALID_ARGUMENT
    Y = (ctypes.c_void_p * 3)(fake, fake, fake + 8)
    assert g(fake, W, Y, 64, arr, 3, fake, 0, 0, fake, need, None) == L.LORA_ERR_INVALID_ARGUMENT
    assert g(fake, W, Y, 64, arr, 3, fake, 0, 8, fake, need, None) == L.LORA_ERR_INVALID_ARGUMENT
    assert g(None, W, Y, 0, arr, 3, None, 0, 0, fake, need, None) == L.LORA_OK


def test_fp8_validation(lib):
    """FP8 entry points: sizes, and every rejection happens on the host."""
    fake = 1 << 20
    P = L.lora_pool_t
    assert L.lora_workspace_bytes_fp8(64, 8, 16, 512, 256) == \
        L.lora_workspace_bytes(64, 8, 16, 256) + 64 * 512 + 256
    assert L.lora_workspace_bytes_fp8(64, 8, 16, 520, 256) == 0           # d_in % 16
    assert L.lora_workspace_bytes_fp8(64, 8, 12, 512, 256) == 0           # bad max_rank
    q = lib.lora_quantize_rows_fp8
    assert q(fake, 4, 24, fake, fake, None) == L.LORA_ERR_INVALID_ARGUMENT
    assert q(fake, -1, 32, fake, fake, None) == L.LORA_ERR_INVALID_ARGUMENT
    assert q(fake, 4, 32, fake + 8, fake, None) == L.LORA_ERR_INVALID_ARGUMENT
    w = lib.lora_quantize_weight_fp8
    assert w(fake, 24, 64, fake, fake, None) == L.LORA_ERR_INVALID_ARGUMENT
    assert w(fake, 32, 60, fake, fake, None) == L.LORA_ERR_INVALID_ARGUMENT
    assert w(None, 32, 64, fake, fake, None) == L.LORA_ERR_INVALID_ARGUMENT
    gm = lib.lora_gemm_fp8
    assert gm(fake, fake, fake, fake, fake, 4, 24, 64, None, 0, None) == L.LORA_ERR_INVALID_ARGUMENT
    assert gm(fake, fake, fake, fake + 4, fake, 4, 32, 64, None, 0, None) == L.LORA_ERR_INVALID_ARGUMENT
    assert gm(None, None, None, None, None, 0, 32, 64, None, 0, None) == L.LORA_OK   # T == 0
    f = lib.lora_linear_forward_fp8
    pool = P(8, 512, 256, 16, L.LORA_BF16, fake, fake, fake, fake)
    need = L.lora_workspace_bytes_fp8(64, 8, 16, 512, 0)
    assert f(fake, fake, fake, fake, 64, ctypes.byref(pool), fake, 0, 0, fake, need - 1, None) == \
        L.LORA_ERR_WORKSPACE_TOO_SMALL
    # the bf16 workspace is too small: the quantized rows of x need room
    assert f(fake, fake, fake, fake, 64, ctypes.byref(pool), fake, 0, 0, fake,
             L.lora_workspace_bytes(64, 8, 16, 0), None) == L.LORA_ERR_WORKSPACE_TOO_SMALL
    f32pool = P(8, 512, 256, 16, L.LORA_F32, fake, fake, fake, fake)
    assert f(fake, fake, fake, fake, 64, ctypes.byref(f32pool), fake, 0, 0, fake, need, None) == \
        L.LORA_ERR_INVALID_ARGUMENT
    odd = P(8, 520, 256, 16, L.LORA_BF16, fake, fake, fake, fake)
    assert f(fake, fake, fake, fake, 64, ctypes.byref(odd), fake, 0, 0, fake, need, None) == \
        L.LORA_ERR_INVALID_ARGUMENT
    assert f(fake, fake, fake + 4, fake, 64, ctypes.byref(pool), fake, 0, 0, fake, need, None) == \
        L.LORA_ERR_INVALID_ARGUMENT
    assert f(fake, fake, fake, fake, 64, ctypes.byref(pool), fake, 3, 0, fake, need, None) == \
        L.LORA_ERR_INVALID_ARGUMENT
    assert f(None, None, None, None, 0, ctypes.byref(pool), None, 0, 0, fake, need, None) == L.LORA_OK
