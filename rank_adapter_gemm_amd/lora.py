"""Python binding of liblora: the C ABI of include/lora.h, same names.

Argument marshalling only: every step of the layer runs in the HIP kernels of
liblora.so.  torch is used for device memory and the current stream.  There
is no fallback: if the library cannot be loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblora.so")

LORA_OK = 0
LORA_ERR_INVALID_ARGUMENT = 1
LORA_ERR_RANK_EXCEEDS_MAX = 2
LORA_ERR_SLOT_OUT_OF_RANGE = 3
LORA_ERR_WORKSPACE_TOO_SMALL = 4
LORA_ERR_UNSUPPORTED = 5
LORA_ERR_HIP = 6

LORA_F32 = 0
LORA_BF16 = 1

LORA_MODE_AUTO = 0
LORA_MODE_BGMV = 1
LORA_MODE_SGMV = 2
LORA_AUTO_SGMV_MIN_ROWS = 512      # AUTO builds segments from this many rows on

LORA_FLAG_SEGMENTS_READY = 0x1
LORA_FLAG_SEPARATE_EXPAND = 0x2


def LORA_FLAG_SHORT_SEGMENT(n: int) -> int:
    """AUTO mode: segments of fewer than n rows take the per-row path."""
    return (int(n) & 0xff) << 8

# Every symbol include/lora.h declares.
EXPORTED = (
    "lora_pool_bytes", "lora_pool_create", "lora_pool_bytes_packed", "lora_pool_create_packed",
    "lora_pool_upload", "lora_pool_clear",
    "lora_workspace_bytes", "lora_workspace_init", "lora_segments_view", "lora_build_segments",
    "lora_shrink", "lora_expand", "lora_gemm", "lora_gemm_expand", "lora_linear_forward",
    "lora_workspace_bytes_sliced", "lora_shrink_sliced", "lora_linear_forward_sliced",
    "lora_pack_host", "lora_cache_create", "lora_cache_destroy", "lora_cache_register", "lora_cache_map",
    "lora_cache_commit", "lora_cache_slot_of", "lora_cache_stats",
    "lora_quantize_rows_fp8", "lora_quantize_weight_fp8", "lora_gemm_fp8", "lora_workspace_bytes_fp8",
    "lora_linear_forward_fp8",
    "lora_linear_forward_noalloc",
    "lora_get_device_error",
    "lora_status_string", "lora_version",
)

LORA_NOALLOC_SCRATCH_BYTES = 64 << 20


class LoraError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, status_string(status), status))


class lora_pool_t(ctypes.Structure):
    _fields_ = [("n_slots", ctypes.c_int32), ("d_in", ctypes.c_int32), ("d_out", ctypes.c_int32),
                ("max_rank", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("a", ctypes.c_void_p), ("b", ctypes.c_void_p),
                ("scale", ctypes.c_void_p), ("rank", ctypes.c_void_p),
                ("row0", ctypes.c_void_p), ("row0_host", ctypes.c_void_p)]


class lora_segments_t(ctypes.Structure):
    _fields_ = [("offsets", ctypes.c_void_p), ("perm", ctypes.c_void_p), ("seg_id", ctypes.c_void_p),
                ("seg_start", ctypes.c_void_p), ("n_seg", ctypes.c_void_p), ("gemm_perm", ctypes.c_void_p),
                ("n_fused", ctypes.c_void_p)]


_lib = None


def _check_single_hip_runtime():
    """liblora must bind to the HIP runtime torch already loaded: two runtimes
    in one process would not share streams or pointers."""
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64.so" in line:
                    paths.add(line.split()[-1])
    except OSError:
        return
    if len(paths) > 1:
        raise RuntimeError("more than one HIP runtime is mapped: %s" % sorted(paths))


def load(path: str = LIB_PATH):
    """Load liblora.so (after torch, so its HIP runtime is the one bound)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("liblora.so is not built (%s): run `python -m rank_adapter_gemm_amd.build`"
                           % path)
    lib = ctypes.CDLL(path)
    _check_single_hip_runtime()
    c_i32, c_sz, c_vp, c_u32, c_f = ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_uint32, ctypes.c_float
    P = ctypes.POINTER
    sig = {
        "lora_pool_bytes": (c_i32, [c_i32, c_i32, c_i32, c_i32, c_i32, P(c_sz), P(c_sz)]),
        "lora_pool_create": (c_i32, [P(lora_pool_t), c_i32, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp]),
        "lora_pool_bytes_packed": (c_i32, [c_i32, c_i32, c_i32, c_vp, c_i32, P(c_sz), P(c_sz)]),
        "lora_pool_create_packed": (c_i32, [P(lora_pool_t), c_i32, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp,
                                            c_vp, c_vp, c_vp, c_vp, c_vp]),
        "lora_pool_upload": (c_i32, [P(lora_pool_t), c_i32, c_vp, c_i32, c_vp, c_i32, c_i32, c_f, c_vp]),
        "lora_pool_clear": (c_i32, [P(lora_pool_t), c_i32, c_vp]),
        "lora_workspace_bytes": (c_sz, [c_i32, c_i32, c_i32, c_i32]),
        "lora_workspace_init": (c_i32, [c_vp, c_sz, c_vp]),
        "lora_segments_view": (c_i32, [c_vp, c_sz, c_i32, c_i32, c_i32, P(lora_segments_t)]),
        "lora_build_segments": (c_i32, [c_vp, c_i32, c_i32, c_i32, c_vp, c_sz, c_vp]),
        "lora_shrink": (c_i32, [c_vp, c_i32, P(lora_pool_t), c_vp, c_i32, c_vp, c_vp, c_sz, c_vp]),
        "lora_expand": (c_i32, [c_vp, c_i32, P(lora_pool_t), c_vp, c_i32, c_vp, c_vp, c_sz, c_vp]),
        "lora_gemm": (c_i32, [c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_vp, c_sz, c_vp]),
        "lora_gemm_expand": (c_i32, [c_vp, c_vp, c_vp, c_i32, P(lora_pool_t), c_vp, c_vp, c_i32, c_vp, c_sz, c_vp]),
        "lora_linear_forward": (c_i32, [c_vp, c_vp, c_vp, c_i32, P(lora_pool_t), c_vp, c_i32, c_u32, c_vp, c_sz, c_vp]),
        "lora_workspace_bytes_sliced": (c_sz, [c_i32, c_i32, c_i32, c_i32, c_i32]),
        "lora_shrink_sliced": (c_i32, [c_vp, c_i32, P(lora_pool_t), c_i32, c_vp, c_i32, c_vp, c_vp, c_sz, c_vp]),
        "lora_linear_forward_sliced": (c_i32, [c_vp, P(c_vp), P(c_vp), c_i32, P(lora_pool_t), c_i32, c_vp,
                                               c_i32, c_u32, c_vp, c_sz, c_vp]),
        "lora_pack_host": (c_i32, [c_i32, c_i32, c_i32, c_i32, c_vp, c_i32, c_vp, c_i32, c_i32, c_vp, c_vp]),
        "lora_cache_create": (c_i32, [P(c_vp), c_i32, P(lora_pool_t), c_i32, c_i32]),
        "lora_cache_destroy": (c_i32, [c_vp]),
        "lora_cache_register": (c_i32, [c_vp, c_i32, P(c_vp), P(c_vp), c_i32, c_f]),
        "lora_cache_map": (c_i32, [c_vp, P(c_i32), c_i32, P(c_i32), c_vp, c_vp]),
        "lora_cache_commit": (c_i32, [c_vp, c_vp]),
        "lora_cache_slot_of": (c_i32, [c_vp, c_i32, P(c_i32)]),
        "lora_cache_stats": (c_i32, [c_vp, P(ctypes.c_int64), P(ctypes.c_int64), P(ctypes.c_int64),
                                     P(ctypes.c_int64)]),
        "lora_quantize_rows_fp8": (c_i32, [c_vp, c_i32, c_i32, c_vp, c_vp, c_vp]),
        "lora_quantize_weight_fp8": (c_i32, [c_vp, c_i32, c_i32, c_vp, c_vp, c_vp]),
        "lora_gemm_fp8": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_vp, c_sz, c_vp]),
        "lora_workspace_bytes_fp8": (c_sz, [c_i32, c_i32, c_i32, c_i32, c_i32]),
        "lora_linear_forward_fp8": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_i32, P(lora_pool_t), c_vp, c_i32, c_u32,
                                            c_vp, c_sz, c_vp]),
        "lora_linear_forward_noalloc": (c_i32, [c_vp, c_vp, c_vp, c_i32, P(lora_pool_t), c_vp, c_i32, c_u32, c_vp,
                                                c_vp]),
        "lora_get_device_error": (c_i32, [c_vp, c_sz, c_vp, P(c_i32)]),
        "lora_status_string": (ctypes.c_char_p, [c_i32]),
        "lora_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().lora_status_string(int(status)).decode()


def _ok(status: int, where: str):
    if status != LORA_OK:
        raise LoraError(status, where)


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return LORA_F32
    if dt == torch.bfloat16:
        return LORA_BF16
    raise TypeError("liblora supports float32 and bfloat16, not %s" % dt)


# ---- a1: pool ---------------------------------------------------------------
def lora_pool_bytes(n_slots, d_in, d_out, max_rank, dtype):
    a = ctypes.c_size_t()
    b = ctypes.c_size_t()
    _ok(load().lora_pool_bytes(n_slots, d_in, d_out, max_rank, dtype, ctypes.byref(a), ctypes.byref(b)),
        "lora_pool_bytes")
    return a.value, b.value


def lora_pool_create(n_slots, d_in, d_out, max_rank, dtype, a, b, scale, rank, stream=None):
    pool = lora_pool_t()
    _ok(load().lora_pool_create(ctypes.byref(pool), n_slots, d_in, d_out, max_rank, dtype, _ptr(a),
                                _ptr(b), _ptr(scale), _ptr(rank), _stream(stream)), "lora_pool_create")
    return pool


def lora_pool_bytes_packed(n_slots, d_in, d_out, capacity, dtype):
    """capacity: a host int32 array (numpy or list) of n_slots rank-row counts."""
    import numpy as np
    cap = np.ascontiguousarray(np.asarray(capacity, dtype=np.int32))
    a = ctypes.c_size_t()
    b = ctypes.c_size_t()
    _ok(load().lora_pool_bytes_packed(n_slots, d_in, d_out, cap.ctypes.data, dtype, ctypes.byref(a),
                                      ctypes.byref(b)), "lora_pool_bytes_packed")
    return a.value, b.value


def lora_pool_create_packed(n_slots, d_in, d_out, max_rank, dtype, capacity, row0_host, a, b, scale, rank, row0,
                            stream=None):
    """capacity: host int32 array [n_slots]; row0_host: host int32 numpy array [n_slots + 1] that the
    caller keeps alive as long as the pool (the descriptor points at it)."""
    import numpy as np
    cap = np.ascontiguousarray(np.asarray(capacity, dtype=np.int32))
    assert row0_host.dtype == np.int32 and row0_host.flags.c_contiguous and row0_host.size == n_slots + 1
    pool = lora_pool_t()
    _ok(load().lora_pool_create_packed(ctypes.byref(pool), n_slots, d_in, d_out, max_rank, dtype, cap.ctypes.data,
                                       row0_host.ctypes.data, _ptr(a), _ptr(b), _ptr(scale), _ptr(rank), _ptr(row0),
                                       _stream(stream)), "lora_pool_create_packed")
    return pool


def lora_pool_upload(pool, slot, A, B, r, alpha, lda=None, ldb=None, stream=None):
    lda = r if lda is None else lda
    ldb = pool.d_out if ldb is None else ldb
    _ok(load().lora_pool_upload(ctypes.byref(pool), slot, _ptr(A), lda, _ptr(B), ldb, r, float(alpha),
                                _stream(stream)), "lora_pool_upload")


def lora_pool_clear(pool, slot, stream=None):
    _ok(load().lora_pool_clear(ctypes.byref(pool), slot, _stream(stream)), "lora_pool_clear")


# ---- workspace / segments -----------------------------------------------------
def lora_workspace_bytes(T, n_slots, max_rank, d_out=0) -> int:
    return int(load().lora_workspace_bytes(T, n_slots, max_rank, d_out))


def lora_workspace_init(ws, stream=None):
    _ok(load().lora_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
        "lora_workspace_init")


def lora_segments_view(ws, T, n_slots, max_rank):
    seg = lora_segments_t()
    _ok(load().lora_segments_view(_ptr(ws), ws.numel() * ws.element_size(), T, n_slots, max_rank,
                                  ctypes.byref(seg)), "lora_segments_view")
    return seg


def lora_build_segments(ids, T, n_slots, max_rank, ws, stream=None):
    _ok(load().lora_build_segments(_ptr(ids), T, n_slots, max_rank, _ptr(ws),
                                   ws.numel() * ws.element_size(), _stream(stream)), "lora_build_segments")


# ---- a4 / a5 / a3 / whole layer ---------------------------------------------------
def lora_shrink(x, T, pool, ids, mode, v, ws, stream=None):
    _ok(load().lora_shrink(_ptr(x), T, ctypes.byref(pool), _ptr(ids), mode, _ptr(v), _ptr(ws),
                           ws.numel() * ws.element_size(), _stream(stream)), "lora_shrink")


def lora_expand(v, T, pool, ids, mode, y, ws, stream=None):
    _ok(load().lora_expand(_ptr(v), T, ctypes.byref(pool), _ptr(ids), mode, _ptr(y), _ptr(ws),
                           ws.numel() * ws.element_size(), _stream(stream)), "lora_expand")


def lora_gemm(x, W, y, T, d_in, d_out, dtype, ws=None, stream=None):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _ok(load().lora_gemm(_ptr(x), _ptr(W), _ptr(y), T, d_in, d_out, dtype, _ptr(ws), nbytes,
                         _stream(stream)), "lora_gemm")


def lora_gemm_expand(x, W, y, T, pool, ids, v, mode, ws, stream=None):
    _ok(load().lora_gemm_expand(_ptr(x), _ptr(W), _ptr(y), T, ctypes.byref(pool), _ptr(ids), _ptr(v),
                                mode, _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
        "lora_gemm_expand")


def lora_linear_forward(x, W, y, T, pool, ids, mode, flags, ws, stream=None):
    _ok(load().lora_linear_forward(_ptr(x), _ptr(W), _ptr(y), T, ctypes.byref(pool), _ptr(ids), mode,
                                   flags, _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
        "lora_linear_forward")


def lora_linear_forward_noalloc(x, W, y, T, pool, ids, mode, flags, err_out=None, stream=None):
    """lora_linear_forward with the library's own device scratch (no workspace argument)."""
    _ok(load().lora_linear_forward_noalloc(_ptr(x), _ptr(W), _ptr(y), T, ctypes.byref(pool), _ptr(ids), mode, flags,
                                           _ptr(err_out), _stream(stream)), "lora_linear_forward_noalloc")


def lora_workspace_bytes_sliced(T, n_slots, max_rank, n_slices, d_out=0) -> int:
    return int(load().lora_workspace_bytes_sliced(T, n_slots, max_rank, n_slices, d_out))


def _pool_array(pools):
    arr = (lora_pool_t * len(pools))()
    for i, p in enumerate(pools):
        arr[i] = p
    return arr


def lora_shrink_sliced(x, T, pools, ids, mode, v, ws, stream=None):
    """pools: a list of lora_pool_t (one per slice)."""
    _ok(load().lora_shrink_sliced(_ptr(x), T, _pool_array(pools), len(pools), _ptr(ids), mode, _ptr(v),
                                  _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
        "lora_shrink_sliced")


def lora_linear_forward_sliced(x, Ws, ys, T, pools, ids, mode, flags, ws, stream=None):
    """Ws, ys: lists of device tensors, one per slice; pools: list of lora_pool_t."""
    n = len(pools)
    w_arr = (ctypes.c_void_p * n)(*[_ptr(w) for w in Ws])
    y_arr = (ctypes.c_void_p * n)(*[_ptr(y) for y in ys])
    _ok(load().lora_linear_forward_sliced(_ptr(x), w_arr, y_arr, T, _pool_array(pools), n, _ptr(ids), mode,
                                          flags, _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
        "lora_linear_forward_sliced")


def lora_pack_host(d_in, d_out, max_rank, dtype, A, B, r, a_slot, b_slot):
    """A [d_in, >= r], B [>= r, d_out] host tensors (row-major) -> a_slot, b_slot
    host tensors of max_rank * d_in and max_rank * d_out elements."""
    for t in (A, B, a_slot, b_slot):
        assert t.device.type == "cpu" and t.is_contiguous()
    _ok(load().lora_pack_host(d_in, d_out, max_rank, dtype, A.data_ptr(), A.shape[1], B.data_ptr(), B.shape[1],
                              r, a_slot.data_ptr(), b_slot.data_ptr()), "lora_pack_host")


class AdapterCache:
    """The host tier + HBM slots residency cache (lora_cache_*).  pools: list
    of lora_pool_t kept in step (empty list: planning only).  Host buffers
    given to register() are kept alive here."""

    def __init__(self, n_slots, pools, max_adapters):
        self.n_pools = len(pools)
        self._h = ctypes.c_void_p()
        arr = _pool_array(pools) if pools else None
        _ok(load().lora_cache_create(ctypes.byref(self._h), n_slots, arr, len(pools), max_adapters),
            "lora_cache_create")
        self._keep = {}

    def register(self, adapter, host_a, host_b, rank, alpha):
        n = self.n_pools
        a_arr = (ctypes.c_void_p * max(n, 1))(*[t.data_ptr() for t in host_a]) if n else None
        b_arr = (ctypes.c_void_p * max(n, 1))(*[t.data_ptr() for t in host_b]) if n else None
        _ok(load().lora_cache_register(self._h, adapter, a_arr, b_arr, rank, alpha), "lora_cache_register")
        self._keep[adapter] = (list(host_a), list(host_b))

    def map(self, adapters, compute=None, copy=None):
        n = len(adapters)
        ids = (ctypes.c_int32 * max(n, 1))(*[int(a) for a in adapters])
        out = (ctypes.c_int32 * max(n, 1))()
        _ok(load().lora_cache_map(self._h, ids, n, out, _stream(compute), _stream(copy)), "lora_cache_map")
        return [out[i] for i in range(n)]

    def commit(self, compute=None):
        _ok(load().lora_cache_commit(self._h, _stream(compute)), "lora_cache_commit")

    def slot_of(self, adapter):
        s = ctypes.c_int32()
        _ok(load().lora_cache_slot_of(self._h, adapter, ctypes.byref(s)), "lora_cache_slot_of")
        return s.value

    def stats(self):
        v = [ctypes.c_int64() for _ in range(4)]
        _ok(load().lora_cache_stats(self._h, *[ctypes.byref(x) for x in v]), "lora_cache_stats")
        return dict(zip(("hits", "misses", "evictions", "bytes"), [x.value for x in v]))

    def close(self):
        if self._h:
            load().lora_cache_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def lora_quantize_rows_fp8(x, T, d, xq, x_scale, stream=None):
    _ok(load().lora_quantize_rows_fp8(_ptr(x), T, d, _ptr(xq), _ptr(x_scale), _stream(stream)),
        "lora_quantize_rows_fp8")


def lora_quantize_weight_fp8(W, d_in, d_out, wq, w_scale, stream=None):
    _ok(load().lora_quantize_weight_fp8(_ptr(W), d_in, d_out, _ptr(wq), _ptr(w_scale), _stream(stream)),
        "lora_quantize_weight_fp8")


def lora_gemm_fp8(xq, x_scale, wq, w_scale, y, T, d_in, d_out, ws=None, stream=None):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _ok(load().lora_gemm_fp8(_ptr(xq), _ptr(x_scale), _ptr(wq), _ptr(w_scale), _ptr(y), T, d_in, d_out,
                             _ptr(ws), nbytes, _stream(stream)), "lora_gemm_fp8")


def lora_workspace_bytes_fp8(T, n_slots, max_rank, d_in, d_out=0) -> int:
    return int(load().lora_workspace_bytes_fp8(T, n_slots, max_rank, d_in, d_out))


def lora_linear_forward_fp8(x, wq, w_scale, y, T, pool, ids, mode, flags, ws, stream=None):
    _ok(load().lora_linear_forward_fp8(_ptr(x), _ptr(wq), _ptr(w_scale), _ptr(y), T, ctypes.byref(pool),
                                       _ptr(ids), mode, flags, _ptr(ws), ws.numel() * ws.element_size(),
                                       _stream(stream)), "lora_linear_forward_fp8")


class Fp8Weight:
    """E4M3 codes [d_out, d_in] and fp32 column scales of a bf16 base weight
    W [d_in, d_out], made on the device by lora_quantize_weight_fp8."""

    def __init__(self, W, stream=None):
        d_in, d_out = W.shape
        self.d_in, self.d_out = d_in, d_out
        self.codes = torch.empty(d_out, d_in, dtype=torch.uint8, device=W.device)
        self.scale = torch.empty(d_out, dtype=torch.float32, device=W.device)
        lora_quantize_weight_fp8(W, d_in, d_out, self.codes, self.scale, stream)


def lora_get_device_error(ws, stream=None) -> int:
    row = ctypes.c_int32()
    _ok(load().lora_get_device_error(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream),
                                     ctypes.byref(row)), "lora_get_device_error")
    return row.value


def lora_version() -> str:
    return load().lora_version().decode()


# ---- plumbing: device buffers held by torch ------------------------------------------
class AdapterPool:
    """Owns the torch device buffers of one pool and its lora_pool_t.  With
    `capacity` (n_slots rank-row counts, multiples of 8) the pool is packed:
    slot s holds capacity[s] rank rows, with no padding to max_rank."""

    def __init__(self, n_slots, d_in, d_out, max_rank, dtype: torch.dtype, device="cuda", stream=None,
                 capacity=None):
        import numpy as np
        code = dtype_code(dtype)
        if capacity is None:
            a_bytes, b_bytes = lora_pool_bytes(n_slots, d_in, d_out, max_rank, code)
        else:
            a_bytes, b_bytes = lora_pool_bytes_packed(n_slots, d_in, d_out, capacity, code)
        self.a = torch.empty(a_bytes, dtype=torch.uint8, device=device)
        self.b = torch.empty(b_bytes, dtype=torch.uint8, device=device)
        self.scale = torch.empty(n_slots, dtype=torch.float32, device=device)
        self.rank = torch.empty(n_slots, dtype=torch.int32, device=device)
        self.dtype = dtype
        if capacity is None:
            self.row0 = self.row0_host = None
            self.pool = lora_pool_create(n_slots, d_in, d_out, max_rank, code, self.a, self.b,
                                         self.scale, self.rank, stream)
        else:
            self.row0 = torch.empty(n_slots + 1, dtype=torch.int32, device=device)
            self.row0_host = np.zeros(n_slots + 1, dtype=np.int32)
            self.pool = lora_pool_create_packed(n_slots, d_in, d_out, max_rank, code, capacity, self.row0_host,
                                                self.a, self.b, self.scale, self.rank, self.row0, stream)

    def upload(self, slot, A, B, r, alpha, lda=None, ldb=None, stream=None):
        lora_pool_upload(self.pool, slot, A, B, r, alpha, lda, ldb, stream)

    def clear(self, slot, stream=None):
        lora_pool_clear(self.pool, slot, stream)

    @property
    def nbytes(self):
        return self.a.numel() + self.b.numel() + 8 * self.scale.numel()


class Workspace:
    """A device workspace sized for (T, n_slots, max_rank, d_out), initialised."""

    def __init__(self, T, n_slots, max_rank, d_out=0, device="cuda", stream=None, n_slices=1, fp8_d_in=0):
        if fp8_d_in:
            if n_slices != 1:
                raise LoraError(LORA_ERR_INVALID_ARGUMENT, "lora_workspace_bytes_fp8")
            n = lora_workspace_bytes_fp8(T, n_slots, max_rank, fp8_d_in, d_out)
        else:
            n = lora_workspace_bytes_sliced(T, n_slots, max_rank, n_slices, d_out)
        if n == 0:
            raise LoraError(LORA_ERR_INVALID_ARGUMENT, "lora_workspace_bytes")
        self.T, self.n_slots, self.max_rank = T, n_slots, max_rank
        self.buf = torch.empty(n, dtype=torch.uint8, device=device)
        lora_workspace_init(self.buf, stream)

    def segments(self, T=None):
        """int32 tensor views of the segment metadata inside the workspace."""
        T = self.T if T is None else T
        seg = lora_segments_view(self.buf, T, self.n_slots, self.max_rank)
        base = self.buf.data_ptr()

        def view(ptr, n):
            off = ptr - base
            return self.buf[off:off + 4 * n].view(torch.int32)

        return {"offsets": view(seg.offsets, self.n_slots + 2), "perm": view(seg.perm, T),
                "seg_id": view(seg.seg_id, self.n_slots), "seg_start": view(seg.seg_start, self.n_slots + 1),
                "n_seg": view(seg.n_seg, 1), "gemm_perm": view(seg.gemm_perm, T), "n_fused": view(seg.n_fused, 1)}
