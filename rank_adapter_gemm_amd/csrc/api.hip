// liblora C ABI: argument validation on the host, then launches on the
// caller's stream.  No allocation, no hidden state.  The contract of every
// entry point is stated in include/lora.h.
#include <string.h>

#include <mutex>

#include "common.hpp"

using namespace lora;

namespace {

inline hipStream_t hs(lora_stream_t s) { return reinterpret_cast<hipStream_t>(s); }
inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool valid_dtype(int32_t d) { return d == LORA_F32 || d == LORA_BF16; }
inline size_t dtype_bytes(int32_t d) { return d == LORA_F32 ? 4 : 2; }

inline bool valid_dims(int32_t n_slots, int32_t d_in, int32_t d_out, int32_t max_rank) {
    return n_slots >= 1 && n_slots <= kMaxSlots && d_in > 0 && d_out > 0 && (d_in % 8) == 0 &&
           (d_out % 8) == 0 && max_rank >= 8 && max_rank <= 128 && (max_rank % 8) == 0 &&
           (int64_t)d_in * max_rank < ((int64_t)1 << 31) && (int64_t)d_out * max_rank < ((int64_t)1 << 31);
}

inline bool valid_pool(const lora_pool_t *p) {
    return p && valid_dims(p->n_slots, p->d_in, p->d_out, p->max_rank) && valid_dtype(p->dtype) &&
           p->a && p->b && p->scale && p->rank && aligned16(p->a) && aligned16(p->b) &&
           (p->row0 == nullptr) == (p->row0_host == nullptr);
}

// Rank rows of one slot: max_rank (padded pool) or its capacity (packed).
inline int32_t slot_capacity(const lora_pool_t *p, int32_t slot) {
    return p->row0_host ? p->row0_host[slot + 1] - p->row0_host[slot] : p->max_rank;
}

// Packed-pool capacities: multiples of 8 in [8, max_rank]; their sum must
// keep every element offset in range.  *rows gets the sum.
inline bool valid_capacities(const int32_t *cap, int32_t n_slots, int32_t d_in, int32_t d_out, int32_t max_rank,
                             int64_t *rows) {
    if (!cap) return false;
    int64_t total = 0;
    for (int32_t s = 0; s < n_slots; ++s) {
        if (cap[s] < 8 || cap[s] > max_rank || (cap[s] % 8)) return false;
        total += cap[s];
    }
    if (total >= ((int64_t)1 << 31)) return false;
    *rows = total;
    return true;
}

inline lora_status_t check_ws(const void *ws, size_t ws_bytes, int32_t T, int32_t n_slots,
                              int32_t max_rank, ws_layout *L) {
    if (!ws || !aligned16(ws)) return LORA_ERR_INVALID_ARGUMENT;
    *L = make_ws_layout(T, n_slots, max_rank, 0);
    if (ws_bytes < L->total) return LORA_ERR_WORKSPACE_TOO_SMALL;
    return LORA_OK;
}

inline lora_status_t check_ws_fp8(const void *ws, size_t ws_bytes, int32_t T, int32_t n_slots,
                                  int32_t max_rank, int32_t d_in, ws_layout *L) {
    if (!ws || !aligned16(ws)) return LORA_ERR_INVALID_ARGUMENT;
    *L = make_ws_layout(T, n_slots, max_rank, 0, d_in);
    if (ws_bytes < L->total) return LORA_ERR_WORKSPACE_TOO_SMALL;
    return LORA_OK;
}

inline bool use_sgmv(lora_mode_t mode, int32_t T) {
    if (mode == LORA_MODE_SGMV) return true;
    if (mode == LORA_MODE_BGMV) return false;
    return T >= LORA_AUTO_SGMV_MIN_ROWS;
}

// Flag bits the forwards accept: the two flags and the short-segment threshold.
constexpr uint32_t kForwardFlags = LORA_FLAG_SEGMENTS_READY | LORA_FLAG_SEPARATE_EXPAND | 0xff00u;

// Segments of fewer rows than this take the per-row path: AUTO mode on bf16
// pools (the threshold from the flags, else the default); SGMV mode groups
// every segment.
inline int32_t short_len_for(lora_mode_t mode, uint32_t flags, int32_t dtype) {
    if (mode != LORA_MODE_AUTO || dtype != LORA_BF16) return 1;
    const int32_t n = (int32_t)((flags >> 8) & 0xffu);
    return n > 0 ? n : kShortSegDefault;
}

inline bool valid_mode(int32_t m) {
    return m == LORA_MODE_AUTO || m == LORA_MODE_BGMV || m == LORA_MODE_SGMV;
}

// Slices must be valid pools that agree on everything the shared shrink uses.
inline lora_status_t check_slices(const lora_pool_t *pools, int32_t n) {
    if (!pools || n < 1) return LORA_ERR_INVALID_ARGUMENT;
    if (n > kMaxSlices) return LORA_ERR_UNSUPPORTED;
    for (int i = 0; i < n; ++i) {
        if (!valid_pool(&pools[i])) return LORA_ERR_INVALID_ARGUMENT;
        if (pools[i].n_slots != pools[0].n_slots || pools[i].d_in != pools[0].d_in ||
            pools[i].max_rank != pools[0].max_rank || pools[i].dtype != pools[0].dtype)
            return LORA_ERR_INVALID_ARGUMENT;
    }
    if ((int64_t)n * pools[0].max_rank > kMaxSliceRanks) return LORA_ERR_UNSUPPORTED;
    return LORA_OK;
}

// Base product plus the low-rank term from v (row stride v_stride), fused
// into the GEMM or as a separate pass.  With segments, the GEMM visits rows
// in the GEMM order (long segments, then short ones), fuses the term of the
// long segments' rows and leaves the short segments' rows to a per-row
// expand after it.
lora_status_t gemm_and_expand(const void *x, const void *W, void *y, int32_t T, const lora_pool_t &p,
                              const int32_t *ids, const float *v, int32_t v_stride, bool sgmv,
                              uint32_t flags, const ws_layout &L, void *ws, size_t ws_bytes,
                              hipStream_t s) {
    const int32_t *gperm = sgmv ? ws_ptr<int32_t>(ws, L.gperm) : nullptr;
    const int32_t *n_fused = sgmv ? ws_ptr<int32_t>(ws, L.header) + kHdrNLong : nullptr;
    float *partial = ws_ptr<float>(ws, L.gemm_partial);
    const size_t partial_bytes = ws_bytes - L.gemm_partial;
    if (flags & LORA_FLAG_SEPARATE_EXPAND) {
        lora_status_t st = launch_gemm(x, W, y, T, p.d_in, p.d_out, p.dtype, nullptr, nullptr, nullptr,
                                       0, nullptr, partial, partial_bytes, s);
        if (st != LORA_OK) return st;
        return launch_expand(v, v_stride, T, p, ids, sgmv, y, L, ws, s);
    }
    lora_status_t st = launch_gemm(x, W, y, T, p.d_in, p.d_out, p.dtype, &p, ids, v, v_stride, gperm, partial,
                                   partial_bytes, s, p.dtype == LORA_BF16 ? n_fused : nullptr);
    if (st == LORA_OK && sgmv) st = launch_expand_short(v, v_stride, T, p, y, L, ws, s);
    return st;
}

// ---------------------------------------------------------------------------
// Workspace of lora_linear_forward_noalloc, for callers that cannot allocate:
// a file-scope device array.  Every GPU the library runs on holds its own
// copy until the process ends.  In host code the array's name is only a
// stand-in: its device address is looked up once per device
// (hipGetSymbolAddress, with that device current) and kept in
// g_scratch_ptr; kernels receive that address, never the name.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
static void *g_scratch_ptr[kMaxDevices];
static std::mutex g_scratch_mu;

lora_status_t scratch_of_current_device(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return LORA_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return LORA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LORA_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return LORA_OK;
}

// err_out[0] = the smallest bad row recorded in the workspace's error word,
// or -1 if none.
__global__ void k_error_out(const int32_t *header, int32_t *err_out) {
    if (threadIdx.x == 0) err_out[0] = header[kHdrErr] == kErrNone ? -1 : header[kHdrErr];
}

}  // namespace

extern "C" {

const char *lora_version(void) { return "liblora 0.1 gfx950"; }

const char *lora_status_string(lora_status_t s) {
    switch (s) {
        case LORA_OK: return "ok";
        case LORA_ERR_INVALID_ARGUMENT: return "invalid argument";
        case LORA_ERR_RANK_EXCEEDS_MAX: return "adapter rank exceeds the pool's max_rank";
        case LORA_ERR_SLOT_OUT_OF_RANGE: return "slot index out of range";
        case LORA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case LORA_ERR_UNSUPPORTED: return "unsupported configuration";
        case LORA_ERR_HIP: return "HIP runtime error at launch";
    }
    return "unknown status";
}

lora_status_t lora_pool_bytes(int32_t n_slots, int32_t d_in, int32_t d_out, int32_t max_rank,
                              lora_dtype_t dtype, size_t *a_bytes, size_t *b_bytes) {
    if (!a_bytes || !b_bytes || !valid_dtype(dtype)) return LORA_ERR_INVALID_ARGUMENT;
    if (n_slots > kMaxSlots) return LORA_ERR_UNSUPPORTED;
    if (!valid_dims(n_slots, d_in, d_out, max_rank)) return LORA_ERR_INVALID_ARGUMENT;
    const size_t eb = dtype_bytes(dtype);
    *a_bytes = (size_t)n_slots * max_rank * d_in * eb;
    *b_bytes = (size_t)n_slots * max_rank * d_out * eb;
    return LORA_OK;
}

lora_status_t lora_pool_create(lora_pool_t *pool, int32_t n_slots, int32_t d_in, int32_t d_out,
                               int32_t max_rank, lora_dtype_t dtype, void *a, void *b,
                               float *scale, int32_t *rank, lora_stream_t stream) {
    size_t ab, bb;
    lora_status_t st = lora_pool_bytes(n_slots, d_in, d_out, max_rank, dtype, &ab, &bb);
    if (st != LORA_OK) return st;
    if (!pool || !a || !b || !scale || !rank || !aligned16(a) || !aligned16(b))
        return LORA_ERR_INVALID_ARGUMENT;
    lora_pool_t p;
    p.n_slots = n_slots;
    p.d_in = d_in;
    p.d_out = d_out;
    p.max_rank = max_rank;
    p.dtype = dtype;
    p.a = a;
    p.b = b;
    p.scale = scale;
    p.rank = rank;
    p.row0 = nullptr;
    p.row0_host = nullptr;
    st = launch_pool_fill(a, ab, b, bb, scale, rank, n_slots, hs(stream));
    if (st == LORA_OK) *pool = p;
    return st;
}

lora_status_t lora_pool_bytes_packed(int32_t n_slots, int32_t d_in, int32_t d_out, const int32_t *capacity,
                                     lora_dtype_t dtype, size_t *a_bytes, size_t *b_bytes) {
    if (!a_bytes || !b_bytes || !valid_dtype(dtype) || !capacity) return LORA_ERR_INVALID_ARGUMENT;
    if (n_slots > kMaxSlots) return LORA_ERR_UNSUPPORTED;
    if (!valid_dims(n_slots, d_in, d_out, 8)) return LORA_ERR_INVALID_ARGUMENT;
    int32_t cmax = 8;
    for (int32_t s = 0; s < n_slots; ++s) cmax = capacity[s] > cmax ? capacity[s] : cmax;
    int64_t rows = 0;
    if (cmax > 128 || !valid_dims(n_slots, d_in, d_out, cmax) ||
        !valid_capacities(capacity, n_slots, d_in, d_out, cmax, &rows))
        return LORA_ERR_INVALID_ARGUMENT;
    const size_t eb = dtype_bytes(dtype);
    *a_bytes = (size_t)rows * d_in * eb;
    *b_bytes = (size_t)rows * d_out * eb;
    return LORA_OK;
}

lora_status_t lora_pool_create_packed(lora_pool_t *pool, int32_t n_slots, int32_t d_in, int32_t d_out,
                                      int32_t max_rank, lora_dtype_t dtype, const int32_t *capacity,
                                      int32_t *row0_host, void *a, void *b, float *scale, int32_t *rank,
                                      int32_t *row0, lora_stream_t stream) {
    if (!pool || !capacity || !row0_host || !row0 || !a || !b || !scale || !rank || !aligned16(a) ||
        !aligned16(b) || !valid_dtype(dtype))
        return LORA_ERR_INVALID_ARGUMENT;
    if (n_slots > kMaxSlots) return LORA_ERR_UNSUPPORTED;
    int64_t rows = 0;
    if (!valid_dims(n_slots, d_in, d_out, max_rank) ||
        !valid_capacities(capacity, n_slots, d_in, d_out, max_rank, &rows))
        return LORA_ERR_INVALID_ARGUMENT;
    if ((int64_t)rows * d_in >= ((int64_t)1 << 40) || (int64_t)rows * d_out >= ((int64_t)1 << 40))
        return LORA_ERR_UNSUPPORTED;
    row0_host[0] = 0;
    for (int32_t s = 0; s < n_slots; ++s) row0_host[s + 1] = row0_host[s] + capacity[s];
    const hipStream_t st_ = hs(stream);
    if (hipMemcpyAsync(row0, row0_host, sizeof(int32_t) * (size_t)(n_slots + 1), hipMemcpyHostToDevice, st_) !=
        hipSuccess)
        return LORA_ERR_HIP;
    lora_pool_t p;
    p.n_slots = n_slots;
    p.d_in = d_in;
    p.d_out = d_out;
    p.max_rank = max_rank;
    p.dtype = dtype;
    p.a = a;
    p.b = b;
    p.scale = scale;
    p.rank = rank;
    p.row0 = row0;
    p.row0_host = row0_host;
    const size_t eb = dtype_bytes(dtype);
    lora_status_t st = launch_pool_fill(a, (size_t)rows * d_in * eb, b, (size_t)rows * d_out * eb, scale, rank,
                                        n_slots, st_);
    if (st == LORA_OK) *pool = p;
    return st;
}

lora_status_t lora_pool_upload(const lora_pool_t *pool, int32_t slot, const void *A, int32_t lda,
                               const void *B, int32_t ldb, int32_t r, float alpha,
                               lora_stream_t stream) {
    if (!valid_pool(pool)) return LORA_ERR_INVALID_ARGUMENT;
    if (slot < 0 || slot >= pool->n_slots) return LORA_ERR_SLOT_OUT_OF_RANGE;
    if (r > pool->max_rank || r > slot_capacity(pool, slot)) return LORA_ERR_RANK_EXCEEDS_MAX;
    if (r < 1 || !A || !B || lda < r || ldb < pool->d_out) return LORA_ERR_INVALID_ARGUMENT;
    return launch_pool_upload(*pool, slot, A, lda, B, ldb, r, alpha, hs(stream));
}

lora_status_t lora_pool_clear(const lora_pool_t *pool, int32_t slot, lora_stream_t stream) {
    if (!valid_pool(pool)) return LORA_ERR_INVALID_ARGUMENT;
    if (slot < 0 || slot >= pool->n_slots) return LORA_ERR_SLOT_OUT_OF_RANGE;
    return launch_pool_clear(*pool, slot, hs(stream));
}

size_t lora_workspace_bytes(int32_t T, int32_t n_slots, int32_t max_rank, int32_t d_out) {
    if (T < 0 || n_slots < 1 || n_slots > kMaxSlots || max_rank < 8 || max_rank > 128 ||
        (max_rank % 8) != 0 || d_out < 0 || (d_out % 8) != 0)
        return 0;
    return make_ws_layout(T, n_slots, max_rank, d_out).total;
}

lora_status_t lora_workspace_init(void *ws, size_t ws_bytes, lora_stream_t stream) {
    if (!ws || !aligned16(ws) || ws_bytes < 256) return LORA_ERR_INVALID_ARGUMENT;
    return launch_ws_init(ws, hs(stream));
}

lora_status_t lora_segments_view(void *ws, size_t ws_bytes, int32_t T, int32_t n_slots,
                                 int32_t max_rank, lora_segments_t *out) {
    if (!out || T < 0 || n_slots < 1 || n_slots > kMaxSlots) return LORA_ERR_INVALID_ARGUMENT;
    ws_layout L;
    lora_status_t st = check_ws(ws, ws_bytes, T, n_slots, max_rank, &L);
    if (st != LORA_OK) return st;
    out->offsets = ws_ptr<int32_t>(ws, L.offsets);
    out->perm = ws_ptr<int32_t>(ws, L.perm);
    out->seg_id = ws_ptr<int32_t>(ws, L.seg_id);
    out->seg_start = ws_ptr<int32_t>(ws, L.seg_start);
    out->n_seg = ws_ptr<int32_t>(ws, L.n_seg);
    out->gemm_perm = ws_ptr<int32_t>(ws, L.gperm);
    out->n_fused = ws_ptr<int32_t>(ws, L.header) + kHdrNLong;
    return LORA_OK;
}

lora_status_t lora_build_segments(const int32_t *ids, int32_t T, int32_t n_slots, int32_t max_rank,
                                  void *ws, size_t ws_bytes, lora_stream_t stream) {
    if (T < 0 || n_slots < 1) return LORA_ERR_INVALID_ARGUMENT;
    if (n_slots > kMaxSlots) return LORA_ERR_UNSUPPORTED;
    if (T > 0 && !ids) return LORA_ERR_INVALID_ARGUMENT;
    ws_layout L;
    lora_status_t st = check_ws(ws, ws_bytes, T, n_slots, max_rank, &L);
    if (st != LORA_OK) return st;
    if (T == 0) return LORA_OK;
    return launch_segments(ids, T, n_slots, L, ws, hs(stream));
}

lora_status_t lora_shrink(const void *x, int32_t T, const lora_pool_t *pool, const int32_t *ids,
                          lora_mode_t mode, float *v, void *ws, size_t ws_bytes,
                          lora_stream_t stream) {
    if (!valid_pool(pool) || T < 0 || !valid_mode(mode)) return LORA_ERR_INVALID_ARGUMENT;
    if (T > 0 && (!x || !ids || !v || !aligned16(x) || !aligned16(v))) return LORA_ERR_INVALID_ARGUMENT;
    ws_layout L;
    lora_status_t st = check_ws(ws, ws_bytes, T, pool->n_slots, pool->max_rank, &L);
    if (st != LORA_OK) return st;
    if (T == 0) return LORA_OK;
    return launch_shrink(x, T, pool, 1, ids, mode == LORA_MODE_SGMV, v, L, ws, hs(stream));
}

lora_status_t lora_expand(const float *v, int32_t T, const lora_pool_t *pool, const int32_t *ids,
                          lora_mode_t mode, void *y, void *ws, size_t ws_bytes,
                          lora_stream_t stream) {
    if (!valid_pool(pool) || T < 0 || !valid_mode(mode)) return LORA_ERR_INVALID_ARGUMENT;
    if (T > 0 && (!v || !ids || !y || !aligned16(y))) return LORA_ERR_INVALID_ARGUMENT;
    ws_layout L;
    lora_status_t st = check_ws(ws, ws_bytes, T, pool->n_slots, pool->max_rank, &L);
    if (st != LORA_OK) return st;
    if (T == 0) return LORA_OK;
    return launch_expand(v, pool->max_rank, T, *pool, ids, mode == LORA_MODE_SGMV, y, L, ws, hs(stream));
}

lora_status_t lora_gemm(const void *x, const void *W, void *y, int32_t T, int32_t d_in,
                        int32_t d_out, lora_dtype_t dtype, void *ws, size_t ws_bytes,
                        lora_stream_t stream) {
    if (T < 0 || !valid_dtype(dtype) || d_in <= 0 || d_out <= 0 || (d_in % 8) || (d_out % 8))
        return LORA_ERR_INVALID_ARGUMENT;
    if (T > 0 && (!x || !W || !y || !aligned16(x) || !aligned16(W) || !aligned16(y)))
        return LORA_ERR_INVALID_ARGUMENT;
    if (ws && !aligned16(ws)) return LORA_ERR_INVALID_ARGUMENT;
    if (T == 0) return LORA_OK;
    return launch_gemm(x, W, y, T, d_in, d_out, dtype, nullptr, nullptr, nullptr, 0, nullptr,
                       ws ? static_cast<float *>(ws) : nullptr, ws ? ws_bytes : 0, hs(stream));
}

lora_status_t lora_gemm_expand(const void *x, const void *W, void *y, int32_t T,
                               const lora_pool_t *pool, const int32_t *ids, const float *v,
                               lora_mode_t mode, void *ws, size_t ws_bytes, lora_stream_t stream) {
    if (!valid_pool(pool) || T < 0 || !valid_mode(mode)) return LORA_ERR_INVALID_ARGUMENT;
    if (T > 0 && (!x || !W || !y || !ids || !v || !aligned16(x) || !aligned16(W) || !aligned16(y)))
        return LORA_ERR_INVALID_ARGUMENT;
    ws_layout L;
    lora_status_t st = check_ws(ws, ws_bytes, T, pool->n_slots, pool->max_rank, &L);
    if (st != LORA_OK) return st;
    if (T == 0) return LORA_OK;
    // SGMV: the GEMM step of a forward -- rows in the GEMM order of the
    // segments in ws, the short segments' rows expanded after the GEMM.
    return gemm_and_expand(x, W, y, T, *pool, ids, v, pool->max_rank, mode == LORA_MODE_SGMV, 0, L, ws, ws_bytes,
                           hs(stream));
}

lora_status_t lora_linear_forward(const void *x, const void *W, void *y, int32_t T,
                                  const lora_pool_t *pool, const int32_t *ids, lora_mode_t mode,
                                  uint32_t flags, void *ws, size_t ws_bytes,
                                  lora_stream_t stream) {
    if (!valid_pool(pool) || T < 0 || !valid_mode(mode) || (flags & ~kForwardFlags))
        return LORA_ERR_INVALID_ARGUMENT;
    if (T > 0 && (!x || !W || !y || !ids || !aligned16(x) || !aligned16(W) || !aligned16(y)))
        return LORA_ERR_INVALID_ARGUMENT;
    ws_layout L;
    lora_status_t st = check_ws(ws, ws_bytes, T, pool->n_slots, pool->max_rank, &L);
    if (st != LORA_OK) return st;
    if (T == 0) return LORA_OK;
    const hipStream_t s = hs(stream);
    const bool sgmv = use_sgmv(mode, T);
    if (sgmv && !(flags & LORA_FLAG_SEGMENTS_READY)) {
        st = launch_segments(ids, T, pool->n_slots, L, ws, s, short_len_for(mode, flags, pool->dtype));
        if (st != LORA_OK) return st;
    }
    // Decode-sized BGMV batches: the shrink runs inside the split-K GEMM,
    // which streams x through LDS anyway (the workspace's v is not written).
    if (!sgmv && !(flags & LORA_FLAG_SEPARATE_EXPAND) && pool->dtype == LORA_BF16 &&
        gemm_fused_shrink_ok(T, pool->d_in, pool->d_out, pool->max_rank, ws_bytes - L.gemm_partial))
        return launch_gemm_fused_shrink(x, W, y, T, pool, ids, ws_ptr<float>(ws, L.partial),
                                        ws_ptr<int32_t>(ws, L.header), ws_ptr<float>(ws, L.gemm_partial),
                                        ws_bytes - L.gemm_partial, s);
    float *v = ws_ptr<float>(ws, L.v);
    st = launch_shrink(x, T, pool, 1, ids, sgmv, v, L, ws, s);
    if (st != LORA_OK) return st;
    return gemm_and_expand(x, W, y, T, *pool, ids, v, pool->max_rank, sgmv, flags, L, ws, ws_bytes, s);
}

size_t lora_workspace_bytes_sliced(int32_t T, int32_t n_slots, int32_t max_rank, int32_t n_slices,
                                   int32_t d_out) {
    if (n_slices < 1 || n_slices > kMaxSlices || (int64_t)n_slices * max_rank > kMaxSliceRanks ||
        max_rank < 8 || (max_rank % 8) != 0)
        return 0;
    return lora_workspace_bytes(T, n_slots, n_slices * max_rank, d_out);
}

lora_status_t lora_shrink_sliced(const void *x, int32_t T, const lora_pool_t *pools,
                                 int32_t n_slices, const int32_t *ids, lora_mode_t mode, float *v,
                                 void *ws, size_t ws_bytes, lora_stream_t stream) {
    lora_status_t st = check_slices(pools, n_slices);
    if (st != LORA_OK) return st;
    if (T < 0 || !valid_mode(mode)) return LORA_ERR_INVALID_ARGUMENT;
    if (T > 0 && (!x || !ids || !v || !aligned16(x) || !aligned16(v))) return LORA_ERR_INVALID_ARGUMENT;
    ws_layout L;
    st = check_ws(ws, ws_bytes, T, pools[0].n_slots, n_slices * pools[0].max_rank, &L);
    if (st != LORA_OK) return st;
    if (T == 0) return LORA_OK;
    return launch_shrink(x, T, pools, n_slices, ids, mode == LORA_MODE_SGMV, v, L, ws, hs(stream));
}

lora_status_t lora_linear_forward_sliced(const void *x, const void *const *W, void *const *y,
                                         int32_t T, const lora_pool_t *pools, int32_t n_slices,
                                         const int32_t *ids, lora_mode_t mode, uint32_t flags,
                                         void *ws, size_t ws_bytes, lora_stream_t stream) {
    lora_status_t st = check_slices(pools, n_slices);
    if (st != LORA_OK) return st;
    if (T < 0 || !valid_mode(mode) || (flags & ~kForwardFlags) || !W || !y) return LORA_ERR_INVALID_ARGUMENT;
    if (T > 0) {
        if (!x || !ids || !aligned16(x)) return LORA_ERR_INVALID_ARGUMENT;
        for (int i = 0; i < n_slices; ++i)
            if (!W[i] || !y[i] || !aligned16(W[i]) || !aligned16(y[i])) return LORA_ERR_INVALID_ARGUMENT;
    }
    const int32_t R = pools[0].max_rank, VS = n_slices * R;
    ws_layout L;
    st = check_ws(ws, ws_bytes, T, pools[0].n_slots, VS, &L);
    if (st != LORA_OK) return st;
    if (T == 0) return LORA_OK;
    const hipStream_t s = hs(stream);
    const bool sgmv = use_sgmv(mode, T);
    // Each slice takes the path lora_linear_forward would take for it:
    // decode-sized BGMV batches compute the shrink inside that slice's GEMM
    // (on the x it streams anyway); the other slices share one shrink.
    const bool try_fused = !sgmv && !(flags & LORA_FLAG_SEPARATE_EXPAND) && pools[0].dtype == LORA_BF16;
    bool fused[kMaxSlices], any_shared = false;
    for (int i = 0; i < n_slices; ++i) {
        fused[i] = try_fused &&
                   gemm_fused_shrink_ok(T, pools[i].d_in, pools[i].d_out, R, ws_bytes - L.gemm_partial);
        any_shared |= !fused[i];
    }
    float *v = ws_ptr<float>(ws, L.v);
    if (any_shared) {
        if (sgmv && !(flags & LORA_FLAG_SEGMENTS_READY)) {
            st = launch_segments(ids, T, pools[0].n_slots, L, ws, s, short_len_for(mode, flags, pools[0].dtype));
            if (st != LORA_OK) return st;
        }
        st = launch_shrink(x, T, pools, n_slices, ids, sgmv, v, L, ws, s);   // one x read for all slices
        if (st != LORA_OK) return st;
    }
    // bf16 slices on the shared shrink: one grouped GEMM with the fused
    // expand, where that fills the chip better than one GEMM per slice
    int32_t Ns[kMaxSlices], nn = 0;
    for (int i = 0; i < n_slices; ++i)
        if (!fused[i]) Ns[nn++] = pools[i].d_out;
    const bool grouped = pools[0].dtype == LORA_BF16 && !(flags & LORA_FLAG_SEPARATE_EXPAND) &&
                         gemm_grouping_pays(T, pools[0].d_in, Ns, nn, ws_bytes - L.gemm_partial);
    const void *gW[kMaxSlices];
    void *gy[kMaxSlices];
    lora_pool_t gp[kMaxSlices];
    int32_t goff[kMaxSlices], ng = 0;
    for (int i = 0; i < n_slices; ++i) {
        if (fused[i])
            st = launch_gemm_fused_shrink(x, W[i], y[i], T, &pools[i], ids, ws_ptr<float>(ws, L.partial),
                                          ws_ptr<int32_t>(ws, L.header), ws_ptr<float>(ws, L.gemm_partial),
                                          ws_bytes - L.gemm_partial, s);
        else if (grouped) {
            gW[ng] = W[i];
            gy[ng] = y[i];
            gp[ng] = pools[i];
            goff[ng++] = i * R;
        } else
            st = gemm_and_expand(x, W[i], y[i], T, pools[i], ids, v + i * R, VS, sgmv, flags, L, ws,
                                 ws_bytes, s);
        if (st != LORA_OK) return st;
    }
    if (ng > 0) {
        st = launch_gemm_grouped(x, gW, gy, T, gp, ng, ids, v, goff, VS,
                                 sgmv ? ws_ptr<int32_t>(ws, L.gperm) : nullptr, ws_ptr<float>(ws, L.gemm_partial),
                                 ws_bytes - L.gemm_partial, s,
                                 sgmv ? ws_ptr<int32_t>(ws, L.header) + kHdrNLong : nullptr);
        for (int i = 0; i < ng && st == LORA_OK && sgmv; ++i)
            st = launch_expand_short(v + goff[i], VS, T, gp[i], gy[i], L, ws, s);
    }
    return st;
}

lora_status_t lora_quantize_rows_fp8(const void *x, int32_t T, int32_t d, uint8_t *xq, float *x_scale,
                                     lora_stream_t stream) {
    if (T < 0 || d <= 0 || (d % 16)) return LORA_ERR_INVALID_ARGUMENT;
    if (T > 0 && (!x || !xq || !x_scale || !aligned16(x) || !aligned16(xq) || !aligned16(x_scale)))
        return LORA_ERR_INVALID_ARGUMENT;
    return launch_quant_rows_fp8(x, T, d, xq, x_scale, hs(stream));
}

lora_status_t lora_quantize_weight_fp8(const void *W, int32_t d_in, int32_t d_out, uint8_t *wq,
                                       float *w_scale, lora_stream_t stream) {
    if (d_in <= 0 || d_out <= 0 || (d_in % 16) || (d_out % 8)) return LORA_ERR_INVALID_ARGUMENT;
    if (!W || !wq || !w_scale || !aligned16(W) || !aligned16(wq) || !aligned16(w_scale))
        return LORA_ERR_INVALID_ARGUMENT;
    return launch_quant_cols_fp8(W, d_in, d_out, wq, w_scale, hs(stream));
}

lora_status_t lora_gemm_fp8(const uint8_t *xq, const float *x_scale, const uint8_t *wq,
                            const float *w_scale, void *y, int32_t T, int32_t d_in, int32_t d_out,
                            void *ws, size_t ws_bytes, lora_stream_t stream) {
    if (T < 0 || d_in <= 0 || d_out <= 0 || (d_in % 16) || (d_out % 8)) return LORA_ERR_INVALID_ARGUMENT;
    if (T > 0 && (!xq || !x_scale || !wq || !w_scale || !y || !aligned16(xq) || !aligned16(wq) ||
                  !aligned16(w_scale) || !aligned16(y)))
        return LORA_ERR_INVALID_ARGUMENT;
    if (ws && !aligned16(ws)) return LORA_ERR_INVALID_ARGUMENT;
    if (T == 0) return LORA_OK;
    return launch_gemm_fp8(xq, x_scale, wq, w_scale, y, T, d_in, d_out, nullptr, nullptr, nullptr, 0, nullptr,
                           ws ? static_cast<float *>(ws) : nullptr, ws ? ws_bytes : 0, hs(stream));
}

size_t lora_workspace_bytes_fp8(int32_t T, int32_t n_slots, int32_t max_rank, int32_t d_in, int32_t d_out) {
    if (lora_workspace_bytes(T, n_slots, max_rank, d_out) == 0 || d_in <= 0 || (d_in % 16)) return 0;
    return make_ws_layout(T, n_slots, max_rank, d_out, d_in).total;
}

lora_status_t lora_linear_forward_fp8(const void *x, const uint8_t *wq, const float *w_scale, void *y,
                                      int32_t T, const lora_pool_t *pool, const int32_t *ids,
                                      lora_mode_t mode, uint32_t flags, void *ws, size_t ws_bytes,
                                      lora_stream_t stream) {
    if (!valid_pool(pool) || pool->dtype != LORA_BF16 || (pool->d_in % 16) || T < 0 || !valid_mode(mode) ||
        (flags & ~kForwardFlags))
        return LORA_ERR_INVALID_ARGUMENT;
    if (T > 0 && (!x || !wq || !w_scale || !y || !ids || !aligned16(x) || !aligned16(wq) ||
                  !aligned16(w_scale) || !aligned16(y)))
        return LORA_ERR_INVALID_ARGUMENT;
    ws_layout L;
    lora_status_t st = check_ws_fp8(ws, ws_bytes, T, pool->n_slots, pool->max_rank, pool->d_in, &L);
    if (st != LORA_OK) return st;
    if (T == 0) return LORA_OK;
    const hipStream_t s = hs(stream);
    const bool sgmv = use_sgmv(mode, T);
    if (sgmv && !(flags & LORA_FLAG_SEGMENTS_READY)) {
        st = launch_segments(ids, T, pool->n_slots, L, ws, s, short_len_for(mode, flags, pool->dtype));
        if (st != LORA_OK) return st;
    }
    uint8_t *xq = ws_ptr<uint8_t>(ws, L.xq);
    float *xs = ws_ptr<float>(ws, L.xs);
    float *v = ws_ptr<float>(ws, L.v);
    if (sgmv) {
        st = launch_quant_rows_fp8(x, T, pool->d_in, xq, xs, s);
        if (st != LORA_OK) return st;
        st = launch_shrink(x, T, pool, 1, ids, sgmv, v, L, ws, s);
    } else {
        // decode rows: quantize each row in the workgroup that shrinks it
        st = launch_quant_shrink_rows(x, T, pool, ids, v, xq, xs, ws_ptr<int32_t>(ws, L.header), s);
    }
    if (st != LORA_OK) return st;
    const int32_t *gperm = sgmv ? ws_ptr<int32_t>(ws, L.gperm) : nullptr;
    float *partial = ws_ptr<float>(ws, L.gemm_partial);
    const size_t partial_bytes = ws_bytes - L.gemm_partial;
    if (flags & LORA_FLAG_SEPARATE_EXPAND) {
        st = launch_gemm_fp8(xq, xs, wq, w_scale, y, T, pool->d_in, pool->d_out, nullptr, nullptr, nullptr, 0,
                             nullptr, partial, partial_bytes, s);
        if (st != LORA_OK) return st;
        return launch_expand(v, pool->max_rank, T, *pool, ids, sgmv, y, L, ws, s);
    }
    st = launch_gemm_fp8(xq, xs, wq, w_scale, y, T, pool->d_in, pool->d_out, pool, ids, v, pool->max_rank, gperm,
                         partial, partial_bytes, s, sgmv ? ws_ptr<int32_t>(ws, L.header) + kHdrNLong : nullptr);
    if (st == LORA_OK && sgmv) st = launch_expand_short(v, pool->max_rank, T, *pool, y, L, ws, s);
    return st;
}

lora_status_t lora_linear_forward_noalloc(const void *x, const void *W, void *y, int32_t T,
                                          const lora_pool_t *pool, const int32_t *ids, lora_mode_t mode,
                                          uint32_t flags, int32_t *err_out, lora_stream_t stream) {
    if (!valid_pool(pool) || T < 0 || !valid_mode(mode) || (flags & ~kForwardFlags))
        return LORA_ERR_INVALID_ARGUMENT;
    if (T > 0 && (!x || !W || !y || !ids || !aligned16(x) || !aligned16(W) || !aligned16(y)))
        return LORA_ERR_INVALID_ARGUMENT;
    if (T == 0) return LORA_OK;
    // the batch's workspace regions (the rest of the scratch holds GEMM
    // split-K partials, which only limits how far K is split)
    const ws_layout L = make_ws_layout(T, pool->n_slots, pool->max_rank, 0);
    if (L.total > kScratchBytes) return LORA_ERR_WORKSPACE_TOO_SMALL;
    void *ws = nullptr;
    lora_status_t st = scratch_of_current_device(&ws);
    if (st != LORA_OK) return st;
    const hipStream_t s = hs(stream);
    st = launch_ws_init(ws, s, true);                     // the error word starts at "none"
    if (st != LORA_OK) return st;
    st = lora_linear_forward(x, W, y, T, pool, ids, mode, flags, ws, kScratchBytes, stream);
    if (st != LORA_OK || !err_out) return st;
    hipLaunchKernelGGL(k_error_out, dim3(1), dim3(64), 0, s, ws_ptr<int32_t>(ws, L.header), err_out);
    return hip_status(hipGetLastError());
}

lora_status_t lora_get_device_error(void *ws, size_t ws_bytes, lora_stream_t stream,
                                    int32_t *first_bad_row) {
    if (!ws || !first_bad_row || ws_bytes < 256 || !aligned16(ws)) return LORA_ERR_INVALID_ARGUMENT;
    int32_t h = 0;
    const hipStream_t s = hs(stream);
    if (hipMemcpyAsync(&h, ws, sizeof h, hipMemcpyDeviceToHost, s) != hipSuccess) return LORA_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return LORA_ERR_HIP;
    *first_bad_row = (h == kErrNone) ? -1 : h;
    return launch_ws_init(ws, s, true);                   // the segments built stay valid
}

}  // extern "C"
