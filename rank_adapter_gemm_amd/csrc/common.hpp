// Shared device/host helpers of liblora (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lora.h"

namespace lora {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// bf16 <-> fp32.  bf16 is the upper half of an fp32; widening is exact, and
// narrowing rounds to nearest with ties to even (NaN stays a quiet NaN).
// Narrowing uses gfx950's v_cvt_pk_bf16_f32 (two values per instruction),
// which matches the integer round-to-nearest-even on every non-NaN fp32
// input (checked over 2^27 bit patterns on the GPU, subnormals and ties
// included).
// ---------------------------------------------------------------------------
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Two fp32 values to bf16, lo in bits 0..15, hi in bits 16..31.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) { return pack_bf16x2(f, f) & 0xffffu; }

// Element-type traits for the two storage types.
template <int DT> struct elem;
template <> struct elem<LORA_F32> {
    typedef float T;
    static constexpr int bytes = 4;
    __device__ static float load(const T *p, int64_t i) { return p[i]; }
    __device__ static void store(T *p, int64_t i, float v) { p[i] = v; }
};
template <> struct elem<LORA_BF16> {
    typedef uint16_t T;
    static constexpr int bytes = 2;
    __device__ static float load(const T *p, int64_t i) { return bf16_to_f32(p[i]); }
    __device__ static void store(T *p, int64_t i, float v) { p[i] = (uint16_t)f32_to_bf16_bits(v); }
};

// 16-byte vector of elements: 8 bf16 or 4 fp32, widened to fp32.
template <int DT> struct vec16;
template <> struct vec16<LORA_BF16> {
    static constexpr int n = 8;
    __device__ static void widen(const uint4 &q, float *f) {
        f[0] = bf16_lo(q.x); f[1] = bf16_hi(q.x);
        f[2] = bf16_lo(q.y); f[3] = bf16_hi(q.y);
        f[4] = bf16_lo(q.z); f[5] = bf16_hi(q.z);
        f[6] = bf16_lo(q.w); f[7] = bf16_hi(q.w);
    }
    __device__ static uint4 narrow(const float *f) {
        return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                          pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
    }
};
template <> struct vec16<LORA_F32> {
    static constexpr int n = 4;
    __device__ static void widen(const uint4 &q, float *f) {
        f[0] = __uint_as_float(q.x); f[1] = __uint_as_float(q.y);
        f[2] = __uint_as_float(q.z); f[3] = __uint_as_float(q.w);
    }
    __device__ static uint4 narrow(const float *f) {
        return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]),
                          __float_as_uint(f[2]), __float_as_uint(f[3]));
    }
};

__device__ __forceinline__ uint4 ldg16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }
__device__ __forceinline__ void stg16(void *p, const uint4 &v) { *reinterpret_cast<uint4 *>(p) = v; }

// A 16-byte zero vector in global memory: the source of the DMA loads of
// masked lanes (rows past T, k past K, columns past N), so those LDS slots
// hold zeros.
static __device__ __attribute__((aligned(16))) uint4 g_zero16[1];


// One 16-byte-per-lane DMA load from global memory straight into LDS: lane
// l's bytes land at lds_wave_base + 16 l (gfx950 global_load_lds_dwordx4).
// Issued as inline assembly so the compiler does not add its own
// conservative vmcnt waits before later LDS reads; the kernel orders these
// loads itself with explicit s_waitcnt vmcnt before each barrier.
__device__ __forceinline__ void dma16(const void *gptr, const void *lds_wave_base) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(
        static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds_wave_base)));
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(m0)
                 : "memory", "m0");
}

// First rank row of slot s in a pool's A^T rows (times d_in: its first
// element) and in its B octet rows (times d_out).  A padded pool (row0 null)
// gives every slot max_rank rows; a packed pool gives slot s the rows
// [row0[s], row0[s+1]).  Kernels read only rows below the slot's rank, and a
// slot's rank never exceeds its row count.
__device__ __forceinline__ int64_t slot_row0(const int32_t *row0, int32_t s, int32_t max_rank) {
    return row0 ? (int64_t)row0[s] : (int64_t)s * max_rank;
}

// Row visited at sorted position p: identity without perm; a perm entry
// outside [0, T) (segments not built for this batch) yields -1 = skip.
__device__ __forceinline__ int32_t perm_row(const int32_t *perm, int32_t p, int32_t T) {
    if (!perm) return p;
    const int32_t t = perm[p];
    return ((uint32_t)t < (uint32_t)T) ? t : -1;
}

// Record a bad adapter id (row index) in the workspace error word: the
// smallest such row wins.  Vector-memory integer atomic.
__device__ __forceinline__ void flag_bad_row(int32_t *err, int32_t row) {
    if (err) atomicMin(err, row);
}

// ---------------------------------------------------------------------------
// Workspace layout (host side).  Regions are 256-byte aligned.
// ---------------------------------------------------------------------------
constexpr int32_t kSegTile = 1024;     // rows per segment-builder tile
// Mixed batches (AUTO mode): adapter segments shorter than this many rows
// take the per-row (BGMV) shrink and expand, longer ones the grouped (SGMV)
// shrink and the expand fused into the base GEMM.
constexpr int32_t kShortSegDefault = 16;
// Workspace header words (int32): the error word, the number of rows whose
// low-rank term is fused into the GEMM (those before the short-segment rows
// in the GEMM's row order), the short-segment threshold of the build and the
// number of short segments.
constexpr int32_t kHdrErr = 0, kHdrNLong = 1, kHdrShortLen = 2, kHdrNShort = 3;
constexpr int32_t kShrinkRows = 32;    // rows of one segment per grouped-shrink work block
constexpr int32_t kMaxKSplit = 16;     // shrink k-split factor bound
constexpr int32_t kMaxSlices = 4;      // pools sharing one shrink (projections that share x)
constexpr int32_t kMaxCachePools = 8;  // pools (projections) one residency cache keeps in step
constexpr int32_t kMaxSliceRanks = 128; // their summed max_rank
constexpr int32_t kMaxSlots = 16000;   // slots per pool (LDS histogram bound, < 64 KiB)
constexpr int32_t kErrNone = 0x7fffffff;
constexpr int32_t kMaxGemmSplit = 16;   // split-K GEMM: most K ranges per tile
// Split-K GEMM partials are fp32 tiles, [tile][split][BM][BN]; one split
// launch has at most about two rounds of 256 workgroups of <= 256 x 256
// tiles, so this bounds the scratch for any shape.
constexpr size_t kGemmPartialCap = size_t(128) << 20;

struct ws_layout {
    size_t header;      // int32[64]: [0] error word (first bad row)
    size_t offsets;     // int32[n_slots + 2]
    size_t seg_id;      // int32[n_slots]
    size_t seg_start;   // int32[n_slots + 1]
    size_t n_seg;       // int32[1]
    size_t blk_start;   // int32[n_slots + 2]: first shrink work block of each segment
    size_t blk_seg;     // int32[ceil(T / kShrinkRows) + n_slots]: segment of each work block
    size_t perm;        // int32[T]
    size_t gperm;       // int32[T]: the GEMM's row order (long-segment rows, then short-segment rows)
    size_t gbase;       // int32[n_slots + 2]: first GEMM position of each key's rows
    size_t srec;        // int4[n_slots]: short segments {key, first GEMM position, rows, 0}, ascending keys;
                        // key 0 from entry n_short to min(n_slots, T)
    size_t tile_hist;   // int32[(n_slots + 1) * n_tiles]
    size_t v;           // fp32[T * max_rank]
    size_t partial;     // fp32[kMaxKSplit * T * max_rank]
    size_t xq;          // FP8 base only: E4M3 codes of x, uint8[T * d_in]
    size_t xs;          // FP8 base only: row scales, fp32[T]
    size_t gemm_partial;  // split-K GEMM partials (fp32 tiles), may be empty
    size_t total;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// q8_d_in > 0 adds the regions of the FP8-base forward (quantized x rows).
inline ws_layout make_ws_layout(int32_t T, int32_t n_slots, int32_t max_rank, int32_t d_out,
                                int32_t q8_d_in = 0) {
    ws_layout L;
    size_t o = 0;
    const size_t t = (size_t)(T > 0 ? T : 1);
    const size_t n_tiles = (t + kSegTile - 1) / kSegTile;
    L.header = o;    o = align256(o + 64 * 4);
    L.offsets = o;   o = align256(o + 4 * (size_t)(n_slots + 2));
    L.seg_id = o;    o = align256(o + 4 * (size_t)(n_slots + 1));
    L.seg_start = o; o = align256(o + 4 * (size_t)(n_slots + 2));
    L.n_seg = o;     o = align256(o + 4);
    L.blk_start = o; o = align256(o + 4 * (size_t)(n_slots + 2));
    L.blk_seg = o;   o = align256(o + 4 * ((t + kShrinkRows - 1) / kShrinkRows + (size_t)n_slots + 1));
    L.perm = o;      o = align256(o + 4 * t);
    L.gperm = o;     o = align256(o + 4 * t);
    L.gbase = o;     o = align256(o + 4 * (size_t)(n_slots + 2));
    L.srec = o;      o = align256(o + 16 * (size_t)n_slots);
    L.tile_hist = o; o = align256(o + 4 * (size_t)(n_slots + 1) * n_tiles);
    L.v = o;         o = align256(o + 4 * t * (size_t)max_rank);
    L.partial = o;   o = align256(o + 4 * (size_t)kMaxKSplit * t * (size_t)max_rank);
    const size_t tq = q8_d_in > 0 ? t : 0;
    L.xq = o;        o = align256(o + tq * (size_t)(q8_d_in > 0 ? q8_d_in : 0));
    L.xs = o;        o = align256(o + 4 * tq);
    L.gemm_partial = o;
    if (d_out > 0 && T > 0) {
        const size_t tp = (t + 255) / 256 * 256, np = ((size_t)d_out + 255) / 256 * 256;
        const size_t need = 4 * (size_t)kMaxGemmSplit * tp * np;
        o = align256(o + (need < kGemmPartialCap ? need : kGemmPartialCap));
    }
    L.total = o;
    return L;
}

template <typename T> inline T *ws_ptr(void *ws, size_t off) {
    return reinterpret_cast<T *>(reinterpret_cast<char *>(ws) + off);
}

inline lora_status_t hip_status(hipError_t e) { return e == hipSuccess ? LORA_OK : LORA_ERR_HIP; }

// Launchers (one per kernel family), implemented in the matching .hip file.
lora_status_t launch_pool_fill(void *a, size_t a_bytes, void *b, size_t b_bytes, float *scale,
                               int32_t *rank, int32_t n_slots, hipStream_t s);
lora_status_t launch_pool_upload(const lora_pool_t &p, int32_t slot, const void *A, int32_t lda,
                                 const void *B, int32_t ldb, int32_t r, float alpha, hipStream_t s);
lora_status_t launch_pool_clear(const lora_pool_t &p, int32_t slot, hipStream_t s);
lora_status_t launch_pool_meta(const lora_pool_t &p, int32_t slot, float scale, int32_t rank, hipStream_t s);
// Scale and rank of up to kMetaBatch slots, written in every pool by one launch.
constexpr int32_t kMetaBatch = 64;
struct meta_batch {
    float *scale[kMaxCachePools];
    int32_t *rank[kMaxCachePools];
    int32_t n_pools, n;
    int32_t slot[kMetaBatch];
    float s[kMetaBatch];
    int32_t r[kMetaBatch];
};
lora_status_t launch_pool_meta_batch(const meta_batch &m, hipStream_t s);
// Up to kCopyBatch copies of whole slot buffers in one launch: src[i] is a
// device-visible address (page-locked host memory mapped into the GPU's
// address space), dst[i] device memory, bytes[i] a multiple of 16.
constexpr int32_t kCopyBatch = 32;
constexpr uint32_t kCopyChunk = 64u << 10;     // bytes per workgroup
struct copy_batch {
    const void *src[kCopyBatch];
    void *dst[kCopyBatch];
    uint32_t bytes[kCopyBatch];
    int32_t n;
    uint32_t max_bytes;
};
lora_status_t launch_copy_batch(const copy_batch &c, hipStream_t s);
lora_status_t launch_ws_init(void *ws, hipStream_t s, bool err_only = false);
// Segments of ids (short_len: segments of fewer rows take the per-row path;
// 1 = none do) into the workspace, with the GEMM's row order.
lora_status_t launch_segments(const int32_t *ids, int32_t T, int32_t n_slots, const ws_layout &L,
                              void *ws, hipStream_t s, int32_t short_len = 1);
// Separate expand of the short segments' rows (the GEMM left their term out),
// one work item per short segment and column chunk.
lora_status_t launch_expand_tiles(const float *v, int32_t v_stride, int32_t T, const lora_pool_t &p,
                                  const int32_t *ids, const int32_t *gperm, const int32_t *n_fused, void *y,
                                  hipStream_t s);
lora_status_t launch_expand_short(const float *v, int32_t v_stride, int32_t T, const lora_pool_t &p, void *y,
                                  const ws_layout &L, void *ws, hipStream_t s);
// Shrink for n_slices pools that share x, ids, n_slots, d_in, max_rank and
// dtype: v[t][s * max_rank + j] for slice s (row stride n_slices * max_rank).
lora_status_t launch_shrink(const void *x, int32_t T, const lora_pool_t *pools, int32_t n_slices,
                            const int32_t *ids, bool sgmv, float *v, const ws_layout &L, void *ws,
                            hipStream_t s);
lora_status_t launch_expand(const float *v, int32_t v_stride, int32_t T, const lora_pool_t &p,
                            const int32_t *ids, bool sgmv, void *y, const ws_layout &L, void *ws,
                            hipStream_t s);
// y = x W (+ s v B when pool != nullptr); rows in perm order when perm != nullptr.
bool gemm_fused_shrink_ok(int32_t T, int32_t d_in, int32_t d_out, int32_t max_rank,
                          size_t partial_bytes);
lora_status_t launch_gemm_fused_shrink(const void *x, const void *W, void *y, int32_t T,
                                       const lora_pool_t *pool, const int32_t *ids, float *vpart,
                                       int32_t *err, float *partial, size_t partial_bytes,
                                       hipStream_t s);
bool gemm_grouping_pays(int32_t T, int32_t K, const int32_t *Ns, int32_t n, size_t partial_bytes);
// n_fused (device, may be null): rows at GEMM positions >= *n_fused get no
// low-rank term here (the short-segment rows; their expand is separate).
lora_status_t launch_gemm_grouped(const void *x, const void *const *W, void *const *y, int32_t T,
                                  const lora_pool_t *pools, int32_t n, const int32_t *ids, const float *v,
                                  const int32_t *v_off, int32_t v_stride, const int32_t *perm, float *partial,
                                  size_t partial_bytes, hipStream_t s, const int32_t *n_fused = nullptr);
lora_status_t launch_gemm(const void *x, const void *W, void *y, int32_t T, int32_t d_in,
                          int32_t d_out, int32_t dtype, const lora_pool_t *pool,
                          const int32_t *ids, const float *v, int32_t v_stride,
                          const int32_t *perm, float *partial, size_t partial_bytes, hipStream_t s,
                          const int32_t *n_fused = nullptr);
// FP8 base (E4M3 codes, fp32 scales): per-row and per-column quantizers and
// y = s_x s_w (xq wq^T) (+ s v B when pool != nullptr), bf16 y.
lora_status_t launch_quant_rows_fp8(const void *x, int32_t T, int32_t K, uint8_t *xq, float *xs, hipStream_t s);
// The BGMV shrink of bf16 rows and their E4M3 quantization (codes xq, scales xs) in one launch.
lora_status_t launch_quant_shrink_rows(const void *x, int32_t T, const lora_pool_t *pool, const int32_t *ids,
                                       float *v, uint8_t *xq, float *xs, int32_t *err, hipStream_t s);
lora_status_t launch_quant_cols_fp8(const void *W, int32_t K, int32_t N, uint8_t *wq, float *wsc, hipStream_t s);
lora_status_t launch_gemm_fp8(const uint8_t *xq, const float *xs, const uint8_t *wq, const float *wsc, void *y,
                              int32_t T, int32_t d_in, int32_t d_out, const lora_pool_t *pool,
                              const int32_t *ids, const float *v, int32_t v_stride, const int32_t *perm,
                              float *partial, size_t partial_bytes, hipStream_t s, const int32_t *n_fused = nullptr);

}  // namespace lora
