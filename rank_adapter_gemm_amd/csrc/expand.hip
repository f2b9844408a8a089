// a5 -- expand as its own pass: y[t,:] += s_a * (v[t, 0:r] B_a).
//
// "Serving multiple LoRAs: segmented matrix multiplies and adapter
// scheduling", section "Not merging the weights, computing in batches": the
// second of the two low-rank products maps the rank-r vector back to d_out
// values, which are added to the base product's row; the scale multiplies
// that product, as in lora_mixed_batch ("LoRAX, in depth", section
// "Computing a batch that mixes adapters").
//
// Three forms, all reading B in rank octets [r/8][d_out][8] (the 8 ranks of
// one output column are 16 contiguous bytes) and only the first ceil(r/8)
// octets of a slot, summing ranks in octet order, and adding to y with one
// rounding:
//  * k_expand_rows (BGMV, and fp32 pools): one workgroup per (token row,
//    2048 columns), rows in their own order;
//  * expand_adapter_rows (rows that share one adapter), used by
//    k_expand_short for the short segments of a mixed batch;
//  * in SGMV mode the long segments' rows go through the LoRA GEMM kernel
//    with no K steps (launch_expand_tiles in gemm.hip), on the matrix cores.
#include "common.hpp"

namespace lora {

// Row at position p (through perm), columns [2048 blockIdx.y, +2048), by one
// 256-thread workgroup (every thread calls it with the same p).  Lane l of
// wave w owns the columns 512 w + 64 c + l (c = 0..7) of the chunk: each load
// instruction of a wave reads the rank octets of 64 consecutive columns.
template <int DT>
__device__ __forceinline__ void expand_row(const float *__restrict__ v, int32_t T, int32_t d_out,
                                           const typename elem<DT>::T *__restrict__ b,
                                           const float *__restrict__ scale, const int32_t *__restrict__ rank,
                                           const int32_t *__restrict__ row0, int32_t n_slots, int32_t max_rank,
                                           int32_t v_stride, const int32_t *__restrict__ ids,
                                           const int32_t *__restrict__ perm, typename elem<DT>::T *__restrict__ y,
                                           int p) {
    typedef typename elem<DT>::T E;
    constexpr int EB = elem<DT>::bytes;
    __shared__ float s_v[128];
    const int t = perm_row(perm, p, T);
    if (t < 0) return;
    const int32_t id = ids[t];
    if (id < 0 || id >= n_slots) return;
    const int32_t r = min(rank[id], max_rank);
    if (r <= 0) return;
    const float s = scale[id];
    for (int j = threadIdx.x; j < max_rank; j += 256) s_v[j] = v[(size_t)t * v_stride + j];
    __syncthreads();
    const int nb = blockIdx.y * 2048 + (threadIdx.x >> 6) * 512 + (threadIdx.x & 63);
    if (nb >= d_out) return;
    const int G = (r + 7) >> 3;
    const E *bs = b + slot_row0(row0, id, max_rank) * d_out;
    float acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = 0.0f;
    for (int g = 0; g < G; ++g) {
        float vv[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) vv[q] = s_v[g * 8 + q];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int n = nb + 64 * c;
            if (n >= d_out) break;
            const E *bg = bs + ((size_t)g * d_out + n) * 8;   // 8 ranks of column n
            float bf[8];
            if (EB == 2) {
                vec16<LORA_BF16>::widen(ldg16(bg), bf);
            } else {
                vec16<LORA_F32>::widen(ldg16(bg), bf);
                vec16<LORA_F32>::widen(ldg16(bg + 4), bf + 4);
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[c] = fmaf(vv[q], bf[q], acc[c]);
        }
    }
    E *yt = y + (size_t)t * d_out;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const int n = nb + 64 * c;
        if (n >= d_out) break;
        elem<DT>::store(yt, n, fmaf(s, acc[c], elem<DT>::load(yt, n)));
    }
}

template <int DT>
__global__ void __launch_bounds__(256) k_expand_rows(const float *__restrict__ v, int32_t T,
                                                     int32_t d_out,
                                                     const typename elem<DT>::T *__restrict__ b,
                                                     const float *__restrict__ scale,
                                                     const int32_t *__restrict__ rank,
                                                     const int32_t *__restrict__ row0,
                                                     int32_t n_slots, int32_t max_rank,
                                                     int32_t v_stride,
                                                     const int32_t *__restrict__ ids,
                                                     const int32_t *__restrict__ perm,
                                                     typename elem<DT>::T *__restrict__ y) {
    expand_row<DT>(v, T, d_out, b, scale, rank, row0, n_slots, max_rank, v_stride, ids, perm, y, blockIdx.x);
}

// Expand of rows that share one adapter: y[t] += s_a (v[t, 0:r] B_a) for
// the rows t = perm[p0 .. p0 + len), columns [512 blockIdx.x, +512) of y, by
// one 256-thread workgroup (every thread calls it with the same arguments).
// Each thread loads all rank octets of B for its two adjacent columns into
// registers once (ranks up to 64; larger ranks stream eight octets at a
// time), before anything that waits on the rows; one load instruction of a
// wave reads the octets of 128 consecutive columns.  Up to kXStage rows are
// staged at once (indices and v in LDS), then computed kXGroup rows at a
// time with the next group's y values already loading.  Ranks are summed in
// octet order before scaling, as the per-row expand does; y is updated in
// fp32 and written back with one rounding.  Measured on the 70B-shaped
// batch's short segments: 13% (d_out 28672) and 40% (d_out 8192) faster
// than 2048-column items that streamed B one octet ahead; staging 16 rows
// at once instead of 4 took the prefill's separate expand from 1243 to
// 1071 us.
constexpr int kXStage = 16;                    // rows whose indices and v are staged at once
constexpr int kXGroup = 8;                     // rows per compute group (y prefetched one group ahead)
constexpr int kCpt = 2;                        // adjacent columns per thread
constexpr int kXCols = 256 * kCpt;             // columns per work item

__device__ __forceinline__ void expand_adapter_rows(int a, int p0, int len, const int32_t *__restrict__ perm,
                                                    const float *__restrict__ v, int32_t v_stride, int32_t T,
                                                    int32_t d_out, const uint16_t *__restrict__ b,
                                                    const float *__restrict__ scale,
                                                    const int32_t *__restrict__ rank,
                                                    const int32_t *__restrict__ row0, int32_t max_rank,
                                                    uint16_t *__restrict__ y, float (*s_v)[128], int32_t *s_t) {
    const int n = blockIdx.x * kXCols + threadIdx.x * kCpt;
    const bool col_ok = n < d_out;                        // d_out % 8 == 0: both columns or neither
    const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
    const int r = min(rank[a], max_rank);
    const float sc = scale[a];
    if (r <= 0) return;                                   // uniform: an empty slot (flagged by the shrink)
    const uint16_t *bs = b + slot_row0(row0, a, max_rank) * d_out + (int64_t)n * 8;
    const int G = (r + 7) >> 3;
    uint4 bq[8][kCpt];
#pragma unroll
    for (int g = 0; g < 8; ++g)
#pragma unroll
        for (int c = 0; c < kCpt; ++c)
            bq[g][c] = (g < G && col_ok) ? ldg16(bs + (int64_t)g * d_out * 8 + c * 8) : zero;
    auto yload = [&](int qb, int nq, uint32_t (&yv)[kXGroup]) {
#pragma unroll
        for (int q = 0; q < kXGroup; ++q) {
            const int32_t t = qb + q < nq ? s_t[qb + q] : -1;
            yv[q] = (t >= 0 && col_ok) ? *reinterpret_cast<const uint32_t *>(y + (size_t)t * d_out + n) : 0u;
        }
    };
    for (int q0 = 0; q0 < len; q0 += kXStage) {
        const int nq = min(kXStage, len - q0);
        __syncthreads();                                  // s_v, s_t are free
        if (threadIdx.x < kXStage)
            s_t[threadIdx.x] = (int)threadIdx.x < nq ? perm_row(perm, p0 + q0 + threadIdx.x, T) : -1;
        __syncthreads();
        for (int e = threadIdx.x; e < nq * max_rank; e += 256) {
            const int qq = e / max_rank, j = e % max_rank;
            const int32_t t = s_t[qq];
            s_v[qq][j] = t >= 0 ? v[(size_t)t * v_stride + j] : 0.0f;
        }
        uint32_t ya[kXGroup], yb[kXGroup];
        yload(0, nq, ya);
        __syncthreads();
        for (int qb = 0; qb < nq; qb += kXGroup) {
            if (qb + kXGroup < nq) yload(qb + kXGroup, nq, yb);   // next group's y, under this group's FMAs
#pragma unroll
            for (int q = 0; q < kXGroup; ++q) {
                if (qb + q >= nq) break;
                float acc[kCpt];
#pragma unroll
                for (int c = 0; c < kCpt; ++c) acc[c] = 0.0f;
                // ranks up to 64 stay in bq; larger ranks stream eight octets at a time
                for (int g0 = 0; g0 < G; g0 += 8) {
                    if (G > 8) {
#pragma unroll
                        for (int g = 0; g < 8; ++g)
#pragma unroll
                            for (int c = 0; c < kCpt; ++c)
                                bq[g][c] = (g0 + g < G && col_ok)
                                               ? ldg16(bs + (int64_t)(g0 + g) * d_out * 8 + c * 8) : zero;
                    }
#pragma unroll
                    for (int g = 0; g < 8; ++g) {
                        if (g0 + g >= G) break;
                        const float4 v0 = *reinterpret_cast<const float4 *>(&s_v[qb + q][8 * (g0 + g)]);
                        const float4 v1 = *reinterpret_cast<const float4 *>(&s_v[qb + q][8 * (g0 + g) + 4]);
#pragma unroll
                        for (int c = 0; c < kCpt; ++c) {
                            float bf[8];
                            vec16<LORA_BF16>::widen(bq[g][c], bf);
                            float s_ = acc[c];
                            s_ = fmaf(v0.x, bf[0], s_); s_ = fmaf(v0.y, bf[1], s_);
                            s_ = fmaf(v0.z, bf[2], s_); s_ = fmaf(v0.w, bf[3], s_);
                            s_ = fmaf(v1.x, bf[4], s_); s_ = fmaf(v1.y, bf[5], s_);
                            s_ = fmaf(v1.z, bf[6], s_); s_ = fmaf(v1.w, bf[7], s_);
                            acc[c] = s_;
                        }
                    }
                }
                const int32_t t = s_t[qb + q];
                if (t >= 0 && col_ok) {
                    const float y0 = fmaf(sc, acc[0], bf16_lo(ya[q])), y1 = fmaf(sc, acc[1], bf16_hi(ya[q]));
                    *reinterpret_cast<uint32_t *>(y + (size_t)t * d_out + n) = pack_bf16x2(y0, y1);
                }
            }
#pragma unroll
            for (int q = 0; q < kXGroup; ++q) ya[q] = yb[q];
        }
    }
}

// The per-row (BGMV) expand of a mixed batch's short segments, whose rows the
// GEMM visits last and leaves without their low-rank term: one work item per
// (short segment, column chunk); a short segment's rows are consecutive in
// the GEMM order.  Item i reads the segment build's record i ({key, first
// GEMM position, rows}; key 0 past the last short segment), so its chain to
// the B loads is one record and the slot's rank.  Every field taken from the
// record is checked against the tables' sizes and T, so tables that
// something else overwrote give wrong rows, never an access outside the
// buffers.  The column chunks of one record are neighbours in the dispatch
// order (grid x), so the workgroups in flight together stream one
// adapter's B octet rows end to end; with the records neighbours instead
// (every workgroup at the same column offset of a different adapter) the
// 70B-shaped batch's gate expand took 124 us against 101.
__global__ void __launch_bounds__(256) k_expand_short(const float *__restrict__ v, int32_t v_stride, int32_t T,
                                                      int32_t d_out, const uint16_t *__restrict__ b,
                                                      const float *__restrict__ scale,
                                                      const int32_t *__restrict__ rank,
                                                      const int32_t *__restrict__ row0, int32_t n_slots,
                                                      int32_t max_rank, const int32_t *__restrict__ gperm,
                                                      const int4 *__restrict__ srec, uint16_t *__restrict__ y) {
    __shared__ __attribute__((aligned(16))) float s_v[kXStage][128];
    __shared__ int32_t s_t[kXStage];
    const int n_rec = min(n_slots, T);                      // records written by the segment build
    for (int i = blockIdx.y; i < n_rec; i += gridDim.y) {
        const int4 rec = srec[i];                           // {key, first GEMM position, rows, 0}
        if (rec.x == 0) break;                              // no short segment from here on
        if (rec.x < 1 || rec.x > n_slots || rec.y < 0 || rec.z < 1 || (int64_t)rec.y + rec.z > T) continue;
        expand_adapter_rows(rec.x - 1, rec.y, rec.z, gperm, v, v_stride, T, d_out, b, scale, rank, row0, max_rank, y,
                            s_v, s_t);
    }
}

lora_status_t launch_expand_short(const float *v, int32_t v_stride, int32_t T, const lora_pool_t &p, void *y,
                                  const ws_layout &L, void *ws, hipStream_t s) {
    if (p.dtype != LORA_BF16) return LORA_OK;
    const int chunks = (p.d_out + kXCols - 1) / kXCols;
    int segs = p.n_slots;                                 // one item per short segment and chunk
    if (segs > T) segs = T;
    if (segs > 65535) segs = 65535;                       // grid y bound; the kernel strides over the rest
    hipLaunchKernelGGL(k_expand_short, dim3(chunks, segs), dim3(256), 0, s, v, v_stride, T, p.d_out,
                       (const uint16_t *)p.b, p.scale, p.rank, p.row0, p.n_slots, p.max_rank,
                       ws_ptr<int32_t>(ws, L.gperm), ws_ptr<int4>(ws, L.srec), (uint16_t *)y);
    return hip_status(hipGetLastError());
}

lora_status_t launch_expand(const float *v, int32_t v_stride, int32_t T, const lora_pool_t &p,
                            const int32_t *ids, bool sgmv, void *y, const ws_layout &L, void *ws,
                            hipStream_t s) {
    const int32_t *perm = sgmv ? ws_ptr<int32_t>(ws, L.perm) : nullptr;
    if (sgmv && p.dtype == LORA_BF16 && T > 0) {
        // as in the fused forward: rows in the GEMM order, long segments on
        // the matrix cores, the short ones per row
        lora_status_t st = launch_expand_tiles(v, v_stride, T, p, ids, ws_ptr<int32_t>(ws, L.gperm),
                                               ws_ptr<int32_t>(ws, L.header) + kHdrNLong, y, s);
        if (st == LORA_OK) st = launch_expand_short(v, v_stride, T, p, y, L, ws, s);
        return st;
    }
    const dim3 grid(T, (p.d_out + 2047) / 2048);
    if (p.dtype == LORA_F32)
        hipLaunchKernelGGL(k_expand_rows<LORA_F32>, grid, dim3(256), 0, s, v, T, p.d_out,
                           (const float *)p.b, p.scale, p.rank, p.row0, p.n_slots, p.max_rank, v_stride, ids, perm,
                           (float *)y);
    else
        hipLaunchKernelGGL(k_expand_rows<LORA_BF16>, grid, dim3(256), 0, s, v, T, p.d_out,
                           (const uint16_t *)p.b, p.scale, p.rank, p.row0, p.n_slots, p.max_rank, v_stride, ids,
                           perm, (uint16_t *)y);
    return hip_status(hipGetLastError());
}

}  // namespace lora
