// a5 -- expand as its own pass: y[t,:] += s_a * (v[t, 0:r] B_a).
//
// "Serving multiple LoRAs: segmented matrix multiplies and adapter
// scheduling", section "Not merging the weights, computing in batches": the
// second of the two low-rank products maps the rank-r vector back to d_out
// values, which are added to the base product's row; the scale multiplies
// that product, as in lora_mixed_batch ("LoRAX, in depth", section
// "Computing a batch that mixes adapters").
//
// One workgroup per (token row, 2048-column chunk); each lane owns 8
// consecutive output columns.  B is stored in rank octets [r/8][d_out][8], so
// for one octet a lane reads its 8 columns x 8 ranks as 8 contiguous 16-byte
// vectors and neighbouring lanes read neighbouring vectors.  Only the first
// ceil(r/8) octets are read.  The row's v values are staged in LDS.  y is read,
// updated in fp32 and written back with one rounding.  In SGMV mode the rows
// are visited in segment order (through perm), so consecutive workgroups
// share the same B in the caches.
#include "common.hpp"

namespace lora {

// Row at position p (through perm), columns [2048 blockIdx.y, +2048), by one
// 256-thread workgroup (every thread calls it with the same p).
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
    const int n0 = (blockIdx.y * 256 + threadIdx.x) * 8;
    if (n0 >= d_out) return;
    const int G = (r + 7) >> 3;
    const E *bs = b + slot_row0(row0, id, max_rank) * d_out;
    float acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = 0.0f;
    for (int g = 0; g < G; ++g) {
        float vv[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) vv[q] = s_v[g * 8 + q];
        const E *bg = bs + ((size_t)g * d_out + n0) * 8;   // 8 columns x 8 ranks
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            float bf[8];
            if (EB == 2) {
                vec16<LORA_BF16>::widen(ldg16(bg + c * 8), bf);
            } else {
                vec16<LORA_F32>::widen(ldg16(bg + c * 8), bf);
                vec16<LORA_F32>::widen(ldg16(bg + c * 8 + 4), bf + 4);
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[c] = fmaf(vv[q], bf[q], acc[c]);
        }
    }
    E *yt = y + (size_t)t * d_out + n0;
    float yf[8];
    if (EB == 2) {
        vec16<LORA_BF16>::widen(ldg16(yt), yf);
    } else {
        vec16<LORA_F32>::widen(ldg16(yt), yf);
        vec16<LORA_F32>::widen(ldg16(yt + 4), yf + 4);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) yf[c] = fmaf(s, acc[c], yf[c]);
    if (EB == 2) {
        stg16(yt, vec16<LORA_BF16>::narrow(yf));
    } else {
        stg16(yt, vec16<LORA_F32>::narrow(yf));
        stg16(yt + 4, vec16<LORA_F32>::narrow(yf + 4));
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

// The per-row (BGMV) expand of a mixed batch's short segments, whose rows the
// GEMM visits last and leaves without their low-rank term.  Work item =
// (short segment, 2048-column chunk): a segment's rows (fewer than the
// build's threshold, consecutive in the GEMM order) share one adapter, so
// its B columns are read once per item and applied to up to kXRows rows at a
// time; each thread owns 8 consecutive columns, loads the rank octets of B
// one octet ahead, and sums ranks in octet order before scaling, as the
// separate expand does.  y is read, updated in fp32 and written back.
constexpr int kXRows = 4;

__global__ void __launch_bounds__(256) k_expand_short(const float *__restrict__ v, int32_t v_stride, int32_t T,
                                                      int32_t d_out, const uint16_t *__restrict__ b,
                                                      const float *__restrict__ scale,
                                                      const int32_t *__restrict__ rank,
                                                      const int32_t *__restrict__ row0, int32_t max_rank,
                                                      const int32_t *__restrict__ gperm,
                                                      const int32_t *__restrict__ offsets,
                                                      const int32_t *__restrict__ gbase,
                                                      const int32_t *__restrict__ skey,
                                                      const int32_t *__restrict__ header,
                                                      uint16_t *__restrict__ y) {
    __shared__ float s_v[kXRows][128];
    const int n_short = header[kHdrNShort];
    const int n0 = (blockIdx.y * 256 + threadIdx.x) * 8;
    for (int i = blockIdx.x; i < n_short; i += gridDim.x) {
        const int key = skey[i], a = key - 1;
        const int p0 = gbase[key], len = offsets[key + 1] - offsets[key];
        const int r = min(rank[a], max_rank);
        const float sc = scale[a];
        if (r <= 0) continue;                             // uniform: an empty slot (flagged by the shrink)
        const uint16_t *bs = b + slot_row0(row0, a, max_rank) * d_out + (int64_t)n0 * 8;
        const int G = (r + 7) >> 3;
        for (int q0 = 0; q0 < len; q0 += kXRows) {
            const int nq = min(kXRows, len - q0);
            __syncthreads();                              // s_v is free
            for (int e = threadIdx.x; e < kXRows * max_rank; e += 256) {
                const int qq = e / max_rank, j = e % max_rank;
                float val = 0.0f;
                if (qq < nq) {
                    const int32_t t = perm_row(gperm, p0 + q0 + qq, T);
                    if (t >= 0) val = v[(size_t)t * v_stride + j];
                }
                s_v[qq][j] = val;
            }
            __syncthreads();
            if (n0 >= d_out) continue;
            float acc[kXRows][8];
#pragma unroll
            for (int qq = 0; qq < kXRows; ++qq)
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[qq][c] = 0.0f;
            uint4 bc[8], bn[8];
#pragma unroll
            for (int c = 0; c < 8; ++c) bc[c] = ldg16(bs + c * 8);
            for (int g = 0; g < G; ++g) {
                if (g + 1 < G) {
#pragma unroll
                    for (int c = 0; c < 8; ++c) bn[c] = ldg16(bs + ((int64_t)(g + 1) * d_out) * 8 + c * 8);
                }
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    float bf[8];
                    vec16<LORA_BF16>::widen(bc[c], bf);
#pragma unroll
                    for (int qq = 0; qq < kXRows; ++qq) {
                        float s_ = acc[qq][c];
#pragma unroll
                        for (int q = 0; q < 8; ++q) s_ = fmaf(s_v[qq][8 * g + q], bf[q], s_);
                        acc[qq][c] = s_;
                    }
                }
#pragma unroll
                for (int c = 0; c < 8; ++c) bc[c] = bn[c];
            }
#pragma unroll
            for (int qq = 0; qq < kXRows; ++qq) {
                if (qq >= nq) break;
                const int32_t t = perm_row(gperm, p0 + q0 + qq, T);
                if (t < 0) continue;
                uint16_t *yt = y + (size_t)t * d_out + n0;
                float yf[8];
                vec16<LORA_BF16>::widen(ldg16(yt), yf);
#pragma unroll
                for (int c = 0; c < 8; ++c) yf[c] = fmaf(sc, acc[qq][c], yf[c]);
                stg16(yt, vec16<LORA_BF16>::narrow(yf));
            }
        }
    }
}

lora_status_t launch_expand_short(const float *v, int32_t v_stride, int32_t T, const lora_pool_t &p, void *y,
                                  const ws_layout &L, void *ws, hipStream_t s) {
    if (p.dtype != LORA_BF16) return LORA_OK;
    const int chunks = (p.d_out + 2047) / 2048;
    int segs = 4096 / chunks;                             // about 4096 workgroups in flight
    if (segs < 64) segs = 64;
    if (segs > p.n_slots) segs = p.n_slots;
    if (segs > T) segs = T;
    hipLaunchKernelGGL(k_expand_short, dim3(segs, chunks), dim3(256), 0, s, v, v_stride, T, p.d_out,
                       (const uint16_t *)p.b, p.scale, p.rank, p.row0, p.max_rank, ws_ptr<int32_t>(ws, L.gperm),
                       ws_ptr<int32_t>(ws, L.offsets), ws_ptr<int32_t>(ws, L.gbase), ws_ptr<int32_t>(ws, L.skey),
                       ws_ptr<int32_t>(ws, L.header), (uint16_t *)y);
    return hip_status(hipGetLastError());
}

lora_status_t launch_expand(const float *v, int32_t v_stride, int32_t T, const lora_pool_t &p,
                            const int32_t *ids, bool sgmv, void *y, const ws_layout &L, void *ws,
                            hipStream_t s) {
    const int32_t *perm = sgmv ? ws_ptr<int32_t>(ws, L.perm) : nullptr;
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
