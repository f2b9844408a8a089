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
    typedef typename elem<DT>::T E;
    constexpr int EB = elem<DT>::bytes;
    __shared__ float s_v[128];
    const int p = blockIdx.x;
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
