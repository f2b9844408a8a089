// a4 -- shrink: v[t, 0:r] = x[t,:] A_a  (fp32 result of rank width).
//
// "Serving multiple LoRAs: segmented matrix multiplies and adapter
// scheduling", section "Not merging the weights, computing in batches"
// (first shrink x -> xA down to r dimensions), and "Serving LoRA adapters:
// from the model name to the wrapped layer", Step 4 (shrink into an fp32
// buffer of rank width).  The BGMV form gathers each token's own A; the SGMV
// form walks adapter-contiguous segments so one read of A serves a segment.
//
// Two kernels:
//  * k_shrink_rows  (BGMV): one workgroup per token row; x[t] is read once
//    with 16-byte coalesced loads, the slot's A^T rows (only the first r)
//    are gathered, each lane keeps per-rank partial sums, which are reduced
//    across the wavefront with a transposing butterfly of cross-lane swaps
//    and then across the 4 wavefronts through LDS.  fp32 or bf16 inputs.
//  * k_shrink_sgmv  (SGMV, bf16): rows in segment order (through perm), 16
//    rows per MFMA tile; for each adapter present in the tile, one bf16 MFMA
//    K-loop with the tile's other rows masked to zero, so all adapters of the
//    tile accumulate into one fp32 result.  The K dimension is split over the
//    4 wavefronts (LDS reduction) and optionally over workgroups (partials,
//    then a fixed-order reduction: deterministic).
#include "common.hpp"

namespace lora {

// ---------------------------------------------------------------------------
// Transposing butterfly: on entry each lane holds N partial sums acc[0..N)
// (N a power of two, N <= 64); on exit lane l holds, in acc[0], the full sum
// over the 64 lanes of index (l % N) ... specifically, after log2(N) halving
// steps each lane owns one index, and the remaining 64/N lanes sharing that
// index are combined with plain xor-shuffles.
// ---------------------------------------------------------------------------
template <int N>
__device__ __forceinline__ float wave_reduce_transpose(float *acc, int lane) {
    // Halving steps: at step with half-width h, lanes with bit h set keep the
    // upper half of the remaining indices, others the lower half.
#pragma unroll
    for (int h = N / 2, bit = 1; h >= 1; h >>= 1, bit <<= 1) {
        const bool upper = (lane & bit) != 0;
#pragma unroll
        for (int i = 0; i < h; ++i) {
            const float send = upper ? acc[i] : acc[i + h];
            const float keep = upper ? acc[i + h] : acc[i];
            acc[i] = keep + __shfl_xor(send, bit, 64);
        }
    }
    float s = acc[0];
    // lanes whose low log2(N) bits agree own the same index: combine them
#pragma unroll
    for (int bit = N; bit < 64; bit <<= 1) s += __shfl_xor(s, bit, 64);
    return s;
}

// Index owned by `lane` after wave_reduce_transpose<N>: bit k of the lane
// selects the upper half at step k, i.e. index = bit-reverse of (lane % N)
// over log2(N) bits ... computed directly.
template <int N>
__device__ __forceinline__ int owned_index(int lane) {
    int idx = 0;
    int h = N / 2;
    for (int bit = 1; h >= 1; h >>= 1, bit <<= 1)
        if (lane & bit) idx += h;
    return idx;
}

template <int DT, int RM>
__global__ void __launch_bounds__(256) k_shrink_rows(const typename elem<DT>::T *__restrict__ x,
                                                     int32_t T, int32_t d_in,
                                                     const typename elem<DT>::T *__restrict__ a,
                                                     const int32_t *__restrict__ rank,
                                                     int32_t n_slots, int32_t max_rank,
                                                     const int32_t *__restrict__ ids,
                                                     const int32_t *__restrict__ perm,
                                                     float *__restrict__ v, int32_t *err) {
    typedef typename elem<DT>::T E;
    constexpr int VN = vec16<DT>::n;
    __shared__ float s_red[4][RM];
    const int p = blockIdx.x;
    const int t = perm_row(perm, p, T);
    if (t < 0) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int32_t id = ids[t];
    const bool in_range = id >= 0 && id < n_slots;
    const int32_t r = in_range ? rank[id] : 0;
    if (tid == 0 && ((id < -1 || id >= n_slots) || (in_range && r == 0))) flag_bad_row(err, t);
    float *vt = v + (size_t)t * max_rank;
    if (r <= 0) {
        for (int j = tid; j < max_rank; j += 256) vt[j] = 0.0f;
        return;
    }
    const E *xt = x + (size_t)t * d_in;
    const E *At = a + (size_t)id * max_rank * d_in;
    float acc[RM];
#pragma unroll
    for (int j = 0; j < RM; ++j) acc[j] = 0.0f;
    const int nvec = d_in / VN;
    for (int kv = tid; kv < nvec; kv += 256) {
        float xf[VN];
        vec16<DT>::widen(ldg16(xt + (size_t)kv * VN), xf);
#pragma unroll
        for (int j = 0; j < RM; ++j) {
            if (j < r) {
                float af[VN];
                vec16<DT>::widen(ldg16(At + (size_t)j * d_in + (size_t)kv * VN), af);
#pragma unroll
                for (int e = 0; e < VN; ++e) acc[j] = fmaf(xf[e], af[e], acc[j]);
            }
        }
    }
    constexpr int NR = RM < 64 ? RM : 64;
#pragma unroll
    for (int c = 0; c < RM / NR; ++c) {
        const float s = wave_reduce_transpose<NR>(acc + c * NR, lane);
        if (lane < NR) s_red[wave][c * NR + owned_index<NR>(lane)] = s;
    }
    __syncthreads();
    for (int j = tid; j < max_rank; j += 256) {
        float s = 0.0f;
        if (j < r) s = (s_red[0][j] + s_red[1][j]) + (s_red[2][j] + s_red[3][j]);
        vt[j] = s;
    }
}

// ---------------------------------------------------------------------------
// SGMV shrink, bf16, MFMA 16x16x32 (fp32 accumulate).
//   grid.x: 16-row tiles of sorted positions; grid.y: k-split chunks.
//   Operand mapping per lane l (wavefront of 64): A operand = x rows,
//   row (l % 16), 8 consecutive k of k-group (l / 16); B operand = A^T rows
//   (one rank per column), column (l % 16) = rank within the 16-rank chunk,
//   the same 8 k.  Output: column (l % 16), rows 4 (l / 16) + 0..3.
// ---------------------------------------------------------------------------
template <int RC>   // number of 16-rank column chunks
__global__ void __launch_bounds__(256) k_shrink_sgmv(const uint16_t *__restrict__ x, int32_t T,
                                                     int32_t d_in, const uint16_t *__restrict__ a,
                                                     const int32_t *__restrict__ rank,
                                                     int32_t n_slots, int32_t max_rank,
                                                     const int32_t *__restrict__ ids,
                                                     const int32_t *__restrict__ perm,
                                                     int32_t k_chunk, float *__restrict__ v,
                                                     float *__restrict__ partial, int32_t *err) {
    __shared__ float s_acc[4][16][RC * 16 + 1];
    __shared__ int32_t s_id[16], s_r[16], s_t[16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int p0 = blockIdx.x * 16;
    if (tid < 16) {
        const int p = p0 + tid;
        int32_t t = -1, id = -1, r = 0;
        if (p < T) t = perm_row(perm, p, T);
        if (t >= 0) {
            const int32_t raw = ids[t];
            const bool in_range = raw >= 0 && raw < n_slots;
            r = in_range ? rank[raw] : 0;
            if (r > 0) id = raw;
            if (blockIdx.y == 0 && ((raw < -1 || raw >= n_slots) || (in_range && r == 0)))
                flag_bad_row(err, t);
        }
        s_t[tid] = t;
        s_id[tid] = id;
        s_r[tid] = r;
    }
    __syncthreads();

    const int k_begin = blockIdx.y * k_chunk;
    const int k_end = min(d_in, k_begin + k_chunk);
    const int row = lane & 15, kg = lane >> 4;
    const int my_t = s_t[row];
    f32x4_t acc[RC];
#pragma unroll
    for (int c = 0; c < RC; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    uint32_t done = 0;                               // processed row slots (uniform)
    for (int guard = 0; guard < 16; ++guard) {
        int first = -1;
        for (int i = 0; i < 16; ++i)
            if (!((done >> i) & 1) && s_id[i] >= 0) { first = i; break; }
        if (first < 0) break;
        const int32_t aid = s_id[first];
        uint32_t mask = 0;
        for (int i = 0; i < 16; ++i)
            if (s_id[i] == aid) mask |= 1u << i;
        done |= mask;
        const int32_t r = s_r[first];
        const bool row_on = (mask >> row) & 1;
        const uint16_t *xrow = x + (size_t)(row_on ? my_t : 0) * d_in;
        const uint16_t *At = a + (size_t)aid * max_rank * d_in;
        for (int k0 = k_begin + wave * 32; k0 < k_end; k0 += 4 * 32) {
            const int kk = k0 + kg * 8;
            uint4 xq = make_uint4(0, 0, 0, 0);
            if (row_on && kk < k_end) xq = ldg16(xrow + kk);
            const bf16x8_t xa = __builtin_bit_cast(bf16x8_t, xq);
#pragma unroll
            for (int c = 0; c < RC; ++c) {
                const int j = c * 16 + row;                 // rank = output column
                uint4 aq = make_uint4(0, 0, 0, 0);
                if (j < r && kk < k_end) aq = ldg16(At + (size_t)j * d_in + kk);
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    xa, __builtin_bit_cast(bf16x8_t, aq), acc[c], 0, 0, 0);
            }
        }
    }
    // cross-wave reduction of the k-subsets
#pragma unroll
    for (int c = 0; c < RC; ++c)
#pragma unroll
        for (int q = 0; q < 4; ++q) s_acc[wave][4 * kg + q][c * 16 + row] = acc[c][q];
    __syncthreads();
    for (int e = tid; e < 16 * max_rank; e += 256) {
        const int i = e / max_rank, j = e % max_rank;
        const int p = p0 + i;
        if (p >= T) continue;
        float s = 0.0f;
        if (j < RC * 16) s = (s_acc[0][i][j] + s_acc[1][i][j]) + (s_acc[2][i][j] + s_acc[3][i][j]);
        if (partial)
            partial[((size_t)blockIdx.y * T + p) * max_rank + j] = s;
        else if (s_t[i] >= 0)
            v[(size_t)s_t[i] * max_rank + j] = s;
    }
}

// v[perm[p]][j] = sum over k-split chunks, in chunk order.
__global__ void __launch_bounds__(256) k_shrink_reduce(const float *__restrict__ partial,
                                                       int32_t n_split, int32_t T,
                                                       int32_t max_rank,
                                                       const int32_t *__restrict__ perm,
                                                       float *__restrict__ v) {
    const size_t n = (size_t)T * max_rank;
    for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < n;
         e += (size_t)gridDim.x * blockDim.x) {
        const int p = (int)(e / max_rank), j = (int)(e % max_rank);
        float s = 0.0f;
        for (int c = 0; c < n_split; ++c) s += partial[(size_t)c * n + e];
        const int t = perm_row(perm, p, T);
        if (t >= 0) v[(size_t)t * max_rank + j] = s;
    }
}

template <int DT>
static void launch_rows(const void *x, int32_t T, const lora_pool_t &p, const int32_t *ids,
                        const int32_t *perm, float *v, int32_t *err, hipStream_t s) {
    typedef typename elem<DT>::T E;
    const E *xe = (const E *)x;
    const E *ae = (const E *)p.a;
#define LORA_SHRINK_ROWS(RMV)                                                                   \
    hipLaunchKernelGGL((k_shrink_rows<DT, RMV>), dim3(T), dim3(256), 0, s, xe, T, p.d_in, ae,   \
                       p.rank, p.n_slots, p.max_rank, ids, perm, v, err)
    if (p.max_rank <= 8) LORA_SHRINK_ROWS(8);
    else if (p.max_rank <= 16) LORA_SHRINK_ROWS(16);
    else if (p.max_rank <= 32) LORA_SHRINK_ROWS(32);
    else if (p.max_rank <= 64) LORA_SHRINK_ROWS(64);
    else LORA_SHRINK_ROWS(128);
#undef LORA_SHRINK_ROWS
}

lora_status_t launch_shrink(const void *x, int32_t T, const lora_pool_t &p, const int32_t *ids,
                            bool sgmv, float *v, const ws_layout &L, void *ws, hipStream_t s) {
    int32_t *err = ws_ptr<int32_t>(ws, L.header);
    const int32_t *perm = sgmv ? ws_ptr<int32_t>(ws, L.perm) : nullptr;
    if (!sgmv || p.dtype == LORA_F32) {
        if (p.dtype == LORA_F32) launch_rows<LORA_F32>(x, T, p, ids, perm, v, err, s);
        else launch_rows<LORA_BF16>(x, T, p, ids, perm, v, err, s);
        return hip_status(hipGetLastError());
    }
    // SGMV bf16: choose a k-split so that the grid has enough workgroups.
    const int32_t tiles = (T + 15) / 16;
    int32_t split = 1;
    while (split < kMaxKSplit && tiles * split < 1024 && p.d_in / (split * 2) >= 256) split *= 2;
    int32_t k_chunk = (p.d_in + split - 1) / split;
    k_chunk = (k_chunk + 31) / 32 * 32;
    split = (p.d_in + k_chunk - 1) / k_chunk;
    float *partial = split > 1 ? ws_ptr<float>(ws, L.partial) : nullptr;
    const uint16_t *xe = (const uint16_t *)x;
    const uint16_t *ae = (const uint16_t *)p.a;
    const int rc = (p.max_rank + 15) / 16;
#define LORA_SHRINK_SGMV(RCV)                                                                    \
    hipLaunchKernelGGL((k_shrink_sgmv<RCV>), dim3(tiles, split), dim3(256), 0, s, xe, T, p.d_in, \
                       ae, p.rank, p.n_slots, p.max_rank, ids, perm, k_chunk, v, partial, err)
    switch (rc) {
        case 1: LORA_SHRINK_SGMV(1); break;
        case 2: LORA_SHRINK_SGMV(2); break;
        case 3: LORA_SHRINK_SGMV(3); break;
        case 4: LORA_SHRINK_SGMV(4); break;
        case 5: LORA_SHRINK_SGMV(5); break;
        case 6: LORA_SHRINK_SGMV(6); break;
        case 7: LORA_SHRINK_SGMV(7); break;
        default: LORA_SHRINK_SGMV(8); break;
    }
#undef LORA_SHRINK_SGMV
    if (split > 1) {
        size_t n = (size_t)T * p.max_rank;
        int g = (int)((n + 255) / 256);
        if (g > 4096) g = 4096;
        hipLaunchKernelGGL(k_shrink_reduce, dim3(g), dim3(256), 0, s, partial, split, T,
                           p.max_rank, perm, v);
    }
    return hip_status(hipGetLastError());
}

}  // namespace lora
