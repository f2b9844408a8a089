// a1 -- the HBM adapter pool: stacked, rank-padded slots.
//
// Activation copies one adapter's A and B into a slot of the stacked
// buffers, and an unused slot is zeroed; buffers are sized for the maximum
// rank ("Serving LoRA adapters: from the model name to the wrapped layer",
// Step 3 "the worker loads and activates adapters", and the closing note on
// slot buffers sized for the maximum LoRA rank; "Serving multiple LoRAs ...",
// exercise 2: kernels allocate by the maximum rank).
//
// Layout per slot (chosen for the kernels' reads), C = max_rank rank rows
// (padded pool) or the slot's own capacity (packed pool, slots back to back
// from row0[s]):
//   A^T [C][d_in]           a rank row is contiguous over d_in, so the
//                           shrink reads only the first r rows;
//   B   [C/8][d_out][8]     8 consecutive ranks of one output column are
//                           16 contiguous bytes (bf16), so the expand
//                           reads only the first ceil(r/8) octets.
#include "common.hpp"

namespace lora {

__global__ void __launch_bounds__(256) k_fill_zero(uint4 *p, size_t n16) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n16;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = make_uint4(0, 0, 0, 0);
}

__global__ void __launch_bounds__(256) k_fill_meta(float *scale, int32_t *rank, int32_t n) {
    for (int32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
        scale[i] = 0.0f;
        rank[i] = 0;
    }
}

template <typename E>
__global__ void __launch_bounds__(256) k_upload(E *a_slot, E *b_slot, const E *A, int32_t lda,
                                                const E *B, int32_t ldb, int32_t r, int32_t d_in,
                                                int32_t d_out, int32_t rows) {
    const size_t na = (size_t)rows * d_in;
    const size_t nb = (size_t)rows * d_out;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < na; e += stride) {
        const int32_t j = (int32_t)(e / d_in), i = (int32_t)(e % d_in);  // A^T[j][i] = A[i][j]
        a_slot[e] = (j < r) ? A[(size_t)i * lda + j] : E(0);
    }
    for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < nb; e += stride) {
        const int32_t g = (int32_t)(e / ((size_t)d_out * 8));
        const int32_t rem = (int32_t)(e % ((size_t)d_out * 8));
        const int32_t n = rem >> 3, j = g * 8 + (rem & 7);   // b[g][n][j%8] = B[j][n]
        b_slot[e] = (j < r) ? B[(size_t)j * ldb + n] : E(0);
    }
}

__global__ void k_set_meta(float *scale, int32_t *rank, int32_t slot, float s, int32_t r) {
    if (threadIdx.x == 0 && blockIdx.x == 0) {
        scale[slot] = s;
        rank[slot] = r;
    }
}

static int grid_for(size_t n, int per_block = 256) {
    size_t g = (n + per_block - 1) / per_block;
    if (g > 4096) g = 4096;
    if (g < 1) g = 1;
    return (int)g;
}

lora_status_t launch_pool_fill(void *a, size_t a_bytes, void *b, size_t b_bytes, float *scale,
                               int32_t *rank, int32_t n_slots, hipStream_t s) {
    hipLaunchKernelGGL(k_fill_zero, dim3(grid_for(a_bytes / 16)), dim3(256), 0, s, (uint4 *)a,
                       a_bytes / 16);
    hipLaunchKernelGGL(k_fill_zero, dim3(grid_for(b_bytes / 16)), dim3(256), 0, s, (uint4 *)b,
                       b_bytes / 16);
    hipLaunchKernelGGL(k_fill_meta, dim3(grid_for(n_slots)), dim3(256), 0, s, scale, rank, n_slots);
    return hip_status(hipGetLastError());
}

// First rank row and rank-row count of a slot (host side): padded pools give
// every slot max_rank rows, packed pools the rows [row0[s], row0[s+1]).
static void slot_rows(const lora_pool_t &p, int32_t slot, size_t &row0, int32_t &rows) {
    if (p.row0_host) {
        row0 = (size_t)p.row0_host[slot];
        rows = p.row0_host[slot + 1] - p.row0_host[slot];
    } else {
        row0 = (size_t)slot * p.max_rank;
        rows = p.max_rank;
    }
}

lora_status_t launch_pool_upload(const lora_pool_t &p, int32_t slot, const void *A, int32_t lda,
                                 const void *B, int32_t ldb, int32_t r, float alpha, hipStream_t s) {
    const size_t eb = p.dtype == LORA_F32 ? 4 : 2;
    size_t row0;
    int32_t rows;
    slot_rows(p, slot, row0, rows);
    const size_t a_slot = (size_t)rows * p.d_in, b_slot = (size_t)rows * p.d_out;
    const size_t n = a_slot > b_slot ? a_slot : b_slot;
    char *a = (char *)p.a + row0 * p.d_in * eb;
    char *b = (char *)p.b + row0 * p.d_out * eb;
    if (p.dtype == LORA_F32)
        hipLaunchKernelGGL(k_upload<uint32_t>, dim3(grid_for(n)), dim3(256), 0, s, (uint32_t *)a,
                           (uint32_t *)b, (const uint32_t *)A, lda, (const uint32_t *)B, ldb, r,
                           p.d_in, p.d_out, rows);
    else
        hipLaunchKernelGGL(k_upload<uint16_t>, dim3(grid_for(n)), dim3(256), 0, s, (uint16_t *)a,
                           (uint16_t *)b, (const uint16_t *)A, lda, (const uint16_t *)B, ldb, r,
                           p.d_in, p.d_out, rows);
    // s = alpha / r in fp32 ("LoRAX, in depth", section "Computing a batch
    // that mixes adapters"), kept per slot and applied at expand time.
    hipLaunchKernelGGL(k_set_meta, dim3(1), dim3(64), 0, s, p.scale, p.rank, slot,
                       alpha / (float)r, r);
    return hip_status(hipGetLastError());
}

__global__ void k_set_meta_batch(meta_batch m) {
    const int i = threadIdx.x;
    if (i < m.n)
        for (int p = 0; p < m.n_pools; ++p) {
            m.scale[p][m.slot[i]] = m.s[i];
            m.rank[p][m.slot[i]] = m.r[i];
        }
}

lora_status_t launch_pool_meta_batch(const meta_batch &m, hipStream_t s) {
    hipLaunchKernelGGL(k_set_meta_batch, dim3(1), dim3(kMetaBatch), 0, s, m);
    return hip_status(hipGetLastError());
}

// Workgroup (chunk, i) copies bytes [64 KB chunk, +64 KB) of copy i; each
// thread keeps four independent 16-byte loads in flight before storing them
// (reads of mapped host memory cross the host link, so depth matters).
__global__ void __launch_bounds__(256) k_copy_batch(copy_batch c) {
    const int i = blockIdx.y;
    if (i >= c.n) return;
    const size_t begin = (size_t)blockIdx.x * kCopyChunk;
    if (begin >= c.bytes[i]) return;
    const size_t n16 = (min((size_t)c.bytes[i], begin + kCopyChunk) - begin) / 16;
    const uint4 *src = reinterpret_cast<const uint4 *>(static_cast<const char *>(c.src[i]) + begin);
    uint4 *dst = reinterpret_cast<uint4 *>(static_cast<char *>(c.dst[i]) + begin);
    for (size_t i0 = threadIdx.x; i0 < n16; i0 += 4 * 256) {
        uint4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (i0 + u * 256 < n16) v[u] = src[i0 + u * 256];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (i0 + u * 256 < n16) dst[i0 + u * 256] = v[u];
    }
}

lora_status_t launch_copy_batch(const copy_batch &c, hipStream_t s) {
    if (c.n <= 0) return LORA_OK;
    const unsigned chunks = (unsigned)((c.max_bytes + kCopyChunk - 1) / kCopyChunk);
    hipLaunchKernelGGL(k_copy_batch, dim3(chunks, c.n), dim3(256), 0, s, c);
    return hip_status(hipGetLastError());
}

lora_status_t launch_pool_meta(const lora_pool_t &p, int32_t slot, float scale, int32_t rank, hipStream_t s) {
    hipLaunchKernelGGL(k_set_meta, dim3(1), dim3(64), 0, s, p.scale, p.rank, slot, scale, rank);
    return hip_status(hipGetLastError());
}

lora_status_t launch_pool_clear(const lora_pool_t &p, int32_t slot, hipStream_t s) {
    const size_t eb = p.dtype == LORA_F32 ? 4 : 2;
    size_t row0;
    int32_t rows;
    slot_rows(p, slot, row0, rows);
    const size_t a_bytes = (size_t)rows * p.d_in * eb, b_bytes = (size_t)rows * p.d_out * eb;
    char *a = (char *)p.a + row0 * p.d_in * eb;
    char *b = (char *)p.b + row0 * p.d_out * eb;
    hipLaunchKernelGGL(k_fill_zero, dim3(grid_for(a_bytes / 16)), dim3(256), 0, s, (uint4 *)a, a_bytes / 16);
    hipLaunchKernelGGL(k_fill_zero, dim3(grid_for(b_bytes / 16)), dim3(256), 0, s, (uint4 *)b, b_bytes / 16);
    hipLaunchKernelGGL(k_set_meta, dim3(1), dim3(64), 0, s, p.scale, p.rank, slot, 0.0f, 0);
    return hip_status(hipGetLastError());
}

}  // namespace lora
