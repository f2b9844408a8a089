// FP8 base GEMM with the bf16 low-rank term in its epilogue: y = s_x[t] s_w[n]
// sum_k xq[t,k] wq[n,k] (+ s_a v[t] B_a), and the E4M3 quantizers that feed it.
//
// A quantized base weight with a half-precision adapter is a common mix; the
// adapter's contribution is added to the base product's accumulator, never
// merged into the packed 8-bit weights ("Multi-LoRA Serving 与 Adapter 隔离",
// section on numerics and mixed precision).  The pages fix no scheme; this
// library uses OCP E4M3 codes with one power-of-two scale per token row of x
// and one per output column of W:
//   scale = 2^e, e the smallest integer with amax <= 448 * 2^e (clamped to
//   [-127, 127]), code = E4M3(v * 2^-e) (an exact scaling; round to nearest
//   even, v_cvt_pk_fp8_f32).  An all-zero row or column gets e = -127 and
//   zero codes.  Inputs must be finite.
// Powers of two are what the matrix cores' E8M0 block scales express, so the
// scales are applied inside the product and the accumulator holds y's base
// part directly.
//
// GEMM (gfx950, v_mfma_scale_f32_32x32x64_f8f6f4, fp32 accumulate):
//   * x codes are [T][K] and W codes [N][K] (K-contiguous, "NT"), so both
//     tiles are rows of K bytes: one DMA plan, one XOR swizzle and
//     ds_read_b128 fragment reads for both operands (no transposing reads).
//   * BM x BN tile, K step 128 codes, NS LDS stages, the same tile order,
//     split-K plan, DMA, stage hand-off, fused expand (before the K loop,
//     while the first stages load) and tile store as the bf16 kernel; split-K
//     pieces write fp32 partials that the bf16 reduction finishes.
// MFMA lane mapping (checked on the GPU): lane l holds 32 codes of row (A) or
// column (B) l % 32, the same k positions for both operands, so a lane may
// take any 32 codes of its row as long as both operands agree; the E8M0
// scale operand of lane l applies to row (column) l % 32 in K-block l / 32 --
// with one scale per row and column, lanes l and l + 32 pass the same one.
// The output layout is that of the bf16 32x32 MFMAs.
#include "gemm_common.hpp"
#include "fp8_common.hpp"

namespace lora {

typedef int i32x8_t __attribute__((ext_vector_type(8)));


// ---------------------------------------------------------------------------
// Quantizers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float block_max256(float m, float *red) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// One token row per workgroup: amax over the row, then the codes (second
// read of the row, from cache).  x bf16 [T][K], K % 16 == 0; xs[t] = 2^e.
__global__ void __launch_bounds__(256) k_quant_rows_fp8(const uint16_t *x, int32_t K, uint8_t *xq, float *xs) {
    __shared__ float red[4];
    const int64_t t = blockIdx.x;
    const uint16_t *row = x + t * K;
    const int nch = K / 8;
    float m = 0.0f;
    for (int c = threadIdx.x; c < nch; c += 256) {
        float f[8];
        vec16<LORA_BF16>::widen(ldg16(row + 8 * c), f);
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
    }
    const int e = scale_exp(block_max256(m, red));
    const float inv = exp2i(-e);
    if (threadIdx.x == 0) xs[t] = exp2i(e);
    uint8_t *out = xq + t * K;
    for (int c = threadIdx.x; c < nch; c += 256) {
        float f[8];
        vec16<LORA_BF16>::widen(ldg16(row + 8 * c), f);
        uint2 q;
        q.x = e4m3x4(f[0] * inv, f[1] * inv, f[2] * inv, f[3] * inv);
        q.y = e4m3x4(f[4] * inv, f[5] * inv, f[6] * inv, f[7] * inv);
        *reinterpret_cast<uint2 *>(out + 8 * c) = q;
    }
}

// 32 output columns per workgroup: column amax over all K, then the codes,
// transposed through LDS 128 k at a time so each lane stores 16 consecutive
// k of one column.  W bf16 [K][N] -> wq [N][K], wsc [N].  K % 16 == 0,
// N % 8 == 0.
__global__ void __launch_bounds__(256) k_quant_cols_fp8(const uint16_t *W, int32_t K, int32_t N, uint8_t *wq,
                                                        float *wsc) {
    __shared__ float red[64][33];
    __shared__ float s_inv[32];
    __shared__ float tile[128][33];
    const int tid = threadIdx.x, n0 = blockIdx.x * 32;
    // pass 1: thread (k lane kl, 8-column chunk cc)
    {
        const int kl = tid >> 2, cc = tid & 3;
        const int n = n0 + 8 * cc;
        float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (n < N)
            for (int k = kl; k < K; k += 64) {
                float f[8];
                vec16<LORA_BF16>::widen(ldg16(W + (int64_t)k * N + n), f);
#pragma unroll
                for (int i = 0; i < 8; ++i) m[i] = fmaxf(m[i], fabsf(f[i]));
            }
#pragma unroll
        for (int i = 0; i < 8; ++i) red[kl][8 * cc + i] = m[i];
    }
    __syncthreads();
    if (tid < 32) {
        float m = 0.0f;
        for (int k = 0; k < 64; ++k) m = fmaxf(m, red[k][tid]);
        const int e = scale_exp(m);
        s_inv[tid] = exp2i(-e);
        if (n0 + tid < N) wsc[n0 + tid] = exp2i(e);
    }
    __syncthreads();
    // pass 2: tiles of 128 k x 32 columns
    const int oc = tid & 31, og = tid >> 5;              // output: column, 16-k group
    const float inv = s_inv[oc];
    for (int k0 = 0; k0 < K; k0 += 128) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int id = tid + 256 * h;                // 512 chunks of 8 columns
            const int kr = id >> 2, cc = id & 3;
            const int k = k0 + kr, n = n0 + 8 * cc;
            float f[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            if (k < K && n < N) vec16<LORA_BF16>::widen(ldg16(W + (int64_t)k * N + n), f);
#pragma unroll
            for (int i = 0; i < 8; ++i) tile[kr][8 * cc + i] = f[i];
        }
        __syncthreads();
        const int k = k0 + 16 * og, n = n0 + oc;
        if (k < K && n < N) {
            float f[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) f[i] = tile[16 * og + i][oc] * inv;
            uint4 q;
            q.x = e4m3x4(f[0], f[1], f[2], f[3]);
            q.y = e4m3x4(f[4], f[5], f[6], f[7]);
            q.z = e4m3x4(f[8], f[9], f[10], f[11]);
            q.w = e4m3x4(f[12], f[13], f[14], f[15]);
            stg16(wq + (int64_t)n * K + k, q);
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// GEMM
// ---------------------------------------------------------------------------

template <int BM, int BN, int NS, int WV, int WR> struct fp8_cfg {
    static constexpr int BK = 128;                          // K codes (bytes) per stage
    static constexpr int WM = BM / WR, WN = BN / (WV / WR); // per-wavefront tile
    static constexpr int RB = WM / 32, CB = WN / 32;        // 32x32 MFMA blocks per wavefront
    static constexpr int CH = BK / 16;                      // 16-byte chunks per LDS row
    static constexpr int XSTAGE = BM * BK, WSTAGE = BN * BK; // bytes
    static constexpr int STAGE = XSTAGE + WSTAGE;
    static constexpr int XI = BM * CH / (64 * WV), WI = BN * CH / (64 * WV);   // DMA instructions per wave
    static constexpr int SLD = WN + 4;
    static constexpr int EPI = WV * 32 * SLD * 4;
    static constexpr int LDS = NS * STAGE > EPI ? NS * STAGE : EPI;
    static_assert(XI * 64 * WV == BM * CH && WI * 64 * WV == BN * CH, "DMA plan must cover the tiles");
};

template <bool LORA, int BM, int BN, int NS, bool SPLIT, int WV = 4, int WR = 2>
__global__ void __launch_bounds__(WV * 64) k_gemm_fp8(gemm_args g) {
    typedef fp8_cfg<BM, BN, NS, WV, WR> C;
    constexpr int BK = C::BK, CH = C::CH, WM = C::WM, WN = C::WN, RB = C::RB, CB = C::CB;
    constexpr int XI = C::XI, WI = C::WI, XSTAGE = C::XSTAGE, STAGE = C::STAGE;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LDS];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w / (WV / WR), wn = w % (WV / WR);
    int tm, tn, split, tidx;
    tile_of(blockIdx.x, gridDim.x, g, tm, tn, split, tidx);
    const int m0 = tm * BM, n0 = tn * BN;
    const int K = g.K, N = g.N, T = g.T;
    const int k_begin = SPLIT ? split * g.k_chunk : 0;
    const int k_end = SPLIT ? min(K, k_begin + g.k_chunk) : K;

    // DMA plan, both operands: chunk c = (w * I + j) * 64 + lane of a stage
    // sits at row c / CH, slot c % CH and holds the row's chunk slot ^ swz(row).
    int64_t xrow[XI], wrow[WI];
    int xcol[XI], wcol[WI];
#pragma unroll
    for (int j = 0; j < XI; ++j) {
        const int c = (w * XI + j) * 64 + lane;
        const int r = c / CH, slot = c % CH;
        const int p = m0 + r;
        const int32_t t = (p < T) ? perm_row(g.perm, p, T) : -1;
        xrow[j] = (t >= 0) ? (int64_t)t * K : -1;
        xcol[j] = 16 * (slot ^ swz_x<64>(r));
    }
#pragma unroll
    for (int j = 0; j < WI; ++j) {
        const int c = (w * WI + j) * 64 + lane;
        const int r = c / CH, slot = c % CH;
        wrow[j] = (n0 + r < N) ? (int64_t)(n0 + r) * K : -1;
        wcol[j] = 16 * (slot ^ swz_x<64>(r));
    }
    auto dma_stage = [&](int kt, int buf) {
        uint8_t *xs = smem + buf * STAGE;
        uint8_t *wsm = xs + XSTAGE;
        const int k0 = k_begin + kt * BK;
#pragma unroll
        for (int j = 0; j < XI; ++j) {
            const int kk = k0 + xcol[j];
            const void *src = (xrow[j] >= 0 && kk < k_end) ? (const void *)(g.xq + xrow[j] + kk)
                                                             : (const void *)g_zero16;
            dma16(src, xs + (w * XI + j) * 64 * 16);
        }
#pragma unroll
        for (int j = 0; j < WI; ++j) {
            const int kk = k0 + wcol[j];
            const void *src = (wrow[j] >= 0 && kk < k_end) ? (const void *)(g.wq + wrow[j] + kk)
                                                             : (const void *)g_zero16;
            dma16(src, wsm + (w * WI + j) * 64 * 16);
        }
    };

    f32x16_t acc[RB][CB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[rb][cb][e] = 0.0f;

    // Fragments: lane reads 32 consecutive codes (two 16-byte chunks) of its
    // row (A) or column (B) for k-substep ks (64 codes).
    const int fr = lane & 31, fh = lane >> 5;
    constexpr int KS = BK / 64;
    i32x8_t af[2][RB], bfr[2][CB];
    auto frag = [&](const uint8_t *base, int r, int ks) {
        const int sw = swz_x<64>(r), c0 = 4 * ks + 2 * fh;
        const uint4 lo = *reinterpret_cast<const uint4 *>(base + r * BK + 16 * (c0 ^ sw));
        const uint4 hi = *reinterpret_cast<const uint4 *>(base + r * BK + 16 * ((c0 + 1) ^ sw));
        i32x8_t v;
        v[0] = (int)lo.x; v[1] = (int)lo.y; v[2] = (int)lo.z; v[3] = (int)lo.w;
        v[4] = (int)hi.x; v[5] = (int)hi.y; v[6] = (int)hi.z; v[7] = (int)hi.w;
        return v;
    };
    auto load_frags = [&](int buf, int ks, i32x8_t *a, i32x8_t *b) {
        const uint8_t *xs = smem + buf * STAGE;
        const uint8_t *wsm = xs + XSTAGE;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) a[rb] = frag(xs, wm * WM + rb * 32 + fr, ks);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) b[cb] = frag(wsm, wn * WN + cb * 32 + fr, ks);
    };
    // per-lane E8M0 scale operands: the row of each A block, the column of each B block
    int esa[RB], esb[CB];
    auto mfmas = [&](const i32x8_t *a, const i32x8_t *b, int rb0, int rb1) {
#pragma unroll
        for (int rb = rb0; rb < rb1; ++rb)
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
                acc[rb][cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[rb], b[cb], acc[rb][cb], 0, 0, 0,
                                                                              esa[rb], 0, esb[cb]);
    };
    constexpr int NREAD = 2 * (RB + CB);                // LDS reads per k-substep

    // Per-row metadata: token row, usable adapter slot or -1, E8M0 code of
    // the row scale (1.0 for rows past T).
    __shared__ int32_t s_meta_t[BM], s_meta_id[BM], s_esx[BM];
    const int32_t n_fused = (LORA && g.n_fused) ? *g.n_fused : T;   // short-segment rows: separate expand
    for (int i = tid; i < BM; i += WV * 64) {
        const int p = m0 + i;
        const int32_t t = (p < T) ? perm_row(g.perm, p, T) : -1;
        int32_t id = -1;
        if (LORA && t >= 0 && (!g.n_fused || p < n_fused)) {
            const int32_t raw = g.ids[t];
            if (raw >= 0 && raw < g.n_slots && g.rank[raw] > 0) id = raw;
        }
        s_meta_t[i] = t;
        s_meta_id[i] = id;
        s_esx[i] = t >= 0 ? e8m0_of(g.xs[t]) : 127;
    }

    const int nk = (k_end - k_begin + BK - 1) / BK;
    constexpr int PER = XI + WI;                          // DMA instructions per stage per wave
    auto wait_stage = [&](int ahead) {                    // later stages still in flight
        if (ahead >= 3) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * PER) : "memory");
        else if (ahead == 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * PER) : "memory");
        else if (ahead == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(PER) : "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    };
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        const int col = n0 + wn * WN + cb * 32 + fr;
        esb[cb] = col < N ? e8m0_of(g.wsc[col]) : 127;
    }
#pragma unroll
    for (int st = 0; st < NS; ++st)
        if (st < nk) dma_stage(st, st);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // metadata stores visible after the barrier
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) esa[rb] = s_esx[wm * WM + rb * 32 + fr];
    // The low-rank term goes into the accumulators before the K loop, while
    // the first stages load (split-K tiles leave it to the reduction).
    if (LORA && !SPLIT)
        lora_pass_impl<RB, CB, (RB >= 4 ? RB : 1), 1, 0>(g, acc, s_meta_t, s_meta_id, n0, wm * WM, n0 + wn * WN, lane);
    wait_stage(min(NS - 1, nk - 1));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    load_frags(0, 0, af[0], bfr[0]);
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt % NS;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int cur = ks & 1, nxt = cur ^ 1;
            if (ks + 1 < KS) {
                load_frags(buf, ks + 1, af[nxt], bfr[nxt]);
                mfmas(af[cur], bfr[cur], 0, RB);
                sched_interleave<NREAD, RB * CB>();
            } else {
                // Stage hand-off (as in the bf16 kernel): all waves are done
                // reading this stage, stage kt+1 has landed, this buffer is
                // refilled with stage kt+NS, and stage kt+1's first fragments
                // are read under the second half of the MFMAs.
                mfmas(af[cur], bfr[cur], 0, RB / 2);
                __builtin_amdgcn_sched_barrier(0);
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                wait_stage(min(NS - 2, nk - 2 - kt));
                __builtin_amdgcn_s_barrier();
                asm volatile("" ::: "memory");
                if (kt + NS < nk) dma_stage(kt + NS, buf);
                __builtin_amdgcn_sched_barrier(0);
                load_frags((kt + 1) % NS, 0, af[nxt], bfr[nxt]);
                mfmas(af[cur], bfr[cur], RB / 2, RB);
                sched_interleave<NREAD, (RB - RB / 2) * CB>();
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    gemm_store_tile<BM, BN, WV, WR, SPLIT, false>(g, acc, reinterpret_cast<float *>(smem), s_meta_t, n0, w, lane,
                                         tidx, split);
}

// NST, WVT: stages and wavefronts of the split-K pieces.
template <int BM, int BN, int NS = 2, int WV = 4, int WR = 2, int NST = NS, int WVT = WV>
static void launch_fp8_cfg(gemm_args g, const gemm_plan &pl, bool lora, hipStream_t s) {
    if (pl.n_dp > 0) {
        g.tile_base = 0;
        g.n_tiles = pl.n_dp;
        g.splits = 1;
        g.k_chunk = g.K;
        if (lora)
            hipLaunchKernelGGL((k_gemm_fp8<true, BM, BN, NS, false, WV, WR>), dim3(pl.n_dp), dim3(WV * 64), 0, s, g);
        else
            hipLaunchKernelGGL((k_gemm_fp8<false, BM, BN, NS, false, WV, WR>), dim3(pl.n_dp), dim3(WV * 64), 0, s, g);
    }
    if (pl.tail > 0) {
        g.tile_base = pl.n_dp;
        g.n_tiles = pl.tail;
        g.splits = pl.splits;
        g.k_chunk = pl.k_chunk;
        hipLaunchKernelGGL((k_gemm_fp8<false, BM, BN, NST, true, WVT, WR>), dim3(pl.tail * pl.splits),
                           dim3(WVT * 64), 0, s, g);
        const dim3 rgrid(pl.tail * (BM / (2048 / BN)));
        if (lora)
            hipLaunchKernelGGL((k_splitk_reduce<true, false, BM, BN>), rgrid, dim3(256), 0, s, g);
        else
            hipLaunchKernelGGL((k_splitk_reduce<false, false, BM, BN>), rgrid, dim3(256), 0, s, g);
    }
}

lora_status_t launch_quant_rows_fp8(const void *x, int32_t T, int32_t K, uint8_t *xq, float *xs, hipStream_t s) {
    if (T <= 0) return LORA_OK;
    hipLaunchKernelGGL(k_quant_rows_fp8, dim3(T), dim3(256), 0, s, (const uint16_t *)x, K, xq, xs);
    return hip_status(hipGetLastError());
}

lora_status_t launch_quant_cols_fp8(const void *W, int32_t K, int32_t N, uint8_t *wq, float *wsc, hipStream_t s) {
    hipLaunchKernelGGL(k_quant_cols_fp8, dim3((N + 31) / 32), dim3(256), 0, s, (const uint16_t *)W, K, N, wq, wsc);
    return hip_status(hipGetLastError());
}

lora_status_t launch_gemm_fp8(const uint8_t *xq, const float *xs, const uint8_t *wq, const float *wsc, void *y,
                              int32_t T, int32_t d_in, int32_t d_out, const lora_pool_t *pool,
                              const int32_t *ids, const float *v, int32_t v_stride, const int32_t *perm,
                              float *partial, size_t partial_bytes, hipStream_t s, const int32_t *n_fused) {
    gemm_args g{};
    g.xq = xq;
    g.wq = wq;
    g.xs = xs;
    g.wsc = wsc;
    g.y = (uint16_t *)y;
    g.T = T;
    g.K = d_in;
    g.N = d_out;
    g.perm = perm;
    g.b = pool ? (const uint16_t *)pool->b : nullptr;
    g.scale = pool ? pool->scale : nullptr;
    g.rank = pool ? pool->rank : nullptr;
    g.row0 = pool ? pool->row0 : nullptr;
    g.n_fused = n_fused;
    g.n_slots = pool ? pool->n_slots : 0;
    g.max_rank = pool ? pool->max_rank : 0;
    g.ids = ids;
    g.v = v;
    g.v_stride = v_stride;
    const gemm_plan pl = plan_gemm(T, d_in, d_out, partial ? partial_bytes : 0, 128);
    g.n_tiles_m = ceil_div(T, pl.bm);
    g.n_tiles_n = ceil_div(d_out, pl.bn);
    g.col_strips = col_strips_pay(T, d_out, g.n_tiles_n);
    g.partial = partial;
    const bool lora = pool != nullptr;
    if (pl.bm == 256 && pl.bn == 256) launch_fp8_cfg<256, 256, 2, 4>(g, pl, lora, s);
    else if (pl.bm == 256 && pl.bn == 128) launch_fp8_cfg<256, 128, 2, 8>(g, pl, lora, s);
    else if (pl.bn == 128) launch_fp8_cfg<128, 128, 2, 4, 2, 4, 8>(g, pl, lora, s);
    else launch_fp8_cfg<128, 64>(g, pl, lora, s);
    return hip_status(hipGetLastError());
}

}  // namespace lora
