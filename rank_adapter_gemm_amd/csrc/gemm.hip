// a3 (+ a5 fused) -- base GEMM y = x W over all token rows, optionally with
// the expand y += s_a v[t] B_a folded into the epilogue so y is written once.
//
// The base product is shared by every request and runs once over all tokens
// ("Multi-LoRA Serving: Architecture for Thousands of Adapters", section "How
// multi-LoRA serving works"; "LoRAX, in depth", section "Computing a batch
// that mixes adapters"; "Serving LoRA adapters ...", Step 4: the base layer
// runs first, then the LoRA output is added).
//
// bf16 kernel (gfx950 MFMA, fp32 accumulate):
//   * 256 x 256 output tile, K step 64, 512 threads = 8 wavefronts in a 2 x 4
//     grid, 128 x 64 outputs per wavefront = 4 x 2 blocks of
//     v_mfma_f32_32x32x16_bf16.
//   * x tile [256][64] and W tile staged in LDS, double-buffered (one barrier
//     per K step); LDS rows padded to 72 elements so the fragment reads of 32
//     rows at one column hit distinct banks.
//   * Both MFMA operands need 8 consecutive k per lane.  x rows already are
//     k-contiguous; W [d_in][d_out] is n-contiguous, so each thread loads a
//     4 (k) x 8 (n) block with four 16-byte loads and transposes it in
//     registers (byte permutes) into 8 columns of 4 k, written to LDS as W^T.
//   * Rows may be visited through `perm` (segment order), gathering x rows on
//     load and scattering y rows on store; nothing is materialised.
//   * Epilogue: fp32 accumulator (+ s_a * sum_j v[t][j] B_a[j][n] for rows
//     with an adapter; v staged in LDS, B read in rank octets), one rounding
//     to bf16 (nearest even).
#include "common.hpp"

namespace lora {

constexpr int GBM = 256, GBN = 256, GBK = 64, GLD = GBK + 8;

struct gemm_args {
    const uint16_t *x;
    const uint16_t *W;
    uint16_t *y;
    int32_t T, K, N;
    const int32_t *perm;
    const uint16_t *b;
    const float *scale;
    const int32_t *rank;
    int32_t n_slots, max_rank;
    const int32_t *ids;
    const float *v;
    int32_t n_tiles_n;
};

template <bool LORA>
__global__ void __launch_bounds__(512) k_gemm_bf16(gemm_args g) {
    __shared__ __attribute__((aligned(16))) uint16_t smem[4 * GBM * GLD];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w >> 2, wn = w & 3;
    const int tm = blockIdx.x / g.n_tiles_n, tn = blockIdx.x % g.n_tiles_n;
    const int m0 = tm * GBM, n0 = tn * GBN;
    const int K = g.K, N = g.N, T = g.T;

    // this thread's four x rows
    int64_t xoff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int p = m0 + (tid >> 3) + 64 * i;
        const int32_t t = (p < T) ? perm_row(g.perm, p, T) : -1;
        xoff[i] = (t >= 0) ? (int64_t)t * K : -1;
    }
    const int xk = (tid & 7) * 8;
    // this thread's 4 x 8 block of W
    const int kb = lane & 15, nb = (lane >> 4) + 4 * w;
    const int wk = 4 * kb, wnn = 8 * nb;
    const bool wcol_ok = (n0 + wnn) < N;

    uint4 xr[4], wr[4];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            xr[i] = make_uint4(0, 0, 0, 0);
            if (xoff[i] >= 0 && k0 + xk < K) xr[i] = ldg16(g.x + xoff[i] + k0 + xk);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int k = k0 + wk + i;
            wr[i] = make_uint4(0, 0, 0, 0);
            if (wcol_ok && k < K) wr[i] = ldg16(g.W + (int64_t)k * N + n0 + wnn);
        }
    };
    auto sstore = [&](int buf) {
        uint16_t *As = smem + buf * GBM * GLD;
        uint16_t *Bs = smem + 2 * GBM * GLD + buf * GBN * GLD;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<uint4 *>(As + ((tid >> 3) + 64 * i) * GLD + xk) = xr[i];
        const uint32_t in0[4] = {wr[0].x, wr[0].y, wr[0].z, wr[0].w};
        const uint32_t in1[4] = {wr[1].x, wr[1].y, wr[1].z, wr[1].w};
        const uint32_t in2[4] = {wr[2].x, wr[2].y, wr[2].z, wr[2].w};
        const uint32_t in3[4] = {wr[3].x, wr[3].y, wr[3].z, wr[3].w};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            // column 2d: low halves; column 2d+1: high halves
            const uint2 lo = make_uint2((in0[d] & 0xffffu) | (in1[d] << 16),
                                        (in2[d] & 0xffffu) | (in3[d] << 16));
            const uint2 hi = make_uint2((in0[d] >> 16) | (in1[d] & 0xffff0000u),
                                        (in2[d] >> 16) | (in3[d] & 0xffff0000u));
            *reinterpret_cast<uint2 *>(Bs + (wnn + 2 * d) * GLD + wk) = lo;
            *reinterpret_cast<uint2 *>(Bs + (wnn + 2 * d + 1) * GLD + wk) = hi;
        }
    };

    f32x16_t acc[4][2];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[rb][cb][e] = 0.0f;

    const int nk = (K + GBK - 1) / GBK;
    gload(0);
    sstore(0);
    __syncthreads();
    const int frag_row = lane & 31, frag_k = (lane >> 5) * 8;
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * GBK);
        const uint16_t *As = smem + buf * GBM * GLD;
        const uint16_t *Bs = smem + 2 * GBM * GLD + buf * GBN * GLD;
#pragma unroll
        for (int ks = 0; ks < GBK / 16; ++ks) {
            bf16x8_t af[4], bfr[2];
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
                af[rb] = *reinterpret_cast<const bf16x8_t *>(
                    As + (wm * 128 + rb * 32 + frag_row) * GLD + ks * 16 + frag_k);
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
                bfr[cb] = *reinterpret_cast<const bf16x8_t *>(
                    Bs + (wn * 64 + cb * 32 + frag_row) * GLD + ks * 16 + frag_k);
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
#pragma unroll
                for (int cb = 0; cb < 2; ++cb)
                    acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[rb], bfr[cb],
                                                                          acc[rb][cb], 0, 0, 0);
        }
        if (kt + 1 < nk) sstore(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue ----
    // Each wavefront moves one 32 x 64 block of its accumulators at a time
    // through its own LDS area; a lane then owns 8 consecutive columns of 4
    // rows, adds s * sum_j v[t][j] B[j][n] for rows with an adapter (B read in
    // rank octets, reused across the lane's rows when they share the slot) and
    // writes 16-byte rows of y after one rounding.
    constexpr int SLD = 68;                                       // staged row stride (floats)
    float *stage = reinterpret_cast<float *>(smem) + w * 32 * SLD;
    int32_t *s_t = reinterpret_cast<int32_t *>(reinterpret_cast<float *>(smem) + 8 * 32 * SLD);
    int32_t *s_id = s_t + GBM;
    int32_t *s_gq = s_id + GBM;
    float *s_sc = reinterpret_cast<float *>(s_gq + GBM);
    for (int i = tid; i < GBM; i += 512) {
        const int p = m0 + i;
        const int32_t t = (p < T) ? perm_row(g.perm, p, T) : -1;
        int32_t id = -1, r = 0;
        float sc = 0.0f;
        if (LORA && t >= 0) {
            const int32_t raw = g.ids[t];
            if (raw >= 0 && raw < g.n_slots) {
                r = g.rank[raw];
                if (r > 0) {
                    id = raw;
                    sc = g.scale[raw];
                } else {
                    r = 0;
                }
            }
        }
        s_t[i] = t;
        s_id[i] = id;
        s_gq[i] = (r + 7) >> 3;
        s_sc[i] = sc;
    }
    const int q = lane & 7, rr = lane >> 3;
    const int n = n0 + wn * 64 + 8 * q;
    const int R = g.max_rank;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
        __syncthreads();
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                stage[(8 * (e >> 2) + 4 * (lane >> 5) + (e & 3)) * SLD + cb * 32 + (lane & 31)] =
                    acc[rb][cb][e];
        __syncthreads();
        int32_t tk[4], idk[4], gk[4];
        float sk[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int i = wm * 128 + rb * 32 + rr + 8 * k;
            tk[k] = s_t[i];
            idk[k] = s_id[i];
            gk[k] = s_gq[i];
            sk[k] = s_sc[i];
        }
        float d[4][8];
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int c = 0; c < 8; ++c) d[k][c] = 0.0f;
        if (LORA && n < N) {
            const bool same = idk[0] >= 0 && idk[1] == idk[0] && idk[2] == idk[0] && idk[3] == idk[0];
            int G = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) G = (idk[k] >= 0 && gk[k] > G) ? gk[k] : G;
            for (int gg = 0; gg < G; ++gg) {
                uint4 bq[8];
                if (same) {
                    const uint16_t *bp = g.b + ((int64_t)idk[0] * R * N + ((int64_t)gg * N + n) * 8);
#pragma unroll
                    for (int c = 0; c < 8; ++c) bq[c] = ldg16(bp + c * 8);
                }
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    if (idk[k] < 0 || gg >= gk[k]) continue;
                    if (!same) {
                        const uint16_t *bp = g.b + ((int64_t)idk[k] * R * N + ((int64_t)gg * N + n) * 8);
#pragma unroll
                        for (int c = 0; c < 8; ++c) bq[c] = ldg16(bp + c * 8);
                    }
                    const float *vp = g.v + (int64_t)tk[k] * R + gg * 8;
                    const float4 v0 = *reinterpret_cast<const float4 *>(vp);
                    const float4 v1 = *reinterpret_cast<const float4 *>(vp + 4);
#pragma unroll
                    for (int c = 0; c < 8; ++c) {
                        float bf[8];
                        vec16<LORA_BF16>::widen(bq[c], bf);
                        float a = d[k][c];
                        a = fmaf(v0.x, bf[0], a); a = fmaf(v0.y, bf[1], a);
                        a = fmaf(v0.z, bf[2], a); a = fmaf(v0.w, bf[3], a);
                        a = fmaf(v1.x, bf[4], a); a = fmaf(v1.y, bf[5], a);
                        a = fmaf(v1.z, bf[6], a); a = fmaf(v1.w, bf[7], a);
                        d[k][c] = a;
                    }
                }
            }
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (tk[k] < 0 || n >= N) continue;
            const float *src = stage + (rr + 8 * k) * SLD + 8 * q;
            const float4 o0 = *reinterpret_cast<const float4 *>(src);
            const float4 o1 = *reinterpret_cast<const float4 *>(src + 4);
            float o[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
            if (LORA && idk[k] >= 0) {
#pragma unroll
                for (int c = 0; c < 8; ++c) o[c] = fmaf(sk[k], d[k][c], o[c]);
            }
            stg16(g.y + (int64_t)tk[k] * N + n, vec16<LORA_BF16>::narrow(o));
        }
    }
}

// ---------------------------------------------------------------------------
// fp32 kernel (plain FMA, no reduced-precision path): 64 x 64 tile, K step
// 16, 256 threads with 4 x 4 outputs each, same epilogue semantics.
// ---------------------------------------------------------------------------
struct gemm_f32_args {
    const float *x;
    const float *W;
    float *y;
    int32_t T, K, N;
    const int32_t *perm;
    const float *b;
    const float *scale;
    const int32_t *rank;
    int32_t n_slots, max_rank;
    const int32_t *ids;
    const float *v;
    int32_t n_tiles_n;
};

template <bool LORA>
__global__ void __launch_bounds__(256) k_gemm_f32(gemm_f32_args g) {
    __shared__ float As[16][64 + 4];
    __shared__ float Bs[16][64 + 4];
    const int tid = threadIdx.x;
    const int tm = blockIdx.x / g.n_tiles_n, tn = blockIdx.x % g.n_tiles_n;
    const int m0 = tm * 64, n0 = tn * 64;
    const int K = g.K, N = g.N, T = g.T;
    const int lr = tid >> 2, lk = (tid & 3) * 4;          // x tile loader
    const int p_load = m0 + lr;
    const int32_t t_load = (p_load < T) ? perm_row(g.perm, p_load, T) : -1;
    const int64_t xrow = (t_load >= 0) ? (int64_t)t_load * K : -1;
    const int wk = tid >> 4, wn4 = (tid & 15) * 4;        // W tile loader
    const int ty = tid >> 4, tx = tid & 15;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += 16) {
        float4 xa = make_float4(0.f, 0.f, 0.f, 0.f), wa = make_float4(0.f, 0.f, 0.f, 0.f);
        if (xrow >= 0 && k0 + lk < K) xa = *reinterpret_cast<const float4 *>(g.x + xrow + k0 + lk);
        if (k0 + wk < K && n0 + wn4 < N)
            wa = *reinterpret_cast<const float4 *>(g.W + (int64_t)(k0 + wk) * N + n0 + wn4);
        __syncthreads();
        As[lk + 0][lr] = xa.x;
        As[lk + 1][lr] = xa.y;
        As[lk + 2][lr] = xa.z;
        As[lk + 3][lr] = xa.w;
        *reinterpret_cast<float4 *>(&Bs[wk][wn4]) = wa;
        __syncthreads();
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            float a[4], bb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[k][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) bb[j] = Bs[k][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], bb[j], acc[i][j]);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int p = m0 + ty * 4 + i;
        if (p >= T) continue;
        const int64_t t = perm_row(g.perm, p, T);
        if (t < 0) continue;
        int32_t id = -1, r = 0;
        float s = 0.0f;
        if (LORA) {
            const int32_t raw = g.ids[t];
            if (raw >= 0 && raw < g.n_slots && g.rank[raw] > 0) {
                id = raw;
                r = g.rank[raw];
                s = g.scale[raw];
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + tx * 4 + j;
            if (n >= N) continue;
            float val = acc[i][j];
            if (LORA && id >= 0) {
                const float *bq = g.b + ((int64_t)id * g.max_rank * N + (int64_t)n * 8);
                const float *vi = g.v + t * g.max_rank;
                float d = 0.0f;
                for (int q = 0; q < r; ++q) d = fmaf(vi[q], bq[(int64_t)(q >> 3) * N * 8 + (q & 7)], d);
                val = fmaf(s, d, val);
            }
            g.y[t * N + n] = val;
        }
    }
}

lora_status_t launch_gemm(const void *x, const void *W, void *y, int32_t T, int32_t d_in,
                          int32_t d_out, int32_t dtype, const lora_pool_t *pool,
                          const int32_t *ids, const float *v, const int32_t *perm,
                          int32_t * /*err*/, hipStream_t s) {
    if (dtype == LORA_BF16) {
        gemm_args g;
        g.x = (const uint16_t *)x;
        g.W = (const uint16_t *)W;
        g.y = (uint16_t *)y;
        g.T = T;
        g.K = d_in;
        g.N = d_out;
        g.perm = perm;
        g.b = pool ? (const uint16_t *)pool->b : nullptr;
        g.scale = pool ? pool->scale : nullptr;
        g.rank = pool ? pool->rank : nullptr;
        g.n_slots = pool ? pool->n_slots : 0;
        g.max_rank = pool ? pool->max_rank : 0;
        g.ids = ids;
        g.v = v;
        g.n_tiles_n = (d_out + GBN - 1) / GBN;
        const int tiles = ((T + GBM - 1) / GBM) * g.n_tiles_n;
        if (pool)
            hipLaunchKernelGGL(k_gemm_bf16<true>, dim3(tiles), dim3(512), 0, s, g);
        else
            hipLaunchKernelGGL(k_gemm_bf16<false>, dim3(tiles), dim3(512), 0, s, g);
    } else {
        gemm_f32_args g;
        g.x = (const float *)x;
        g.W = (const float *)W;
        g.y = (float *)y;
        g.T = T;
        g.K = d_in;
        g.N = d_out;
        g.perm = perm;
        g.b = pool ? (const float *)pool->b : nullptr;
        g.scale = pool ? pool->scale : nullptr;
        g.rank = pool ? pool->rank : nullptr;
        g.n_slots = pool ? pool->n_slots : 0;
        g.max_rank = pool ? pool->max_rank : 0;
        g.ids = ids;
        g.v = v;
        g.n_tiles_n = (d_out + 63) / 64;
        const int tiles = ((T + 63) / 64) * g.n_tiles_n;
        if (pool)
            hipLaunchKernelGGL(k_gemm_f32<true>, dim3(tiles), dim3(256), 0, s, g);
        else
            hipLaunchKernelGGL(k_gemm_f32<false>, dim3(tiles), dim3(256), 0, s, g);
    }
    return hip_status(hipGetLastError());
}

}  // namespace lora
