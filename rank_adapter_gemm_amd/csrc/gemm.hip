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

constexpr int GBM = 256, GBN = 256;
// K step and number of LDS stages of the bf16 kernel (2 x 64 KB).
constexpr int kGemmBK = 64, kGemmNS = 2;

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
    int32_t n_tiles_m, n_tiles_n;
};

// Tile order: workgroups are dispatched round-robin over the 8 XCDs (each
// with its own L2), so workgroup b runs on XCD b % 8.  Give each XCD a
// contiguous range of tiles, walked in groups of GROUP_M row tiles (down M
// first, then across N) so the tiles resident on one XCD share x rows and W
// columns in its L2.
constexpr int kXcds = 8, kGroupM = 8;

__device__ __forceinline__ void tile_of(int b, int total, int n_tiles_m, int n_tiles_n, int &tm, int &tn) {
    const int q = total / kXcds, r = total % kXcds;
    const int x = b % kXcds, slot = b / kXcds;
    const int v = x * q + min(x, r) + slot;
    const int per_group = kGroupM * n_tiles_n;
    const int grp = v / per_group;
    const int first_m = grp * kGroupM;
    const int gm = min(kGroupM, n_tiles_m - first_m);
    const int in = v - grp * per_group;
    tm = first_m + in % gm;
    tn = in / gm;
}

// A 16-byte zero vector in global memory: the source of the DMA loads of
// masked lanes (rows past T, k past K, columns past N), so those LDS slots
// hold zeros.
__device__ __attribute__((aligned(16))) uint4 g_zero16[1];

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;

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

// XOR swizzles of the 16-byte chunk index inside an LDS row (see the tile
// layouts below): conflict-free fragment reads for 32 and for 64 LDS banks.
template <int BK> __device__ __forceinline__ int swz_x(int r) {
    return BK == 64 ? ((r ^ (r >> 3)) & 7) : (((r >> 2) ^ (r >> 1)) & 3);
}
__device__ __forceinline__ int swz_w(int k) {
    return (0xCA60 >> (4 * (k & 3))) & 0xF;            // 0, 6, 10, 12 for k % 4 = 0..3
}

// LDS tiles per stage (no padding; rows written by DMA 1 KB at a time):
//   x: [256 rows][BK] bf16, row chunk c (8 k) stored at slot c ^ swz_x(row)
//   W: [BK rows (k)][256 n] bf16, row chunk c (8 n) stored at slot c ^ swz_w(k)
// MFMA A fragments: ds_read_b128 of 8 consecutive k of one x row.
// MFMA B fragments: two ds_read_b64_tr_b16 per lane, each returning 4
// consecutive k of one W column from a 4 x 16 block read by 16 lanes.
template <bool LORA, int BK, int NS>
__global__ void __launch_bounds__(256, 1) k_gemm_bf16(gemm_args g) {
    constexpr int XCH = BK / 8;                         // 16-byte chunks per x row
    constexpr int XSTAGE = GBM * BK, WSTAGE = BK * GBN; // elements per stage
    __shared__ __attribute__((aligned(1024))) uint16_t smem[NS * (XSTAGE + WSTAGE) > 4 * 32 * 132 * 2 + 4 * GBM * 2
                                                                  ? NS * (XSTAGE + WSTAGE)
                                                                  : 4 * 32 * 132 * 2 + 4 * GBM * 2];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w >> 1, wn = w & 1;                  // 2 x 2 wavefronts, 128 x 128 each
    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, g.n_tiles_m, g.n_tiles_n, tm, tn);
    const int m0 = tm * GBM, n0 = tn * GBN;
    const int K = g.K, N = g.N, T = g.T;

    // DMA plan.  x: the stage is 256 * XCH chunks; wave w issues XI = 256*XCH/256
    // instructions of 64 chunks, chunk index c = (w * XI + j) * 64 + lane.
    constexpr int XI = GBM * XCH / 256, WI = BK * 32 / 256;
    int64_t xrow[XI];
    int xcol[XI];
#pragma unroll
    for (int j = 0; j < XI; ++j) {
        const int c = (w * XI + j) * 64 + lane;
        const int r = c / XCH, slot = c % XCH;
        const int p = m0 + r;
        const int32_t t = (p < T) ? perm_row(g.perm, p, T) : -1;
        xrow[j] = (t >= 0) ? (int64_t)t * K : -1;
        xcol[j] = 8 * (slot ^ swz_x<BK>(r));
    }
    // W: the stage is BK rows * 32 chunks; chunk index c = (w * WI + j) * 64 + lane
    int wrow[WI], wcol[WI];
#pragma unroll
    for (int j = 0; j < WI; ++j) {
        const int c = (w * WI + j) * 64 + lane;
        const int k = c >> 5, slot = c & 31;
        wrow[j] = k;
        wcol[j] = n0 + 8 * (slot ^ swz_w(k));
    }
    auto dma_stage = [&](int kt, int buf) {
        uint16_t *xs = smem + buf * (XSTAGE + WSTAGE);
        uint16_t *wsm = xs + XSTAGE;
        const int k0 = kt * BK;
#pragma unroll
        for (int j = 0; j < XI; ++j) {
            const int kk = k0 + xcol[j];
            const void *src = (xrow[j] >= 0 && kk < K) ? (const void *)(g.x + xrow[j] + kk) : (const void *)g_zero16;
            dma16(src, xs + (w * XI + j) * 64 * 8);
        }
#pragma unroll
        for (int j = 0; j < WI; ++j) {
            const int k = k0 + wrow[j];
            const void *src = (k < K && wcol[j] < N) ? (const void *)(g.W + (int64_t)k * N + wcol[j]) : (const void *)g_zero16;
            dma16(src, wsm + (w * WI + j) * 64 * 8);
        }
    };

    f32x16_t acc[4][4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[rb][cb][e] = 0.0f;

    // fragment addressing
    const int fr = lane & 31, fk = lane >> 5;           // A: row within block, k-group
    const int grp = lane >> 4, s16 = lane & 15;         // B: 16-lane group, lane in group
    const int b_kofs = 8 * (grp >> 1) + (s16 >> 2);     // + 16 ks + 4 inst
    const int b_col = 16 * (grp & 1) + 4 * (s16 & 3);   // + wn*128 + cb*32
    constexpr int KS = BK / 16;                         // MFMA k-substeps per stage
    bf16x8_t af[2][4], bfr[2][4];
    auto load_frags = [&](int buf, int ks, bf16x8_t *a, bf16x8_t *b) {
        const uint16_t *xs = smem + buf * (XSTAGE + WSTAGE);
        const uint16_t *wsm = xs + XSTAGE;
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            const int r = wm * 128 + rb * 32 + fr;
            const int c = (2 * ks + fk) ^ swz_x<BK>(r);
            a[rb] = *reinterpret_cast<const bf16x8_t *>(xs + r * BK + 8 * c);
        }
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            const int col = wn * 128 + cb * 32 + b_col;          // multiple of 4
            short4_t h[2];
#pragma unroll
            for (int inst = 0; inst < 2; ++inst) {
                const int k = 16 * ks + 4 * inst + b_kofs;
                const int chunk = (col >> 3) ^ swz_w(k);
                const uint16_t *addr = wsm + k * GBN + 8 * chunk + (col & 7);
                h[inst] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_short4_t *)(reinterpret_cast<uintptr_t>(addr)));
            }
            typedef short short8_t __attribute__((ext_vector_type(8)));
            const short8_t hv = {h[0][0], h[0][1], h[0][2], h[0][3], h[1][0], h[1][1], h[1][2], h[1][3]};
            b[cb] = __builtin_bit_cast(bf16x8_t, hv);
        }
    };
    auto mfmas = [&](const bf16x8_t *a, const bf16x8_t *b, int rb0, int rb1) {
#pragma unroll
        for (int rb = rb0; rb < rb1; ++rb)
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
                acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[rb], b[cb], acc[rb][cb], 0, 0, 0);
    };
    // Scheduling patterns (sched_group_barrier masks: 0x008 MFMA, 0x100 LDS read).
    auto interleave_16_12 = [&]() {          // 16 MFMAs; the 12 reads of the next fragments early
#pragma unroll
        for (int i = 0; i < 6; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 10, 0);
    };
    auto interleave_8_12 = [&]() {           // 8 MFMAs; 12 reads early
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    };

    const int nk = (K + BK - 1) / BK;
    constexpr int PER = XI + WI;                          // DMA instructions per stage per wave
    auto wait_stage = [&](int ahead) {                    // later stages still in flight
        if (ahead >= 3) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * PER) : "memory");
        else if (ahead == 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * PER) : "memory");
        else if (ahead == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(PER) : "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    };
#pragma unroll
    for (int st = 0; st < NS; ++st)
        if (st < nk) dma_stage(st, st);
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
                mfmas(af[cur], bfr[cur], 0, 4);
                interleave_16_12();
            } else {
                // Stage hand-off, between the two halves of the last MFMAs of
                // this stage: every wave has finished reading this stage from
                // LDS (lgkmcnt), stage kt+1 has landed for all waves after the
                // barrier, this stage's buffer is refilled with stage kt+NS,
                // and the first fragments of stage kt+1 are read under the
                // second half of the MFMAs (after the last stage they are read
                // and not used).
                mfmas(af[cur], bfr[cur], 0, 2);
                __builtin_amdgcn_sched_barrier(0);
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                wait_stage(min(NS - 2, nk - 2 - kt));
                __builtin_amdgcn_s_barrier();
                asm volatile("" ::: "memory");
                if (kt + NS < nk) dma_stage(kt + NS, buf);
                __builtin_amdgcn_sched_barrier(0);
                load_frags((kt + 1) % NS, 0, af[nxt], bfr[nxt]);
                mfmas(af[cur], bfr[cur], 2, 4);
                interleave_8_12();
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // ---- epilogue ----
    // Each wavefront moves one 32 x 128 block of its accumulators at a time
    // through its own LDS area; a lane then owns 8 consecutive columns of 8
    // rows, adds s * sum_j v[t][j] B[j][n] for rows with an adapter (B read in
    // rank octets, reused across the lane's rows while they share the slot)
    // and writes 16-byte rows of y after one rounding.
    constexpr int SLD = 132;                                      // staged row stride (floats)
    float *stage = reinterpret_cast<float *>(smem) + w * 32 * SLD;
    int32_t *s_t = reinterpret_cast<int32_t *>(reinterpret_cast<float *>(smem) + 4 * 32 * SLD);
    int32_t *s_id = s_t + GBM;
    int32_t *s_gq = s_id + GBM;
    float *s_sc = reinterpret_cast<float *>(s_gq + GBM);
    for (int i = tid; i < GBM; i += 256) {
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
    const int q = lane & 15, rr = lane >> 4;
    const int n = n0 + wn * 128 + 8 * q;
    const int R = g.max_rank;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
        __syncthreads();
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                stage[(8 * (e >> 2) + 4 * (lane >> 5) + (e & 3)) * SLD + cb * 32 + (lane & 31)] =
                    acc[rb][cb][e];
        __syncthreads();
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            int32_t tk[4], idk[4], gk[4];
            float sk[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int i = wm * 128 + rb * 32 + rr + 4 * (k + 4 * half);
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
                const float *src = stage + (rr + 4 * (k + 4 * half)) * SLD + 8 * q;
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
        g.n_tiles_m = (T + GBM - 1) / GBM;
        const int tiles = g.n_tiles_m * g.n_tiles_n;
        if (pool)
            hipLaunchKernelGGL((k_gemm_bf16<true, kGemmBK, kGemmNS>), dim3(tiles), dim3(256), 0, s, g);
        else
            hipLaunchKernelGGL((k_gemm_bf16<false, kGemmBK, kGemmNS>), dim3(tiles), dim3(256), 0, s, g);
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
