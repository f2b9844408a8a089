// a3 (+ a5 fused) -- base GEMM y = x W over all token rows, optionally with
// the expand y += s_a v[t] B_a folded into the epilogue so y is written once.
//
// The base product is shared by every request and runs once over all tokens
// ("Multi-LoRA Serving: Architecture for Thousands of Adapters", section "How
// multi-LoRA serving works"; "LoRAX, in depth", section "Computing a batch
// that mixes adapters"; "Serving LoRA adapters ...", Step 4: the base layer
// runs first, then the LoRA output is added).
//
// bf16 kernel (gfx950, v_mfma_f32_32x32x16_bf16, fp32 accumulate):
//   * BM x BN output tile (256x256, 256x128, 128x128 or 128x64), 4 wavefronts
//     in a 2 x 2 grid, each owning (BM/2) x (BN/2) outputs.
//   * K step BK, NS LDS stages.  Both tiles are loaded with DMA
//     (global_load_lds: global memory straight into LDS, no registers), stored
//     unpadded with XOR-swizzled 16-byte chunks; A fragments are ds_read_b128
//     of x rows, B fragments ds_read_b64_tr_b16 (transposing reads) of the
//     n-contiguous W tile.
//   * Rows may be visited through `perm` (segment order), gathering x rows on
//     load and scattering y rows on store; nothing is materialised.
//   * Epilogue: fp32 accumulator (+ s_a * sum_j v[t][j] B_a[j][n] for rows
//     with an adapter, B read in rank octets), one rounding to bf16 (nearest
//     even), 16-byte stores.
//   * Split-K (small grids): each workgroup sums a K range and writes fp32
//     partials in sorted-row order; k_splitk_reduce adds them in split order
//     (deterministic, no atomics) and applies the same epilogue.
#include "gemm_common.hpp"

namespace lora {

template <int BM, int BN, int BK, int NS, bool SH, int WV = 4, int WR = 2> struct gemm_cfg {
    // WV wavefronts in a WR x (WV/WR) grid; each owns a WM x WN tile
    static constexpr int WM = BM / WR, WN = BN / (WV / WR); // per-wavefront tile
    static constexpr int RB = WM / 32, CB = WN / 32;        // 32x32 MFMA blocks per wavefront
    static constexpr int XCH = BK / 8, WCH = BN / 8;        // 16-byte chunks per LDS row
    static constexpr int XSTAGE = BM * BK, WSTAGE = BK * BN;
    // fused shrink: per stage, 64/R rows x R ranks x BK k of A^T (8 BK chunks)
    static constexpr int ACH = BK / 8, ASTAGE = SH ? 64 * BK : 0;
    static constexpr int STAGE = XSTAGE + WSTAGE + ASTAGE;  // uint16 elements per ring stage
    static constexpr int XI = BM * XCH / (64 * WV), WI = BK * WCH / (64 * WV);   // DMA instructions per wave
    static constexpr int AI = SH ? BK / (8 * WV) : 0;              // A^T stage: 8 BK chunks over WV waves
    static constexpr int SLD = WN + 4;                      // epilogue staging row stride (floats)
    static constexpr int EPI = WV * 32 * SLD * 4;            // epilogue LDS bytes
    static constexpr int LDS = NS * STAGE * 2 > EPI ? NS * STAGE * 2 : EPI;
};

template <bool LORA, int BM, int BN, int BK, int NS, bool SPLIT, bool SH = false, int WV = 4, int WR = 2>
__global__ void __launch_bounds__(WV * 64) k_gemm_bf16(gemm_args g) {
    static_assert(!SH || SPLIT, "the fused shrink runs in split-K mode");
    static_assert(!SH || (WV == 4 || WV == 8), "the fused shrink maps 4 or 8 threads to a (row, rank) pair");
    // The single-stage LoRA instantiation is the expand-only pass
    // (launch_expand_tiles: no K steps): it adds its tile to y.
    constexpr bool ADD = LORA && !SPLIT && NS == 1;
    typedef gemm_cfg<BM, BN, BK, NS, SH, WV, WR> C;
    constexpr int WM = C::WM, WN = C::WN, RB = C::RB, CB = C::CB;
    constexpr int XCH = C::XCH, WCH = C::WCH, XSTAGE = C::XSTAGE, WSTAGE = C::WSTAGE;
    constexpr int XI = C::XI, WI = C::WI, AI = C::AI, ACH = C::ACH, STAGE = C::STAGE;
    __shared__ __attribute__((aligned(1024))) uint16_t smem[C::LDS / 2];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w / (WV / WR), wn = w % (WV / WR);
    int tm, tn, split, tidx;
    tile_of(blockIdx.x, gridDim.x, g, tm, tn, split, tidx);
    tn = select_slice(g, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int K = g.K, N = g.N, T = g.T;
    const int k_begin = SPLIT ? split * g.k_chunk : 0;
    const int k_end = SPLIT ? min(K, k_begin + g.k_chunk) : K;

    // DMA plan.  x stage: BM rows x XCH chunks; wave w issues XI instructions of
    // 64 chunks, chunk c = (w * XI + j) * 64 + lane at row c / XCH, slot c % XCH,
    // holding the row's chunk slot ^ swz_x(row).
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
    // W stage: BK rows x WCH chunks, chunk c at row c / WCH, slot c % WCH,
    // holding the row's chunk slot ^ swz_w(row).
    int wrow[WI], wcol[WI];
#pragma unroll
    for (int j = 0; j < WI; ++j) {
        const int c = (w * WI + j) * 64 + lane;
        const int k = c / WCH, slot = c % WCH;
        wrow[j] = k;
        wcol[j] = n0 + 8 * (slot ^ swz_w<BN>(k));
    }
    // Fused shrink (decode-sized batches): this workgroup also computes the
    // rank partials v[t][j] over its K range for the rows
    // t = m0 + tn + i * n_tiles_n (i < 64 / R) that fall in its row tile.
    // The A^T slices of those rows' adapters ride along in every DMA stage
    // (chunk c: row i, rank j, 8 k), so x, already in LDS for the base
    // product, is read from HBM once.  Only the slot's first r rank rows are
    // read from the pool; the stage slots of ranks past r take the zero
    // vector, so A's bytes follow each adapter's true rank.
    int64_t arow[AI > 0 ? AI : 1];
    int acol[AI > 0 ? AI : 1];
    const int R = g.max_rank;
    if (SH) {
#pragma unroll
        for (int jj = 0; jj < AI; ++jj) {
            const int c = (w * AI + jj) * 64 + lane;
            const int i = c / (R * ACH), rem = c % (R * ACH);
            const int j = rem / ACH, q = rem % ACH;
            const int t = m0 + tn + i * g.n_tiles_n;
            int64_t off = -1;
            if (t < T && t - m0 < BM) {
                const int32_t id = g.ids[t];
                if (id >= 0 && id < g.n_slots && j < g.rank[id]) off = (slot_row0(g.row0, id, R) + j) * K;
            }
            arow[jj] = off;
            acol[jj] = 8 * q;
        }
    }
    // Bad ids of those rows (outside [-1, n_slots) or an empty slot) are
    // flagged once, by the first K range; the slot's rank is loaded now and
    // checked after the K loop.
    int32_t fl_t = -1, fl_id = -1, fl_rank = 1;
    if (SH && split == 0 && tid < 64 / R) {
        const int t = m0 + tn + tid * g.n_tiles_n;
        if (t < T && t - m0 < BM) {
            fl_t = t;
            fl_id = g.ids[t];
            if (fl_id >= 0 && fl_id < g.n_slots) fl_rank = g.rank[fl_id];
        }
    }
    auto dma_stage = [&](int kt, int buf) {
        uint16_t *xs = smem + buf * STAGE;
        uint16_t *wsm = xs + XSTAGE;
        uint16_t *as = wsm + WSTAGE;
        const int k0 = k_begin + kt * BK;
#pragma unroll
        for (int j = 0; j < XI; ++j) {
            const int kk = k0 + xcol[j];
            const void *src = (xrow[j] >= 0 && kk < k_end) ? (const void *)(g.x + xrow[j] + kk)
                                                             : (const void *)g_zero16;
            dma16(src, xs + (w * XI + j) * 64 * 8);
        }
#pragma unroll
        for (int j = 0; j < WI; ++j) {
            const int k = k0 + wrow[j];
            const void *src = (k < k_end && wcol[j] < N) ? (const void *)(g.W + (int64_t)k * N + wcol[j])
                                                          : (const void *)g_zero16;
            dma16(src, wsm + (w * WI + j) * 64 * 8);
        }
#pragma unroll
        for (int jj = 0; jj < AI; ++jj) {
            const int k = k0 + acol[jj];
            const void *src = (arow[jj] >= 0 && k < k_end) ? (const void *)(g.a + arow[jj] + k)
                                                            : (const void *)g_zero16;
            dma16(src, as + (w * AI + jj) * 64 * 8);
        }
    };

    f32x16_t acc[RB][CB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[rb][cb][e] = 0.0f;

    // fragment addressing
    const int fr = lane & 31, fk = lane >> 5;           // A: row within block, k-group
    const int grp = lane >> 4, s16 = lane & 15;         // B: 16-lane group, lane in group
    const int b_kofs = 8 * (grp >> 1) + (s16 >> 2);     // + 16 ks + 4 inst
    const int b_col = 16 * (grp & 1) + 4 * (s16 & 3);   // + wn*WN + cb*32
    constexpr int KS = BK / 16;                         // MFMA k-substeps per stage
    bf16x8_t af[2][RB], bfr[2][CB];
    auto load_frags = [&](int buf, int ks, bf16x8_t *a, bf16x8_t *b) {
        const uint16_t *xs = smem + buf * STAGE;
        const uint16_t *wsm = xs + XSTAGE;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const int r = wm * WM + rb * 32 + fr;
            const int c = (2 * ks + fk) ^ swz_x<BK>(r);
            a[rb] = *reinterpret_cast<const bf16x8_t *>(xs + r * BK + 8 * c);
        }
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            const int col = wn * WN + cb * 32 + b_col;          // multiple of 4
            short4_t h[2];
#pragma unroll
            for (int inst = 0; inst < 2; ++inst) {
                const int k = 16 * ks + 4 * inst + b_kofs;
                const int chunk = (col >> 3) ^ swz_w<BN>(k);
                const uint16_t *addr = wsm + k * BN + 8 * chunk + (col & 7);
                h[inst] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_short4_t *)(reinterpret_cast<uintptr_t>(addr)));
            }
            const short8_t hv = {h[0][0], h[0][1], h[0][2], h[0][3], h[1][0], h[1][1], h[1][2], h[1][3]};
            b[cb] = __builtin_bit_cast(bf16x8_t, hv);
        }
    };
    auto mfmas = [&](const bf16x8_t *a, const bf16x8_t *b, int rb0, int rb1) {
#pragma unroll
        for (int rb = rb0; rb < rb1; ++rb)
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
                acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[rb], b[cb], acc[rb][cb], 0, 0, 0);
    };
    constexpr int NREAD = RB + 2 * CB;                  // LDS reads per k-substep

    // Per-row metadata of a whole tile (token row; usable adapter slot or
    // -1).  Split pieces keep none: they write every row of their partial
    // tile (rows past T hold zeros) and the reduction skips those rows.
    int32_t *s_meta_t = nullptr, *s_meta_id = nullptr;
    if constexpr (!SPLIT) {
        __shared__ int32_t s_meta_t_buf[BM], s_meta_id_buf[BM];
        s_meta_t = s_meta_t_buf;
        s_meta_id = s_meta_id_buf;
        // mixed batches: rows from GEMM position n_fused on (short segments)
        // get their low-rank term from the separate per-row expand
        const int32_t n_fused = (LORA && g.n_fused) ? *g.n_fused : T;
        for (int i = tid; i < BM; i += WV * 64) {
            const int p = m0 + i;
            const int32_t t = (p < T) ? perm_row(g.perm, p, T) : -1;
            int32_t id = -1;
            if (LORA && t >= 0 && (!g.n_fused || p < n_fused)) {
                const int32_t raw = g.ids[t];
                if (raw >= 0 && raw < g.n_slots && g.rank[raw] > 0) id = raw;
            }
            s_meta_t[i] = (ADD && id < 0) ? -1 : t;   // adding: rows without a term stay untouched
            s_meta_id[i] = id;
        }
    }

    const int nk = (k_end - k_begin + BK - 1) / BK;
    constexpr int PER = XI + WI + AI;                     // DMA instructions per stage per wave
    // fused shrink: thread = (row slot i, rank j, k group gq) of a stage:
    // 64 pairs of row slot and rank, WV groups of the stage's k per pair
    const int sh_i = tid / (WV * R), sh_j = (tid / WV) % R, sh_gq = tid % WV;
    const int sh_t = SH && tn + sh_i * g.n_tiles_n < BM ? m0 + tn + sh_i * g.n_tiles_n : T;
    float sh_acc = 0.0f;
    // A stage's shrink operands are read from LDS at the stage hand-off and
    // multiplied after the stage's first MFMA group, so the FMAs never wait
    // on LDS in front of the matrix cores.
    constexpr int SHC = ACH / WV > 0 ? ACH / WV : 1;     // chunks of 8 k per thread and stage
    uint4 sh_xq[SHC], sh_aq[SHC];
    auto shrink_load = [&](int buf) {
        if (!SH || sh_t >= T) return;
        const uint16_t *xs = smem + buf * STAGE;
        const uint16_t *as = xs + XSTAGE + WSTAGE;
        const int r = sh_t - m0;
#pragma unroll
        for (int h = 0; h < SHC; ++h) {                    // this thread's chunks of 8 k
            const int c = SHC * sh_gq + h;
            sh_xq[h] = *reinterpret_cast<const uint4 *>(xs + r * BK + 8 * (c ^ swz_x<BK>(r)));
            sh_aq[h] = *reinterpret_cast<const uint4 *>(as + ((sh_i * R + sh_j) * ACH + c) * 8);
        }
    };
    auto shrink_fma = [&]() {
        if (!SH || sh_t >= T) return;
#pragma unroll
        for (int h = 0; h < SHC; ++h) {
            float xf[8], af[8];
            vec16<LORA_BF16>::widen(sh_xq[h], xf);
            vec16<LORA_BF16>::widen(sh_aq[h], af);
#pragma unroll
            for (int e = 0; e < 8; ++e) sh_acc = fmaf(xf[e], af[e], sh_acc);
        }
    };
    static_assert((NS - 1) * PER <= 63, "vmcnt counts at most 63 loads");
    // vmcnt immediates of the stage counts a ring of NS stages can reach
    // (counts past 63 only for depths this ring never has)
    constexpr int V1 = PER, V2 = 2 * PER > 63 ? 63 : 2 * PER, V3 = 3 * PER > 63 ? 63 : 3 * PER;
    constexpr int V4 = 4 * PER > 63 ? 63 : 4 * PER, V5 = 5 * PER > 63 ? 63 : 5 * PER;
    auto wait_stage = [&](int ahead) {                    // later stages still in flight
        if (ahead >= 5) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(V5) : "memory");
        else if (ahead == 4) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(V4) : "memory");
        else if (ahead == 3) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(V3) : "memory");
        else if (ahead == 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(V2) : "memory");
        else if (ahead == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(V1) : "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    };
#pragma unroll
    for (int st = 0; st < NS; ++st)
        if (st < nk) dma_stage(st, st);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // The low-rank term goes into the accumulators before the K loop, while
    // the first stages load.  (Split-K tiles leave it to the reduction, whose
    // one-thread-per-row-chunk layout hides the per-row loads of B.)
    if (LORA && !SPLIT)
        lora_pass_impl<RB, CB, (RB >= 2 ? 2 : 1), 1, (RB >= 2 ? 2 : 1)>(g, acc, s_meta_t, s_meta_id, n0, wm * WM, n0 + wn * WN,
                                                    lane);
    wait_stage(min(NS - 1, nk - 1));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    load_frags(0, 0, af[0], bfr[0]);
    if (SH && nk > 0) shrink_load(0);
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt % NS;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int cur = ks & 1, nxt = cur ^ 1;
            if (ks + 1 < KS) {
                load_frags(buf, ks + 1, af[nxt], bfr[nxt]);
                mfmas(af[cur], bfr[cur], 0, RB);
                sched_interleave<NREAD, RB * CB>();
                if (SH && ks == 0) shrink_fma();
            } else {
                // Stage hand-off, between the two halves of the last MFMAs of
                // this stage: every wave has finished reading this stage from
                // LDS (lgkmcnt), stage kt+1 has landed for all waves after the
                // barrier, this stage's buffer is refilled with stage kt+NS,
                // and the first fragments of stage kt+1 are read under the
                // second half of the MFMAs (after the last stage they are read
                // and not used).
                mfmas(af[cur], bfr[cur], 0, RB / 2);
                __builtin_amdgcn_sched_barrier(0);
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                wait_stage(min(NS - 2, nk - 2 - kt));
                __builtin_amdgcn_s_barrier();
                asm volatile("" ::: "memory");
                if (kt + NS < nk) dma_stage(kt + NS, buf);
                __builtin_amdgcn_sched_barrier(0);
                load_frags((kt + 1) % NS, 0, af[nxt], bfr[nxt]);
                if (SH && kt + 1 < nk) shrink_load((kt + 1) % NS);
                mfmas(af[cur], bfr[cur], RB / 2, RB);
                sched_interleave<NREAD, RB / 2 * CB>();
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (SH) {
        // rank partial of this K range: sum the WV k groups (adjacent lanes)
        float vsum = sh_acc;
#pragma unroll
        for (int o = 1; o < WV; o <<= 1) vsum += __shfl_xor(vsum, o, 64);
        if (sh_gq == 0 && sh_t < T) g.vpart[((int64_t)split * T + sh_t) * R + sh_j] = vsum;
        if (fl_t >= 0 && fl_id != -1 && !(fl_id >= 0 && fl_id < g.n_slots && fl_rank > 0))
            flag_bad_row(g.err, fl_t);
    }

    gemm_store_tile<BM, BN, WV, WR, SPLIT, ADD>(g, acc, reinterpret_cast<float *>(smem), s_meta_t, n0, w, lane,
                                              tidx, split);
}

struct gemm_f32_args {
    const float *x;
    const float *W;
    float *y;
    int32_t T, K, N;
    const int32_t *perm;
    const float *b;
    const float *scale;
    const int32_t *rank;
    const int32_t *row0;
    int32_t n_slots, max_rank;
    const int32_t *ids;
    const float *v;
    int32_t v_stride;
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
                r = min(g.rank[raw], g.max_rank);
                s = g.scale[raw];
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + tx * 4 + j;
            if (n >= N) continue;
            float val = acc[i][j];
            if (LORA && id >= 0) {
                const float *bq = g.b + (slot_row0(g.row0, id, g.max_rank) * N + (int64_t)n * 8);
                const float *vi = g.v + t * g.v_stride;
                float d = 0.0f;
                for (int q = 0; q < r; ++q) d = fmaf(vi[q], bq[(int64_t)(q >> 3) * N * 8 + (q & 7)], d);
                val = fmaf(s, d, val);
            }
            g.y[t * N + n] = val;
        }
    }
}

// NST, WVT: stages and wavefronts of the split-K pieces (their LDS holds no
// row tables).
template <int BM, int BN, int NS = 2, int WV = 4, int WR = 2, int BK = 64, int NST = NS, int WVT = WV>
static void launch_cfg(gemm_args g, const gemm_plan &pl, bool lora, hipStream_t s) {
    if (pl.n_dp > 0) {
        g.tile_base = 0;
        g.n_tiles = pl.n_dp;
        g.splits = 1;
        g.k_chunk = g.K;
        if (lora)
            hipLaunchKernelGGL((k_gemm_bf16<true, BM, BN, BK, NS, false, false, WV, WR>), dim3(pl.n_dp), dim3(WV * 64),
                               0, s, g);
        else
            hipLaunchKernelGGL((k_gemm_bf16<false, BM, BN, BK, NS, false, false, WV, WR>), dim3(pl.n_dp), dim3(WV * 64),
                               0, s, g);
    }
    if (pl.tail > 0) {
        g.tile_base = pl.n_dp;
        g.n_tiles = pl.tail;
        g.splits = pl.splits;
        g.k_chunk = pl.k_chunk;
        hipLaunchKernelGGL((k_gemm_bf16<false, BM, BN, BK, NST, true, false, WVT, WR>), dim3(pl.tail * pl.splits),
                           dim3(WVT * 64), 0, s, g);
        const dim3 rgrid(pl.tail * (BM / (2048 / BN)));
        if (lora)
            hipLaunchKernelGGL((k_splitk_reduce<true, false, BM, BN>), rgrid, dim3(256), 0, s, g);
        else
            hipLaunchKernelGGL((k_splitk_reduce<false, false, BM, BN>), rgrid, dim3(256), 0, s, g);
    }
}

// The fused shrink applies to decode-sized split-K plans (T <= 256): every
// row of a row tile must be one of the 64 / R rows that some column tile
// takes on.  128 x 128 tiles (four stages in LDS) where their column tiles
// cover the rows, else one 256-row tile of 64-column tiles (twice the
// column tiles: max ranks 32 and 64 with narrower outputs).
static bool fused_shrink_plan(int32_t T, int32_t d_in, int32_t d_out, int32_t max_rank, size_t partial_bytes,
                              gemm_plan &pl) {
    if (T <= 0 || T > 256) return false;
    if (max_rank != 8 && max_rank != 16 && max_rank != 32 && max_rank != 64) return false;
    for (int wide = 0; wide <= 1; ++wide) {
        pl = plan_gemm(T, d_in, d_out, partial_bytes, 64, wide == 1);
        if (pl.n_dp != 0 || pl.splits <= 1 || pl.splits > kMaxKSplit) continue;
        if (!(pl.bm == 128 && pl.bn == 128) && !(pl.bm == 256 && pl.bn == 64)) continue;
        if ((int64_t)ceil_div(d_out, pl.bn) * (64 / max_rank) >= (T < pl.bm ? T : pl.bm)) return true;
    }
    return false;
}

bool gemm_fused_shrink_ok(int32_t T, int32_t d_in, int32_t d_out, int32_t max_rank,
                          size_t partial_bytes) {
    gemm_plan pl;
    return fused_shrink_plan(T, d_in, d_out, max_rank, partial_bytes, pl);
}

lora_status_t launch_gemm_fused_shrink(const void *x, const void *W, void *y, int32_t T,
                                       const lora_pool_t *pool, const int32_t *ids, float *vpart,
                                       int32_t *err, float *partial, size_t partial_bytes,
                                       hipStream_t s) {
    gemm_args g{};
    g.x = (const uint16_t *)x;
    g.W = (const uint16_t *)W;
    g.y = (uint16_t *)y;
    g.T = T;
    g.K = pool->d_in;
    g.N = pool->d_out;
    g.perm = nullptr;
    g.b = (const uint16_t *)pool->b;
    g.scale = pool->scale;
    g.rank = pool->rank;
    g.row0 = pool->row0;
    g.n_slots = pool->n_slots;
    g.max_rank = pool->max_rank;
    g.ids = ids;
    g.v = nullptr;
    g.v_stride = pool->max_rank;
    gemm_plan pl;
    if (!fused_shrink_plan(T, g.K, g.N, g.max_rank, partial_bytes, pl)) return LORA_ERR_UNSUPPORTED;
    g.n_tiles_m = ceil_div(T, pl.bm);
    g.n_tiles_n = ceil_div(g.N, pl.bn);
    g.tile_base = 0;
    g.n_tiles = pl.tail;
    g.splits = pl.splits;
    g.k_chunk = pl.k_chunk;
    g.partial = partial;
    g.a = (const uint16_t *)pool->a;
    g.vpart = vpart;
    g.err = err;
    if (pl.bm == 128) {
        hipLaunchKernelGGL((k_gemm_bf16<false, 128, 128, 64, 4, true, true, 8, 2>), dim3(pl.tail * pl.splits),
                           dim3(512), 0, s, g);
        hipLaunchKernelGGL((k_splitk_reduce<true, true, 128, 128>), dim3(pl.tail * (128 / 16)), dim3(256), 0, s,
                           g);
    } else {
        hipLaunchKernelGGL((k_gemm_bf16<false, 256, 64, 64, 3, true, true>), dim3(pl.tail * pl.splits),
                           dim3(256), 0, s, g);
        hipLaunchKernelGGL((k_splitk_reduce<true, true, 256, 64>), dim3(pl.tail * (256 / 32)), dim3(256), 0, s,
                           g);
    }
    return hip_status(hipGetLastError());
}

// Whether slices of these widths gain from one grouped launch: not when each
// alone already runs whole tiles of the largest size (measured: two 28672-
// or 14336-wide slices run 3-9% slower grouped than one after the other),
// but when some slice alone would take smaller tiles or split K.
bool gemm_grouping_pays(int32_t T, int32_t K, const int32_t *Ns, int32_t n, size_t partial_bytes) {
    if (n < 2) return false;
    for (int i = 0; i < n; ++i) {
        const gemm_plan pl = plan_gemm(T, K, Ns[i], partial_bytes);
        if (pl.bm != 256 || pl.bn != 256 || pl.tail != 0) return true;
    }
    return false;
}

// The separate expand of rows in the GEMM order on the matrix cores: the
// LoRA kernel with no K steps runs its expand pass (s v in three bf16 parts
// times B, fp32 accumulators) on each 256 x 256 tile of rows and adds the
// tile to y (read, fp32 sum, one rounding to bf16).  Rows without a usable
// adapter, and rows at GEMM positions from *n_fused on (short segments, left
// to the per-row expand), are neither read nor written.
lora_status_t launch_expand_tiles(const float *v, int32_t v_stride, int32_t T, const lora_pool_t &p,
                                  const int32_t *ids, const int32_t *gperm, const int32_t *n_fused, void *y,
                                  hipStream_t s) {
    if (p.dtype != LORA_BF16 || T <= 0) return LORA_ERR_INVALID_ARGUMENT;
    gemm_args g{};
    g.T = T;
    g.K = 0;
    g.N = p.d_out;
    g.y = (uint16_t *)y;
    g.perm = gperm;
    g.n_fused = n_fused;
    g.b = (const uint16_t *)p.b;
    g.scale = p.scale;
    g.rank = p.rank;
    g.row0 = p.row0;
    g.n_slots = p.n_slots;
    g.max_rank = p.max_rank;
    g.ids = ids;
    g.v = v;
    g.v_stride = v_stride;
    g.n_tiles_m = ceil_div(T, 256);
    g.n_tiles_n = ceil_div(p.d_out, 256);
    g.tile_base = 0;
    g.n_tiles = g.n_tiles_m * g.n_tiles_n;
    g.splits = 1;
    g.k_chunk = 0;
    g.col_strips = col_strips_pay(T, p.d_out, g.n_tiles_n);
    // no K steps: one small stage keeps the LDS at the epilogue's size (the
    // single-stage instantiation is the one that adds its tile to y)
    hipLaunchKernelGGL((k_gemm_bf16<true, 256, 256, 16, 1, false, false, 8, 2>), dim3(g.n_tiles), dim3(512), 0, s, g);
    return hip_status(hipGetLastError());
}

// Base products of several outputs that share x (projections of one
// layer), each with its own adapter pool and rank columns v + v_off[i], in
// one launch: the column tiles of all slices form one grid, so a layer of
// narrow projections still fills the chip with large tiles.
lora_status_t launch_gemm_grouped(const void *x, const void *const *W, void *const *y, int32_t T,
                                  const lora_pool_t *pools, int32_t n, const int32_t *ids, const float *v,
                                  const int32_t *v_off, int32_t v_stride, const int32_t *perm, float *partial,
                                  size_t partial_bytes, hipStream_t s, const int32_t *n_fused) {
    if (n < 1 || n > kMaxSlices || pools[0].dtype != LORA_BF16) return LORA_ERR_INVALID_ARGUMENT;
    int32_t Ns[kMaxSlices];
    for (int i = 0; i < n; ++i) Ns[i] = pools[i].d_out;
    gemm_args g{};
    g.x = (const uint16_t *)x;
    g.T = T;
    g.K = pools[0].d_in;
    g.perm = perm;
    g.n_slots = pools[0].n_slots;
    g.max_rank = pools[0].max_rank;
    g.ids = ids;
    g.v = v;
    g.v_stride = v_stride;
    g.n_fused = n_fused;
    const gemm_plan pl = plan_gemm(T, g.K, Ns, n, partial ? partial_bytes : 0);
    g.n_slices = n;
    int tn0 = 0;
    for (int i = 0; i < n; ++i) {
        g.sl[i] = gemm_slice{(const uint16_t *)W[i], (uint16_t *)y[i], Ns[i], tn0, (const uint16_t *)pools[i].b,
                             pools[i].scale, pools[i].rank, pools[i].row0, v_off[i]};
        tn0 += ceil_div(Ns[i], pl.bn);
    }
    // fields a slice overrides start at slice 0 (never read before selection)
    g.W = g.sl[0].W;
    g.y = g.sl[0].y;
    g.N = g.sl[0].N;
    g.b = g.sl[0].b;
    g.scale = g.sl[0].scale;
    g.rank = g.sl[0].rank;
    g.row0 = g.sl[0].row0;
    g.n_tiles_m = ceil_div(T, pl.bm);
    g.n_tiles_n = tn0;
    g.col_strips = col_strips_pay(T, tn0 * pl.bn, tn0);
    g.partial = partial;
    if (pl.bm == 256 && pl.bn == 256) launch_cfg<256, 256, 2, 8>(g, pl, true, s);
    else if (pl.bm == 256 && pl.bn == 128) launch_cfg<256, 128, 2, 8>(g, pl, true, s);
    else if (pl.bn == 128) launch_cfg<128, 128, 2, 4, 2, 64, 4, 8>(g, pl, true, s);
    else launch_cfg<128, 64>(g, pl, true, s);
    return hip_status(hipGetLastError());
}

lora_status_t launch_gemm(const void *x, const void *W, void *y, int32_t T, int32_t d_in,
                          int32_t d_out, int32_t dtype, const lora_pool_t *pool,
                          const int32_t *ids, const float *v, int32_t v_stride,
                          const int32_t *perm, float *partial, size_t partial_bytes, hipStream_t s,
                          const int32_t *n_fused) {
    if (dtype == LORA_BF16) {
        gemm_args g{};
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
        g.row0 = pool ? pool->row0 : nullptr;
        g.n_slots = pool ? pool->n_slots : 0;
        g.max_rank = pool ? pool->max_rank : 0;
        g.ids = ids;
        g.v = v;
        g.v_stride = v_stride;
        g.n_fused = n_fused;
        const gemm_plan pl = plan_gemm(T, d_in, d_out, partial ? partial_bytes : 0);
        g.n_tiles_m = ceil_div(T, pl.bm);
        g.n_tiles_n = ceil_div(d_out, pl.bn);
        g.col_strips = col_strips_pay(T, d_out, g.n_tiles_n);
        g.partial = partial;
        g.a = nullptr;
        g.vpart = nullptr;
        g.err = nullptr;
        const bool lora = pool != nullptr;
        // 256-row tiles and the 128 x 128 split pieces run 8 wavefronts (two
        // per SIMD: one issues MFMAs while the other waits on LDS or the
        // barrier); other tiles 4.
        if (pl.bm == 256 && pl.bn == 256) launch_cfg<256, 256, 2, 8>(g, pl, lora, s);
        else if (pl.bm == 256 && pl.bn == 128) launch_cfg<256, 128, 2, 8>(g, pl, lora, s);
        else if (pl.bn == 128) launch_cfg<128, 128, 2, 4, 2, 64, 4, 8>(g, pl, lora, s);
        else launch_cfg<128, 64>(g, pl, lora, s);
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
        g.row0 = pool ? pool->row0 : nullptr;
        g.n_slots = pool ? pool->n_slots : 0;
        g.max_rank = pool ? pool->max_rank : 0;
        g.ids = ids;
        g.v = v;
        g.v_stride = v_stride;
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
