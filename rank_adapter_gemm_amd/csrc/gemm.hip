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
#include "common.hpp"

namespace lora {

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
    const float *v;                // [T][v_stride] fp32, this pool's ranks at columns 0..max_rank-1
    int32_t v_stride;
    int32_t n_tiles_m, n_tiles_n;
    int32_t tile_base, n_tiles;    // this launch: tiles [tile_base, tile_base + n_tiles) in tile order
    int32_t splits, k_chunk;       // split-K: number of K ranges and their length
    float *partial;                // split-K: fp32 [n_tiles][splits][BM][BN] (tile-major)
    const uint16_t *a;             // fused shrink: the pool's A^T [n_slots][max_rank][K]
    float *vpart;                  // fused shrink: fp32 [splits][T][max_rank] rank partials
    int32_t *err;                  // fused shrink: the workspace error word
};

// Tile order: workgroups are dispatched round-robin over the 8 XCDs (each
// with its own L2), so workgroup b runs on XCD b % 8.  Give each XCD a
// contiguous range of work items, walked in groups of GROUP_M row tiles (down
// M first, then across N) so the tiles resident on one XCD share x rows and W
// columns in its L2.  With split-K the split index varies slowest.
constexpr int kXcds = 8, kGroupM = 8;

__device__ __forceinline__ void grouped_tile(int v, int n_tiles_m, int n_tiles_n, int &tm, int &tn) {
    const int per_group = kGroupM * n_tiles_n;
    const int grp = v / per_group;
    const int first_m = grp * kGroupM;
    const int gm = min(kGroupM, n_tiles_m - first_m);
    const int in = v - grp * per_group;
    tm = first_m + in % gm;
    tn = in / gm;
}

// Work item of workgroup b in a launch of `total` workgroups covering
// n_tiles tiles (from tile_base, in tile order) times the split count.
// Returns the tile (tm, tn), the split, and the launch-local tile index.
__device__ __forceinline__ void tile_of(int b, int total, const gemm_args &g, int &tm, int &tn,
                                        int &split, int &tidx) {
    const int q = total / kXcds, r = total % kXcds;
    const int x = b % kXcds, slot = b / kXcds;
    int v = x * q + min(x, r) + slot;
    split = v / g.n_tiles;
    tidx = v - split * g.n_tiles;
    grouped_tile(g.tile_base + tidx, g.n_tiles_m, g.n_tiles_n, tm, tn);
}

// A 16-byte zero vector in global memory: the source of the DMA loads of
// masked lanes (rows past T, k past K, columns past N), so those LDS slots
// hold zeros.
__device__ __attribute__((aligned(16))) uint4 g_zero16[1];

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));
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

// XOR swizzles of the 16-byte chunk index inside an LDS row: conflict-free
// fragment reads for 32 and for 64 LDS banks.
//   x rows (BK bf16): ds_read_b128 of 16 consecutive rows at one chunk.
//   W rows (BN bf16): ds_read_b64_tr_b16 of 4 rows x 64 bytes per half-wave.
template <int BK> __device__ __forceinline__ int swz_x(int r) {
    return BK == 64 ? ((r ^ (r >> 3)) & 7) : (((r >> 2) ^ (r >> 1)) & 3);
}
template <int BN> __device__ __forceinline__ int swz_w(int k) {
    // rows of >= 16 chunks: 0, 6, 10, 12 for k % 4 = 0..3; rows of 8 chunks: 0, 2, 4, 6
    return BN >= 128 ? ((0xCA60 >> (4 * (k & 3))) & 0xF) : 2 * (k & 3);
}

// Scheduling pattern for one group of NMFMA MFMAs and the NREAD LDS reads of
// the next fragments (sched_group_barrier masks: 0x100 LDS read, 0x008 MFMA):
// the reads go out early, at least two per MFMA.
template <int NREAD, int NMFMA> __device__ __forceinline__ void sched_interleave() {
    constexpr int per = (NREAD + NMFMA - 1) / NMFMA > 2 ? (NREAD + NMFMA - 1) / NMFMA : 2;
#pragma unroll
    for (int i = 0; i < NMFMA; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, per, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
}

// The expand on MFMA: acc[rb][cb] += (s_a v[t]) B_a for the rows of each
// distinct adapter a among a wavefront's 32-row block (found with ballots;
// other rows get zero operands).  v is split into bf16 high and low parts so
// the fp32 intermediate keeps about 16 mantissa bits; B octets (8 ranks of
// one column, 16 bytes) are exactly the MFMA B operand of one lane.
// Operand mapping of v_mfma_f32_32x32x16_bf16 per lane l: A = row (l % 32),
// ranks 16 ks + 8 (l / 32) + 0..7; B = column (l % 32), the same ranks.
template <int RB, int CB>
__device__ __forceinline__ void lora_pass_impl(const gemm_args &g, f32x16_t (&acc)[RB][CB],
                                               const int32_t *s_t, const int32_t *s_id, int n0,
                                               int wrow0, int wcol0, int lane) {
    const int R = g.max_rank, RO = g.max_rank / 8, N = g.N;
    const int half = lane >> 5;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int row = wrow0 + rb * 32 + (lane & 31);
        const int32_t my_id = s_id[row];
        const int32_t my_t = s_t[row];
        uint64_t pend = __ballot(my_id >= 0) & 0xffffffffull;
        while (pend) {
            const int first = __ffsll((long long)pend) - 1;
            const int32_t a = __shfl(my_id, first, 64);
            pend &= ~(__ballot(my_id == a) & 0xffffffffull);
            const int32_t ra = g.rank[a];
            const float sa = g.scale[a];
            const uint32_t vm = (my_id == a) ? ~0u : 0u;
            const float *vrow = g.v + (int64_t)(my_id == a ? my_t : 0) * g.v_stride;
            for (int ks = 0; ks * 16 < ra; ++ks) {
                const int j0 = 16 * ks + 8 * half;
                const int oct = 2 * ks + half;
                const bool j_ok = j0 < ra;              // octets past the slot's rank: not read
                const float *vp = vrow + (j_ok ? j0 : 0);
                float4 v0 = *reinterpret_cast<const float4 *>(vp);
                float4 v1 = *reinterpret_cast<const float4 *>(vp + 4);
                uint4 bq[CB];
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) {
                    const int col = wcol0 + cb * 32 + (lane & 31);
                    const bool ok = j_ok && col < N;
                    bq[cb] = ldg16(g.b + ((int64_t)a * R * N + ((int64_t)(ok ? oct : 0) * N + (ok ? col : 0)) * 8));
                    const uint32_t m = ok ? ~0u : 0u;
                    bq[cb] = make_uint4(bq[cb].x & m, bq[cb].y & m, bq[cb].z & m, bq[cb].w & m);
                }
                const uint32_t m = j_ok ? vm : 0u;
                float vv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
                uint32_t hi[4], lo[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float f0 = __uint_as_float(__float_as_uint(sa * vv[2 * e]) & m);
                    const float f1 = __uint_as_float(__float_as_uint(sa * vv[2 * e + 1]) & m);
                    const uint32_t h0 = f32_to_bf16_bits(f0), h1 = f32_to_bf16_bits(f1);
                    hi[e] = h0 | (h1 << 16);
                    lo[e] = f32_to_bf16_bits(f0 - __uint_as_float(h0 << 16)) |
                            (f32_to_bf16_bits(f1 - __uint_as_float(h1 << 16)) << 16);
                }
                const bf16x8_t ahi = __builtin_bit_cast(bf16x8_t, make_uint4(hi[0], hi[1], hi[2], hi[3]));
                const bf16x8_t alo = __builtin_bit_cast(bf16x8_t, make_uint4(lo[0], lo[1], lo[2], lo[3]));
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) {
                    const bf16x8_t bb = __builtin_bit_cast(bf16x8_t, bq[cb]);
                    acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, bb, acc[rb][cb], 0, 0, 0);
                    acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, bb, acc[rb][cb], 0, 0, 0);
                }
            }
        }
    }
}

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
    static constexpr int AI = SH ? BK / 32 : 0;
    static constexpr int SLD = WN + 4;                      // epilogue staging row stride (floats)
    static constexpr int EPI = WV * 32 * SLD * 4;            // epilogue LDS bytes
    static constexpr int LDS = NS * STAGE * 2 > EPI ? NS * STAGE * 2 : EPI;
};

template <bool LORA, int BM, int BN, int BK, int NS, bool SPLIT, bool SH = false, int WV = 4, int WR = 2>
__global__ void __launch_bounds__(WV * 64) k_gemm_bf16(gemm_args g) {
    static_assert(!SH || SPLIT, "the fused shrink runs in split-K mode");
    static_assert(!SH || WV == 4, "the fused shrink maps 256 threads");
    typedef gemm_cfg<BM, BN, BK, NS, SH, WV, WR> C;
    constexpr int WM = C::WM, WN = C::WN, RB = C::RB, CB = C::CB;
    constexpr int XCH = C::XCH, WCH = C::WCH, XSTAGE = C::XSTAGE, WSTAGE = C::WSTAGE;
    constexpr int XI = C::XI, WI = C::WI, AI = C::AI, ACH = C::ACH, STAGE = C::STAGE;
    __shared__ __attribute__((aligned(1024))) uint16_t smem[C::LDS / 2];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w / (WV / WR), wn = w % (WV / WR);
    int tm, tn, split, tidx;
    tile_of(blockIdx.x, gridDim.x, g, tm, tn, split, tidx);
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
    // Fused shrink (decode-sized batches, one M tile): this workgroup also
    // computes the rank partials v[t][j] over its K range for the rows
    // t = tn + i * n_tiles_n (i < 64 / R).  The A^T slices of those rows'
    // adapters ride along in every DMA stage (chunk c: row i, rank j, 8 k),
    // so x, already in LDS for the base product, is read from HBM once.
    int64_t arow[AI > 0 ? AI : 1];
    int acol[AI > 0 ? AI : 1];
    const int R = g.max_rank;
    if (SH) {
#pragma unroll
        for (int jj = 0; jj < AI; ++jj) {
            const int c = (w * AI + jj) * 64 + lane;
            const int i = c / (R * ACH), rem = c % (R * ACH);
            const int j = rem / ACH, q = rem % ACH;
            const int t = tn + i * g.n_tiles_n;
            int64_t off = -1;
            if (t < T) {
                const int32_t id = g.ids[t];
                if (id >= 0 && id < g.n_slots && j < g.rank[id]) off = ((int64_t)id * R + j) * K;
            }
            arow[jj] = off;
            acol[jj] = 8 * q;
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

    // Per-row metadata of the tile (token row; usable adapter slot or -1).
    __shared__ int32_t s_meta_t[BM], s_meta_id[BM];
    for (int i = tid; i < BM; i += WV * 64) {
        const int p = m0 + i;
        const int32_t t = (p < T) ? perm_row(g.perm, p, T) : -1;
        int32_t id = -1;
        if (LORA && t >= 0) {
            const int32_t raw = g.ids[t];
            if (raw >= 0 && raw < g.n_slots && g.rank[raw] > 0) id = raw;
        }
        s_meta_t[i] = t;
        s_meta_id[i] = id;
    }

    const int nk = (k_end - k_begin + BK - 1) / BK;
    constexpr int PER = XI + WI + AI;                     // DMA instructions per stage per wave
    // fused shrink: thread = (row slot i, rank j, 16-k group gq) of a stage
    const int sh_i = tid / (4 * R), sh_j = (tid >> 2) % R, sh_gq = tid & 3;
    const int sh_t = SH ? tn + sh_i * g.n_tiles_n : -1;
    float sh_acc = 0.0f;
    auto shrink_stage = [&](int buf) {
        if (!SH || sh_t >= T) return;
        const uint16_t *xs = smem + buf * STAGE;
        const uint16_t *as = xs + XSTAGE + WSTAGE;
        const int r = sh_t - m0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int c = 2 * sh_gq + h;
            const uint4 xq = *reinterpret_cast<const uint4 *>(xs + r * BK + 8 * (c ^ swz_x<BK>(r)));
            const uint4 aq = *reinterpret_cast<const uint4 *>(as + ((sh_i * R + sh_j) * ACH + c) * 8);
            float xf[8], af[8];
            vec16<LORA_BF16>::widen(xq, xf);
            vec16<LORA_BF16>::widen(aq, af);
#pragma unroll
            for (int e = 0; e < 8; ++e) sh_acc = fmaf(xf[e], af[e], sh_acc);
        }
    };
    auto wait_stage = [&](int ahead) {                    // later stages still in flight
        if (ahead >= 3) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * PER) : "memory");
        else if (ahead == 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * PER) : "memory");
        else if (ahead == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(PER) : "memory");
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
        lora_pass_impl<RB, CB>(g, acc, s_meta_t, s_meta_id, n0, wm * WM, n0 + wn * WN, lane);
    wait_stage(min(NS - 1, nk - 1));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    load_frags(0, 0, af[0], bfr[0]);
    if (SH && nk > 0) shrink_stage(0);
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
                if (SH && kt + 1 < nk) shrink_stage((kt + 1) % NS);
                mfmas(af[cur], bfr[cur], RB / 2, RB);
                sched_interleave<NREAD, RB / 2 * CB>();
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (SH) {
        // rank partial of this K range: sum the four 16-k groups (adjacent lanes)
        float vsum = sh_acc;
        vsum += __shfl_xor(vsum, 1, 64);
        vsum += __shfl_xor(vsum, 2, 64);
        if (sh_gq == 0 && sh_t < T) g.vpart[((int64_t)split * T + sh_t) * R + sh_j] = vsum;
    }

    // ---- epilogue ----
    // Each wavefront moves one 32 x WN block of its accumulators at a time
    // through its own LDS area; a lane then owns 8 consecutive columns of
    // several rows and writes them with 16-byte stores after one rounding (the
    // low-rank term is already in the accumulators).  In split-K mode the
    // staged fp32 rows go to the partial buffer instead.
    constexpr int SLD = C::SLD;
    constexpr int QN = WN / 8, RPP = 64 / QN, PASSES = 32 / RPP;
    float *stage = reinterpret_cast<float *>(smem) + w * 32 * SLD;
    const int q = lane % QN, rr = lane / QN;
    const int n = n0 + wn * WN + 8 * q;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        __syncthreads();
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                stage[(8 * (e >> 2) + 4 * (lane >> 5) + (e & 3)) * SLD + cb * 32 + (lane & 31)] =
                    acc[rb][cb][e];
        __syncthreads();
#pragma unroll
        for (int k = 0; k < PASSES; ++k) {
            const int i = wm * WM + rb * 32 + rr + RPP * k;
            const int32_t tk = s_meta_t[i];
            if (tk < 0 || n >= N) continue;
            const float *src = stage + (rr + RPP * k) * SLD + 8 * q;
            const float4 o0 = *reinterpret_cast<const float4 *>(src);
            const float4 o1 = *reinterpret_cast<const float4 *>(src + 4);
            if (SPLIT) {
                float *dst = g.partial + (((int64_t)tidx * g.splits + split) * BM + i) * BN + (n - n0);
                *reinterpret_cast<float4 *>(dst) = o0;
                *reinterpret_cast<float4 *>(dst + 4) = o1;
            } else {
                const float o[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
                stg16(g.y + (int64_t)tk * N + n, vec16<LORA_BF16>::narrow(o));
            }
        }
    }
}

// s * sum_j v[j] B[j][n..n+8] for one row: G rank octets of slot `id`, 8
// consecutive columns starting at n (B in rank octets [R/8][N][8]).
__device__ __forceinline__ void lora_delta8(const uint16_t *b, int32_t id, int32_t R, int32_t N,
                                            int32_t n, int32_t G, const float *vrow, float *d) {
    for (int gg = 0; gg < G; ++gg) {
        const uint16_t *bp = b + ((int64_t)id * R * N + ((int64_t)gg * N + n) * 8);
        const float4 v0 = *reinterpret_cast<const float4 *>(vrow + gg * 8);
        const float4 v1 = *reinterpret_cast<const float4 *>(vrow + gg * 8 + 4);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            float bf[8];
            vec16<LORA_BF16>::widen(ldg16(bp + c * 8), bf);
            float a = d[c];
            a = fmaf(v0.x, bf[0], a); a = fmaf(v0.y, bf[1], a);
            a = fmaf(v0.z, bf[2], a); a = fmaf(v0.w, bf[3], a);
            a = fmaf(v1.x, bf[4], a); a = fmaf(v1.y, bf[5], a);
            a = fmaf(v1.z, bf[6], a); a = fmaf(v1.w, bf[7], a);
            d[c] = a;
        }
    }
}

// Split-K reduction over the tiles of one split launch.  A workgroup takes
// RW = 2048 / BN rows of one tile; a thread owns 8 consecutive columns of one
// row: y[t][n..n+8] = bf16(sum_s partial[tile][s][r][c..c+8]
//                          (+ s_a * sum_j v[t][j] B_a[j][n..n+8])), t = perm[p].
// The partials of an element are summed in split order (deterministic).
// With VP (fused shrink) the rows' v are first summed from the K-range rank
// partials (in range order) into LDS, and the first column tile flags bad ids.
template <bool LORA, bool VP, int BM, int BN>
__global__ void __launch_bounds__(256) k_splitk_reduce(gemm_args g) {
    constexpr int RW = 2048 / BN, CPR = BN / 8, CHUNKS = BM / RW;
    const int tidx = blockIdx.x / CHUNKS, chunk = blockIdx.x % CHUNKS;
    int tm, tn;
    grouped_tile(g.tile_base + tidx, g.n_tiles_m, g.n_tiles_n, tm, tn);
    const int T = g.T, N = g.N, R = g.max_rank;
    const int r = chunk * RW + threadIdx.x / CPR, c = (threadIdx.x % CPR) * 8;
    const int p = tm * BM + r, n = tn * BN + c;
    __shared__ __attribute__((aligned(16))) float s_v[VP ? RW * 64 : 1];
    if (VP) {
        for (int e = threadIdx.x; e < RW * R; e += 256) {
            const int rr = e / R, j = e % R;
            const int pp = tm * BM + chunk * RW + rr;
            float sum = 0.0f;
            if (pp < T) {
                const int32_t tt = perm_row(g.perm, pp, T);
                if (tt >= 0) {
                    for (int sidx = 0; sidx < g.splits; ++sidx)
                        sum += g.vpart[((int64_t)sidx * T + tt) * R + j];
                    if (j == 0 && tn == 0) {
                        const int32_t raw = g.ids[tt];
                        const bool ok = raw == -1 || (raw >= 0 && raw < g.n_slots && g.rank[raw] > 0);
                        if (!ok) flag_bad_row(g.err, tt);
                    }
                }
            }
            s_v[rr * R + j] = sum;
        }
        __syncthreads();
    }
    if (p >= T || n >= N) return;
    const int32_t t = perm_row(g.perm, p, T);
    if (t < 0) return;
    float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int sidx = 0; sidx < g.splits; ++sidx) {
        const float *src = g.partial + (((int64_t)tidx * g.splits + sidx) * BM + r) * BN + c;
        const float4 a = *reinterpret_cast<const float4 *>(src);
        const float4 b = *reinterpret_cast<const float4 *>(src + 4);
        o[0] += a.x; o[1] += a.y; o[2] += a.z; o[3] += a.w;
        o[4] += b.x; o[5] += b.y; o[6] += b.z; o[7] += b.w;
    }
    if (LORA) {
        const int32_t raw = g.ids[t];
        if (raw >= 0 && raw < g.n_slots) {
            const int32_t rk = g.rank[raw];
            if (rk > 0) {
                float d[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
                lora_delta8(g.b, raw, R, N, n, (rk + 7) >> 3,
                            VP ? s_v + (r - chunk * RW) * R : g.v + (int64_t)t * g.v_stride, d);
                const float sc = g.scale[raw];
#pragma unroll
                for (int q = 0; q < 8; ++q) o[q] = fmaf(sc, d[q], o[q]);
            }
        }
    }
    stg16(g.y + (int64_t)t * N + n, vec16<LORA_BF16>::narrow(o));
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
                const float *vi = g.v + t * g.v_stride;
                float d = 0.0f;
                for (int q = 0; q < r; ++q) d = fmaf(vi[q], bq[(int64_t)(q >> 3) * N * 8 + (q & 7)], d);
                val = fmaf(s, d, val);
            }
            g.y[t * N + n] = val;
        }
    }
}

// Tile configuration and K split for one bf16 GEMM shape.
struct gemm_plan {
    int bm, bn;
    int n_dp;          // tiles computed whole (with the fused expand), from tile 0
    int tail;          // tiles after those, computed as split-K pieces + reduction
    int splits, k_chunk;
};

static int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// Largest tile that still gives close to one workgroup per CU.  When the last
// round of tiles would leave most CUs idle (a tail of at most 160 of 256),
// those tail tiles are split over K so every CU takes a share.  Grids that
// stay small (few token rows) split K for all tiles.  Split-K needs room for
// the fp32 partials in the workspace.
static gemm_plan plan_gemm(int T, int K, int N, size_t partial_bytes) {
    static const int cfg[4][2] = {{256, 256}, {256, 128}, {128, 128}, {128, 64}};
    for (int c = 0; c < 4; ++c) {
        const int bm = cfg[c][0], bn = cfg[c][1];
        const int tiles = ceil_div(T, bm) * ceil_div(N, bn);
        if (tiles < 224) continue;
        gemm_plan p{bm, bn, tiles, 0, 1, K};
        const int full = tiles / 256 * 256, rem = tiles - full;
        if (full > 0 && rem > 0 && rem <= 160 && K >= 1024) {
            int sp = 256 / rem;
            if (sp > kMaxGemmSplit) sp = kMaxGemmSplit;
            if (sp > K / 512) sp = K / 512;
            while (sp > 1 && (size_t)sp * rem * bm * bn * 4 > partial_bytes) --sp;
            if (sp >= 2) {
                const int kc = ceil_div(ceil_div(K, sp), 64) * 64;
                p = gemm_plan{bm, bn, full, rem, ceil_div(K, kc), kc};
            }
        }
        return p;
    }
    // Small grid (decode-sized T): split K.  One 256-row tile covers T <= 256,
    // so W is read once; narrow 64-column tiles keep the number of fp32
    // partial copies (written and read back) low for the same grid size.
    const int bm = T <= 256 ? 256 : 128, bn = T <= 256 ? 64 : 128;
    const int tiles = ceil_div(T, bm) * ceil_div(N, bn);
    int splits = ceil_div(256, tiles);
    const int max_by_k = K / 256 > 0 ? K / 256 : 1;
    if (splits > max_by_k) splits = max_by_k;
    if (splits > kMaxGemmSplit) splits = kMaxGemmSplit;
    while (splits > 1 && (size_t)splits * tiles * bm * bn * 4 > partial_bytes) --splits;
    if (splits <= 1) {
        const int t2 = ceil_div(T, 128) * ceil_div(N, 64);
        return t2 > tiles ? gemm_plan{128, 64, t2, 0, 1, K} : gemm_plan{bm, bn, tiles, 0, 1, K};
    }
    const int k_chunk = ceil_div(ceil_div(K, splits), 64) * 64;
    return {bm, bn, 0, tiles, ceil_div(K, k_chunk), k_chunk};
}

template <int BM, int BN, int NS = 2, int WV = 4, int WR = 2, int BK = 64>
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
        hipLaunchKernelGGL((k_gemm_bf16<false, BM, BN, BK, NS, true, false, WV, WR>), dim3(pl.tail * pl.splits),
                           dim3(WV * 64), 0, s, g);
        const dim3 rgrid(pl.tail * (BM / (2048 / BN)));
        if (lora)
            hipLaunchKernelGGL((k_splitk_reduce<true, false, BM, BN>), rgrid, dim3(256), 0, s, g);
        else
            hipLaunchKernelGGL((k_splitk_reduce<false, false, BM, BN>), rgrid, dim3(256), 0, s, g);
    }
}

// The fused shrink applies to the decode-sized split-K plan (one 256-row
// tile, 64-column tiles): every row must be one of the 64 / R rows that some
// column tile takes on.
bool gemm_fused_shrink_ok(int32_t T, int32_t d_in, int32_t d_out, int32_t max_rank,
                          size_t partial_bytes) {
    if (T <= 0 || T > 256) return false;
    if (max_rank != 8 && max_rank != 16 && max_rank != 32 && max_rank != 64) return false;
    const gemm_plan pl = plan_gemm(T, d_in, d_out, partial_bytes);
    if (pl.n_dp != 0 || pl.splits <= 1 || pl.bm != 256 || pl.bn != 64) return false;
    if (pl.splits > kMaxKSplit) return false;
    return (int64_t)ceil_div(d_out, pl.bn) * (64 / max_rank) >= T;
}

lora_status_t launch_gemm_fused_shrink(const void *x, const void *W, void *y, int32_t T,
                                       const lora_pool_t *pool, const int32_t *ids, float *vpart,
                                       int32_t *err, float *partial, size_t partial_bytes,
                                       hipStream_t s) {
    gemm_args g;
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
    g.n_slots = pool->n_slots;
    g.max_rank = pool->max_rank;
    g.ids = ids;
    g.v = nullptr;
    g.v_stride = pool->max_rank;
    const gemm_plan pl = plan_gemm(T, g.K, g.N, partial_bytes);
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
    hipLaunchKernelGGL((k_gemm_bf16<false, 256, 64, 64, 3, true, true>), dim3(pl.tail * pl.splits), dim3(256),
                       0, s, g);
    hipLaunchKernelGGL((k_splitk_reduce<true, true, 256, 64>), dim3(pl.tail * (256 / 32)), dim3(256), 0, s, g);
    return hip_status(hipGetLastError());
}

lora_status_t launch_gemm(const void *x, const void *W, void *y, int32_t T, int32_t d_in,
                          int32_t d_out, int32_t dtype, const lora_pool_t *pool,
                          const int32_t *ids, const float *v, int32_t v_stride,
                          const int32_t *perm, float *partial, size_t partial_bytes, hipStream_t s) {
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
        g.v_stride = v_stride;
        const gemm_plan pl = plan_gemm(T, d_in, d_out, partial ? partial_bytes : 0);
        g.n_tiles_m = ceil_div(T, pl.bm);
        g.n_tiles_n = ceil_div(d_out, pl.bn);
        g.partial = partial;
        g.a = nullptr;
        g.vpart = nullptr;
        g.err = nullptr;
        const bool lora = pool != nullptr;
        // 256-row tiles run 8 wavefronts (two per SIMD: one issues MFMAs while
        // the other waits on LDS or the barrier); smaller tiles 4.
        if (pl.bm == 256 && pl.bn == 256) launch_cfg<256, 256, 2, 8>(g, pl, lora, s);
        else if (pl.bm == 256 && pl.bn == 128) launch_cfg<256, 128, 2, 8>(g, pl, lora, s);
        else if (pl.bm == 256) launch_cfg<256, 64, 3>(g, pl, lora, s);
        else if (pl.bn == 128) launch_cfg<128, 128>(g, pl, lora, s);
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
