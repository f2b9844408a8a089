// Pieces shared by the bf16 and FP8 base GEMM kernels: kernel arguments,
// XCD-aware tile order, LDS DMA, swizzles, the fused low-rank pass on MFMA,
// the tile store, the split-K reduction and the tile/split planner.
#pragma once

#include "common.hpp"

namespace lora {

// One output slice of a grouped launch (projections that share x): its
// weight, output, width, first column tile in the launch's tile numbering,
// adapter pool (B, scale, rank) and the offset of its rank columns in v.
struct gemm_slice {
    const uint16_t *W;
    uint16_t *y;
    int32_t N, tn0;
    const uint16_t *b;
    const float *scale;
    const int32_t *rank;
    const int32_t *row0;
    int32_t v_off;
};

struct gemm_args {
    const uint16_t *x;
    const uint16_t *W;
    uint16_t *y;
    int32_t T, K, N;
    const int32_t *perm;
    const uint16_t *b;
    const float *scale;
    const int32_t *rank;
    const int32_t *row0;           // packed pool: first rank row per slot; padded: null
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
    const uint8_t *xq;             // FP8 base: E4M3 codes of the x rows [T][K]
    const uint8_t *wq;             // FP8 base: E4M3 codes of the W columns [N][K]
    const float *xs;               // FP8 base: row scales [T] (powers of two)
    const float *wsc;              // FP8 base: column scales [N] (powers of two)
    const int32_t *n_fused;        // mixed batches: rows at positions >= *n_fused get no low-rank term here
    int32_t col_strips;            // tile order: 1 = strips of kGroupN column tiles (see grouped_tile)
    int32_t n_slices;              // grouped launch: 0 (one output), else slices sl[0..n_slices)
    gemm_slice sl[kMaxSlices];     // column tiles numbered slice after slice
};

// Grouped launch: point g at the slice that owns global column tile tn and
// return the tile's index within that slice (identity without slices).  The
// slice is chosen with constant indices only, so the arguments stay in
// registers.
__device__ __forceinline__ int select_slice(gemm_args &g, int tn) {
    if (g.n_slices <= 0) return tn;
    gemm_slice q = g.sl[0];
#pragma unroll
    for (int i = 1; i < kMaxSlices; ++i)
        if (i < g.n_slices && tn >= g.sl[i].tn0) q = g.sl[i];
    g.W = q.W;
    g.y = q.y;
    g.N = q.N;
    g.b = q.b;
    g.scale = q.scale;
    g.rank = q.rank;
    g.row0 = q.row0;
    if (g.v) g.v += q.v_off;
    return tn - q.tn0;
}

// Tile order: workgroups are dispatched round-robin over the 8 XCDs (each
// with its own L2), so workgroup b runs on XCD b % 8.  Give each XCD a
// contiguous range of work items.  By default the range is walked in groups
// of kGroupM row tiles (down M first, then across N), so the 32 tiles an XCD
// runs at once (8 rows x 4 columns) share x rows and W columns in its L2,
// and each XCD owns a band of rows: x is read once, W by every XCD.  With
// col_strips the groups are kGroupN column tiles wide and span all row
// tiles (same 8 x 4 tiles at once), so each XCD owns a band of columns: W
// is read once, x by every XCD -- the cheaper split when x is the smaller
// operand (T < N), and every XCD gets every row tile, so rows that cost more
// (blocks of many adapters) do not pile up on the XCD of the last row band.
// With split-K the split index varies slowest.
constexpr int kXcds = 8, kGroupM = 8, kGroupN = 4;

__device__ __forceinline__ void grouped_tile(int v, int n_tiles_m, int n_tiles_n, int col_strips, int &tm,
                                             int &tn) {
    // one walk for both orders: groups of `gs` tiles along the banded
    // dimension (rows, or columns with col_strips), walking the other
    const int gs = col_strips ? kGroupN : kGroupM;
    const int nb = col_strips ? n_tiles_n : n_tiles_m;     // banded dimension
    const int nw = col_strips ? n_tiles_m : n_tiles_n;     // walked dimension
    const int per_group = gs * nw;
    const int grp = v / per_group;
    const int first = grp * gs;
    const int gb = min(gs, nb - first);
    const int in = v - grp * per_group;
    const int b = first + in % gb, wk = in / gb;
    tm = col_strips ? wk : b;
    tn = col_strips ? b : wk;
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
    grouped_tile(g.tile_base + tidx, g.n_tiles_m, g.n_tiles_n, g.col_strips, tm, tn);
}

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;

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
// other rows get zero operands).  s v is split into three bf16 parts, which
// carry its full fp32 value; B octets (8 ranks of one column, 16 bytes) are
// exactly the MFMA B operand of one lane.
// Operand mapping of v_mfma_f32_32x32x16_bf16 per lane l: A = row (l % 32),
// ranks 16 ks + 8 (l / 32) + 0..7; B = column (l % 32), the same ranks.

// Loads of one 16-rank step ks of adapter a for one lane: its row's 8 ranks
// of v (zeroed later unless the row belongs to a) and its columns' B octets
// (zero past the slot's rank or the last column).
// A slot's first rank row (see slot_row0), as a 32-bit index: loaded beside
// the slot's rank and scale, so the B loads below wait for one round trip.
__device__ __forceinline__ int32_t slot_row0_i(const gemm_args &g, int32_t a) {
    return a < 0 ? 0 : (g.row0 ? g.row0[a] : a * g.max_rank);
}

// A value every lane of the wavefront holds (taken from one lane by a
// shuffle), moved to a scalar register; the loads that depend on it become
// scalar loads, which keeps the vector registers for the accumulators.
__device__ __forceinline__ int32_t uniform_i(int32_t v) { return __builtin_amdgcn_readfirstlane(v); }

template <int CB>
__device__ __forceinline__ void lora_step_load(const gemm_args &g, int32_t a, int32_t ra, int32_t ro, bool mine,
                                               int32_t my_t, int ks, int half, int wcol0, int lane,
                                               float4 &v0, float4 &v1, uint4 (&bq)[CB]) {
    const int N = g.N;
    const int j0 = 16 * ks + 8 * half;
    const int oct = 2 * ks + half;
    const bool j_ok = a >= 0 && j0 < ra;              // octets past the slot's rank: not read
    const float *vp = g.v + (mine && j_ok ? (int64_t)my_t * g.v_stride + j0 : 0);
    v0 = *reinterpret_cast<const float4 *>(vp);
    v1 = *reinterpret_cast<const float4 *>(vp + 4);
    const int64_t abase = (int64_t)ro * N;            // slot a's first B octet row (ro = its first rank row)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        const int col = wcol0 + cb * 32 + (lane & 31);
        const bool ok = j_ok && col < N;
        bq[cb] = ldg16(g.b + (abase + ((int64_t)(ok ? oct : 0) * N + (ok ? col : 0)) * 8));
        const uint32_t m = ok ? ~0u : 0u;
        bq[cb] = make_uint4(bq[cb].x & m, bq[cb].y & m, bq[cb].z & m, bq[cb].w & m);
    }
}

// acc += (s_a v) B for one step from loaded operands; lanes with `use` false
// (rows of other adapters, ranks past the slot's) contribute zero.
template <int CB>
__device__ __forceinline__ void lora_step_mfma(f32x16_t (&acc)[CB], float sa, bool use, const float4 &v0,
                                               const float4 &v1, const uint4 (&bq)[CB]) {
    const uint32_t m = use ? ~0u : 0u;
    const float vv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    // s v as three bf16 parts: hi = bf16(f), mid = bf16(f - hi), lo =
    // bf16(f - hi - mid), each difference exact in fp32, so hi + mid + lo is
    // f to within 2^-27 |f| (below fp32's own rounding): v enters the expand
    // at fp32 precision, and the products with B's bf16 values are exact.
    uint32_t hi[4], md[4], lo[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float f0 = __uint_as_float(__float_as_uint(sa * vv[2 * e]) & m);
        const float f1 = __uint_as_float(__float_as_uint(sa * vv[2 * e + 1]) & m);
        hi[e] = pack_bf16x2(f0, f1);
        const float r0 = f0 - bf16_lo(hi[e]), r1 = f1 - bf16_hi(hi[e]);
        md[e] = pack_bf16x2(r0, r1);
        lo[e] = pack_bf16x2(r0 - bf16_lo(md[e]), r1 - bf16_hi(md[e]));
    }
    const bf16x8_t ahi = __builtin_bit_cast(bf16x8_t, make_uint4(hi[0], hi[1], hi[2], hi[3]));
    const bf16x8_t amd = __builtin_bit_cast(bf16x8_t, make_uint4(md[0], md[1], md[2], md[3]));
    const bf16x8_t alo = __builtin_bit_cast(bf16x8_t, make_uint4(lo[0], lo[1], lo[2], lo[3]));
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        const bf16x8_t bb = __builtin_bit_cast(bf16x8_t, bq[cb]);
        acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, bb, acc[cb], 0, 0, 0);
        acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(amd, bb, acc[cb], 0, 0, 0);
        acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, bb, acc[cb], 0, 0, 0);
    }
}

// The whole pass over a wavefront's RB x CB blocks.  Every block first takes
// the adapter of its lowest row with one (the only adapter of the block in
// segment order): the operands of KB rank steps of RG blocks are loaded
// before any of their MFMAs, so the wavefront waits for memory once per
// group, not once per block and step.  Rows of further adapters in a block
// (unsorted batches, or the short segments of decode rows in a sorted one)
// are then taken one adapter per block and round, for RF blocks at a time,
// so RF blocks' loads are in flight together; before that loop each lane
// loads its own row's slot rank and scale, and the loop takes an adapter's
// from the lane of its lowest row, so finding the next adapter needs no
// memory access.  RF = 0 keeps one block and one adapter at a time, with
// the slot's rank and scale read per adapter (kernels with no registers to
// spare).  Per block the MFMAs run in the same order either way: adapters
// by lowest row, ranks ascending.
template <int RB, int CB, int RG = 1, int KB = 1, int RF = 1>
__device__ __forceinline__ void lora_pass_impl(const gemm_args &g, f32x16_t (&acc)[RB][CB],
                                               const int32_t *s_t, const int32_t *s_id, int n0,
                                               int wrow0, int wcol0, int lane) {
    static_assert(RB % RG == 0 && (RF == 0 || RB % RF == 0), "row blocks come in whole groups");
    constexpr int RFG = RF > 0 ? RF : 1;
    const int half = lane >> 5;
    int32_t my_id[RB], my_t[RB], my_r[RB], my_o[RB], a0[RB], ra0[RB], ro0[RB];
    float my_s[RB], sa0[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int row = wrow0 + rb * 32 + (lane & 31);
        my_id[rb] = s_id[row];
        my_t[rb] = s_t[row];
        const uint64_t pend = __ballot(my_id[rb] >= 0) & 0xffffffffull;
        a0[rb] = uniform_i(pend ? __shfl(my_id[rb], __ffsll((long long)pend) - 1, 64) : -1);
        ra0[rb] = a0[rb] >= 0 ? g.rank[a0[rb]] : 0;
        sa0[rb] = a0[rb] >= 0 ? g.scale[a0[rb]] : 0.0f;
        ro0[rb] = slot_row0_i(g, a0[rb]);
    }
#pragma unroll
    for (int r0 = 0; r0 < RB; r0 += RG) {
        int nks = 0;
#pragma unroll
        for (int i = 0; i < RG; ++i) nks = max(nks, (ra0[r0 + i] + 15) >> 4);
        for (int ks0 = 0; ks0 < nks; ks0 += KB) {
            float4 v0[RG][KB], v1[RG][KB];
            uint4 bq[RG][KB][CB];
#pragma unroll
            for (int i = 0; i < RG; ++i)
#pragma unroll
                for (int u = 0; u < KB; ++u)
                    lora_step_load<CB>(g, a0[r0 + i], ra0[r0 + i], ro0[r0 + i], my_id[r0 + i] == a0[r0 + i],
                                       my_t[r0 + i], ks0 + u, half, wcol0, lane, v0[i][u], v1[i][u], bq[i][u]);
#pragma unroll
            for (int i = 0; i < RG; ++i)
#pragma unroll
                for (int u = 0; u < KB; ++u)
                    if (16 * (ks0 + u) < ra0[r0 + i])      // wave-uniform
                        lora_step_mfma<CB>(acc[r0 + i], sa0[r0 + i],
                                           my_id[r0 + i] == a0[r0 + i] && 16 * (ks0 + u) + 8 * half < ra0[r0 + i],
                                           v0[i][u], v1[i][u], bq[i][u]);
        }
    }
    if (RF == 0) {
        // further adapters of a block, one at a time (kernels at their
        // register limit: no per-row rank and scale)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            uint64_t pend = __ballot(my_id[rb] >= 0 && my_id[rb] != a0[rb]) & 0xffffffffull;
            while (pend) {
                const int first = __ffsll((long long)pend) - 1;
                const int32_t a = uniform_i(__shfl(my_id[rb], first, 64));
                pend &= ~(__ballot(my_id[rb] == a) & 0xffffffffull);
                const int32_t ra = g.rank[a];
                const float sa = g.scale[a];
                const int32_t ro = slot_row0_i(g, a);
                const bool mine = my_id[rb] == a;
                for (int ks = 0; ks * 16 < ra; ++ks) {
                    float4 v0, v1;
                    uint4 bq[CB];
                    lora_step_load<CB>(g, a, ra, ro, mine, my_t[rb], ks, half, wcol0, lane, v0, v1, bq);
                    lora_step_mfma<CB>(acc[rb], sa, mine && 16 * ks + 8 * half < ra, v0, v1, bq);
                }
            }
        }
        return;
    }
    // further adapters of the blocks, RF blocks at a time
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        my_r[rb] = my_id[rb] >= 0 ? g.rank[my_id[rb]] : 0;
        my_s[rb] = my_id[rb] >= 0 ? g.scale[my_id[rb]] : 0.0f;
        my_o[rb] = slot_row0_i(g, my_id[rb]);
    }
#pragma unroll
    for (int r0 = 0; r0 < RB; r0 += RFG) {
        uint64_t pend[RFG];
        uint64_t any = 0;
#pragma unroll
        for (int i = 0; i < RFG; ++i) {
            pend[i] = __ballot(my_id[r0 + i] >= 0 && my_id[r0 + i] != a0[r0 + i]) & 0xffffffffull;
            any |= pend[i];
        }
        while (any) {                                       // wave-uniform
            int32_t a[RFG], ra[RFG], ro[RFG];
            float sa[RFG];
            bool mine[RFG];
            int nks = 0;
            any = 0;
#pragma unroll
            for (int i = 0; i < RFG; ++i) {
                a[i] = -1;
                ra[i] = 0;
                ro[i] = 0;
                sa[i] = 0.0f;
                if (pend[i]) {
                    const int first = __ffsll((long long)pend[i]) - 1;
                    a[i] = uniform_i(__shfl(my_id[r0 + i], first, 64));
                    ra[i] = uniform_i(__shfl(my_r[r0 + i], first, 64));
                    ro[i] = uniform_i(__shfl(my_o[r0 + i], first, 64));
                    sa[i] = __int_as_float(uniform_i(__float_as_int(__shfl(my_s[r0 + i], first, 64))));
                    pend[i] &= ~(__ballot(my_id[r0 + i] == a[i]) & 0xffffffffull);
                }
                mine[i] = a[i] >= 0 && my_id[r0 + i] == a[i];
                nks = max(nks, (ra[i] + 15) >> 4);
                any |= pend[i];
            }
            for (int ks = 0; ks < nks; ++ks) {
                float4 v0[RFG], v1[RFG];
                uint4 bq[RFG][CB];
#pragma unroll
                for (int i = 0; i < RFG; ++i)
                    lora_step_load<CB>(g, a[i], ra[i], ro[i], mine[i], my_t[r0 + i], ks, half, wcol0, lane, v0[i],
                                       v1[i], bq[i]);
#pragma unroll
                for (int i = 0; i < RFG; ++i)
                    if (16 * ks < ra[i])                   // wave-uniform
                        lora_step_mfma<CB>(acc[r0 + i], sa[i], mine[i] && 16 * ks + 8 * half < ra[i], v0[i], v1[i],
                                           bq[i]);
            }
        }
    }
}

// Tile store after the K loop.
// Each wavefront moves one 32 x WN block of its accumulators at a time
// through its own LDS area; a lane then owns 8 consecutive columns of
// several rows and writes them with 16-byte stores after one rounding (the
// low-rank term is already in the accumulators).  In split-K mode the
// staged fp32 rows go to the partial buffer instead.  ADD (the expand-only
// pass) adds the tile to y instead: the block's y values load before its
// staging, and the sum is rounded once.  It is a template parameter so that
// the kernels that only store keep their registers (the y staging would
// make the FP8 LoRA kernel spill).
template <int BM, int BN, int WV, int WR, bool SPLIT, bool ADD, int RB, int CB>
__device__ __forceinline__ void gemm_store_tile(const gemm_args &g, f32x16_t (&acc)[RB][CB], float *smem_f,
                                                const int32_t *s_meta_t, int n0, int w, int lane,
                                                int tidx, int split) {
    static_assert(!(ADD && SPLIT), "split pieces store fp32 partials");
    constexpr int WM = BM / WR, WN = BN / (WV / WR), SLD = WN + 4;
    const int wm = w / (WV / WR), wn = w % (WV / WR);
    const int N = g.N;
    constexpr int QN = WN / 8, RPP = 64 / QN, PASSES = 32 / RPP;
    float *stage = smem_f + w * 32 * SLD;
    const int q = lane % QN, rr = lane / QN;
    const int n = n0 + wn * WN + 8 * q;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        // adding to y: this block's y values load before the staging below
        uint4 yq[ADD ? PASSES : 1];
        if constexpr (ADD) {
#pragma unroll
            for (int k = 0; k < PASSES; ++k) {
                const int i = wm * WM + rb * 32 + rr + RPP * k;
                const int32_t tk = s_meta_t ? s_meta_t[i] : -1;
                yq[k] = (tk >= 0 && n < N) ? ldg16(g.y + (int64_t)tk * N + n) : make_uint4(0u, 0u, 0u, 0u);
            }
        }
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
            const int32_t tk = s_meta_t ? s_meta_t[i] : 0;   // no row table: every row of a partial tile
            if (tk < 0 || n >= N) continue;
            const float *src = stage + (rr + RPP * k) * SLD + 8 * q;
            const float4 o0 = *reinterpret_cast<const float4 *>(src);
            const float4 o1 = *reinterpret_cast<const float4 *>(src + 4);
            if (SPLIT) {
                float *dst = g.partial + (((int64_t)tidx * g.splits + split) * BM + i) * BN + (n - n0);
                *reinterpret_cast<float4 *>(dst) = o0;
                *reinterpret_cast<float4 *>(dst + 4) = o1;
            } else {
                float o[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
                if constexpr (ADD) {
                    float yf[8];
                    vec16<LORA_BF16>::widen(yq[k], yf);
#pragma unroll
                    for (int e = 0; e < 8; ++e) o[e] += yf[e];
                }
                stg16(g.y + (int64_t)tk * N + n, vec16<LORA_BF16>::narrow(o));
            }
        }
    }
}

// Split-K reduction over the tiles of one split launch.  A workgroup takes
// RW = 2048 / BN rows of one tile; a thread owns 8 consecutive columns of one
// row: y[t][n..n+8] = bf16(sum_s partial[tile][s][r][c..c+8]
//                          (+ s_a * sum_j v[t][j] B_a[j][n..n+8])), t = perm[p].
// The partials of an element are summed in split order (deterministic).
// With VP (fused shrink) the rows' v are first summed from the K-range rank
// partials (in range order) into LDS (the GEMM has flagged bad ids).
template <bool LORA, bool VP, int BM, int BN>
__global__ void __launch_bounds__(256) k_splitk_reduce(gemm_args g0) {
    constexpr int RW = 2048 / BN, CPR = BN / 8, CHUNKS = BM / RW;
    constexpr int SP = 4;                                 // split partials loaded ahead
    constexpr int GP = 2;                                 // rank octets of B loaded ahead
    // Each XCD takes a contiguous range of (tile, row chunk) items, so it
    // owns whole tiles: the B columns of a tile are fetched into one L2 for
    // all of its rows (with chunk = XCD, every XCD read B for every column).
    const int per = gridDim.x / kXcds, rem = gridDim.x % kXcds;
    const int xcd = blockIdx.x % kXcds;
    const int item = xcd * per + min(xcd, rem) + blockIdx.x / kXcds;
    const int tidx = item / CHUNKS, chunk = item % CHUNKS;
    int tm, tn;
    grouped_tile(g0.tile_base + tidx, g0.n_tiles_m, g0.n_tiles_n, g0.col_strips, tm, tn);
    gemm_args g = g0;
    tn = select_slice(g, tn);
    const int T = g.T, N = g.N, R = g.max_rank;
    const int rloc = threadIdx.x / CPR, c = (threadIdx.x % CPR) * 8;
    const int r = chunk * RW + rloc;                      // row within the tile
    const int p = tm * BM + r, n = tn * BN + c;
    __shared__ __attribute__((aligned(16))) float s_v[VP ? RW * 64 : 1];
    // Loads that do not depend on the rank vector go out first, so their
    // latency overlaps the summing of the rank partials below: the row's
    // adapter, the first SP splits' partials, and the adapter's first GP rank
    // octets of B.  The B loads need the slot only, not its rank (a slot's
    // ranks past its own are zero in the pool and are not summed), so they
    // wait for one round trip (the id), not two.
    const int32_t t = (p < T && n < N) ? perm_row(g.perm, p, T) : -1;
    const bool fused = !g.n_fused || p < *g.n_fused;      // short-segment rows: expanded separately
    const int32_t raw = (LORA && t >= 0 && fused) ? g.ids[t] : -1;
    const bool slot_ok = raw >= 0 && raw < g.n_slots;
    float4 pa[SP], pb[SP];
    uint4 bq[GP][8];
    // B of a padded slot is prefetched from its first GP octets (at most
    // max_rank ranks, all inside the slot, zero past its rank); a packed
    // slot's octets past its capacity belong to the next slot, so there only
    // the first octet (every slot holds at least 8 ranks) is prefetched.
    const int gp_pre = g.row0 ? 1 : GP;
    int64_t bbase = 0;
    if (t >= 0) {
#pragma unroll
        for (int sidx = 0; sidx < SP; ++sidx)
            if (sidx < g.splits) {
                const float *src = g.partial + (((int64_t)tidx * g.splits + sidx) * BM + r) * BN + c;
                pa[sidx] = *reinterpret_cast<const float4 *>(src);
                pb[sidx] = *reinterpret_cast<const float4 *>(src + 4);
            }
        if (LORA && slot_ok) {
            bbase = slot_row0(g.row0, raw, R) * N;
#pragma unroll
            for (int gg = 0; gg < GP; ++gg)
                if (8 * gg < R && gg < gp_pre) {
                    const uint16_t *bp = g.b + (bbase + ((int64_t)gg * N + n) * 8);
#pragma unroll
                    for (int q = 0; q < 8; ++q) bq[gg][q] = ldg16(bp + q * 8);
                }
        }
    }
    int32_t rk = 0;
    float sc = 0.0f;
    if (LORA && t >= 0 && slot_ok) {
        rk = min(g.rank[raw], R);
        sc = g.scale[raw];
    }
    const int G = (rk + 7) >> 3;
    if (VP) {
        for (int e = threadIdx.x; e < RW * R; e += 256) {
            const int rr = e / R, j = e % R;
            const int pp = tm * BM + chunk * RW + rr;
            float sum = 0.0f;
            if (pp < T) {
                const int32_t tt = perm_row(g.perm, pp, T);
                if (tt >= 0)
                    for (int sidx = 0; sidx < g.splits; ++sidx)
                        sum += g.vpart[((int64_t)sidx * T + tt) * R + j];
            }
            s_v[rr * R + j] = sum;
        }
        __syncthreads();
    }
    if (t < 0) return;
    // partials summed in split order
    float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int sidx = 0; sidx < g.splits; ++sidx) {
        float4 a, b;
        if (sidx < SP) {
            a = pa[sidx];
            b = pb[sidx];
        } else {
            const float *src = g.partial + (((int64_t)tidx * g.splits + sidx) * BM + r) * BN + c;
            a = *reinterpret_cast<const float4 *>(src);
            b = *reinterpret_cast<const float4 *>(src + 4);
        }
        o[0] += a.x; o[1] += a.y; o[2] += a.z; o[3] += a.w;
        o[4] += b.x; o[5] += b.y; o[6] += b.z; o[7] += b.w;
    }
    if (LORA && rk > 0) {
        // s * sum_j v[j] B[j][n..n+8]: rank octets in order, ranks of an octet in order
        const float *vrow = VP ? s_v + rloc * R : g.v + (int64_t)t * g.v_stride;
        float d[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int gg = 0; gg < G; ++gg) {
            const float4 v0 = *reinterpret_cast<const float4 *>(vrow + gg * 8);
            const float4 v1 = *reinterpret_cast<const float4 *>(vrow + gg * 8 + 4);
            const uint16_t *bp = g.b + (bbase + ((int64_t)gg * N + n) * 8);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                uint4 bw;
                if (gg < GP && gg < gp_pre) {
#pragma unroll
                    for (int u = 0; u < GP; ++u)
                        if (u == gg) bw = bq[u][q];
                } else {
                    bw = ldg16(bp + q * 8);
                }
                float bf[8];
                vec16<LORA_BF16>::widen(bw, bf);
                float a = d[q];
                a = fmaf(v0.x, bf[0], a); a = fmaf(v0.y, bf[1], a);
                a = fmaf(v0.z, bf[2], a); a = fmaf(v0.w, bf[3], a);
                a = fmaf(v1.x, bf[4], a); a = fmaf(v1.y, bf[5], a);
                a = fmaf(v1.z, bf[6], a); a = fmaf(v1.w, bf[7], a);
                d[q] = a;
            }
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) o[q] = fmaf(sc, d[q], o[q]);
    }
    stg16(g.y + (int64_t)t * N + n, vec16<LORA_BF16>::narrow(o));
}

// Column bands per XCD (col_strips) for wide grids whose x is the smaller
// operand.  Measured on the layer sets: 112 column tiles (70B gate, up)
// -12% (bf16) and -29% (FP8) per call; 32-56 column tiles +1-4%.
inline bool col_strips_pay(int T, int N, int n_tiles_n) { return T < N && n_tiles_n >= 64; }

// Tile configuration and K split for one GEMM shape (bf16 or FP8).
struct gemm_plan {
    int bm, bn;
    int n_dp;          // tiles computed whole (with the fused expand), from tile 0
    int tail;          // tiles after those, computed as split-K pieces + reduction
    int splits, k_chunk;
};

inline int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// Largest tile that still gives close to one workgroup per CU.  When the last
// round of tiles would leave most CUs idle (a tail of at most 160 of 256),
// those tail tiles are split over K so every CU takes a share.  Grids that
// stay small (few token rows) split K for all tiles.  Split-K needs room for
// the fp32 partials in the workspace.  K ranges are multiples of kgran
// elements (one K step of the kernel).
inline int tiles_n(const int32_t *Ns, int nN, int bn) {
    int t = 0;
    for (int i = 0; i < nN; ++i) t += ceil_div(Ns[i], bn);
    return t;
}

inline gemm_plan plan_gemm(int T, int K, const int32_t *Ns, int nN, size_t partial_bytes, int kgran = 64,
                           bool wide_small = false) {
    static const int cfg[4][2] = {{256, 256}, {256, 128}, {128, 128}, {128, 64}};
    for (int c = 0; c < 4; ++c) {
        const int bm = cfg[c][0], bn = cfg[c][1];
        const int tiles = ceil_div(T, bm) * tiles_n(Ns, nN, bn);
        // 208-223 of the largest tiles still fill the chip in one round
        // better than twice as many half tiles in two (2240 x 4096 x 6144:
        // 216 tiles of 256 x 256 7% faster than 432 of 256 x 128)
        if (tiles < 224 && !(c == 0 && tiles >= 208)) continue;
        gemm_plan p{bm, bn, tiles, 0, 1, K};
        const int full = tiles / 256 * 256, rem = tiles - full;
        if (full > 0 && rem > 0 && rem <= 160 && K >= 1024) {
            int sp = 256 / rem;
            if (sp > kMaxGemmSplit) sp = kMaxGemmSplit;
            if (sp > K / 512) sp = K / 512;
            while (sp > 1 && (size_t)sp * rem * bm * bn * 4 > partial_bytes) --sp;
            if (sp >= 2) {
                const int kc = ceil_div(ceil_div(K, sp), kgran) * kgran;
                p = gemm_plan{bm, bn, full, rem, ceil_div(K, kc), kc};
            }
        }
        return p;
    }
    // Small grid (decode-sized T): split K, on 128 x 128 tiles.  Their x and
    // W stages are 32 KB, a fifth less than one 256-row tile of 64 columns
    // (which reads W once but x four times as often), so four stages fit in
    // LDS; the two row tiles of a column run on one XCD and share W through
    // its L2.  wide_small asks for the 256 x 64 tiles (T <= 256): twice the
    // column tiles, which the fused shrink needs for max ranks 32 and 64.
    const bool wide = T <= 256 && wide_small;
    const int bm = wide ? 256 : 128, bn = wide ? 64 : 128;
    const int tiles = ceil_div(T, bm) * tiles_n(Ns, nN, bn);
    int splits = ceil_div(256, tiles);
    const int max_by_k = K / 256 > 0 ? K / 256 : 1;
    if (splits > max_by_k) splits = max_by_k;
    if (splits > kMaxGemmSplit) splits = kMaxGemmSplit;
    while (splits > 1 && (size_t)splits * tiles * bm * bn * 4 > partial_bytes) --splits;
    if (splits <= 1) {
        const int t2 = ceil_div(T, 128) * tiles_n(Ns, nN, 64);
        return t2 > tiles ? gemm_plan{128, 64, t2, 0, 1, K} : gemm_plan{bm, bn, tiles, 0, 1, K};
    }
    const int k_chunk = ceil_div(ceil_div(K, splits), kgran) * kgran;
    return {bm, bn, 0, tiles, ceil_div(K, k_chunk), k_chunk};
}

// One output of width N.
inline gemm_plan plan_gemm(int T, int K, int N, size_t partial_bytes, int kgran = 64,
                           bool wide_small = false) {
    const int32_t n = N;
    return plan_gemm(T, K, &n, 1, partial_bytes, kgran, wide_small);
}

}  // namespace lora
