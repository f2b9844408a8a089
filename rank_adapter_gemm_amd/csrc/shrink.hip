// a4 -- shrink: v[t, 0:r] = x[t,:] A_a  (fp32 result of rank width).
//
// "Serving multiple LoRAs: segmented matrix multiplies and adapter
// scheduling", section "Not merging the weights, computing in batches": the
// low-rank term is computed in two products, and this is the first, which
// maps each token row from d_in values to r; "Serving LoRA adapters: from the
// model name to the wrapped layer", Step 4: its result is kept in an fp32
// buffer of rank width.  The BGMV form gathers each token's own A; the SGMV
// form walks adapter-contiguous segments so one read of A serves a segment.
//
// Two kernels:
//  * k_shrink_rows  (BGMV): one 512-thread workgroup per token row; x[t] is
//    read once with 16-byte coalesced loads, the slot's first r A^T rows (its
//    true rank) are gathered in batches of independent loads, each lane keeps
//    per-rank partial sums, which are reduced across the wavefront with a
//    transposing butterfly of cross-lane swaps and then across the 8
//    wavefronts through LDS.  fp32 or bf16 inputs.
//  * k_shrink_grouped (SGMV, bf16): work blocks of up to 32 rows of one
//    adapter segment (rows through perm), MFMA 16x16x32 with fp32 accumulate;
//    K is split over the 4 wavefronts (LDS reduction) and optionally over
//    workgroups (partials, then a fixed-order reduction: deterministic).
#include "common.hpp"
#include "fp8_common.hpp"

namespace lora {

// Pools that share x, ids, n_slots, d_in, max_rank and dtype (projections
// fed by the same input): one shrink reads x once for all of them and
// writes v[t][s * max_rank + j] for slice s.
struct slice_set {
    const void *a[kMaxSlices];
    const int32_t *rank[kMaxSlices];
    const int32_t *row0[kMaxSlices];     // packed pools: first rank row per slot; padded: null
    int32_t n;
};

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

// Q8 (FP8-base forward, bf16 rows, no perm): the workgroup also writes the
// row's E4M3 codes and power-of-two scale, as k_quant_rows_fp8 does (amax
// over the row, then the codes), after the shrink, with x from cache: one
// launch and one HBM read of x for both.
// The shrink of the row at position p (through perm), by one 512-thread
// workgroup (every thread calls it with the same p).
template <int DT, int RM, bool Q8>
__device__ __forceinline__ void shrink_row(const typename elem<DT>::T *__restrict__ x, int32_t T, int32_t d_in,
                                           const slice_set &ss, int32_t n_slots, int32_t max_rank,
                                           const int32_t *__restrict__ ids, const int32_t *__restrict__ perm,
                                           float *__restrict__ v, int32_t *err, uint8_t *__restrict__ xq,
                                           float *__restrict__ xs, int p) {
    static_assert(!Q8 || DT == LORA_BF16, "the FP8 base quantizes bf16 rows");
    typedef typename elem<DT>::T E;
    constexpr int VN = vec16<DT>::n;
    constexpr int NW = 8;                                 // wavefronts per workgroup
    constexpr int RC = RM < 16 ? RM : (RM > 32 ? 8 : 16); // rank rows per batch of loads
    __shared__ float s_red[NW][RM];
    const int t = perm_row(perm, p, T);
    if (t < 0) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int32_t id = ids[t];
    const bool in_range = id >= 0 && id < n_slots;
    const int VS = ss.n * max_rank;                       // v row stride
    const E *xt = x + (size_t)t * d_in;
    // One slice after the other: x[t] comes from HBM for the first and from
    // the cache for the rest.
    for (int sl = 0; sl < ss.n; ++sl) {
    float *vt = v + (size_t)t * VS + sl * max_rank;
    if (!in_range) {                                      // uniform: a base row (or a bad id)
        for (int j = tid; j < max_rank; j += NW * 64) vt[j] = 0.0f;
        continue;
    }
    // Only the slot's first r rank rows are read (its rank and, in a packed
    // pool, its first row come one round trip after the id): the bytes of A
    // follow the adapter's true rank, not the pool's max_rank.
    const int32_t r = min(ss.rank[sl][id], max_rank);
    const E *At = reinterpret_cast<const E *>(ss.a[sl]) + slot_row0(ss.row0[sl], id, max_rank) * d_in;
    float acc[RM];
#pragma unroll
    for (int j = 0; j < RM; ++j) acc[j] = 0.0f;
    const int nvec = d_in / VN;
    for (int kv = tid; kv < nvec; kv += NW * 64) {
        const uint4 xq = ldg16(xt + (size_t)kv * VN);
        float xf[VN];
        if (r > 0) vec16<DT>::widen(xq, xf);
#pragma unroll
        for (int c = 0; c < RM; c += RC) {
            if (c < r) {                                  // uniform: rank rows left in the slot
                // RC independent loads in flight; rows past the rank re-read
                // the last rank row (a cache hit) and are masked out below.
                uint4 aq[RC];
#pragma unroll
                for (int j = 0; j < RC; ++j) {
                    const int row = min(c + j, r - 1);
                    aq[j] = ldg16(At + (size_t)row * d_in + (size_t)kv * VN);
                }
#pragma unroll
                for (int j = 0; j < RC; ++j) {
                    float af[VN];
                    vec16<DT>::widen(aq[j], af);
                    float d = 0.0f;
#pragma unroll
                    for (int e = 0; e < VN; ++e) d = fmaf(xf[e], af[e], d);
                    acc[c + j] += (c + j < r) ? d : 0.0f;
                }
            }
        }
    }
    constexpr int NR = RM < 64 ? RM : 64;
#pragma unroll
    for (int c = 0; c < RM / NR; ++c) {
        const float sum = wave_reduce_transpose<NR>(acc + c * NR, lane);
        if (lane < NR) s_red[wave][c * NR + owned_index<NR>(lane)] = sum;
    }
    __syncthreads();
    for (int j = tid; j < max_rank; j += NW * 64) {
        float sum = 0.0f;
        if (j < r) {
#pragma unroll
            for (int w2 = 0; w2 < NW; ++w2) sum += s_red[w2][j];
        }
        vt[j] = sum;
    }
    __syncthreads();                                      // s_red is reused by the next slice
    }
    // Bad ids (out of range, or a slot empty in some slice), flagged last so
    // that no load above waits on the ranks.
    if (tid == 0) {
        bool any_empty = false;
        if (in_range)
            for (int sl = 0; sl < ss.n; ++sl) any_empty |= ss.rank[sl][id] <= 0;
        if ((id < -1 || id >= n_slots) || any_empty) flag_bad_row(err, t);
    }
    if constexpr (Q8) {
        __shared__ float s_max[NW];
        const int nch = d_in / 8;
        float m = 0.0f;
        for (int c = tid; c < nch; c += NW * 64) {
            float f[8];
            vec16<LORA_BF16>::widen(ldg16(xt + 8 * c), f);
#pragma unroll
            for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
        if (lane == 0) s_max[wave] = m;
        __syncthreads();
        float amax = s_max[0];
#pragma unroll
        for (int w2 = 1; w2 < NW; ++w2) amax = fmaxf(amax, s_max[w2]);
        const int e = scale_exp(amax);
        const float inv = exp2i(-e);
        if (tid == 0) xs[t] = exp2i(e);
        uint8_t *out = xq + (size_t)t * d_in;
        for (int c = tid; c < nch; c += NW * 64) {
            float f[8];
            vec16<LORA_BF16>::widen(ldg16(xt + 8 * c), f);
            uint2 q;
            q.x = e4m3x4(f[0] * inv, f[1] * inv, f[2] * inv, f[3] * inv);
            q.y = e4m3x4(f[4] * inv, f[5] * inv, f[6] * inv, f[7] * inv);
            *reinterpret_cast<uint2 *>(out + 8 * c) = q;
        }
    }
}

// BGMV: one workgroup per row (position blockIdx.x through perm).
template <int DT, int RM, bool Q8 = false>
__global__ void __launch_bounds__(512) k_shrink_rows(const typename elem<DT>::T *__restrict__ x,
                                                     int32_t T, int32_t d_in, slice_set ss,
                                                     int32_t n_slots, int32_t max_rank,
                                                     const int32_t *__restrict__ ids,
                                                     const int32_t *__restrict__ perm,
                                                     float *__restrict__ v, int32_t *err,
                                                     uint8_t *__restrict__ xq, float *__restrict__ xs) {
    shrink_row<DT, RM, Q8>(x, T, d_in, ss, n_slots, max_rank, ids, perm, v, err, xq, xs, blockIdx.x);
}


// ---------------------------------------------------------------------------
// SGMV shrink, bf16: a grouped product over adapter segments.
//   Work block w (grid.x) covers up to kShrinkRows consecutive sorted rows of
//   ONE segment (the block table comes from the segment builder); grid.y
//   splits K.  Rows of a segment share one adapter, so the block is a small
//   GEMM: its x rows (gathered through perm) times the adapter's A^T rows.
//   Both operands are K-contiguous rows, so they go global -> LDS by DMA
//   (global_load_lds, whole 16-byte chunks of a row per lane: full cache
//   lines), NS stages of 128 k (NS - 1 in flight), stored with an XOR swizzle of the
//   16-byte chunk index by row (conflict-free fragment reads); masked rows,
//   ranks past the slot's and k past the range load the zero vector.  Each of
//   the 4 wavefronts takes one 32-k quarter of every stage
//   (v_mfma_f32_16x16x32_bf16, fp32 accumulate), and the 4 partial sums are
//   added in LDS in a fixed order.  Extra workgroups past the work blocks
//   write the zero v rows of the base-only block (and of bad ids) so every
//   row of v is defined.
//   Operand mapping per lane l: A operand = x row (l % 16) of a 16-row block,
//   8 consecutive k of k-group (l / 16); B operand = A^T row (rank) (l % 16) of
//   a 16-rank chunk, the same 8 k.  Output: rank (l % 16), rows 4 (l / 16) + q.
// ---------------------------------------------------------------------------
template <int RCH, int NS_> struct shrink_cfg {
    static constexpr int BR = kShrinkRows;               // rows per work block
    static constexpr int NR = RCH * 16;                  // rank columns
    static constexpr int BK = 128;                       // k per stage
    static constexpr int CH = BK / 8;                    // 16-byte chunks per LDS row
    static constexpr int XST = BR * BK, AST = NR * BK;   // elements per stage
    static constexpr int STAGE = XST + AST;
    static constexpr int NS = NS_;                       // stages in LDS
    static constexpr int XI = BR * CH / 256, AI = NR * CH / 256;   // DMA instructions per wave per stage
    static constexpr int RED = 4 * BR * (NR + 1);        // fp32 reduction buffer
    static constexpr int LDS_BYTES = NS * STAGE * 2 > RED * 4 ? NS * STAGE * 2 : RED * 4;
    static_assert(XI * 256 == BR * CH && AI * 256 == NR * CH, "DMA plan must cover the stage");
};

template <int RCH, int NS_>   // 16-rank chunks, LDS stages
__global__ void __launch_bounds__(256) k_shrink_grouped(
    const uint16_t *__restrict__ x, int32_t T, int32_t d_in, slice_set ss, int32_t max_rank,
    const int32_t *__restrict__ perm, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ seg_id,
    const int32_t *__restrict__ seg_start, const int32_t *__restrict__ n_seg_p,
    const int32_t *__restrict__ blk_start, const int32_t *__restrict__ blk_seg,
    int32_t n_work_upper, int32_t n_slots, int32_t k_chunk,
    float *__restrict__ v, float *__restrict__ partial, int32_t *err) {
    typedef shrink_cfg<RCH, NS_> C;
    constexpr int BR = C::BR, NR = C::NR, BK = C::BK, CH = C::CH, XST = C::XST, STAGE = C::STAGE;
    constexpr int NS = C::NS, XI = C::XI, AI = C::AI, PER = XI + AI;
    constexpr int RBN = BR / 16;                         // 16-row MFMA blocks
    __shared__ __attribute__((aligned(1024))) uint16_t smem[C::LDS_BYTES / 2];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wid = blockIdx.x;
    const int VS = ss.n * max_rank;                      // v row stride: all slices
    if (wid >= n_work_upper) {
        // base-only block: sorted positions [0, offsets[1]) get v = 0
        if (blockIdx.y != 0) return;
        const int p0 = (wid - n_work_upper) * BR;
        const int pend = min(min(offsets[1], p0 + BR), T);
        for (int e = tid; e < BR * VS; e += 256) {
            const int p = p0 + e / VS, j = e % VS;
            if (p < pend) {
                const int32_t t = perm_row(perm, p, T);
                if (t >= 0) v[(size_t)t * VS + j] = 0.0f;
            }
        }
        return;
    }
    // Every index taken from the segment tables is checked against the
    // tables' sizes (n_slots + 2 entries; wid is below the block table's
    // size) and T: overwritten tables give wrong rows, never an access
    // outside the buffers.
    const int nseg = min(*n_seg_p, n_slots);
    if (nseg <= 0 || wid >= blk_start[nseg]) return;
    const int lo = blk_seg[wid];                         // this block's segment
    if (lo < 0 || lo >= nseg) return;
    const int32_t aid = seg_id[lo];
    if (aid < 0 || aid >= n_slots) return;
    const int64_t s0 = seg_start[lo], s1 = seg_start[lo + 1];
    const int64_t q0 = s0 + ((int64_t)wid - blk_start[lo]) * BR;
    if (s0 < 0 || s1 > T || q0 < s0 || q0 >= s1) return;
    const int p0 = (int)q0;
    const int pend = (int)(s1 < q0 + BR ? s1 : q0 + BR);
    bool any_rank = false, any_empty = false;
    for (int sl = 0; sl < ss.n; ++sl) {
        const int32_t rs = ss.rank[sl][aid];
        any_rank |= rs > 0;
        any_empty |= rs <= 0;
    }
    const int k_begin = blockIdx.y * k_chunk;
    const int k_end = min(d_in, k_begin + k_chunk);

    // DMA plan: chunk c = (w * I + j) * 64 + lane of a stage sits at LDS row
    // c / CH, slot c % CH, and holds the row's chunk slot ^ (row % CH).
    int64_t xrow[XI];
    const uint16_t *arow[AI];                            // the rank's A^T row, or null (zero rank)
    int xcol[XI], acol[AI];
#pragma unroll
    for (int j = 0; j < XI; ++j) {
        const int c = (wave * XI + j) * 64 + lane;
        const int r = c / CH, slot = c % CH;
        const int p = p0 + r;
        const int32_t t = p < pend ? perm_row(perm, p, T) : -1;
        xrow[j] = t >= 0 ? (int64_t)t * d_in : -1;
        xcol[j] = 8 * (slot ^ (r % CH));
    }
#pragma unroll
    for (int j = 0; j < AI; ++j) {
        const int c = (wave * AI + j) * 64 + lane;
        const int r = c / CH, slot = c % CH;
        // rank column r of the concatenated slices: slice r / max_rank
        const int sl = r / max_rank, jj = r - sl * max_rank;
        const int32_t rs = sl < ss.n ? ss.rank[sl][aid] : 0;
        arow[j] = jj < rs ? reinterpret_cast<const uint16_t *>(ss.a[sl]) +
                                (slot_row0(ss.row0[sl], aid, max_rank) + jj) * d_in
                          : nullptr;
        acol[j] = 8 * (slot ^ (r % CH));
    }
    auto dma_stage = [&](int kt, int buf) {
        uint16_t *xs = smem + buf * STAGE;
        uint16_t *as = xs + XST;
        const int k0 = k_begin + kt * BK;
#pragma unroll
        for (int j = 0; j < XI; ++j) {
            const int kk = k0 + xcol[j];
            const void *src = (xrow[j] >= 0 && kk < k_end) ? (const void *)(x + xrow[j] + kk) : (const void *)g_zero16;
            dma16(src, xs + (wave * XI + j) * 64 * 8);
        }
#pragma unroll
        for (int j = 0; j < AI; ++j) {
            const int kk = k0 + acol[j];
            const void *src = (arow[j] && kk < k_end) ? (const void *)(arow[j] + kk) : (const void *)g_zero16;
            dma16(src, as + (wave * AI + j) * 64 * 8);
        }
    };
    auto wait_stage = [&](int ahead) {                    // stages issued after the awaited one
        if (ahead >= 3) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * PER) : "memory");
        else if (ahead == 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * PER) : "memory");
        else if (ahead == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(PER) : "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    };

    f32x4_t acc[RBN][RCH];
#pragma unroll
    for (int rb = 0; rb < RBN; ++rb)
#pragma unroll
        for (int rc = 0; rc < RCH; ++rc) acc[rb][rc] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int lr = lane & 15, kg = lane >> 4;
    const int nk = any_rank ? (k_end - k_begin + BK - 1) / BK : 0;
    // NS - 1 stages ahead; iteration kt waits for stage kt, then (after the
    // barrier, when every wave is done with stage kt - 1) refills that buffer
    // with stage kt + NS - 1 and computes stage kt.
#pragma unroll
    for (int st = 0; st < NS - 1; ++st)
        if (st < nk) dma_stage(st, st);
    for (int kt = 0; kt < nk; ++kt) {
        wait_stage(min(NS - 2, nk - 1 - kt));
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (kt + NS - 1 < nk) dma_stage(kt + NS - 1, (kt + NS - 1) % NS);
        const uint16_t *xs = smem + (kt % NS) * STAGE;
        const uint16_t *as = xs + XST;
        const int c = 4 * wave + kg;                     // this lane's logical chunk
        uint4 xq[RBN], aq[RCH];
#pragma unroll
        for (int rb = 0; rb < RBN; ++rb) {
            const int r = rb * 16 + lr;
            xq[rb] = *reinterpret_cast<const uint4 *>(xs + r * BK + 8 * (c ^ (r % CH)));
        }
#pragma unroll
        for (int rc = 0; rc < RCH; ++rc) {
            const int r = rc * 16 + lr;
            aq[rc] = *reinterpret_cast<const uint4 *>(as + r * BK + 8 * (c ^ (r % CH)));
        }
#pragma unroll
        for (int rb = 0; rb < RBN; ++rb)
#pragma unroll
            for (int rc = 0; rc < RCH; ++rc)
                acc[rb][rc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8_t, xq[rb]), __builtin_bit_cast(bf16x8_t, aq[rc]), acc[rb][rc], 0, 0, 0);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (any_empty && blockIdx.y == 0 && tid < BR && p0 + tid < pend)
        flag_bad_row(err, perm_row(perm, p0 + tid, T));     // segment of an empty slot
    __syncthreads();                                     // all waves done with the stages
    float (*s_acc)[BR][NR + 1] = reinterpret_cast<float (*)[BR][NR + 1]>(smem);
#pragma unroll
    for (int rb = 0; rb < RBN; ++rb)
#pragma unroll
        for (int rc = 0; rc < RCH; ++rc)
#pragma unroll
            for (int q = 0; q < 4; ++q) s_acc[wave][rb * 16 + 4 * kg + q][rc * 16 + lr] = acc[rb][rc][q];
    __syncthreads();
    for (int e = tid; e < BR * VS; e += 256) {
        const int i = e / VS, j = e % VS;
        const int p = p0 + i;
        if (p >= pend) continue;
        float sum = 0.0f;
        if (j < NR) sum = (s_acc[0][i][j] + s_acc[1][i][j]) + (s_acc[2][i][j] + s_acc[3][i][j]);
        if (partial) {
            partial[((size_t)blockIdx.y * T + p) * VS + j] = sum;
        } else {
            const int32_t t = perm_row(perm, p, T);
            if (t >= 0) v[(size_t)t * VS + j] = sum;
        }
    }
}

// v[perm[p]][j] = sum over k-split chunks, in chunk order, for the adapter
// rows (sorted positions from offsets[1] on).
__global__ void __launch_bounds__(256) k_shrink_reduce(const float *__restrict__ partial,
                                                       int32_t n_split, int32_t T,
                                                       int32_t max_rank,
                                                       const int32_t *__restrict__ perm,
                                                       const int32_t *__restrict__ offsets,
                                                       float *__restrict__ v) {
    const size_t n = (size_t)T * max_rank;
    const int32_t o1 = offsets[1];                        // first adapter row (sorted order)
    const size_t e0 = (size_t)(o1 < 0 ? 0 : (o1 > T ? T : o1)) * max_rank;
    for (size_t e = e0 + blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < n;
         e += (size_t)gridDim.x * blockDim.x) {
        const int p = (int)(e / max_rank), j = (int)(e % max_rank);
        float sum = 0.0f;
        for (int c = 0; c < n_split; ++c) sum += partial[(size_t)c * n + e];
        const int t = perm_row(perm, p, T);
        if (t >= 0) v[(size_t)t * max_rank + j] = sum;
    }
}

template <int DT>
static void launch_rows(const void *x, int32_t T, const lora_pool_t &p, const slice_set &ss,
                        const int32_t *ids, const int32_t *perm, float *v, int32_t *err,
                        hipStream_t s) {
    typedef typename elem<DT>::T E;
    const E *xe = (const E *)x;
#define LORA_SHRINK_ROWS(RMV)                                                                   \
    hipLaunchKernelGGL((k_shrink_rows<DT, RMV>), dim3(T), dim3(512), 0, s, xe, T, p.d_in, ss,   \
                       p.n_slots, p.max_rank, ids, perm, v, err, nullptr, nullptr)
    if (p.max_rank <= 8) LORA_SHRINK_ROWS(8);
    else if (p.max_rank <= 16) LORA_SHRINK_ROWS(16);
    else if (p.max_rank <= 32) LORA_SHRINK_ROWS(32);
    else if (p.max_rank <= 64) LORA_SHRINK_ROWS(64);
    else LORA_SHRINK_ROWS(128);
#undef LORA_SHRINK_ROWS
}

// FP8-base forward, BGMV rows: the shrink and the row quantizer in one launch.
lora_status_t launch_quant_shrink_rows(const void *x, int32_t T, const lora_pool_t *pool, const int32_t *ids,
                                       float *v, uint8_t *xq, float *xs, int32_t *err, hipStream_t s) {
    slice_set ss;
    ss.n = 1;
    for (int i = 0; i < kMaxSlices; ++i) {
        ss.a[i] = pool->a;
        ss.rank[i] = pool->rank;
        ss.row0[i] = pool->row0;
    }
    const uint16_t *xe = (const uint16_t *)x;
#define LORA_QSHRINK_ROWS(RMV)                                                                            \
    hipLaunchKernelGGL((k_shrink_rows<LORA_BF16, RMV, true>), dim3(T), dim3(512), 0, s, xe, T, pool->d_in, ss, \
                       pool->n_slots, pool->max_rank, ids, nullptr, v, err, xq, xs)
    if (pool->max_rank <= 8) LORA_QSHRINK_ROWS(8);
    else if (pool->max_rank <= 16) LORA_QSHRINK_ROWS(16);
    else if (pool->max_rank <= 32) LORA_QSHRINK_ROWS(32);
    else if (pool->max_rank <= 64) LORA_QSHRINK_ROWS(64);
    else LORA_QSHRINK_ROWS(128);
#undef LORA_QSHRINK_ROWS
    return hip_status(hipGetLastError());
}

lora_status_t launch_shrink(const void *x, int32_t T, const lora_pool_t *pools, int32_t n_slices,
                            const int32_t *ids, bool sgmv, float *v, const ws_layout &L, void *ws,
                            hipStream_t s) {
    const lora_pool_t &p = pools[0];
    slice_set ss;
    ss.n = n_slices;
    for (int i = 0; i < kMaxSlices; ++i) {
        const lora_pool_t &q = pools[i < n_slices ? i : 0];
        ss.a[i] = q.a;
        ss.rank[i] = q.rank;
        ss.row0[i] = q.row0;
    }
    const int32_t VS = n_slices * p.max_rank;
    int32_t *err = ws_ptr<int32_t>(ws, L.header);
    const int32_t *perm = sgmv ? ws_ptr<int32_t>(ws, L.perm) : nullptr;
    if (!sgmv || p.dtype == LORA_F32) {
        if (p.dtype == LORA_F32) launch_rows<LORA_F32>(x, T, p, ss, ids, perm, v, err, s);
        else launch_rows<LORA_BF16>(x, T, p, ss, ids, perm, v, err, s);
        return hip_status(hipGetLastError());
    }
    // SGMV bf16: grouped over segment blocks; split K so that about 512
    // workgroups have work.
    const int32_t row_blocks = (T + kShrinkRows - 1) / kShrinkRows;
    const int32_t n_work_upper = row_blocks + (T < p.n_slots ? T : p.n_slots);
    int32_t split = (512 + row_blocks) / (row_blocks + 1);
    if (split > kMaxKSplit) split = kMaxKSplit;
    while (split > 1 && p.d_in / split < 256) --split;
    int32_t k_chunk = (p.d_in + split - 1) / split;
    k_chunk = (k_chunk + 31) / 32 * 32;
    split = (p.d_in + k_chunk - 1) / k_chunk;
    float *partial = split > 1 ? ws_ptr<float>(ws, L.partial) : nullptr;
    const uint16_t *xe = (const uint16_t *)x;
    const int rc = (VS + 15) / 16;
    const int32_t *offsets = ws_ptr<int32_t>(ws, L.offsets);
    const dim3 grid(n_work_upper + row_blocks, split);
    // Stages: 3 for narrow rank sets streaming long K ranges (more bytes in
    // flight per workgroup), else 2 (more workgroups resident per CU, which
    // serves short K ranges and wide rank sets better).
    const bool deep = rc <= 2 && k_chunk >= 8 * 128;
#define LORA_SHRINK_GROUPED(RCV, NSV)                                                             \
    hipLaunchKernelGGL((k_shrink_grouped<RCV, NSV>), grid, dim3(256), 0, s, xe, T, p.d_in, ss,    \
                       p.max_rank, perm, offsets, ws_ptr<int32_t>(ws, L.seg_id),                  \
                       ws_ptr<int32_t>(ws, L.seg_start), ws_ptr<int32_t>(ws, L.n_seg),            \
                       ws_ptr<int32_t>(ws, L.blk_start), ws_ptr<int32_t>(ws, L.blk_seg),          \
                       n_work_upper, p.n_slots, k_chunk, v, partial, err)
    switch (rc) {
        case 1: if (deep) LORA_SHRINK_GROUPED(1, 3); else LORA_SHRINK_GROUPED(1, 2); break;
        case 2: if (deep) LORA_SHRINK_GROUPED(2, 3); else LORA_SHRINK_GROUPED(2, 2); break;
        case 3: LORA_SHRINK_GROUPED(3, 2); break;
        case 4: LORA_SHRINK_GROUPED(4, 2); break;
        case 5: LORA_SHRINK_GROUPED(5, 2); break;
        case 6: LORA_SHRINK_GROUPED(6, 2); break;
        case 7: LORA_SHRINK_GROUPED(7, 2); break;
        default: LORA_SHRINK_GROUPED(8, 2); break;
    }
#undef LORA_SHRINK_GROUPED
    if (split > 1) {
        size_t n = (size_t)T * VS;
        int g = (int)((n + 255) / 256);
        if (g > 4096) g = 4096;
        hipLaunchKernelGGL(k_shrink_reduce, dim3(g), dim3(256), 0, s, partial, split, T, VS, perm,
                           offsets, v);
    }
    return hip_status(hipGetLastError());
}

}  // namespace lora
