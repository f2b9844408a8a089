// a2 -- integer segment builder: histogram -> exclusive prefix sum -> stable
// scatter of row indices -> compaction of non-empty adapter segments.
//
// It produces what the SGMV routine of "Serving multiple LoRAs: segmented
// matrix multiplies and adapter scheduling" (section "Not merging the
// weights, computing in batches") obtains with a stable argsort by adapter id
// and consecutive-unique counts, and what lora_mixed_batch in "LoRAX, in
// depth" consumes as segment boundaries plus the owner of each segment.  The
// kernels never move x or y: later kernels index rows through `perm`, the
// offsets-instead-of-gather idea of "Multi-LoRA Serving 与 Adapter 隔离"
// (adapter ownership in one continuous batch).
//
// Key of row t: ids[t] + 1 (so "no adapter" = key 0 sorts first); ids outside
// [-1, n_slots) count as key 0 and are flagged in the error word.
//
// Three launches, all integer, no floating point:
//   1. per 1024-row tile, an LDS histogram of keys -> tile_hist[key][tile]
//   2. one workgroup: exclusive scan of tile_hist in (key, tile) order, so
//      entry (key, tile) becomes the first output position of that tile's rows
//      with that key; offsets[], the GEMM order's key bases (long segments
//      first, short ones last), then the compaction of non-empty keys >= 1
//   3. per tile, each row's rank among the earlier rows of its tile with the
//      same key (stable: the tile's (key, row) pairs sorted in LDS),
//      perm[base + rank] = t, and its place in the GEMM order.
#include "common.hpp"

namespace lora {

// Workspace header: the error word to "none"; with `all`, every other
// header word (the segment build's) to zero as well.
__global__ void k_ws_init(int32_t *header, int32_t all) {
    const int i = threadIdx.x;
    if (i == 0) header[0] = kErrNone;
    else if (all && i < 64) header[i] = 0;
}

__device__ __forceinline__ int32_t row_key(int32_t id, int32_t n_slots) {
    return (id >= -1 && id < n_slots) ? id + 1 : 0;
}

__global__ void __launch_bounds__(256) k_seg_hist(const int32_t *__restrict__ ids, int32_t T,
                                                  int32_t n_slots, int32_t *__restrict__ tile_hist,
                                                  int32_t n_tiles, int32_t *err) {
    extern __shared__ int32_t hist[];
    const int32_t nb = n_slots + 1, tile = blockIdx.x;
    for (int32_t k = threadIdx.x; k < nb; k += blockDim.x) hist[k] = 0;
    __syncthreads();
    const int32_t t0 = tile * kSegTile;
    const int32_t t1 = min(T, t0 + kSegTile);
    for (int32_t t = t0 + threadIdx.x; t < t1; t += blockDim.x) {
        const int32_t id = ids[t];
        if (!(id >= -1 && id < n_slots)) flag_bad_row(err, t);
        atomicAdd(&hist[row_key(id, n_slots)], 1);
    }
    __syncthreads();
    for (int32_t k = threadIdx.x; k < nb; k += blockDim.x)
        tile_hist[(size_t)k * n_tiles + tile] = hist[k];
}

// Block-wide exclusive scan of one value per thread (1024 threads = 16
// waves of 64).  Returns the exclusive prefix; *total gets the block sum.
__device__ __forceinline__ int32_t block_exclusive_scan(int32_t v, int32_t *s_wave, int32_t *total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int32_t inc = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int32_t o = __shfl_up(inc, d, 64);
        if (lane >= d) inc += o;
    }
    if (lane == 63) s_wave[wave] = inc;
    __syncthreads();
    if (wave == 0) {
        const int nw = blockDim.x >> 6;
        int32_t w = (lane < nw) ? s_wave[lane] : 0;
        int32_t winc = w;
#pragma unroll
        for (int d = 1; d < 16; d <<= 1) {
            const int32_t o = __shfl_up(winc, d, 64);
            if (lane >= d) winc += o;
        }
        if (lane < nw) s_wave[16 + lane] = winc - w;   // exclusive wave prefix
        if (lane == nw - 1) s_wave[32] = winc;
    }
    __syncthreads();
    const int32_t res = s_wave[16 + wave] + inc - v;
    *total = s_wave[32];
    __syncthreads();
    return res;
}

// Compaction of non-empty adapter keys (k >= 1) in ascending order, and the
// grouped shrink's work table: segment i covers work blocks [blk_start[i],
// blk_start[i+1]) of kShrinkRows rows each.  s_off: the keys' first output
// positions (s_off[nb] = T), in LDS; every thread of the block calls it.
__device__ void compact_segments(const int32_t *s_off, int32_t nb, int32_t T, int32_t *s_wave,
                                 int32_t *__restrict__ seg_id, int32_t *__restrict__ seg_start,
                                 int32_t *__restrict__ n_seg, int32_t *__restrict__ blk_start,
                                 int32_t *__restrict__ blk_seg) {
    int32_t seg_carry = 0, blk_carry = 0;
    for (int32_t k0 = 1; k0 < nb; k0 += blockDim.x) {
        const int32_t k = k0 + threadIdx.x;
        const int32_t len = (k < nb) ? (s_off[k + 1] - s_off[k]) : 0;
        const int32_t nonempty = len > 0;
        const int32_t nblk = (len + kShrinkRows - 1) / kShrinkRows;
        int32_t tot, btot;
        const int32_t idx = block_exclusive_scan(nonempty, s_wave, &tot) + seg_carry;
        const int32_t bidx = block_exclusive_scan(nblk, s_wave, &btot) + blk_carry;
        if (nonempty) {
            seg_id[idx] = k - 1;
            seg_start[idx] = s_off[k];
            blk_start[idx] = bidx;
            for (int32_t b = 0; b < nblk; ++b) blk_seg[bidx + b] = idx;
        }
        seg_carry += tot;
        blk_carry += btot;
    }
    if (threadIdx.x == 0) {
        seg_start[seg_carry] = T;
        blk_start[seg_carry] = blk_carry;
        *n_seg = seg_carry;
    }
}

// The GEMM's row order: the rows of the base block and of the segments of at
// least short_len rows, in sorted order, then the rows of the shorter
// segments, in sorted order (a stable partition of perm).  gbase[k] is the
// first GEMM position of key k's rows; srec lists the short segments in
// ascending key order as {key, first GEMM position, rows, 0}, then key 0 up
// to entry min(n_slots, T) (so the per-row expand reads one record per
// item); header[kHdrNLong] is the number of rows before the short ones and
// header[kHdrNShort] the number of short segments.  Every thread of the
// block calls it.
__device__ void gemm_order(const int32_t *s_off, int32_t nb, int32_t T, int32_t short_len, int32_t *s_wave,
                           int32_t *__restrict__ gbase, int4 *__restrict__ srec, int32_t *__restrict__ header) {
    int32_t n_short = 0;
    for (int32_t k0 = 0; k0 < nb; k0 += blockDim.x) {
        const int32_t k = k0 + threadIdx.x;
        const int32_t len = (k < nb) ? (s_off[k + 1] - s_off[k]) : 0;
        int32_t tot;
        block_exclusive_scan((k >= 1 && len > 0 && len < short_len) ? len : 0, s_wave, &tot);
        n_short += tot;
    }
    const int32_t n_long = T - n_short;
    int32_t long_carry = 0, short_carry = 0, seg_carry = 0;
    for (int32_t k0 = 0; k0 < nb; k0 += blockDim.x) {
        const int32_t k = k0 + threadIdx.x;
        const int32_t len = (k < nb) ? (s_off[k + 1] - s_off[k]) : 0;
        const bool is_short = k >= 1 && len > 0 && len < short_len;
        int32_t lt, st, nt;
        const int32_t lp = block_exclusive_scan(is_short ? 0 : len, s_wave, &lt) + long_carry;
        const int32_t sp = block_exclusive_scan(is_short ? len : 0, s_wave, &st) + short_carry;
        const int32_t si = block_exclusive_scan(is_short ? 1 : 0, s_wave, &nt) + seg_carry;
        if (k < nb) gbase[k] = is_short ? n_long + sp : lp;
        if (is_short) srec[si] = make_int4(k, n_long + sp, len, 0);
        long_carry += lt;
        short_carry += st;
        seg_carry += nt;
    }
    const int32_t n_rec = min(nb - 1, T);
    for (int32_t i = seg_carry + threadIdx.x; i < n_rec; i += blockDim.x) srec[i] = make_int4(0, 0, 0, 0);
    if (threadIdx.x == 0) {
        header[kHdrNLong] = n_long;
        header[kHdrShortLen] = short_len;
        header[kHdrNShort] = seg_carry;
    }
}

// The (key, row) pairs of one tile of kSegTile rows (rows t0 ...), sorted
// ascending in LDS by a bitonic network; rows are distinct, so the order is
// total and rows of one key stay in row order (stable).  Returns thread i's
// sorted key (INT32_MAX for padding past T) and row, and the key's first
// sorted position, so i - first is the row's rank among the tile's rows of
// its key.  Every thread of the block (kSegTile of them) calls it.
__device__ void sort_tile(const int32_t *__restrict__ ids, int32_t T, int32_t n_slots, int32_t t0,
                          int32_t *s_key, int32_t *s_row, int32_t &key, int32_t &row, int32_t &first) {
    const int i = threadIdx.x;
    const int32_t t = t0 + i;
    s_key[i] = (t < T) ? row_key(ids[t], n_slots) : INT32_MAX;         // padding sorts last
    s_row[i] = t;
    __syncthreads();
    for (int k = 2; k <= kSegTile; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            const int p = i ^ j;
            if (p > i) {
                const int32_t ka = s_key[i], kb = s_key[p], ra = s_row[i], rb = s_row[p];
                const bool a_gt_b = ka > kb || (ka == kb && ra > rb);
                if (a_gt_b == ((i & k) == 0)) {                      // ascending where bit k of i is clear
                    s_key[i] = kb; s_key[p] = ka;
                    s_row[i] = rb; s_row[p] = ra;
                }
            }
            __syncthreads();
        }
    }
    key = s_key[i];
    row = s_row[i];
    int lo = 0, hi = i;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (s_key[mid] < key) lo = mid + 1;
        else hi = mid;
    }
    first = lo;
}

constexpr int kScanItems = 4;

__global__ void __launch_bounds__(1024) k_seg_scan(int32_t *__restrict__ tile_hist, int32_t n_slots,
                                                   int32_t n_tiles, int32_t T, int32_t short_len,
                                                   int32_t *__restrict__ offsets,
                                                   int32_t *__restrict__ seg_id,
                                                   int32_t *__restrict__ seg_start,
                                                   int32_t *__restrict__ n_seg,
                                                   int32_t *__restrict__ blk_start,
                                                   int32_t *__restrict__ blk_seg,
                                                   int32_t *__restrict__ gbase,
                                                   int4 *__restrict__ srec,
                                                   int32_t *__restrict__ header) {
    extern __shared__ int32_t s_off[];        // [n_slots + 2]
    __shared__ int32_t s_wave[48];
    const int32_t nb = n_slots + 1;
    const int64_t N = (int64_t)nb * n_tiles;
    int32_t carry = 0;
    const int64_t chunk = (int64_t)blockDim.x * kScanItems;
    for (int64_t c0 = 0; c0 < N; c0 += chunk) {
        const int64_t e0 = c0 + (int64_t)threadIdx.x * kScanItems;
        int32_t vals[kScanItems], sum = 0;
#pragma unroll
        for (int q = 0; q < kScanItems; ++q) {
            vals[q] = (e0 + q < N) ? tile_hist[e0 + q] : 0;
            sum += vals[q];
        }
        int32_t tot;
        int32_t run = block_exclusive_scan(sum, s_wave, &tot) + carry;
#pragma unroll
        for (int q = 0; q < kScanItems; ++q) {
            const int64_t e = e0 + q;
            if (e < N) {
                tile_hist[e] = run;
                if (e % n_tiles == 0) s_off[e / n_tiles] = run;   // first tile of key e / n_tiles
            }
            run += vals[q];
        }
        carry += tot;
    }
    if (threadIdx.x == 0) s_off[nb] = T;
    __syncthreads();
    for (int32_t k = threadIdx.x; k <= nb; k += blockDim.x) offsets[k] = s_off[k];

    gemm_order(s_off, nb, T, short_len, s_wave, gbase, srec, header);
    compact_segments(s_off, nb, T, s_wave, seg_id, seg_start, n_seg, blk_start, blk_seg);
}

__global__ void __launch_bounds__(1024) k_seg_scatter(const int32_t *__restrict__ ids, int32_t T,
                                                      int32_t n_slots,
                                                      const int32_t *__restrict__ tile_hist,
                                                      int32_t n_tiles, int32_t *__restrict__ perm,
                                                      const int32_t *__restrict__ offsets,
                                                      const int32_t *__restrict__ gbase,
                                                      int32_t *__restrict__ gperm) {
    __shared__ int32_t s_key[kSegTile], s_row[kSegTile];
    int32_t key, row, first;
    sort_tile(ids, T, n_slots, blockIdx.x * kSegTile, s_key, s_row, key, row, first);
    if (key == INT32_MAX) return;
    const int32_t pos = tile_hist[(size_t)key * n_tiles + blockIdx.x] + ((int)threadIdx.x - first);
    perm[pos] = row;
    gperm[gbase[key] + (pos - offsets[key])] = row;      // same place within its key's block
}

lora_status_t launch_ws_init(void *ws, hipStream_t s, bool err_only) {
    hipLaunchKernelGGL(k_ws_init, dim3(1), dim3(64), 0, s, ws_ptr<int32_t>(ws, 0), err_only ? 0 : 1);
    return hip_status(hipGetLastError());
}

lora_status_t launch_segments(const int32_t *ids, int32_t T, int32_t n_slots, const ws_layout &L,
                              void *ws, hipStream_t s, int32_t short_len) {
    if (short_len < 1) short_len = 1;
    const int32_t n_tiles = (T + kSegTile - 1) / kSegTile;
    int32_t *err = ws_ptr<int32_t>(ws, L.header);
    int32_t *tile_hist = ws_ptr<int32_t>(ws, L.tile_hist);
    const size_t lds_hist = sizeof(int32_t) * (size_t)(n_slots + 1);
    const size_t lds_off = sizeof(int32_t) * (size_t)(n_slots + 2);
    hipLaunchKernelGGL(k_seg_hist, dim3(n_tiles), dim3(256), lds_hist, s, ids, T, n_slots,
                       tile_hist, n_tiles, err);
    hipLaunchKernelGGL(k_seg_scan, dim3(1), dim3(1024), lds_off, s, tile_hist, n_slots, n_tiles, T, short_len,
                       ws_ptr<int32_t>(ws, L.offsets), ws_ptr<int32_t>(ws, L.seg_id),
                       ws_ptr<int32_t>(ws, L.seg_start), ws_ptr<int32_t>(ws, L.n_seg),
                       ws_ptr<int32_t>(ws, L.blk_start), ws_ptr<int32_t>(ws, L.blk_seg),
                       ws_ptr<int32_t>(ws, L.gbase), ws_ptr<int4>(ws, L.srec), ws_ptr<int32_t>(ws, L.header));
    hipLaunchKernelGGL(k_seg_scatter, dim3(n_tiles), dim3(kSegTile), 0, s, ids, T, n_slots,
                       tile_hist, n_tiles, ws_ptr<int32_t>(ws, L.perm), ws_ptr<int32_t>(ws, L.offsets),
                       ws_ptr<int32_t>(ws, L.gbase), ws_ptr<int32_t>(ws, L.gperm));
    return hip_status(hipGetLastError());
}

}  // namespace lora
