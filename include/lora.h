/*
 * lora.h -- C ABI of liblora, the mixed-adapter LoRA linear layer for one
 * MI355X (gfx950) GPU.
 *
 * The operation (row-vector form):  for every token row t of a batch
 *
 *     y[t,:] = x[t,:] W  +  s_a * (x[t,:] A_a) B_a        a = ids[t]
 *
 * where W is the shared base weight [d_in, d_out], A_a [d_in, r_a] and
 * B_a [r_a, d_out] are the low-rank pair of adapter slot a, s_a = alpha_a/r_a,
 * and a = -1 means "no adapter" (base row only).
 *   - The forward y = xW + s (xA) B with A of shape d x r and B of shape r x d'
 *     and the BGMV / SGMV ways of batching it: "Serving multiple LoRAs:
 *     segmented matrix multiplies and adapter scheduling", section "Not
 *     merging the weights, computing in batches".
 *   - s = alpha / r, the shared base product over all tokens and the
 *     per-segment delta: "LoRAX, in depth", section "Computing a batch that
 *     mixes adapters".
 *   - Stacked per-slot buffers, the slot copy on activation, zeroing of an
 *     unused slot, slot buffers sized for the maximum rank, shrink into an
 *     fp32 rank-width buffer followed by an expand added to the output, and
 *     -1 as the slot of a token without adapter: "Serving LoRA adapters: from
 *     the model name to the wrapped layer", Steps 3, 4 and 5.
 *
 * Conventions for every function below
 *   - Pointers named as DEVICE point to GPU memory owned by the caller (the
 *     library never allocates or frees device memory).  HOST pointers point
 *     to host memory owned by the caller.
 *   - All GPU work is enqueued on the caller's `stream` and is asynchronous;
 *     the caller keeps every buffer alive until the stream has passed the
 *     call.  Work on one stream is ordered, so uploading into a slot after a
 *     forward on the same stream is safe; use an event across streams.
 *   - Arguments are validated on the host before anything is enqueued; on
 *     any status other than LORA_OK nothing was enqueued.
 *   - Row-major everywhere.  x, W, y and the pool share one element type
 *     (fp32 or bf16); accumulation is always fp32; v is always fp32.
 *   - d_in and d_out must be positive multiples of 8; max_rank a multiple of
 *     8 in [8, 128]; T >= 0 (T == 0 is a no-op returning LORA_OK).
 *   - Device pointers must be 16-byte aligned.
 *   - Bad adapter ids found on the device (outside [-1, n_slots) or naming a
 *     slot of rank 0) never fault: the row is computed as a base row and the
 *     smallest such row index is recorded in the workspace's error word,
 *     read (and cleared) by lora_get_device_error.
 *   - No function keeps hidden state; all are reentrant.  Two calls that
 *     share a workspace must be ordered (same stream or events).
 *   - Results are deterministic: the same inputs and workspace size give
 *     bitwise the same outputs (no floating-point atomics; the workspace
 *     size can change how the GEMM splits K, see lora_workspace_bytes).
 */
#ifndef LORA_H_
#define LORA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *lora_stream_t; /* a hipStream_t; NULL = the null stream */

typedef enum {
    LORA_OK = 0,
    LORA_ERR_INVALID_ARGUMENT = 1,   /* null pointer, bad size, bad dtype, misaligned pointer */
    LORA_ERR_RANK_EXCEEDS_MAX = 2,   /* upload with r > max_rank ("Serving LoRA adapters ...", Step 3: the rank check against the maximum LoRA rank) */
    LORA_ERR_SLOT_OUT_OF_RANGE = 3,  /* slot outside [0, n_slots) */
    LORA_ERR_WORKSPACE_TOO_SMALL = 4,
    LORA_ERR_UNSUPPORTED = 5,        /* combination not implemented (e.g. too many slots) */
    LORA_ERR_HIP = 6                 /* the HIP runtime reported an error at launch */
} lora_status_t;

typedef enum { LORA_F32 = 0, LORA_BF16 = 1 } lora_dtype_t;

/* How the low-rank term is batched ("Serving multiple LoRAs ...", section
 * "Not merging the weights, computing in batches": BGMV gathers each
 * request's adapter, the form for decode; SGMV shares one adapter read per
 * segment, the form for prefill; "Multi-LoRA Serving: Architecture for
 * Thousands of Adapters", section "S-LoRA, Punica and the batched kernels":
 * separate prefill and decode kernels):
 *   BGMV: every row gathers its own adapter (rows in their original order);
 *   SGMV: rows are grouped into adapter-contiguous segments (a stable sort by
 *         slot, built by lora_build_segments) and each segment shares one
 *         read of its adapter;
 *   AUTO: in the forwards, a batch of fewer than LORA_AUTO_SGMV_MIN_ROWS
 *         rows is all BGMV (its segments are short, and up to 256 rows the
 *         shrink can ride inside the base GEMM); a larger one is built into
 *         segments, whose shrink is grouped (one read of each adapter's A
 *         per segment block), and split per segment for the expand:
 *         segments of at least L rows (the prefill chunks) take SGMV's
 *         expand fused into the base GEMM, shorter ones (decode rows) a
 *         per-row expand after the GEMM that reads each segment's B once.
 *         L is 16 by default, or LORA_FLAG_SHORT_SEGMENT(L) for bf16 pools.
 *         In lora_shrink and lora_expand (which cannot know whether
 *         segments were built), AUTO is BGMV.
 * The result does not depend on the mode beyond fp32 rounding order. */
typedef enum { LORA_MODE_AUTO = 0, LORA_MODE_BGMV = 1, LORA_MODE_SGMV = 2 } lora_mode_t;

/* AUTO's batch size from which the forwards build segments (see above).
 * Measured on 512 decode rows of a 70B-shaped q projection (8192 x 8192,
 * ranks 8-64, 218 distinct adapters): 245 us with segments against 266 us
 * per row; on 256 rows of a 4096 x 4096 projection (rank 16) the per-row
 * path with the shrink inside the GEMM takes 33 us against 71 us. */
#define LORA_AUTO_SGMV_MIN_ROWS 512

/* Flags for the forwards (lora_linear_forward, _sliced, _fp8). */
#define LORA_FLAG_SEGMENTS_READY 0x1  /* segments already built in this workspace for these ids */
#define LORA_FLAG_SEPARATE_EXPAND 0x2 /* expand as its own read-modify-write pass, not in the GEMM epilogue */
/* AUTO mode: segments of fewer than L rows (1 <= L <= 255) take the per-row
 * path; 0 (no flag) means the default, 16.  Used when the forward builds
 * the segments (a later call with LORA_FLAG_SEGMENTS_READY follows the
 * build). */
#define LORA_FLAG_SHORT_SEGMENT(L) ((((uint32_t)(L)) & 0xffu) << 8)

/*
 * The HBM adapter pool of one projection: n_slots stacked slots (the stacked
 * buffers of "Serving LoRA adapters ...", Step 3/4).  A plain descriptor
 * filled by lora_pool_create or lora_pool_create_packed and not modified
 * afterwards.  Two forms:
 *   padded (lora_pool_create): every slot holds max_rank rank rows, so any
 *     adapter of rank <= max_rank fits any slot (the slots sized for the
 *     maximum rank of "Serving LoRA adapters ...", Step 3, and of "Serving
 *     multiple LoRAs ...", section "Scheduling the adapters");
 *   packed (lora_pool_create_packed): slot s holds c_s rank rows, c_s a
 *     multiple of 8 chosen per slot, stored back to back with no padding to
 *     max_rank (the heterogeneous-rank, non-contiguous layout of "Multi-LoRA
 *     Serving: Architecture for Thousands of Adapters", section
 *     "Heterogeneous batching and rank"); row0[s] is the first rank row of
 *     slot s and row0[n_slots] the total.
 * Internal layout of slot s, whose rank rows start at R0 = s * max_rank
 * (padded) or row0[s] (packed) and number C = max_rank or c_s (the library's
 * choice, documented for tools):
 *   a: A transposed, rank rows R0 .. R0+C-1 of d_in elements each
 *   b: B in rank octets, rows R0/8 .. (R0+C)/8-1 of [d_out][8] elements
 *      (8 ranks of one output column are 16 contiguous bytes in bf16)
 * Rank rows at and beyond the slot's rank are zero.  Kernels read only the
 * rank rows (octets) below the rank of the slot they serve.
 */
typedef struct {
    int32_t n_slots, d_in, d_out, max_rank;
    int32_t dtype;     /* lora_dtype_t */
    void *a;           /* DEVICE, lora_pool_bytes[_packed](...).a_bytes */
    void *b;           /* DEVICE, lora_pool_bytes[_packed](...).b_bytes */
    float *scale;      /* DEVICE [n_slots], s = alpha / r (0 for an empty slot) */
    int32_t *rank;     /* DEVICE [n_slots], true rank, 0 = empty slot */
    int32_t *row0;     /* packed: DEVICE [n_slots + 1] first rank row per slot; padded: NULL */
    const int32_t *row0_host;  /* packed: HOST copy of row0 (caller-owned, kept valid); padded: NULL */
} lora_pool_t;

/* Device views of the segment metadata held in a workspace (see
 * lora_segments_view).  For T rows and n_slots slots, with key = id + 1
 * (ids outside [-1, n_slots) count as -1):
 *   offsets   [n_slots + 2]  exclusive prefix sum of per-key row counts
 *   perm      [T]            rows in (key, original row) order -- a stable sort
 *   seg_id    [n_slots]      slot of each non-empty adapter segment, ascending
 *   seg_start [n_slots + 1]  first sorted position of each segment; entry n_seg is T
 *   n_seg     [1]            number of adapter segments (the -1 block is not one)
 * ("Serving multiple LoRAs ...": the stable argsort by adapter and the
 * consecutive-unique counts of the SGMV routine; "LoRAX, in depth":
 * segment boundaries of length n_segments + 1 and the owner of each).
 * Two more arrays order the rows for the base GEMM of a mixed batch:
 *   gemm_perm [T]            the rows of the -1 block and of every segment of
 *                            at least L rows, in perm order, then the rows of
 *                            the shorter segments, in perm order (a stable
 *                            partition of perm; L is the short-segment
 *                            threshold of the build, 1 for lora_build_segments,
 *                            so there gemm_perm equals perm)
 *   n_fused   [1]            the number of rows before the short segments'. */
typedef struct {
    int32_t *offsets, *perm, *seg_id, *seg_start, *n_seg;
    int32_t *gemm_perm, *n_fused;
} lora_segments_t;

/* ---- a1: adapter pool ----------------------------------------------------- */

/* Bytes of the caller-allocated pool buffers.  HOST outputs. */
lora_status_t lora_pool_bytes(int32_t n_slots, int32_t d_in, int32_t d_out, int32_t max_rank,
                              lora_dtype_t dtype, size_t *a_bytes, size_t *b_bytes);

/* Fill *pool (HOST) with the given DEVICE buffers and zero all slots on
 * `stream` (every slot starts empty: rank 0, scale 0). */
lora_status_t lora_pool_create(lora_pool_t *pool, int32_t n_slots, int32_t d_in, int32_t d_out,
                               int32_t max_rank, lora_dtype_t dtype, void *a, void *b,
                               float *scale, int32_t *rank, lora_stream_t stream);

/* A packed pool: slot s holds capacity[s] rank rows (HOST [n_slots], each a
 * multiple of 8 in [8, max_rank]; max_rank is the largest).  Bytes of the
 * caller-allocated a and b buffers (HOST outputs), for rows
 * sum_s capacity[s] instead of n_slots * max_rank. */
lora_status_t lora_pool_bytes_packed(int32_t n_slots, int32_t d_in, int32_t d_out, const int32_t *capacity,
                                     lora_dtype_t dtype, size_t *a_bytes, size_t *b_bytes);

/* Fill *pool (HOST) as a packed pool: writes the prefix sums of capacity
 * (HOST [n_slots]) into row0_host (HOST [n_slots + 1], caller-owned; it must
 * stay valid and unchanged while the pool is used: uploads validate against
 * it) and copies them to row0 (DEVICE [n_slots + 1]) on `stream`, then zeroes
 * every slot as lora_pool_create does.  max_rank (the v row width of every
 * call on this pool) must be at least the largest capacity.  Errors:
 * LORA_ERR_INVALID_ARGUMENT for a capacity that is not a multiple of 8 in
 * [8, max_rank], or the conditions of lora_pool_create. */
lora_status_t lora_pool_create_packed(lora_pool_t *pool, int32_t n_slots, int32_t d_in, int32_t d_out,
                                      int32_t max_rank, lora_dtype_t dtype, const int32_t *capacity,
                                      int32_t *row0_host, void *a, void *b, float *scale, int32_t *rank,
                                      int32_t *row0, lora_stream_t stream);

/* Copy one adapter into `slot` (activation of an adapter into a slot):
 *   A: DEVICE [d_in, r] row-major with row stride lda >= r elements,
 *   B: DEVICE [r, d_out] row-major with row stride ldb >= d_out elements,
 * both in the pool's dtype.  The slot's rank rows r.. (up to max_rank, or
 * to its capacity in a packed pool) are zeroed, scale[slot] = alpha / r
 * (computed in fp32), rank[slot] = r.
 * Errors: LORA_ERR_SLOT_OUT_OF_RANGE, LORA_ERR_RANK_EXCEEDS_MAX (r > max_rank,
 * or r above the slot's capacity in a packed pool),
 * LORA_ERR_INVALID_ARGUMENT (r < 1, null, lda < r, ldb < d_out). */
lora_status_t lora_pool_upload(const lora_pool_t *pool, int32_t slot, const void *A, int32_t lda,
                               const void *B, int32_t ldb, int32_t r, float alpha,
                               lora_stream_t stream);

/* Empty one slot: zero its A and B, rank = 0, scale = 0 (the zeroing of an
 * unused slot in "Serving LoRA adapters ...", Step 3). */
lora_status_t lora_pool_clear(const lora_pool_t *pool, int32_t slot, lora_stream_t stream);

/* ---- workspace ------------------------------------------------------------- */

/* Bytes of workspace for batches of up to T rows against a pool of n_slots
 * slots and max_rank, for every entry point below.  d_out is the widest
 * output the workspace serves (0: none): with it the workspace also holds
 * fp32 partial tiles (at most 128 MiB) that let the GEMM split K -- for all
 * tiles of small batches, and for the last, mostly idle round of tiles of
 * larger ones; without it every tile runs whole.  The two differ in fp32
 * summation order and in how the low-rank term is added: a whole tile feeds
 * s_a * v to the matrix cores as three bf16 parts (its full fp32 value) and
 * sums in the accumulator's order, a split tile's reduction sums it on the
 * vector units.  Returns 0 on bad arguments. */
size_t lora_workspace_bytes(int32_t T, int32_t n_slots, int32_t max_rank, int32_t d_out);

/* Prepare a freshly allocated DEVICE workspace: clears the error word and
 * the internal counters.  Call once after allocation (it is kept valid by
 * every later call). */
lora_status_t lora_workspace_init(void *ws, size_t ws_bytes, lora_stream_t stream);

/* HOST-only pointer arithmetic: device views of the segment metadata that
 * lora_build_segments writes into `ws` for (T, n_slots, max_rank). */
lora_status_t lora_segments_view(void *ws, size_t ws_bytes, int32_t T, int32_t n_slots,
                                 int32_t max_rank, lora_segments_t *out);

/* ---- a2: segment builder ---------------------------------------------------- */

/* Build the segment metadata of DEVICE ids[T] into `ws`: a histogram of keys,
 * an exclusive prefix sum, a stable scatter of row indices and a compaction
 * of non-empty adapter segments.  Bad ids are counted as -1 and recorded in
 * the error word. */
lora_status_t lora_build_segments(const int32_t *ids, int32_t T, int32_t n_slots, int32_t max_rank,
                                  void *ws, size_t ws_bytes, lora_stream_t stream);

/* ---- a4: shrink ------------------------------------------------------------- */

/* The first of the two low-rank products, per row: v[t, 0:r_a] = x[t,:] A_a
 * for rows with a usable adapter a = ids[t]; all other entries of
 * v[t, 0:max_rank] are zero ("Serving multiple LoRAs ...", section "Not
 * merging the weights, computing in batches": the rank-r intermediate xA,
 * per request (BGMV) or per adapter segment (SGMV); "Serving LoRA adapters
 * ...", Step 4: the shrink writes an fp32 buffer of rank width).
 *   x: DEVICE [T, d_in] (pool dtype);  v: DEVICE fp32 [T, max_rank].
 * SGMV requires lora_build_segments on the same ids and ws beforehand. */
lora_status_t lora_shrink(const void *x, int32_t T, const lora_pool_t *pool, const int32_t *ids,
                          lora_mode_t mode, float *v, void *ws, size_t ws_bytes,
                          lora_stream_t stream);

/* ---- a5: expand ------------------------------------------------------------- */

/* The second low-rank product, added to the output:
 * y[t,:] += s_a * v[t, 0:r_a] B_a for rows with a usable adapter a = ids[t];
 * other rows are not touched ("Serving multiple LoRAs ...", section "Not
 * merging the weights, computing in batches": the rank vector times B is
 * added to the row's base output; "LoRAX, in depth", section "Computing a
 * batch that mixes adapters": the scale multiplies that product; "Serving
 * LoRA adapters ...", Step 4: the expand is added to the base layer's
 * output).  A read-modify-write of y (bf16 y is rounded once, to nearest
 * even, after the fp32 sum).  In SGMV mode with a bf16 pool the rows of
 * segments of at least the build's threshold go through the matrix cores
 * (s v as three bf16 parts, i.e. its full fp32 value) and shorter ones per
 * row; the sums differ from BGMV's only in fp32 rounding order.
 *   v: DEVICE fp32 [T, max_rank];  y: DEVICE [T, d_out] (pool dtype).
 * SGMV requires lora_build_segments on the same ids and ws beforehand. */
lora_status_t lora_expand(const float *v, int32_t T, const lora_pool_t *pool, const int32_t *ids,
                          lora_mode_t mode, void *y, void *ws, size_t ws_bytes,
                          lora_stream_t stream);

/* ---- a3: base GEMM ---------------------------------------------------------- */

/* The shared base product, once over every token row of the batch
 * ("Multi-LoRA Serving: Architecture for Thousands of Adapters", section "How
 * multi-LoRA serving works"; "LoRAX, in depth", section "Computing a batch
 * that mixes adapters": the base output of all rows first).
 * y = x W (no adapters): x DEVICE [T, d_in], W DEVICE [d_in, d_out],
 * y DEVICE [T, d_out], all of `dtype`; fp32 accumulation, one rounding.
 * ws (DEVICE, may be NULL) is scratch for a K split, used from its first byte
 * and only if ws_bytes holds the fp32 partials: a forward workspace passed
 * here loses its segments (build them again before an SGMV call on it).
 * Kernels that read segment tables check every index they take from them,
 * so tables overwritten this way give wrong rows, not invalid accesses. */
lora_status_t lora_gemm(const void *x, const void *W, void *y, int32_t T, int32_t d_in,
                        int32_t d_out, lora_dtype_t dtype, void *ws, size_t ws_bytes,
                        lora_stream_t stream);

/* ---- a3 + a5 fused ------------------------------------------------------------ */

/* y = x W + s_a v[t, 0:r_a] B_a per row (the expand inside the GEMM
 * epilogue, one rounding), with v from lora_shrink on the same ids.  In SGMV
 * mode the GEMM visits rows in the GEMM order of the segments built in ws
 * (lora_build_segments, or a forward, on the same ids first): the rows of
 * segments shorter than the build's threshold come last and get their term
 * from a per-row expand after the GEMM (bf16 pools; two roundings for those
 * rows), exactly the GEMM step of lora_linear_forward.  BGMV and AUTO keep
 * the original row order.  Shapes and dtypes as for lora_linear_forward;
 * v DEVICE fp32 [T, max_rank]. */
lora_status_t lora_gemm_expand(const void *x, const void *W, void *y, int32_t T,
                               const lora_pool_t *pool, const int32_t *ids, const float *v,
                               lora_mode_t mode, void *ws, size_t ws_bytes, lora_stream_t stream);

/* ---- a3-a8: the whole layer -------------------------------------------------- */

/* The mixed-adapter LoRA linear layer ("Serving multiple LoRAs ...", section
 * "Not merging the weights, computing in batches": y = xW + s (xA) B with
 * each request's own adapter, by BGMV or SGMV; "LoRAX, in depth", section
 * "Computing a batch that mixes adapters": one base product over all rows,
 * then the low-rank term per adapter segment, none for rows without one;
 * "Serving LoRA adapters ...", Steps 4 and 5: the wrapped layer and the
 * token-to-slot mapping with -1 for no adapter):
 * y = x W + s_a (x A_a) B_a per row (a = ids[t], -1 = none).
 * x DEVICE [T, pool->d_in], W DEVICE [d_in, d_out], y DEVICE [T, d_out]
 * (overwritten), ids DEVICE int32 [T].  `mode` picks BGMV/SGMV (AUTO by T);
 * in SGMV the segments are built in `ws` unless LORA_FLAG_SEGMENTS_READY says
 * they already are for these ids (reuse across the projections of one
 * layer).  By default the expand runs inside the GEMM epilogue (one rounding
 * of base + delta); LORA_FLAG_SEPARATE_EXPAND runs it as its own pass. */
lora_status_t lora_linear_forward(const void *x, const void *W, void *y, int32_t T,
                                  const lora_pool_t *pool, const int32_t *ids, lora_mode_t mode,
                                  uint32_t flags, void *ws, size_t ws_bytes,
                                  lora_stream_t stream);

/* ---- several projections that share x (multi-slice) ------------------------- */

/* Projections fed by the same input -- q, k and v of an attention block, or
 * gate and up of an MLP -- each with its own pool, share one shrink: it
 * reads x once and computes every slice's rank vector in one launch (the
 * stacked per-slice buffers and output slices of "Serving LoRA adapters
 * ...", Step 4).  The pools of one call (HOST array pools[0..n_slices)) must
 * agree on n_slots, d_in, max_rank and dtype (d_out may differ); a slot
 * number names the same adapter in every slice, with its own rank and scale
 * there.  1 <= n_slices <= 4 and n_slices * max_rank <= 128, else
 * LORA_ERR_UNSUPPORTED.  A row is flagged as bad (see lora_get_device_error)
 * if its id is out of range or its slot is empty in any slice; each slice
 * then computes it as a base row where its own slot is empty. */

/* Workspace bytes for sliced calls (lora_workspace_bytes with v of
 * n_slices * max_rank columns); 0 on bad arguments. */
size_t lora_workspace_bytes_sliced(int32_t T, int32_t n_slots, int32_t max_rank, int32_t n_slices,
                                   int32_t d_out);

/* v DEVICE fp32 [T, n_slices * max_rank]: slice s in columns
 * [s * max_rank, (s + 1) * max_rank), each as lora_shrink would write it for
 * pools[s] (bitwise the same values). */
lora_status_t lora_shrink_sliced(const void *x, int32_t T, const lora_pool_t *pools,
                                 int32_t n_slices, const int32_t *ids, lora_mode_t mode, float *v,
                                 void *ws, size_t ws_bytes, lora_stream_t stream);

/* y[s] = x W[s] + s_a (x A_a^s) B_a^s for each slice s: W and y are HOST
 * arrays of n_slices DEVICE pointers ([d_in, pools[s].d_out] and
 * [T, pools[s].d_out]).  Same modes and flags as lora_linear_forward.
 * Segments (SGMV) are built once and the shrink runs once for all slices.
 * A slice that lora_linear_forward would run on its decode-sized fused path
 * (the shrink inside the GEMM, on the x it streams anyway) runs that way
 * here too, bitwise as that call.  The other slices of a bf16 pool share one
 * GEMM launch whose grid spans every slice's column tiles (each with its own
 * W, y and expand) when some of them alone would not fill the chip with the
 * largest tiles; their results may then differ from lora_linear_forward's
 * where a tile is computed whole in one call and split over K in the other
 * (see lora_workspace_bytes; the GEMM is planned for all slices' tiles at
 * once).  Otherwise, and for fp32 pools and LORA_FLAG_SEPARATE_EXPAND,
 * each slice runs its own GEMM, bitwise as lora_linear_forward.  For the
 * grouped GEMM's K split, size the workspace with d_out = the sum of the
 * slices' widths (a smaller d_out only limits the split). */
lora_status_t lora_linear_forward_sliced(const void *x, const void *const *W, void *const *y,
                                         int32_t T, const lora_pool_t *pools, int32_t n_slices,
                                         const int32_t *ids, lora_mode_t mode, uint32_t flags,
                                         void *ws, size_t ws_bytes, lora_stream_t stream);

/* ---- adapter residency: a host tier and the HBM slots as its cache ------------ */

/* Adapters live in host DRAM and are brought into the pool's GPU slots on
 * demand, least recently used out ("Multi-LoRA Serving: Architecture for
 * Thousands of Adapters", sections "Unified paging of adapters and KV cache"
 * and "A worked memory example"; "Serving LoRA adapters ...", Step 3: a fixed
 * number of slots, LRU eviction, activation copies an adapter into its slot).
 *
 * Pack one adapter for a host tier: A HOST [d_in, r] (leading dimension lda)
 * and B HOST [r, d_out] (ldb) into a_slot HOST [max_rank * d_in] and b_slot
 * HOST [max_rank * d_out] elements in the pool's slot layout (A^T rank rows,
 * B rank octets, zero rows past r), so that promotion into a slot is a plain
 * copy.  Host only; no GPU work. */
lora_status_t lora_pack_host(int32_t d_in, int32_t d_out, int32_t max_rank, lora_dtype_t dtype,
                             const void *A, int32_t lda, const void *B, int32_t ldb, int32_t r,
                             void *a_slot, void *b_slot);

/* A residency cache over slots 0..n_slots-1 of n_pools pools (the projections
 * of one layer set, kept in step: slot s holds the same adapter in every pool;
 * every pool has at least n_slots slots, and all share one max_rank and one
 * dtype; packed pools are not supported: LORA_ERR_UNSUPPORTED) for adapter ids
 * 0..max_adapters-1.  n_pools == 0 gives a planning-only cache: the same
 * bookkeeping with no GPU work (for tests and schedulers).  The cache object
 * is host memory owned by the library until lora_cache_destroy; it creates
 * HIP events (one per slot plus one) but no device memory.  Not thread-safe:
 * one host thread at a time per cache. */
typedef struct lora_cache lora_cache_t;
lora_status_t lora_cache_create(lora_cache_t **cache, int32_t n_slots, const lora_pool_t *pools,
                                int32_t n_pools, int32_t max_adapters);
lora_status_t lora_cache_destroy(lora_cache_t *cache);

/* Register (or replace) an adapter in the host tier: host_a[p], host_b[p]
 * HOST pointers, one per pool, to lora_pack_host output of that pool's
 * shapes; they must stay valid, and unchanged, while the cache may copy from
 * them.  Page-locked memory that the HIP runtime maps into the GPU's address
 * space (hipHostMalloc, or a pinned torch tensor), 16-byte aligned, is read
 * directly by a copy kernel on the copy stream (tens of GB/s); other memory
 * is copied with hipMemcpyAsync.  rank <= max_rank
 * (LORA_ERR_RANK_EXCEEDS_MAX), s = alpha / rank.  Re-registering a resident
 * adapter drops its slot, so the next batch loads the new version. */
lora_status_t lora_cache_register(lora_cache_t *cache, int32_t adapter, const void *const *host_a,
                                  const void *const *host_b, int32_t rank, float alpha);

/* Map a batch: adapters HOST [n] (adapter ids or -1) -> slots HOST [n] (slot
 * of each id, -1 for -1), making every distinct adapter of the batch
 * resident.  A miss takes an empty slot, else the least recently used slot
 * the batch does not need.  The copy waits (on `copy`) for the victim slot's
 * last use, then copies A, B, scale and rank; `compute` then waits for the
 * copies, so kernels enqueued on `compute` after this call see the batch's
 * adapters.  An unknown or unregistered id (LORA_ERR_INVALID_ARGUMENT) or
 * more distinct adapters than slots (LORA_ERR_UNSUPPORTED; the per-step
 * adapter limit of "Serving LoRA adapters ...", Step 2) changes nothing. */
lora_status_t lora_cache_map(lora_cache_t *cache, const int32_t *adapters, int32_t n, int32_t *slots,
                             lora_stream_t compute, lora_stream_t copy);

/* After enqueuing the mapped batch's kernels on `compute`: record each of
 * its slots' last use, which later evictions wait for. */
lora_status_t lora_cache_commit(lora_cache_t *cache, lora_stream_t compute);

/* Slot of an adapter (HOST out; -1 if not resident), and counters since
 * creation: batch lookups that hit or missed, evictions, bytes copied. */
lora_status_t lora_cache_slot_of(const lora_cache_t *cache, int32_t adapter, int32_t *slot);
lora_status_t lora_cache_stats(const lora_cache_t *cache, int64_t *hits, int64_t *misses,
                               int64_t *evictions, int64_t *bytes_uploaded);

/* ---- FP8 base weight with a bf16 adapter ----------------------------------- */

/* A quantized base weight with a half-precision adapter is a common serving
 * mix, and the adapter's contribution belongs in the base product's
 * accumulator, never merged into the packed 8-bit weight ("Multi-LoRA
 * Serving 与 Adapter 隔离", section on numerics and mixed precision).  The
 * pages fix no scheme; this library uses OCP E4M3 codes (largest finite 448,
 * subnormals, 0x7f / 0xff NaN) with one power-of-two scale per token row of x
 * and one per output column of W:
 *     scale = 2^e, e the smallest integer with amax <= 448 * 2^e, clamped to
 *     [-127, 127];  code = E4M3(v * 2^-e)  (exact scaling, round to nearest
 *     even); an all-zero row or column gets e = -127 and zero codes.
 * Inputs must be finite.  The matrix cores apply the scales inside the
 * product (E8M0 block scales), so scales passed to lora_gemm_fp8 must be
 * such powers of two (as the quantizers below write them).  The layer is
 *     y[t,n] = s_x[t] s_w[n] sum_k dq(xq[t,k]) dq(wq[n,k]) + s_a ((x A_a) B_a)[n]
 * with the low-rank term from the bf16 x, fp32 accumulation and one rounding
 * of y to bf16.  The FP8 products are exact; the matrix cores add each block
 * of 64 of them with an error below about 2^-12 of the block's largest
 * product, so results are not bitwise equal to an fp32 sum of the products.
 * For all of these: d_in a positive multiple of 16, d_out of 8. */

/* Codes and scales of DEVICE x bf16 [T, d]: xq DEVICE uint8 [T, d],
 * x_scale DEVICE fp32 [T] (each 2^e). */
lora_status_t lora_quantize_rows_fp8(const void *x, int32_t T, int32_t d, uint8_t *xq, float *x_scale,
                                     lora_stream_t stream);

/* Codes and scales of a base weight, once at load: W DEVICE bf16
 * [d_in, d_out] -> wq DEVICE uint8 [d_out, d_in] (row n holds column n of W,
 * K-contiguous), w_scale DEVICE fp32 [d_out] (each 2^e). */
lora_status_t lora_quantize_weight_fp8(const void *W, int32_t d_in, int32_t d_out, uint8_t *wq,
                                       float *w_scale, lora_stream_t stream);

/* Base product only: y = s_x s_w (xq wq^T), y DEVICE bf16 [T, d_out]; the
 * scales are powers of two 2^e, e in [-127, 127] (only their exponents are
 * read).  ws (DEVICE, may be NULL) as for lora_gemm. */
lora_status_t lora_gemm_fp8(const uint8_t *xq, const float *x_scale, const uint8_t *wq,
                            const float *w_scale, void *y, int32_t T, int32_t d_in, int32_t d_out,
                            void *ws, size_t ws_bytes, lora_stream_t stream);

/* Workspace of lora_linear_forward_fp8: that of lora_workspace_bytes plus
 * the quantized rows of x (T * d_in bytes and T scales).  0 on bad
 * arguments. */
size_t lora_workspace_bytes_fp8(int32_t T, int32_t n_slots, int32_t max_rank, int32_t d_in,
                                int32_t d_out);

/* The whole layer on an FP8 base weight: quantizes x into `ws`, computes the
 * shrink from the bf16 x, then the FP8 GEMM with the expand in its epilogue
 * (or, with LORA_FLAG_SEPARATE_EXPAND, as its own pass).  x DEVICE bf16
 * [T, d_in], wq / w_scale from lora_quantize_weight_fp8, y DEVICE bf16
 * [T, d_out], pool bf16 with pool->d_in == d_in and pool->d_out == d_out;
 * mode and flags as for lora_linear_forward.  ws sized by
 * lora_workspace_bytes_fp8. */
lora_status_t lora_linear_forward_fp8(const void *x, const uint8_t *wq, const float *w_scale, void *y,
                                      int32_t T, const lora_pool_t *pool, const int32_t *ids,
                                      lora_mode_t mode, uint32_t flags, void *ws, size_t ws_bytes,
                                      lora_stream_t stream);

/* ---- the layer without a caller workspace ---------------------------------------- */

/* For callers that cannot allocate device memory at call time: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * lora_linear_forward with its workspace in a library-owned device array of
 * 64 MiB (LORA_NOALLOC_SCRATCH_BYTES) per GPU, held until the process ends
 * and looked up at the first call on each device (that first call must not
 * be under stream capture).  It calls no hipMalloc, hipFree or allocating
 * library routine.  Arguments as for lora_linear_forward, on the current
 * device's stream; err_out (DEVICE int32 [1], may be NULL) receives the
 * smallest row index with a bad adapter id in this call, or -1.
 * Limits: a batch whose workspace regions (segments, v, shrink partials:
 * lora_workspace_bytes(T, n_slots, max_rank, 0)) exceed the array returns
 * LORA_ERR_WORKSPACE_TOO_SMALL before enqueuing anything; the rest of the
 * array holds GEMM split-K partials, so it can split K less far than a
 * larger caller workspace would (results then differ in fp32 summation
 * order only).  Every call on one GPU shares the array and it keeps the
 * last call's contents: calls that overlap on one GPU (different streams
 * without ordering) race and are not allowed; LORA_FLAG_SEGMENTS_READY
 * refers to the segments left by the previous call on this GPU. */
#define LORA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
lora_status_t lora_linear_forward_noalloc(const void *x, const void *W, void *y, int32_t T,
                                          const lora_pool_t *pool, const int32_t *ids, lora_mode_t mode,
                                          uint32_t flags, int32_t *err_out, lora_stream_t stream);

/* ---- errors ------------------------------------------------------------------- */

/* Synchronise `stream`, read the workspace's error word into *first_bad_row
 * (HOST; -1 if no bad id was seen since the last call) and clear it. */
lora_status_t lora_get_device_error(void *ws, size_t ws_bytes, lora_stream_t stream,
                                    int32_t *first_bad_row);

/* Static string for a status code. */
const char *lora_status_string(lora_status_t status);

/* Library version string, e.g. "liblora 0.1 gfx950". */
const char *lora_version(void);

#ifdef __cplusplus
}
#endif
#endif /* LORA_H_ */
