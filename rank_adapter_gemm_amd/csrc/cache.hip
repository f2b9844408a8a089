// Adapter residency: a host tier of registered adapters and the pool's HBM
// slots as a cache over it, with least-recently-used replacement.
//
// The tiers and their movement follow "Multi-LoRA Serving: Architecture for
// Thousands of Adapters" (sections "Unified paging of adapters and KV cache"
// and "A worked memory example": adapters kept in host DRAM and brought into
// GPU memory on demand) and "Serving LoRA adapters: from the model name to
// the wrapped layer", Step 3 (a fixed number of GPU slots, the least recently
// used adapter evicted to make room, activation copying an adapter into its
// slot).  Two failure modes listed in "Multi-LoRA Serving 与 Adapter 隔离"
// shape the ordering: an adapter's storage is never overwritten while
// in-flight kernels may still read it (each slot's last use is an event the
// copy waits for), and a re-registered adapter is never served from its old
// copy (registration drops residency).
//
// Registered adapters live in HOST memory already in the slot layout (see
// lora_pack_host), so promotion is a plain copy per buffer on the caller's
// copy stream, overlapping compute.  Buffers in page-locked memory that the
// HIP runtime maps into the GPU's address space are copied by one gather
// kernel per 32 buffers, reading them directly over the host link (an
// asynchronous memory copy per buffer costs tens of microseconds of fixed
// overhead, which dominates slot-sized buffers); other buffers go through
// hipMemcpyAsync.  Scale and rank are published by one kernel per batch of
// slots after the copies.
#include <cstring>
#include <new>
#include <vector>

#include "common.hpp"

struct lora_cache {
    int32_t n_slots = 0, n_pools = 0, max_adapters = 0;
    lora_pool_t pools[lora::kMaxCachePools];
    struct adapter {
        bool registered = false;
        int32_t rank = 0;
        float alpha = 0.0f;
        const void *a[lora::kMaxCachePools] = {};
        const void *b[lora::kMaxCachePools] = {};
        const void *dev_a[lora::kMaxCachePools] = {};   // device-visible address of a[p], or null
        const void *dev_b[lora::kMaxCachePools] = {};
    };
    std::vector<adapter> adapters;
    std::vector<int32_t> slot_of;     // adapter -> slot, -1 if not resident
    std::vector<int32_t> owner;       // slot -> adapter, -1 if empty
    std::vector<uint64_t> touched;    // slot -> LRU clock of its last batch
    std::vector<hipEvent_t> last_use; // slot -> event after the last batch that used it
    std::vector<char> used;           // last_use has been recorded
    hipEvent_t ready = nullptr;       // after a batch's uploads, on the copy stream
    std::vector<int32_t> batch;       // slots of the last mapped batch
    uint64_t clock = 0;
    int64_t hits = 0, misses = 0, evictions = 0, bytes = 0;
};

namespace {

inline hipStream_t hs(lora_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

// The address at which a kernel can read host buffer p: page-locked host
// memory that the runtime reports as mapped into the device's address
// space, 16-byte aligned; else null (the buffer is copied by the runtime).
const void *device_view(const void *p) {
    if (!p || (reinterpret_cast<uintptr_t>(p) & 15u)) return nullptr;
    hipPointerAttribute_t at;
    if (hipPointerGetAttributes(&at, p) != hipSuccess) {
        (void)hipGetLastError();                      // pageable memory: not an error here
        return nullptr;
    }
    if (at.type != hipMemoryTypeHost || !at.devicePointer) return nullptr;
    const char *host_base = at.hostPointer ? static_cast<const char *>(at.hostPointer) : static_cast<const char *>(p);
    const char *dev = static_cast<const char *>(at.devicePointer) + (static_cast<const char *>(p) - host_base);
    return (reinterpret_cast<uintptr_t>(dev) & 15u) ? nullptr : dev;
}

}  // namespace

extern "C" {

lora_status_t lora_pack_host(int32_t d_in, int32_t d_out, int32_t max_rank, lora_dtype_t dtype,
                             const void *A, int32_t lda, const void *B, int32_t ldb, int32_t r,
                             void *a_slot, void *b_slot) {
    if ((dtype != LORA_F32 && dtype != LORA_BF16) || d_in <= 0 || d_out <= 0 || (d_in % 8) ||
        (d_out % 8) || max_rank < 8 || max_rank > 128 || (max_rank % 8))
        return LORA_ERR_INVALID_ARGUMENT;
    if (r > max_rank) return LORA_ERR_RANK_EXCEEDS_MAX;
    if (r < 1 || !A || !B || !a_slot || !b_slot || lda < r || ldb < d_out) return LORA_ERR_INVALID_ARGUMENT;
    const size_t eb = dtype == LORA_F32 ? 4 : 2;
    const char *Ab = static_cast<const char *>(A), *Bb = static_cast<const char *>(B);
    char *ab = static_cast<char *>(a_slot), *bb = static_cast<char *>(b_slot);
    // A^T [max_rank][d_in]: rank row j holds column j of A; rows >= r are zero
    for (int32_t j = 0; j < max_rank; ++j)
        for (int32_t i = 0; i < d_in; ++i) {
            char *dst = ab + ((size_t)j * d_in + i) * eb;
            if (j < r) memcpy(dst, Ab + ((size_t)i * lda + j) * eb, eb);
            else memset(dst, 0, eb);
        }
    // B in rank octets [max_rank/8][d_out][8]
    for (int32_t g = 0; g < max_rank / 8; ++g)
        for (int32_t n = 0; n < d_out; ++n)
            for (int32_t q = 0; q < 8; ++q) {
                const int32_t j = g * 8 + q;
                char *dst = bb + (((size_t)g * d_out + n) * 8 + q) * eb;
                if (j < r) memcpy(dst, Bb + ((size_t)j * ldb + n) * eb, eb);
                else memset(dst, 0, eb);
            }
    return LORA_OK;
}

lora_status_t lora_cache_create(lora_cache_t **out, int32_t n_slots, const lora_pool_t *pools,
                                int32_t n_pools, int32_t max_adapters) {
    if (!out || n_slots < 1 || n_slots > lora::kMaxSlots || n_pools < 0 || max_adapters < 1 ||
        (n_pools > 0 && !pools))
        return LORA_ERR_INVALID_ARGUMENT;
    if (n_pools > lora::kMaxCachePools) return LORA_ERR_UNSUPPORTED;
    for (int32_t p = 0; p < n_pools; ++p) {
        const lora_pool_t &q = pools[p];
        if (q.n_slots < n_slots || !q.a || !q.b || !q.scale || !q.rank || q.max_rank < 8 ||
            q.max_rank > 128 || q.max_rank != pools[0].max_rank || q.dtype != pools[0].dtype)
            return LORA_ERR_INVALID_ARGUMENT;
        if (q.row0 || q.row0_host) return LORA_ERR_UNSUPPORTED;   // slots of one size only
    }
    lora_cache *c = new (std::nothrow) lora_cache;
    if (!c) return LORA_ERR_UNSUPPORTED;
    c->n_slots = n_slots;
    c->n_pools = n_pools;
    c->max_adapters = max_adapters;
    for (int32_t p = 0; p < n_pools; ++p) c->pools[p] = pools[p];
    c->adapters.resize(max_adapters);
    c->slot_of.assign(max_adapters, -1);
    c->owner.assign(n_slots, -1);
    c->touched.assign(n_slots, 0);
    c->used.assign(n_slots, 0);
    if (n_pools > 0) {
        c->last_use.assign(n_slots, nullptr);
        bool ok = hipEventCreateWithFlags(&c->ready, hipEventDisableTiming) == hipSuccess;
        for (int32_t s = 0; ok && s < n_slots; ++s)
            ok = hipEventCreateWithFlags(&c->last_use[s], hipEventDisableTiming) == hipSuccess;
        if (!ok) {
            lora_cache_destroy(c);
            return LORA_ERR_HIP;
        }
    }
    *out = c;
    return LORA_OK;
}

lora_status_t lora_cache_destroy(lora_cache_t *c) {
    if (!c) return LORA_ERR_INVALID_ARGUMENT;
    for (hipEvent_t e : c->last_use)
        if (e) (void)hipEventDestroy(e);
    if (c->ready) (void)hipEventDestroy(c->ready);
    delete c;
    return LORA_OK;
}

lora_status_t lora_cache_register(lora_cache_t *c, int32_t adapter, const void *const *host_a,
                                  const void *const *host_b, int32_t rank, float alpha) {
    if (!c || adapter < 0 || adapter >= c->max_adapters) return LORA_ERR_INVALID_ARGUMENT;
    if (c->n_pools > 0 && rank > c->pools[0].max_rank) return LORA_ERR_RANK_EXCEEDS_MAX;
    if (rank < 1) return LORA_ERR_INVALID_ARGUMENT;
    if (c->n_pools > 0) {
        if (!host_a || !host_b) return LORA_ERR_INVALID_ARGUMENT;
        for (int32_t p = 0; p < c->n_pools; ++p)
            if (!host_a[p] || !host_b[p]) return LORA_ERR_INVALID_ARGUMENT;
    }
    lora_cache::adapter &ad = c->adapters[adapter];
    ad.registered = true;
    ad.rank = rank;
    ad.alpha = alpha;
    for (int32_t p = 0; p < c->n_pools; ++p) {
        ad.a[p] = host_a[p];
        ad.b[p] = host_b[p];
        ad.dev_a[p] = device_view(host_a[p]);
        ad.dev_b[p] = device_view(host_b[p]);
    }
    // a new version of a resident adapter must not be served from the old copy
    const int32_t s = c->slot_of[adapter];
    if (s >= 0) {
        c->owner[s] = -1;
        c->slot_of[adapter] = -1;
    }
    return LORA_OK;
}

lora_status_t lora_cache_map(lora_cache_t *c, const int32_t *adapters, int32_t n, int32_t *slots,
                             lora_stream_t compute, lora_stream_t copy) {
    if (!c || n < 0 || (n > 0 && (!adapters || !slots))) return LORA_ERR_INVALID_ARGUMENT;
    // validate first: an invalid batch changes nothing
    std::vector<int32_t> distinct;
    std::vector<char> seen(c->max_adapters, 0);
    for (int32_t i = 0; i < n; ++i) {
        const int32_t a = adapters[i];
        if (a == -1) continue;
        if (a < 0 || a >= c->max_adapters || !c->adapters[a].registered) return LORA_ERR_INVALID_ARGUMENT;
        if (!seen[a]) {
            seen[a] = 1;
            distinct.push_back(a);
        }
    }
    if ((int32_t)distinct.size() > c->n_slots) return LORA_ERR_UNSUPPORTED;

    // slots this batch needs: resident adapters keep theirs
    std::vector<char> needed(c->n_slots, 0);
    for (int32_t a : distinct)
        if (c->slot_of[a] >= 0) needed[c->slot_of[a]] = 1;
    // misses take an empty slot, else the least recently used one not needed here
    std::vector<std::pair<int32_t, int32_t>> uploads;   // (slot, adapter)
    for (int32_t a : distinct) {
        if (c->slot_of[a] >= 0) {
            ++c->hits;
            continue;
        }
        int32_t best = -1;
        for (int32_t s = 0; s < c->n_slots; ++s) {
            if (needed[s]) continue;
            if (best < 0) best = s;
            const bool empty_s = c->owner[s] < 0, empty_b = c->owner[best] < 0;
            if ((empty_s && !empty_b) || (empty_s == empty_b && c->touched[s] < c->touched[best])) best = s;
        }
        if (c->owner[best] >= 0) {
            c->slot_of[c->owner[best]] = -1;
            ++c->evictions;
        }
        c->owner[best] = a;
        c->slot_of[a] = best;
        needed[best] = 1;
        ++c->misses;
        uploads.push_back({best, a});
    }
    ++c->clock;
    c->batch.clear();
    for (int32_t a : distinct) {
        c->touched[c->slot_of[a]] = c->clock;
        c->batch.push_back(c->slot_of[a]);
    }
    for (int32_t i = 0; i < n; ++i) slots[i] = adapters[i] == -1 ? -1 : c->slot_of[adapters[i]];
    if (c->n_pools == 0 || uploads.empty()) return LORA_OK;

    // device side: wait for the victims' last uses, then every copy (gather
    // kernels over mapped host memory, runtime copies for the rest), then one
    // kernel per kMetaBatch slots that publishes scale and rank in all pools
    const hipStream_t cs = hs(copy), ks = hs(compute);
    const size_t eb = c->pools[0].dtype == LORA_F32 ? 4 : 2;
    for (const auto &u : uploads)
        if (c->used[u.first] && hipStreamWaitEvent(cs, c->last_use[u.first], 0) != hipSuccess)
            return LORA_ERR_HIP;
    lora::copy_batch cb;
    cb.n = 0;
    cb.max_bytes = 0;
    auto flush = [&]() -> lora_status_t {
        const lora_status_t st = lora::launch_copy_batch(cb, cs);
        cb.n = 0;
        cb.max_bytes = 0;
        return st;
    };
    // one buffer: into the gather kernel's batch if the kernel can read it, else a runtime copy
    auto copy_one = [&](void *dst, const void *host, const void *dev, size_t bytes) -> lora_status_t {
        if (dev && bytes < (size_t(1) << 31)) {
            cb.src[cb.n] = dev;
            cb.dst[cb.n] = dst;
            cb.bytes[cb.n] = (uint32_t)bytes;
            cb.max_bytes = cb.max_bytes > (uint32_t)bytes ? cb.max_bytes : (uint32_t)bytes;
            return ++cb.n == lora::kCopyBatch ? flush() : LORA_OK;
        }
        return hipMemcpyAsync(dst, host, bytes, hipMemcpyHostToDevice, cs) == hipSuccess ? LORA_OK : LORA_ERR_HIP;
    };
    for (const auto &u : uploads) {
        const int32_t s = u.first;
        const lora_cache::adapter &ad = c->adapters[u.second];
        for (int32_t p = 0; p < c->n_pools; ++p) {
            const lora_pool_t &q = c->pools[p];
            const size_t ab = (size_t)q.max_rank * q.d_in * eb, bb = (size_t)q.max_rank * q.d_out * eb;
            lora_status_t st = copy_one((char *)q.a + (size_t)s * ab, ad.a[p], ad.dev_a[p], ab);
            if (st == LORA_OK) st = copy_one((char *)q.b + (size_t)s * bb, ad.b[p], ad.dev_b[p], bb);
            if (st != LORA_OK) return st;
            c->bytes += (int64_t)(ab + bb);
        }
    }
    if (cb.n > 0) {
        const lora_status_t st = flush();
        if (st != LORA_OK) return st;
    }
    for (size_t i0 = 0; i0 < uploads.size(); i0 += lora::kMetaBatch) {
        lora::meta_batch m;
        m.n_pools = c->n_pools;
        for (int32_t p = 0; p < lora::kMaxCachePools; ++p) {
            m.scale[p] = p < c->n_pools ? c->pools[p].scale : nullptr;
            m.rank[p] = p < c->n_pools ? c->pools[p].rank : nullptr;
        }
        m.n = 0;
        for (size_t i = i0; i < uploads.size() && m.n < lora::kMetaBatch; ++i, ++m.n) {
            const lora_cache::adapter &ad = c->adapters[uploads[i].second];
            m.slot[m.n] = uploads[i].first;
            m.s[m.n] = ad.alpha / (float)ad.rank;
            m.r[m.n] = ad.rank;
        }
        lora_status_t st = lora::launch_pool_meta_batch(m, cs);
        if (st != LORA_OK) return st;
    }
    if (hipEventRecord(c->ready, cs) != hipSuccess || hipStreamWaitEvent(ks, c->ready, 0) != hipSuccess)
        return LORA_ERR_HIP;
    return LORA_OK;
}

lora_status_t lora_cache_commit(lora_cache_t *c, lora_stream_t compute) {
    if (!c) return LORA_ERR_INVALID_ARGUMENT;
    if (c->n_pools == 0) return LORA_OK;
    for (int32_t s : c->batch) {
        if (hipEventRecord(c->last_use[s], hs(compute)) != hipSuccess) return LORA_ERR_HIP;
        c->used[s] = 1;
    }
    return LORA_OK;
}

lora_status_t lora_cache_slot_of(const lora_cache_t *c, int32_t adapter, int32_t *slot) {
    if (!c || !slot || adapter < 0 || adapter >= c->max_adapters) return LORA_ERR_INVALID_ARGUMENT;
    *slot = c->slot_of[adapter];
    return LORA_OK;
}

lora_status_t lora_cache_stats(const lora_cache_t *c, int64_t *hits, int64_t *misses,
                               int64_t *evictions, int64_t *bytes_uploaded) {
    if (!c || !hits || !misses || !evictions || !bytes_uploaded) return LORA_ERR_INVALID_ARGUMENT;
    *hits = c->hits;
    *misses = c->misses;
    *evictions = c->evictions;
    *bytes_uploaded = c->bytes;
    return LORA_OK;
}

}  // extern "C"
