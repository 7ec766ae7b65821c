// C ABI of the HBM expert-slot cache (include/moe.h): LRU metadata on the
// host (expert_cache_core), one hipMemcpyAsync per miss from host memory into
// the slot on a copy stream (pageable records through pinned bounce buffers
// filled by host threads), per-slot events for ordering.
//
// Sources: WISP launch post, section "통찰" (lookups in the fastest tier
// that holds the expert, LRU promotion) and section "더블 버퍼 비동기
// 파이프라인" (expert loads from pinned RAM overlap GPU compute); WASTE
// article, section "유휴 가중치는 메모리가 아니라 제때 닿기만 하면 된다" (one
// aligned record per expert, so a miss costs exactly one transfer).
#include "expert_cache.h"

#include <algorithm>
#include <climits>
#include <cstring>
#include <new>

namespace moe {
int fail(int code, const char *fmt, ...);
int hip_fail(hipError_t e, const char *what);

int cache_wait(moe_cache *c, int32_t slot, hipStream_t s) {
    if (!c) return fail(MOE_E_INVAL, "cache is NULL");
    if (slot < 0 || slot >= c->core.capacity()) return fail(MOE_E_STATE, "slot %d out of range", slot);
    if (!c->filled[slot]) return fail(MOE_E_STATE, "slot %d has never been filled", slot);
    // a copy that has landed already needs no wait on the stream
    hipError_t e = hipEventQuery(c->ready[slot]);
    if (e == hipSuccess) return MOE_OK;
    if (e != hipErrorNotReady) return hip_fail(e, "hipEventQuery(ready)");
    e = hipStreamWaitEvent(s, c->ready[slot], 0);
    if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent(ready)");
    return MOE_OK;
}

int cache_release_many(moe_cache *c, const int32_t *slots, int n, hipStream_t s) {
    if (!c) return fail(MOE_E_INVAL, "cache is NULL");
    for (int i = 0; i < n; i++)
        if (slots[i] < 0 || slots[i] >= c->core.capacity()) return fail(MOE_E_STATE, "slot %d out of range", slots[i]);
    if (n <= 0) return MOE_OK;
    int32_t ev;
    if (!c->use_free.empty()) {
        ev = c->use_free.back();
        c->use_free.pop_back();
    } else {
        hipEvent_t h = nullptr;
        hipError_t e = hipEventCreateWithFlags(&h, hipEventDisableTiming);
        if (e != hipSuccess) return hip_fail(e, "hipEventCreateWithFlags(readers)");
        ev = (int32_t)c->use_ev.size();
        c->use_ev.push_back(h);
        c->use_refs.push_back(0);
    }
    hipError_t e = hipEventRecord(c->use_ev[ev], s);
    if (e != hipSuccess) {
        c->use_free.push_back(ev);
        return hip_fail(e, "hipEventRecord(readers)");
    }
    for (int i = 0; i < n; i++) {
        int32_t &u = c->slot_use[slots[i]];
        if (u == ev) continue;               // the slot appears twice in the batch
        if (u >= 0 && --c->use_refs[u] == 0) c->use_free.push_back(u);
        u = ev;
        c->use_refs[ev]++;
    }
    return MOE_OK;
}

int cache_release(moe_cache *c, int32_t slot, hipStream_t s) { return cache_release_many(c, &slot, 1, s); }

hipError_t cache_wait_readers(moe_cache *c, int32_t slot, hipStream_t s) {
    const int32_t u = c->slot_use[slot];
    if (u < 0) return hipSuccess;
    // readers long done (the usual case for an LRU victim): no wait enqueued
    const hipError_t q = hipEventQuery(c->use_ev[u]);
    if (q == hipSuccess) return hipSuccess;
    if (q != hipErrorNotReady) return q;
    return hipStreamWaitEvent(s, c->use_ev[u], 0);
}
}  // namespace moe

using namespace moe;

namespace {
void destroy_events(moe_cache *c) {
    if (c->ps2) (void)hipStreamSynchronize(c->ps2);   // its copies record the events below
    for (hipEvent_t e : c->ready)
        if (e) (void)hipEventDestroy(e);
    for (hipEvent_t e : c->use_ev)
        if (e) (void)hipEventDestroy(e);
    c->ready.clear();
    c->use_ev.clear();
    if (c->h_idx) (void)hipHostFree(c->h_idx);
    c->h_idx = nullptr;
    if (c->idx_ev) (void)hipEventDestroy(c->idx_ev);
    if (c->ahead_ev) (void)hipEventDestroy(c->ahead_ev);
    c->idx_ev = c->ahead_ev = nullptr;
    if (c->ps2) (void)hipStreamDestroy(c->ps2);
    if (c->ps2_done) (void)hipEventDestroy(c->ps2_done);
    c->ps2 = nullptr;
    c->ps2_done = nullptr;
    for (int b = 0; b < moe::kBounce; b++) {
        if (c->bounce_used[b]) (void)hipEventSynchronize(c->bounce_done[b]);
        if (c->bounce_done[b]) (void)hipEventDestroy(c->bounce_done[b]);
        if (c->bounce[b]) (void)hipHostFree(c->bounce[b]);
        c->bounce_done[b] = nullptr;
        c->bounce[b] = nullptr;
        c->bounce_used[b] = false;
    }
    delete c->copier;
    c->copier = nullptr;
}

bool page_locked(const void *p) {
    hipPointerAttribute_t at;
    if (hipPointerGetAttributes(&at, p) != hipSuccess) {
        (void)hipGetLastError();          // pageable memory may be reported as an error
        return false;
    }
    return at.type == hipMemoryTypeHost;
}
}  // namespace

namespace moe {
bool host_page_locked(const void *p) { return page_locked(p); }

CopyPool::CopyPool(int n) : n_((size_t)n) {
    th_.reserve(n_);
    for (int i = 0; i < n; i++) th_.emplace_back(&CopyPool::worker, this, i);
}
CopyPool::~CopyPool() {
    {
        std::lock_guard<std::mutex> g(m_);
        stop_ = true;
    }
    go_.notify_all();
    for (auto &t : th_) t.join();
}
void CopyPool::worker(int i) {
    unsigned seen = 0;
    for (;;) {
        char *dst;
        const char *src;
        size_t bytes;
        {
            std::unique_lock<std::mutex> l(m_);
            go_.wait(l, [&] { return stop_ || gen_ != seen; });
            if (stop_) return;
            seen = gen_;
            dst = dst_;
            src = src_;
            bytes = bytes_;
        }
        // slice i of n, on 4 KiB boundaries
        const size_t n = n_, pages = (bytes + 4095) / 4096;
        const size_t a = std::min(bytes, pages * i / n * 4096), b = std::min(bytes, pages * (i + 1) / n * 4096);
        if (b > a) std::memcpy(dst + a, src + a, b - a);
        std::lock_guard<std::mutex> g(m_);
        if (--pending_ == 0) done_.notify_one();
    }
}
void CopyPool::copy(void *dst, const void *src, size_t bytes) {
    std::unique_lock<std::mutex> l(m_);
    dst_ = (char *)dst;
    src_ = (const char *)src;
    bytes_ = bytes;
    pending_ = (int)n_;
    gen_++;
    go_.notify_all();
    done_.wait(l, [&] { return pending_ == 0; });
}

hipError_t cache_copy_in(moe_cache *c, int32_t s, const void *src, hipStream_t ps, bool *enqueued) {
    char *dst = c->pool + (size_t)s * c->slot_bytes;
    *enqueued = false;
    if (page_locked(src)) {
        const hipError_t e = hipMemcpyAsync(dst, src, c->slot_bytes, hipMemcpyHostToDevice, ps);
        *enqueued = e == hipSuccess;
        return e;
    }
    hipError_t e = hipSuccess;
    if (!c->copier) {
        for (int b = 0; e == hipSuccess && b < kBounce; b++) {
            e = hipHostMalloc((void **)&c->bounce[b], c->slot_bytes, hipHostMallocDefault);
            if (e == hipSuccess) e = hipEventCreateWithFlags(&c->bounce_done[b], hipEventDisableTiming);
        }
        if (e != hipSuccess) return e;
        const unsigned hw = std::thread::hardware_concurrency();
        c->copier = new (std::nothrow) CopyPool((int)std::max(1u, std::min(8u, hw ? hw : 1u)));
        if (!c->copier) return hipErrorOutOfMemory;
    }
    const int b = c->bounce_next;
    c->bounce_next = (b + 1) % kBounce;
    if (c->bounce_used[b] && (e = hipEventSynchronize(c->bounce_done[b])) != hipSuccess) return e;
    c->bounce_used[b] = false;
    c->copier->copy(c->bounce[b], src, c->slot_bytes);
    e = hipMemcpyAsync(dst, c->bounce[b], c->slot_bytes, hipMemcpyHostToDevice, ps);
    if (e != hipSuccess) return e;
    *enqueued = true;
    e = hipEventRecord(c->bounce_done[b], ps);
    if (e != hipSuccess) {
        // the buffer's transfer is in flight but cannot be waited on: drain
        // the copy stream so that the buffer can be refilled safely
        (void)hipStreamSynchronize(ps);
        c->bounce_used[b] = false;
        return e;
    }
    c->bounce_used[b] = true;
    return hipSuccess;
}
}  // namespace moe

extern "C" {

int expert_cache_create(int32_t capacity, uint64_t slot_bytes, void *pool_dev, moe_cache **out) {
    if (!out) return fail(MOE_E_INVAL, "out is NULL");
    *out = nullptr;
    if (capacity < 1) return fail(MOE_E_INVAL, "capacity %d < 1", capacity);
    if (slot_bytes == 0 || slot_bytes % 256) return fail(MOE_E_INVAL, "slot_bytes must be a positive multiple of 256");
    if (!pool_dev) return fail(MOE_E_INVAL, "pool is NULL");
    moe_cache *c = new (std::nothrow) moe_cache(capacity);
    if (!c) return fail(MOE_E_NOMEM, "host allocation failed");
    c->pool = (char *)pool_dev;
    c->slot_bytes = slot_bytes;
    c->ready.assign(capacity, nullptr);
    c->slot_use.assign(capacity, -1);
    c->filled.assign(capacity, 0);
    hipError_t e = hipGetDevice(&c->device);
    for (int s = 0; e == hipSuccess && s < capacity; s++) {
        e = hipEventCreateWithFlags(&c->ready[s], hipEventDisableTiming);
    }
    if (e == hipSuccess) e = hipHostMalloc((void **)&c->h_idx, (kIdsFlag + 1) * sizeof(int32_t), hipHostMallocDefault);
    if (e == hipSuccess) c->h_idx[kIdsFlag] = 0;   // no sequence number yet (they start at 1)
    if (e == hipSuccess) e = hipEventCreateWithFlags(&c->idx_ev, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&c->ahead_ev, hipEventDisableTiming);
    if (e == hipSuccess) e = hipStreamCreateWithFlags(&c->ps2, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&c->ps2_done, hipEventDisableTiming);
    if (e != hipSuccess) {
        destroy_events(c);
        delete c;
        return hip_fail(e, "expert_cache_create");
    }
    *out = c;
    return MOE_OK;
}

void expert_cache_destroy(moe_cache *c) {
    if (!c) return;
    destroy_events(c);
    delete c;
}

int expert_cache_lookup(moe_cache *c, uint32_t key, int32_t *slot) {
    if (!c || !slot) return fail(MOE_E_INVAL, "cache and slot must be non-NULL");
    *slot = c->core.lookup(key);
    return MOE_OK;
}

int expert_cache_insert(moe_cache *c, uint32_t key, const void *host_src, void *copy_stream, int32_t *slot,
                        uint32_t *evicted) {
    if (!c || !host_src || !slot || !evicted) return fail(MOE_E_INVAL, "cache, host_src, slot, evicted must be non-NULL");
    if (key == MOE_NO_KEY) return fail(MOE_E_INVAL, "key 0xFFFFFFFF is reserved");
    uint32_t victim = kNoKey;
    const int s = c->core.plan_insert(key, &victim);
    if (s < 0) return fail(MOE_E_STATE, "key %u is already cached", key);
    hipStream_t cs = (hipStream_t)copy_stream;
    hipError_t e = hipSuccess;
    e = cache_wait_readers(c, s, cs);      // readers of the victim first
    if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent(readers)");
    bool enqueued = false;
    e = moe::cache_copy_in(c, s, host_src, cs, &enqueued);
    if (e != hipSuccess) {
        if (enqueued) {
            // the slot's bytes are being overwritten: the victim it held is
            // gone, so forget it and leave the slot free
            c->core.drop_slot(s);
            c->filled[s] = 0;
        }
        // otherwise nothing was enqueued: the cache is unchanged
        return hip_fail(e, "copy into slot");
    }
    e = hipEventRecord(c->ready[s], cs);
    if (e != hipSuccess) {
        // the copy is in flight but cannot be waited on: the slot no longer
        // holds the victim, so forget it and leave the slot free
        c->core.drop_slot(s);
        c->filled[s] = 0;
        return hip_fail(e, "hipEventRecord(ready)");
    }
    c->filled[s] = 1;
    c->core.commit_insert(key, s, victim);
    *slot = s;
    *evicted = victim;
    return MOE_OK;
}

int expert_cache_wait(moe_cache *c, int32_t slot, void *compute_stream) {
    return cache_wait(c, slot, (hipStream_t)compute_stream);
}

int expert_cache_release(moe_cache *c, int32_t slot, void *compute_stream) {
    return cache_release(c, slot, (hipStream_t)compute_stream);
}

int expert_cache_slot_ptr(moe_cache *c, int32_t slot, void **ptr) {
    if (!c || !ptr) return fail(MOE_E_INVAL, "cache and ptr must be non-NULL");
    if (slot < 0 || slot >= c->core.capacity()) return fail(MOE_E_STATE, "slot %d out of range", slot);
    *ptr = c->pool + (size_t)slot * c->slot_bytes;
    return MOE_OK;
}

int expert_cache_trace(moe_cache *c, moe_trace_rec *buf, int64_t cap, int64_t *n) {
    if (!c || !n) return fail(MOE_E_INVAL, "cache and n must be non-NULL");
    const auto &tr = c->core.trace();
    *n = (int64_t)tr.size();
    const int64_t m = cap < *n ? cap : *n;
    if (m > 0 && !buf) return fail(MOE_E_INVAL, "buf is NULL");
    for (int64_t i = 0; i < m; i++) buf[i] = {tr[i].key, tr[i].hit, tr[i].slot, tr[i].evicted};
    if (cap < *n) return fail(MOE_E_SPACE, "trace holds %lld records, buffer %lld", (long long)*n, (long long)cap);
    return MOE_OK;
}

int expert_cache_trace_reset(moe_cache *c) {
    if (!c) return fail(MOE_E_INVAL, "cache is NULL");
    c->core.trace_reset();
    return MOE_OK;
}

int moe_lru_stack_distances(const uint32_t *keys, int64_t n, int32_t *dist) {
    if (n < 0) return fail(MOE_E_INVAL, "n=%lld < 0", (long long)n);
    if (n > 0 && (!keys || !dist)) return fail(MOE_E_INVAL, "keys and dist must be non-NULL");
    if (n > INT32_MAX) return fail(MOE_E_INVAL, "n=%lld exceeds the 32-bit distance range", (long long)n);
    try {
        lru_stack_distances(keys, n, dist);
    } catch (const std::bad_alloc &) {
        return fail(MOE_E_SPACE, "out of host memory for %lld references", (long long)n);
    }
    return MOE_OK;
}

int expert_cache_stats_ahead(moe_cache *c, int64_t *inserted, int64_t *present, int64_t *used, int64_t *wasted) {
    if (!c) return fail(MOE_E_INVAL, "cache is NULL");
    if (inserted) *inserted = c->core.ahead_inserts;
    if (present) *present = c->core.ahead_present;
    if (used) *used = c->core.ahead_used;
    if (wasted) *wasted = c->core.ahead_wasted;
    return MOE_OK;
}

int expert_cache_stats(moe_cache *c, int64_t *lookups, int64_t *hits, int64_t *inserts, int64_t *evictions) {
    if (!c) return fail(MOE_E_INVAL, "cache is NULL");
    if (lookups) *lookups = c->core.lookups;
    if (hits) *hits = c->core.hits;
    if (inserts) *inserts = c->core.inserts;
    if (evictions) *evictions = c->core.evictions;
    return MOE_OK;
}

}  // extern "C"
