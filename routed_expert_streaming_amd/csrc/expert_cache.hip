// C ABI of the HBM expert-slot cache (include/moe.h): LRU metadata on the
// host (expert_cache_core), one hipMemcpyAsync per miss from pinned host
// memory into the slot on a copy stream, per-slot events for ordering.
//
// Sources: WISP launch post, section "통찰" (lookups in the fastest tier
// that holds the expert, LRU promotion) and section "더블 버퍼 비동기
// 파이프라인" (expert loads from pinned RAM overlap GPU compute); WASTE
// article, section "유휴 가중치는 메모리가 아니라 제때 닿기만 하면 된다" (one
// aligned record per expert, so a miss costs exactly one transfer).
#include "expert_cache.h"

#include <climits>
#include <new>

namespace moe {
int fail(int code, const char *fmt, ...);
int hip_fail(hipError_t e, const char *what);

int cache_wait(moe_cache *c, int32_t slot, hipStream_t s) {
    if (!c) return fail(MOE_E_INVAL, "cache is NULL");
    if (slot < 0 || slot >= c->core.capacity()) return fail(MOE_E_STATE, "slot %d out of range", slot);
    if (!c->filled[slot]) return fail(MOE_E_STATE, "slot %d has never been filled", slot);
    hipError_t e = hipStreamWaitEvent(s, c->ready[slot], 0);
    if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent(ready)");
    return MOE_OK;
}

int cache_release(moe_cache *c, int32_t slot, hipStream_t s) {
    if (!c) return fail(MOE_E_INVAL, "cache is NULL");
    if (slot < 0 || slot >= c->core.capacity()) return fail(MOE_E_STATE, "slot %d out of range", slot);
    hipError_t e = hipEventRecord(c->last_use[slot], s);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord(last_use)");
    c->used[slot] = 1;
    return MOE_OK;
}
}  // namespace moe

using namespace moe;

namespace {
void destroy_events(moe_cache *c) {
    for (hipEvent_t e : c->ready)
        if (e) (void)hipEventDestroy(e);
    for (hipEvent_t e : c->last_use)
        if (e) (void)hipEventDestroy(e);
    c->ready.clear();
    c->last_use.clear();
    if (c->h_idx) (void)hipHostFree(c->h_idx);
    c->h_idx = nullptr;
}
}  // namespace

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
    c->last_use.assign(capacity, nullptr);
    c->filled.assign(capacity, 0);
    c->used.assign(capacity, 0);
    hipError_t e = hipGetDevice(&c->device);
    for (int s = 0; e == hipSuccess && s < capacity; s++) {
        e = hipEventCreateWithFlags(&c->ready[s], hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&c->last_use[s], hipEventDisableTiming);
    }
    if (e == hipSuccess) e = hipHostMalloc((void **)&c->h_idx, 2 * MOE_MAX_K * sizeof(int32_t), hipHostMallocDefault);
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
    if (c->used[s]) e = hipStreamWaitEvent(cs, c->last_use[s], 0);      // readers of the victim first
    if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent(last_use)");
    e = hipMemcpyAsync(c->pool + (size_t)s * c->slot_bytes, host_src, c->slot_bytes, hipMemcpyHostToDevice, cs);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(slot)");    // nothing enqueued: cache unchanged
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
