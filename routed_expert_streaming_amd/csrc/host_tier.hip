// Third tier of the streamed decode: expert records in a file, read with
// O_DIRECT (no OS page cache) through a small pageable bounce buffer per I/O
// thread into a pinned host slot pool kept as LRU; it is the source of the
// HBM slot cache's misses.
//
// Sources: WASTE article ("2.78조 파라미터 모델을 노트북에서: NVMe 스트리밍 추론
// 엔진 WASTE"), section "유휴 가중치는 메모리가 아니라 제때 닿기만 하면 된다"
// (one 4 KiB-aligned record per expert, so a miss costs one aligned read;
// reads bypass the page cache so that measured hit rates are real); WISP
// launch post, section "통찰" (VRAM, then RAM, then NVMe: each lookup goes to
// the fastest tier that holds the expert, and LRU promotes what is used).
#include "host_tier.h"

#include <fcntl.h>
#include <sys/stat.h>
#include <unistd.h>

#include <cerrno>
#include <cstdlib>
#include <chrono>
#include <cstring>
#include <algorithm>
#include <new>
#include <thread>

namespace moe {
int fail(int code, const char *fmt, ...);
int hip_fail(hipError_t e, const char *what);

namespace {
// Read one record into dst (4 KiB-aligned) at its file offset; false on a
// short read or an error.
bool read_record(int fd, char *dst, uint64_t bytes, int64_t index) {
    uint64_t done = 0;
    const off_t base = (off_t)((uint64_t)index * bytes);
    while (done < bytes) {
        const ssize_t r = pread(fd, dst + done, bytes - done, base + (off_t)done);
        if (r < 0 && errno == EINTR) continue;
        if (r <= 0) return false;
        done += (uint64_t)r;
    }
    return true;
}
}  // namespace

// Records recs[q] into dst[q] (q < nt), spread over the I/O threads; on a
// failed read returns an error with *bad = its index.
int read_parallel(moe_host_tier *t, const int64_t *recs, char *const *dst, int nt, int *bad) {
    if (!nt) return MOE_OK;
    const auto t0 = std::chrono::steady_clock::now();
    bool ok[MOE_MAX_K];
    int err[MOE_MAX_K];
    const int nthr = std::min(nt, t->io_threads);
    auto worker = [&](int w) {
        for (int q = w; q < nt; q += nthr) {
            errno = 0;
            ok[q] = read_record(t->fd, t->bounce[w], t->record_bytes, recs[q]);
            err[q] = ok[q] ? 0 : (errno ? errno : EIO);
            if (ok[q]) memcpy(dst[q], t->bounce[w], t->record_bytes);
        }
    };
    if (nthr <= 1) {
        worker(0);
    } else {
        std::thread th[MOE_MAX_K];
        int started = 0;
        try {
            for (int w = 1; w < nthr; w++, started++) th[w] = std::thread(worker, w);
        } catch (...) {
        }
        worker(0);
        for (int w = 1; w <= started; w++) th[w].join();
        for (int w = started + 1; w < nthr; w++) worker(w);   // threads that could not start
    }
    t->read_ns += (int64_t)std::chrono::duration_cast<std::chrono::nanoseconds>(std::chrono::steady_clock::now() - t0)
                      .count();
    for (int q = 0; q < nt; q++) {
        if (!ok[q]) {
            *bad = q;
            return fail(MOE_E_HIP, "read of record %lld failed: %s", (long long)recs[q], strerror(err[q]));
        }
        t->reads++;
        t->read_bytes += (int64_t)t->record_bytes;
    }
    return MOE_OK;
}

int tier_fetch(moe_host_tier *t, const int64_t *recs, int n, const char **ptrs) {
    if (n > t->core.capacity())
        return fail(MOE_E_INVAL, "%d records requested at once from a host tier of %d slots", n, t->core.capacity());
    int32_t slot[MOE_MAX_K];
    bool need[MOE_MAX_K];
    for (int i = 0; i < n; i++) {
        if (recs[i] < 0 || recs[i] >= t->n_records)
            return fail(MOE_E_INVAL, "record %lld outside the file's %lld", (long long)recs[i], (long long)t->n_records);
        const uint32_t key = (uint32_t)recs[i];
        int32_t s = t->core.lookup(key);
        need[i] = s < 0;
        if (s < 0) {
            uint32_t victim = kNoKey;
            s = t->core.plan_insert(key, &victim);
            // the slot's last host-to-device copy must be done before it is overwritten
            if (t->pending[s]) {
                hipError_t e = hipEventSynchronize(t->copied[s]);
                if (e != hipSuccess) return hip_fail(e, "wait for a host slot's last copy");
                t->pending[s] = 0;
            }
            t->core.commit_insert(key, s, victim);
        }
        slot[i] = s;
        ptrs[i] = t->pool + (size_t)slot[i] * t->record_bytes;
    }
    // the reads of this batch, spread over the I/O threads
    int64_t rr[MOE_MAX_K];
    char *dst[MOE_MAX_K];
    int todo[MOE_MAX_K], nt = 0;
    for (int i = 0; i < n; i++)
        if (need[i]) {
            todo[nt] = i;
            rr[nt] = recs[i];
            dst[nt++] = (char *)ptrs[i];
        }
    int bad = -1;
    const int rc = read_parallel(t, rr, dst, nt, &bad);
    if (rc) t->core.drop_slot(slot[todo[bad]]);
    return rc;
}

int tier_copied(moe_host_tier *t, const char *src, hipStream_t copy_stream) {
    return tier_page_copied(t, (int32_t)((src - t->pool) / (ptrdiff_t)t->record_bytes), copy_stream);
}

int tier_page_copied(moe_host_tier *t, int32_t page, hipStream_t copy_stream) {
    hipError_t e = hipEventRecord(t->copied[page], copy_stream);
    if (e != hipSuccess) return hip_fail(e, "record a host page's copy");
    t->pending[page] = 1;
    return MOE_OK;
}

int tier_take_page(moe_host_tier *t, bool cpu_write, hipStream_t copy_stream, int32_t *page) {
    if (t->free_pages.empty()) return fail(MOE_E_STATE, "exclusive host tier: no free page");
    const int32_t p = t->free_pages.back();
    if (t->pending[p]) {
        hipError_t e = hipEventQuery(t->copied[p]);
        if (e == hipErrorNotReady)
            e = cpu_write ? hipEventSynchronize(t->copied[p]) : hipStreamWaitEvent(copy_stream, t->copied[p], 0);
        if (e != hipSuccess) return hip_fail(e, "wait for a host page's last copy");
        if (cpu_write) t->pending[p] = 0;
    }
    t->free_pages.pop_back();
    *page = p;
    return MOE_OK;
}

int tier_read_pages(moe_host_tier *t, const int64_t *recs, const int32_t *pages, int n) {
    char *dst[MOE_MAX_K];
    for (int q = 0; q < n; q++) dst[q] = tier_page(t, pages[q]);
    int bad = -1;
    return read_parallel(t, recs, dst, n, &bad);
}
}  // namespace moe

using namespace moe;

namespace {
int create_tier(const char *path, uint64_t record_bytes, int64_t n_records, int32_t slots, void *pinned_pool,
                int32_t io_threads, bool exclusive, moe_host_tier **out) {
    if (!out) return fail(MOE_E_INVAL, "out is NULL");
    *out = nullptr;
    if (!path || !pinned_pool) return fail(MOE_E_INVAL, "path and pinned_pool must be non-NULL");
    if (record_bytes == 0 || record_bytes % 4096)
        return fail(MOE_E_INVAL, "record_bytes must be a positive multiple of 4096 (O_DIRECT)");
    if ((uintptr_t)pinned_pool % 4096) return fail(MOE_E_INVAL, "pinned_pool must be 4096-byte aligned");
    if (n_records < 1 || n_records > (int64_t)kNoKey) return fail(MOE_E_INVAL, "n_records=%lld", (long long)n_records);
    if (slots < 1) return fail(MOE_E_INVAL, "slots=%d < 1", slots);
    if (exclusive && slots <= MOE_MAX_K)
        return fail(MOE_E_INVAL, "an exclusive host tier needs more than %d slots (got %d)", MOE_MAX_K, slots);
    if (io_threads < 1 || io_threads > MOE_MAX_K) return fail(MOE_E_INVAL, "io_threads must be in 1..%d", MOE_MAX_K);
    const int fd = open(path, O_RDONLY | O_DIRECT);
    if (fd < 0) return fail(MOE_E_INVAL, "open(%s, O_DIRECT): %s", path, strerror(errno));
    struct stat st;
    if (fstat(fd, &st) != 0 || (uint64_t)st.st_size < record_bytes * (uint64_t)n_records) {
        close(fd);
        return fail(MOE_E_INVAL, "%s holds fewer than %lld records of %llu bytes", path, (long long)n_records,
                    (unsigned long long)record_bytes);
    }
    moe_host_tier *t = new (std::nothrow) moe_host_tier(exclusive ? slots - MOE_MAX_K : slots);
    if (!t) {
        close(fd);
        return fail(MOE_E_NOMEM, "host allocation failed");
    }
    t->fd = fd;
    t->record_bytes = record_bytes;
    t->n_records = n_records;
    t->pool = (char *)pinned_pool;
    t->io_threads = io_threads;
    t->exclusive = exclusive;
    t->page_of.resize(t->core.capacity());
    for (int i = 0; i < t->core.capacity(); i++) t->page_of[i] = exclusive ? -1 : i;
    if (exclusive)
        for (int p = slots - 1; p >= 0; p--) t->free_pages.push_back(p);   // lowest page taken first
    t->copied.assign(slots, nullptr);
    t->pending.assign(slots, 0);
    t->bounce.assign(io_threads, nullptr);
    for (int i = 0; i < io_threads; i++) {
        t->bounce[i] = (char *)aligned_alloc(4096, record_bytes);
        if (!t->bounce[i]) {
            moe_host_tier_destroy(t);
            return fail(MOE_E_NOMEM, "bounce buffer allocation failed");
        }
    }
    hipError_t e = hipSuccess;
    for (int s = 0; e == hipSuccess && s < slots; s++) e = hipEventCreateWithFlags(&t->copied[s], hipEventDisableTiming);
    if (e == hipSuccess && exclusive) e = hipStreamCreateWithFlags(&t->down, hipStreamNonBlocking);
    if (e != hipSuccess) {
        moe_host_tier_destroy(t);
        return hip_fail(e, "hipEventCreate");
    }
    *out = t;
    return MOE_OK;
}
}  // namespace

extern "C" {

int moe_host_tier_create(const char *path, uint64_t record_bytes, int64_t n_records, int32_t slots,
                         void *pinned_pool, int32_t io_threads, moe_host_tier **out) {
    return create_tier(path, record_bytes, n_records, slots, pinned_pool, io_threads, false, out);
}

int moe_host_tier_create_exclusive(const char *path, uint64_t record_bytes, int64_t n_records, int32_t slots,
                                   void *pinned_pool, int32_t io_threads, moe_host_tier **out) {
    return create_tier(path, record_bytes, n_records, slots, pinned_pool, io_threads, true, out);
}

int moe_host_tier_demotions(moe_host_tier *t, int64_t *demotions) {
    if (!t || !demotions) return fail(MOE_E_INVAL, "host tier and demotions must be non-NULL");
    *demotions = t->demotions;
    return MOE_OK;
}

void moe_host_tier_destroy(moe_host_tier *t) {
    if (!t) return;
    for (size_t s = 0; s < t->copied.size(); s++) {
        if (!t->copied[s]) continue;
        if (t->pending[s]) (void)hipEventSynchronize(t->copied[s]);
        (void)hipEventDestroy(t->copied[s]);
    }
    for (char *b : t->bounce) free(b);
    if (t->down) (void)hipStreamDestroy(t->down);
    if (t->fd >= 0) close(t->fd);
    delete t;
}

int moe_host_tier_stats(moe_host_tier *t, int64_t *lookups, int64_t *hits, int64_t *reads, int64_t *read_bytes,
                        int64_t *read_ns) {
    if (!t) return fail(MOE_E_INVAL, "host tier is NULL");
    if (lookups) *lookups = t->core.lookups;
    if (hits) *hits = t->core.hits;
    if (reads) *reads = t->reads;
    if (read_bytes) *read_bytes = t->read_bytes;
    if (read_ns) *read_ns = t->read_ns;
    return MOE_OK;
}

int moe_host_tier_trace(moe_host_tier *t, moe_trace_rec *buf, int64_t cap, int64_t *n) {
    if (!t || !n) return fail(MOE_E_INVAL, "host tier and n must be non-NULL");
    const auto &tr = t->core.trace();
    *n = (int64_t)tr.size();
    const int64_t m = cap < *n ? cap : *n;
    if (m > 0 && !buf) return fail(MOE_E_INVAL, "buf is NULL");
    for (int64_t i = 0; i < m; i++) buf[i] = {tr[i].key, tr[i].hit, tr[i].slot, tr[i].evicted};
    if (cap < *n) return fail(MOE_E_SPACE, "trace holds %lld records, buffer %lld", (long long)*n, (long long)cap);
    return MOE_OK;
}

}  // extern "C"
