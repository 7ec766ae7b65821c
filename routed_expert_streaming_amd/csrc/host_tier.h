// Host side of the file tier (host_tier.hip): LRU over pinned host slots
// holding whole records, filled by O_DIRECT reads (inclusive), or by the HBM
// cache's evicted records (exclusive).  The pool is divided into pages of one
// record; page_of maps an LRU slot to its page (the identity when inclusive;
// an exclusive tier has MOE_MAX_K more pages than slots, for the records in
// transit during one layer call).
#pragma once

#include <hip/hip_runtime.h>

#include <vector>

#include "expert_cache_core.h"
#include "moe.h"

struct moe_host_tier {
    moe::LruCore core;                 // keys: record index in the file
    int fd = -1;
    uint64_t record_bytes = 0;
    int64_t n_records = 0;
    char *pool = nullptr;              // caller-owned pinned memory, pages x record_bytes
    int io_threads = 1;
    bool exclusive = false;
    std::vector<int32_t> page_of;      // LRU slot -> page
    std::vector<int32_t> free_pages;   // exclusive: pages with no key and no copy of the current call
    std::vector<hipEvent_t> copied;    // per page: recorded on the copy stream after its last copy
    std::vector<uint8_t> pending;      // copied[] recorded and not waited for since
    int64_t demotions = 0;
    hipStream_t down = nullptr;        // exclusive: device-to-host copies of the HBM cache's evicted records
    std::vector<char *> bounce;        // per I/O thread: 4 KiB-aligned pageable buffer of one record (O_DIRECT
                                       // cannot target the pinned pool: the kernel will not map it for I/O)
    int64_t reads = 0, read_bytes = 0, read_ns = 0;

    explicit moe_host_tier(int slots) : core(slots) {}
};

namespace moe {
// Host pointers of n records (at most the tier's slot count, at most
// MOE_MAX_K), reading the ones not in the tier: looks each up in order (hits
// move to MRU), inserts the misses (a reused slot first waits for its last
// copy), then reads them in parallel on the tier's I/O threads.
int tier_fetch(moe_host_tier *t, const int64_t *recs, int n, const char **ptrs);
// A copy from src (a slot of t) was enqueued on copy_stream: the slot is not
// rewritten before it completes.
int tier_copied(moe_host_tier *t, const char *src, hipStream_t copy_stream);

// Exclusive tier, one layer call.  tier_take_page: a free page for a record
// in transit; before the host writes it (cpu_write) its last copy is waited
// for, else copy_stream waits for it.  tier_read_pages: records recs[i] from
// the file into pages[i], in parallel on the I/O threads.  tier_page_copied:
// a copy to or from the page was enqueued on copy_stream.
int tier_take_page(moe_host_tier *t, bool cpu_write, hipStream_t copy_stream, int32_t *page);
int tier_read_pages(moe_host_tier *t, const int64_t *recs, const int32_t *pages, int n);
int tier_page_copied(moe_host_tier *t, int32_t page, hipStream_t copy_stream);
inline char *tier_page(moe_host_tier *t, int32_t page) { return t->pool + (size_t)page * t->record_bytes; }
}  // namespace moe
