// Host side of the file tier (host_tier.hip): LRU over pinned host slots
// holding whole records, filled by O_DIRECT reads.
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
    char *pool = nullptr;              // caller-owned pinned memory, slots x record_bytes
    int io_threads = 1;
    std::vector<hipEvent_t> copied;    // recorded on the copy stream after a slot's last host-to-device copy
    std::vector<uint8_t> pending;      // copied[] recorded and not waited for since
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
}  // namespace moe
