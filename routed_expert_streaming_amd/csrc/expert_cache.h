// HIP side of the expert-slot cache: the slot pool, per-slot ready events
// (copy landed) and readers' events (write-after-read guard for evictions).
#pragma once

#include <hip/hip_runtime.h>

#include <condition_variable>
#include <mutex>
#include <thread>
#include <vector>

#include "expert_cache_core.h"
#include "moe.h"

namespace moe {
// Persistent host threads that split one memcpy between them (pageable
// records into a pinned bounce buffer).
class CopyPool {
public:
    explicit CopyPool(int n);
    ~CopyPool();
    void copy(void *dst, const void *src, size_t bytes);   // returns when all of it is copied
private:
    void worker(int i);
    std::mutex m_;
    std::condition_variable go_, done_;
    std::vector<std::thread> th_;
    size_t n_ = 0;                 // threads (fixed before any starts)
    char *dst_ = nullptr;
    const char *src_ = nullptr;
    size_t bytes_ = 0;
    unsigned gen_ = 0;
    int pending_ = 0;
    bool stop_ = false;
};
constexpr int kBounce = 4;   // pinned bounce buffers per cache
constexpr int kIdsFlag = 3 * MOE_MAX_K;   // word of moe_cache::h_idx holding the ids' sequence flag
}  // namespace moe

struct moe_cache {
    moe::LruCore core;
    char *pool = nullptr;                 // caller-owned device pool
    uint64_t slot_bytes = 0;
    std::vector<hipEvent_t> ready;        // recorded on a copy stream after a slot's copy
    std::vector<uint8_t> filled;          // slot has had a copy enqueued
    // Readers' events: one event is recorded on a compute stream after the
    // readers of a whole batch of slots (one release call), and every slot of
    // the batch refers to it; an event no slot refers to any more is free for
    // reuse (re-recording it then cannot delay a copy that waits for an older
    // recording, since no slot waits for that one).
    std::vector<hipEvent_t> use_ev;
    std::vector<int32_t> use_refs;        // slots referring to each event
    std::vector<int32_t> use_free;        // events with no referring slot
    std::vector<int32_t> slot_use;        // per slot: its readers' event, or -1
    int32_t *h_idx = nullptr;             // pinned staging: the router's expert ids, the look-ahead ids and
                                          // (bits of) the look-ahead weights, MOE_MAX_K each, then the
                                          // ids' sequence flag (word kIdsFlag)
    uint32_t ids_seq = 0;                 // the last sequence number the top-k was asked to write
    hipEvent_t idx_ev = nullptr;          // recorded after the top-k that writes the ids to h_idx
    hipEvent_t ahead_ev = nullptr;        // recorded after the look-ahead top-k
    // A second copy stream of the cache's own: a streamed layer alternates its
    // misses' copies between the caller's copy stream and this one, so that
    // one copy's start-up overlaps the other's transfer; the caller's copy
    // stream then waits for this one (ps2_done), so it still completes after
    // every copy of the call.
    hipStream_t ps2 = nullptr;
    hipEvent_t ps2_done = nullptr;
    int device = 0;
    // records in pageable host memory go through pinned bounce buffers
    // (allocated on first use) filled by host threads
    char *bounce[moe::kBounce] = {};
    hipEvent_t bounce_done[moe::kBounce] = {};   // recorded on a copy stream after the buffer's copy
    bool bounce_used[moe::kBounce] = {};
    int bounce_next = 0;
    moe::CopyPool *copier = nullptr;

    explicit moe_cache(int capacity) : core(capacity) {}
};

namespace moe {
int cache_wait(moe_cache *c, int32_t slot, hipStream_t s);
int cache_release(moe_cache *c, int32_t slot, hipStream_t s);
// Records one event on s after the readers of n distinct slots and makes it
// their readers' event.
int cache_release_many(moe_cache *c, const int32_t *slots, int n, hipStream_t s);
// Makes stream s wait for the readers of slot s_ (if any were recorded).
hipError_t cache_wait_readers(moe_cache *c, int32_t slot, hipStream_t s);
// Enqueue the copy of one record (slot_bytes at src, host memory) into slot
// s on stream ps: straight from page-locked memory; from pageable memory
// through the next bounce buffer, which host threads fill after its previous
// copy has completed (the runtime's own staging of pageable copies reaches a
// fraction of the link rate).
// *enqueued tells whether the copy into the slot was enqueued (then, even on
// an error, the slot's previous contents are gone).
hipError_t cache_copy_in(moe_cache *c, int32_t s, const void *src, hipStream_t ps, bool *enqueued);
// Whether host memory at p is page-locked (a copy from it needs no staging).
bool host_page_locked(const void *p);
}  // namespace moe
