// HIP side of the expert-slot cache: the slot pool, per-slot ready events
// (copy landed) and last-use events (write-after-read guard for evictions).
#pragma once

#include <hip/hip_runtime.h>

#include <vector>

#include "expert_cache_core.h"
#include "moe.h"

struct moe_cache {
    moe::LruCore core;
    char *pool = nullptr;                 // caller-owned device pool
    uint64_t slot_bytes = 0;
    std::vector<hipEvent_t> ready;        // recorded on the copy stream after a slot's copy
    std::vector<hipEvent_t> last_use;     // recorded on a compute stream after the slot's readers
    std::vector<uint8_t> filled;          // slot has had a copy enqueued
    std::vector<uint8_t> used;            // last_use has been recorded
    int32_t *h_idx = nullptr;             // pinned staging for the router's expert ids
    int device = 0;

    explicit moe_cache(int capacity) : core(capacity) {}
};

namespace moe {
int cache_wait(moe_cache *c, int32_t slot, hipStream_t s);
int cache_release(moe_cache *c, int32_t slot, hipStream_t s);
}  // namespace moe
