// Host-only LRU core of the HBM expert-slot cache: O(1) lookup and insert
// (hash map + intrusive doubly linked list over slots), lowest-free-slot
// allocation, a lookup trace and counters.  No HIP dependency, so it can be
// built and tested on its own.
//
// Policy (WISP launch post, section "통찰": an LRU cache promotes the experts
// the router keeps choosing): a hit moves the key to most-recently-used; a
// new key takes the lowest-numbered free slot, else the least recently used
// key is evicted and its slot reused; the new key becomes most-recently-used.
#pragma once

#include <cstddef>
#include <cstdint>
#include <set>
#include <unordered_map>
#include <vector>

namespace moe {

constexpr uint32_t kNoKey = 0xFFFFFFFFu;

// Trace record kinds (CacheTraceRec::hit).
enum TraceKind : int32_t {
    kTraceMiss = 0,          // lookup missed; the key was inserted
    kTraceHit = 1,           // lookup hit; the key moved to MRU
    kTraceAheadInsert = 2,   // look-ahead: key absent, inserted ahead of its lookup
    kTraceAheadPresent = 3,  // look-ahead: key present, moved to MRU
    kTraceAbsent = 4,        // lower tier of two: lookup found nothing, nothing inserted
    kTraceDemote = 5,        // lower tier of two: the upper tier's victim inserted
};

struct CacheTraceRec {
    uint32_t key;
    int32_t hit;        // TraceKind
    int32_t slot;
    uint32_t evicted;   // kNoKey if none
};

class LruCore {
public:
    explicit LruCore(int capacity);

    int capacity() const { return capacity_; }
    int size() const { return (int)map_.size(); }
    bool contains(uint32_t key) const { return map_.count(key) != 0; }

    // Hit: returns the slot, moves the key to MRU and appends a hit record.
    // Miss: returns -1 and changes nothing but the lookup counter.
    int lookup(uint32_t key);

    // Slot a new key would take and the key it would evict (kNoKey if a slot
    // is free).  Returns -1 if the key is already cached.  Changes nothing.
    int plan_insert(uint32_t key, uint32_t *victim) const;

    // Apply a planned insert: evict the victim (if any), map key -> slot at
    // MRU and append a miss record.
    void commit_insert(uint32_t key, int slot, uint32_t victim);

    // Look-ahead touch of a key predicted for a later lookup: present -> move
    // to MRU (a kTraceAheadPresent record); absent -> insert exactly like a
    // miss (kTraceAheadInsert record, *inserted = true).  Returns the slot.
    // Either way the LRU order changes as it would for a lookup of the key,
    // but the lookup and hit counters do not.
    int touch_ahead(uint32_t key, uint32_t *victim, bool *inserted);

    // Lookup that also records a miss (kTraceAbsent, slot -1) and inserts
    // nothing: the lower tier of two exclusive tiers, whose keys arrive only
    // by demotion.  A hit moves the key to MRU as lookup() does.
    int probe(uint32_t key);

    // Insert an absent key (kind: the trace record's kind) at the slot and
    // with the victim plan_insert gives; returns the slot, -1 if present.
    int insert_kind(uint32_t key, int32_t kind, uint32_t *victim);

    // Forget whatever key a slot holds (the slot becomes free).
    void drop_slot(int slot);

    // Key held by a slot, or kNoKey.
    uint32_t key_of(int slot) const { return key_of_[slot]; }

    // Keys from most to least recently used.
    std::vector<uint32_t> order() const;

    const std::vector<CacheTraceRec> &trace() const { return trace_; }
    void trace_reset() { trace_.clear(); }

    int64_t lookups = 0, hits = 0, inserts = 0, evictions = 0;
    // look-ahead: keys inserted ahead, keys found present, inserted keys later
    // hit by a lookup, inserted keys evicted (or dropped) before any lookup
    int64_t ahead_inserts = 0, ahead_present = 0, ahead_used = 0, ahead_wasted = 0;

private:
    void unlink(int s);
    void push_front(int s);

    int capacity_;
    std::unordered_map<uint32_t, int> map_;
    void insert_at(uint32_t key, int slot, uint32_t victim, int32_t kind);

    std::vector<uint32_t> key_of_;
    std::vector<uint8_t> ahead_;     // slot holds a key inserted ahead and not looked up since
    std::vector<int> prev_, next_;
    int head_ = -1, tail_ = -1;
    std::set<int> free_;
    std::vector<CacheTraceRec> trace_;
};

// dist[i] = distinct keys referenced since the previous reference to
// keys[i] (0: it was the most recent one), or -1 at a first reference.  An
// LRU cache of capacity C hits exactly the references with 0 <= dist < C.
void lru_stack_distances(const uint32_t *keys, int64_t n, int32_t *dist);

}  // namespace moe
