// Host-only LRU core of the HBM expert-slot cache (see expert_cache_core.h).
#include "expert_cache_core.h"

namespace moe {

LruCore::LruCore(int capacity)
    : capacity_(capacity), key_of_(capacity, kNoKey), ahead_(capacity, 0), prev_(capacity, -1), next_(capacity, -1) {
    map_.reserve((size_t)capacity * 2);
    for (int s = 0; s < capacity; s++) free_.insert(s);
}

void LruCore::unlink(int s) {
    if (prev_[s] != -1) next_[prev_[s]] = next_[s];
    else head_ = next_[s];
    if (next_[s] != -1) prev_[next_[s]] = prev_[s];
    else tail_ = prev_[s];
    prev_[s] = next_[s] = -1;
}

void LruCore::push_front(int s) {
    prev_[s] = -1;
    next_[s] = head_;
    if (head_ != -1) prev_[head_] = s;
    head_ = s;
    if (tail_ == -1) tail_ = s;
}

int LruCore::lookup(uint32_t key) {
    lookups++;
    auto it = map_.find(key);
    if (it == map_.end()) return -1;
    const int s = it->second;
    hits++;
    if (ahead_[s]) {
        ahead_used++;
        ahead_[s] = 0;
    }
    unlink(s);
    push_front(s);
    trace_.push_back({key, kTraceHit, s, kNoKey});
    return s;
}

int LruCore::plan_insert(uint32_t key, uint32_t *victim) const {
    if (map_.count(key)) return -1;
    if (!free_.empty()) {
        *victim = kNoKey;
        return *free_.begin();
    }
    *victim = key_of_[tail_];
    return tail_;
}

void LruCore::insert_at(uint32_t key, int slot, uint32_t victim, int32_t kind) {
    if (victim != kNoKey) {
        map_.erase(victim);
        unlink(slot);
        evictions++;
        if (ahead_[slot]) ahead_wasted++;
    } else {
        free_.erase(slot);
    }
    key_of_[slot] = key;
    map_[key] = slot;
    ahead_[slot] = kind == kTraceAheadInsert;
    push_front(slot);
    inserts++;
    trace_.push_back({key, kind, slot, victim});
}

void LruCore::commit_insert(uint32_t key, int slot, uint32_t victim) {
    insert_at(key, slot, victim, kTraceMiss);
}

int LruCore::touch_ahead(uint32_t key, uint32_t *victim, bool *inserted) {
    auto it = map_.find(key);
    if (it != map_.end()) {
        const int s = it->second;
        unlink(s);
        push_front(s);
        ahead_present++;
        trace_.push_back({key, kTraceAheadPresent, s, kNoKey});
        *victim = kNoKey;
        *inserted = false;
        return s;
    }
    const int s = plan_insert(key, victim);
    insert_at(key, s, *victim, kTraceAheadInsert);
    ahead_inserts++;
    *inserted = true;
    return s;
}

int LruCore::probe(uint32_t key) {
    const int s = lookup(key);
    if (s < 0) trace_.push_back({key, kTraceAbsent, -1, kNoKey});
    return s;
}

int LruCore::insert_kind(uint32_t key, int32_t kind, uint32_t *victim) {
    const int s = plan_insert(key, victim);
    if (s >= 0) insert_at(key, s, *victim, kind);
    return s;
}

void LruCore::drop_slot(int slot) {
    const uint32_t k = key_of_[slot];
    if (k == kNoKey) return;
    if (ahead_[slot]) ahead_wasted++;
    ahead_[slot] = 0;
    map_.erase(k);
    unlink(slot);
    key_of_[slot] = kNoKey;
    free_.insert(slot);
}

std::vector<uint32_t> LruCore::order() const {
    std::vector<uint32_t> v;
    for (int s = head_; s != -1; s = next_[s]) v.push_back(key_of_[s]);
    return v;
}

// LRU stack distances in one pass (Mattson, Gecsei, Slutz and Traiger,
// "Evaluation techniques for storage hierarchies", 1970): a Fenwick tree over
// reference times holds a 1 at each key's latest reference, so the distinct
// keys referenced since key k's previous reference p are the ones in (p, i).
void lru_stack_distances(const uint32_t *keys, int64_t n, int32_t *dist) {
    std::vector<int32_t> tree((size_t)n + 1, 0);
    auto add = [&](int64_t i, int32_t v) {
        for (++i; i <= n; i += i & -i) tree[(size_t)i] += v;
    };
    auto prefix = [&](int64_t i) {   // sum over positions [0, i)
        int64_t s = 0;
        for (; i > 0; i -= i & -i) s += tree[(size_t)i];
        return s;
    };
    std::unordered_map<uint32_t, int64_t> last;
    last.reserve((size_t)n);
    for (int64_t i = 0; i < n; i++) {
        auto it = last.find(keys[i]);
        if (it == last.end()) {
            dist[i] = -1;
            last.emplace(keys[i], i);
        } else {
            const int64_t p = it->second;
            dist[i] = (int32_t)(prefix(i) - prefix(p + 1));
            add(p, -1);
            it->second = i;
        }
        add(i, 1);
    }
}

}  // namespace moe
