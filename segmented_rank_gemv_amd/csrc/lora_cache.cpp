// Adapter slot cache: which adapter occupies which slot of the device stacks.
//
// Activation follows the two pages' managers: an adapter that is already
// active keeps its slot and becomes the most recently used ([vLLM] §5.3
// activate_adapter returns early for an active id; §7 LRU touch); a new one
// takes the first free slot ([vLLM] §5.3); when no slot is free, the LRU
// policy evicts the least recently used adapter that is not pinned and
// reuses its slot ([MAX-V3] activate_adapter; [vLLM] §7 remove_oldest, then
// the first free slot), and the no-evict policy fails ([vLLM] §5.3 "No free
// lora slots").  Unloading frees the slot ([MAX-V3] unload_adapter); pinned
// adapters are never evicted ([vLLM] §7 pin_adapter).  Host only; a cache
// is not thread-safe.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <vector>

#include "lora_sgmv.h"

struct lora_slot_cache {
    int32_t policy;
    std::vector<int64_t> id;         // adapter in each slot, -1 = free
    std::vector<uint64_t> last_use;  // activation tick of each slot's adapter
    std::vector<uint8_t> pinned;
    uint64_t tick = 0;
};

namespace {

constexpr int32_t kMaxSlots = 1 << 20;

int slot_of(const lora_slot_cache& c, int64_t id)
{
    for (size_t s = 0; s < c.id.size(); ++s)
        if (c.id[s] == id)
            return (int)s;
    return -1;
}

// Activate one adapter.  Slots whose last use is at or after `protect_from`
// (the adapters a batch activated so far) are not evicted.
lora_status_t activate(lora_slot_cache& c, int64_t id, uint64_t protect_from, int32_t* slot,
                       int32_t* needs_load, int64_t* evicted)
{
    *evicted = -1;
    int s = slot_of(c, id);
    if (s >= 0) {
        c.last_use[s] = ++c.tick;
        *slot = s;
        *needs_load = 0;
        return LORA_OK;
    }
    for (size_t i = 0; i < c.id.size() && s < 0; ++i)
        if (c.id[i] < 0)
            s = (int)i;
    if (s < 0) {
        if (c.policy != LORA_CACHE_LRU)
            return LORA_ERR_NO_FREE_SLOT;
        for (size_t i = 0; i < c.id.size(); ++i)
            if (!c.pinned[i] && c.last_use[i] < protect_from && (s < 0 || c.last_use[i] < c.last_use[s]))
                s = (int)i;
        if (s < 0)
            return LORA_ERR_NO_FREE_SLOT;
        *evicted = c.id[s];
    }
    c.id[s] = id;
    c.last_use[s] = ++c.tick;
    c.pinned[s] = 0;
    *slot = s;
    *needs_load = 1;
    return LORA_OK;
}

}  // namespace

extern "C" {

lora_status_t lora_cache_create(int32_t num_slots, int32_t policy, lora_slot_cache_t** cache)
{
    if (!cache || num_slots <= 0 || num_slots > kMaxSlots ||
        (policy != LORA_CACHE_LRU && policy != LORA_CACHE_NO_EVICT))
        return LORA_ERR_INVALID_ARGUMENT;
    lora_slot_cache* c = new (std::nothrow) lora_slot_cache;
    if (!c)
        return LORA_ERR_UNSPECIFIED;
    c->policy = policy;
    c->id.assign(num_slots, -1);
    c->last_use.assign(num_slots, 0);
    c->pinned.assign(num_slots, 0);
    *cache = c;
    return LORA_OK;
}

void lora_cache_destroy(lora_slot_cache_t* cache) { delete cache; }

lora_status_t lora_cache_activate(lora_slot_cache_t* cache, int64_t adapter_id, int32_t* slot,
                                  int32_t* needs_load, int64_t* evicted_id)
{
    if (!cache || adapter_id < 0 || !slot || !needs_load || !evicted_id)
        return LORA_ERR_INVALID_ARGUMENT;
    return activate(*cache, adapter_id, UINT64_MAX, slot, needs_load, evicted_id);
}

lora_status_t lora_cache_activate_batch(lora_slot_cache_t* cache, int32_t num_requests,
                                        const int64_t* adapter_ids, int32_t* request_slot,
                                        int32_t* load_slots, int64_t* load_ids, int32_t* num_loads)
{
    if (!cache || num_requests < 0 || (num_requests > 0 && (!adapter_ids || !request_slot)) || !load_slots ||
        !load_ids || !num_loads)
        return LORA_ERR_INVALID_ARGUMENT;
    for (int32_t i = 0; i < num_requests; ++i)
        if (adapter_ids[i] < -1)
            return LORA_ERR_INVALID_ARGUMENT;
    // work on a copy: on an error the cache is left as it was
    lora_slot_cache c = *cache;
    const uint64_t batch_from = c.tick + 1;
    int32_t nl = 0;
    std::vector<int32_t> out(num_requests, -1);
    // the batch's adapters that already hold a slot are touched first (in
    // first-appearance order), so that loading the others cannot evict them
    for (int32_t i = 0; i < num_requests; ++i) {
        const int prev = adapter_ids[i] >= 0 ? slot_of(c, adapter_ids[i]) : -1;
        if (prev >= 0 && c.last_use[prev] < batch_from)
            c.last_use[prev] = ++c.tick;
    }
    for (int32_t i = 0; i < num_requests; ++i) {
        if (adapter_ids[i] < 0)
            continue;
        int32_t s, load;
        int64_t ev;
        const int prev = slot_of(c, adapter_ids[i]);
        if (prev >= 0 && c.last_use[prev] >= batch_from) {
            out[i] = prev;  // active already, or loaded by an earlier request of this batch
            continue;
        }
        const lora_status_t st = activate(c, adapter_ids[i], batch_from, &s, &load, &ev);
        if (st != LORA_OK)
            return st;
        out[i] = s;
        if (load) {
            // a slot loaded earlier in this batch is never evicted again in it
            load_slots[nl] = s;
            load_ids[nl] = adapter_ids[i];
            ++nl;
        }
    }
    *cache = c;
    std::copy(out.begin(), out.end(), request_slot);
    *num_loads = nl;
    return LORA_OK;
}

lora_status_t lora_cache_unload(lora_slot_cache_t* cache, int64_t adapter_id, int32_t* slot)
{
    if (!cache || adapter_id < 0 || !slot)
        return LORA_ERR_INVALID_ARGUMENT;
    const int s = slot_of(*cache, adapter_id);
    if (s < 0)
        return LORA_ERR_NOT_ACTIVE;
    cache->id[s] = -1;
    cache->last_use[s] = 0;
    cache->pinned[s] = 0;
    *slot = s;
    return LORA_OK;
}

lora_status_t lora_cache_pin(lora_slot_cache_t* cache, int64_t adapter_id, int32_t pinned, int32_t* slot,
                             int32_t* needs_load, int64_t* evicted_id)
{
    if (!cache || adapter_id < 0 || !slot || !needs_load || !evicted_id)
        return LORA_ERR_INVALID_ARGUMENT;
    if (!pinned) {
        const int s = slot_of(*cache, adapter_id);
        if (s < 0)
            return LORA_ERR_NOT_ACTIVE;
        cache->pinned[s] = 0;
        *slot = s;
        *needs_load = 0;
        *evicted_id = -1;
        return LORA_OK;
    }
    const lora_status_t st = activate(*cache, adapter_id, UINT64_MAX, slot, needs_load, evicted_id);
    if (st == LORA_OK)
        cache->pinned[*slot] = 1;
    return st;
}

lora_status_t lora_cache_lookup(const lora_slot_cache_t* cache, int64_t adapter_id, int32_t* slot)
{
    if (!cache || adapter_id < 0 || !slot)
        return LORA_ERR_INVALID_ARGUMENT;
    *slot = slot_of(*cache, adapter_id);
    return LORA_OK;
}

lora_status_t lora_cache_slot_table(const lora_slot_cache_t* cache, int32_t capacity, int64_t* slot_ids,
                                    uint8_t* pinned)
{
    if (!cache || !slot_ids || capacity < (int32_t)cache->id.size())
        return cache && slot_ids ? LORA_ERR_CAPACITY : LORA_ERR_INVALID_ARGUMENT;
    std::copy(cache->id.begin(), cache->id.end(), slot_ids);
    if (pinned)
        std::copy(cache->pinned.begin(), cache->pinned.end(), pinned);
    return LORA_OK;
}

}  // extern "C"
