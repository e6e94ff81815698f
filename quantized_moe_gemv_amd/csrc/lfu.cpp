// Host-side slot cache for a routed-expert pool kept in host memory
// ("Load and ownership": each layer owns a fixed group of expert slots; the
// cache records which expert occupies each slot; least-frequently-used
// eviction with recency as the tie-breaker; a hit reuses its slot, a miss
// takes an evictable slot and starts a bounded read; distinct misses may be
// read in parallel but never two into one slot).
//
// All state lives in a caller buffer (no allocation).  One plan call takes
// the expert ids a layer call will use, counts one use for each distinct
// expert, keeps the slots of resident experts, gives every missing expert a
// slot that no expert of the same call uses (empty slots first, then the
// resident expert with the fewest uses, ties to the one used longest ago,
// then the lower slot), and reports the misses to fill.
#include <string.h>

#include "../../include/moegemv.h"

namespace {

constexpr uint32_t kMagic = 0x4C465531u;   // "LFU1"

struct Header {
    uint32_t magic;
    int32_t E, S;
    int32_t pad;
    uint64_t clock;          // plan calls so far
};

struct View {
    Header* h;
    int32_t* slot_of_expert;   // [E], -1: not resident
    int32_t* expert_of_slot;   // [S], -1: empty
    uint64_t* uses;            // [E] calls that used the expert
    uint64_t* last_use;        // [S] the clock of the last call that used the slot
    uint64_t* mark;            // [S] the clock of the call holding the slot (this plan)
    uint64_t* seen;            // [E] stamp of the plan call that last saw the expert (2 clock, then 2 clock + 1 once counted)
};

size_t state_bytes(int32_t E, int32_t S) {
    return sizeof(Header) + (size_t)E * 4 + (size_t)S * 4 + (size_t)E * 8 + (size_t)S * 16 + (size_t)E * 8 + 64;
}

bool view(void* state, size_t bytes, View* v) {
    if (!state || ((uintptr_t)state % 8) || bytes < sizeof(Header)) return false;
    Header* h = (Header*)state;
    if (h->magic != kMagic || h->E <= 0 || h->S <= 0 || bytes < state_bytes(h->E, h->S)) return false;
    uint8_t* p = (uint8_t*)state + sizeof(Header);
    v->h = h;
    v->uses = (uint64_t*)p;
    p += (size_t)h->E * 8;
    v->seen = (uint64_t*)p;
    p += (size_t)h->E * 8;
    v->last_use = (uint64_t*)p;
    p += (size_t)h->S * 8;
    v->mark = (uint64_t*)p;
    p += (size_t)h->S * 8;
    v->slot_of_expert = (int32_t*)p;
    p += (size_t)h->E * 4;
    v->expert_of_slot = (int32_t*)p;
    return true;
}

}  // namespace

extern "C" size_t mq_lfu_state_bytes(int32_t num_experts, int32_t num_slots) {
    if (num_experts <= 0 || num_slots <= 0 || num_experts > (1 << 20) || num_slots > (1 << 20)) return 0;
    return state_bytes(num_experts, num_slots);
}

extern "C" mq_status mq_lfu_init(void* state, size_t state_bytes_, int32_t num_experts, int32_t num_slots) {
    if (!state) return MQ_ERR_NULL;
    if ((uintptr_t)state % 8) return MQ_ERR_ALIGN;
    const size_t need = mq_lfu_state_bytes(num_experts, num_slots);
    if (need == 0) return MQ_ERR_SHAPE;
    if (state_bytes_ < need) return MQ_ERR_BUFFER;
    memset(state, 0, need);
    Header* h = (Header*)state;
    h->magic = kMagic;
    h->E = num_experts;
    h->S = num_slots;
    View v;
    view(state, state_bytes_, &v);
    for (int e = 0; e < num_experts; ++e) v.slot_of_expert[e] = -1;
    for (int s = 0; s < num_slots; ++s) v.expert_of_slot[s] = -1;
    return MQ_OK;
}

extern "C" mq_status mq_lfu_plan(void* state, size_t state_bytes_, const int32_t* ids, int32_t n,
                                 int32_t* slot_of_id, int32_t* miss_expert, int32_t* miss_slot, int32_t* n_miss) {
    if (!state || (n > 0 && (!ids || !slot_of_id || !miss_expert || !miss_slot)) || !n_miss) return MQ_ERR_NULL;
    View v;
    if (!view(state, state_bytes_, &v)) return MQ_ERR_BUFFER;
    if (n < 0) return MQ_ERR_SHAPE;
    const int E = v.h->E, S = v.h->S;
    // validate and count the distinct experts before changing anything
    const uint64_t now = v.h->clock + 1, seen_st = 2 * now, counted_st = 2 * now + 1;
    for (int i = 0; i < n; ++i)
        if (ids[i] < 0 || ids[i] >= E) return MQ_ERR_SHAPE;
    int distinct = 0;
    for (int i = 0; i < n; ++i) {
        if (v.seen[ids[i]] != seen_st) {
            v.seen[ids[i]] = seen_st;
            ++distinct;
        }
    }
    if (distinct > S) {
        for (int i = 0; i < n; ++i) v.seen[ids[i]] = 0;   // leave no trace of the refused call
        return MQ_ERR_SHAPE;
    }
    v.h->clock = now;
    // hits: count the use and hold the slot for this call
    for (int i = 0; i < n; ++i) {
        const int e = ids[i];
        if (v.seen[e] != seen_st) continue;   // counted already in this call
        v.seen[e] = counted_st;
        ++v.uses[e];
        if (v.slot_of_expert[e] >= 0) v.mark[v.slot_of_expert[e]] = now;
    }
    // misses, in order of first appearance
    int nm = 0;
    for (int i = 0; i < n; ++i) {
        const int e = ids[i];
        if (v.slot_of_expert[e] >= 0) continue;
        int best = -1;
        for (int s = 0; s < S; ++s) {
            if (v.mark[s] == now) continue;
            if (best < 0) {
                best = s;
                continue;
            }
            const int a = v.expert_of_slot[s], b = v.expert_of_slot[best];
            if (b < 0) continue;                     // an empty slot is taken first
            if (a < 0) {
                best = s;
                continue;
            }
            if (v.uses[a] < v.uses[b] || (v.uses[a] == v.uses[b] && v.last_use[s] < v.last_use[best])) best = s;
        }
        // best >= 0: distinct <= S and every held slot belongs to a distinct expert of this call
        const int old = v.expert_of_slot[best];
        if (old >= 0) v.slot_of_expert[old] = -1;
        v.expert_of_slot[best] = e;
        v.slot_of_expert[e] = best;
        v.mark[best] = now;
        miss_expert[nm] = e;
        miss_slot[nm] = best;
        ++nm;
    }
    for (int i = 0; i < n; ++i) {
        const int s = v.slot_of_expert[ids[i]];
        v.last_use[s] = now;
        slot_of_id[i] = s;
    }
    *n_miss = nm;
    return MQ_OK;
}
