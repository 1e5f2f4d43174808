/*
 * expert_cache.cpp -- host-side slot cache and pass planner of the tiered
 * expert store, and its C ABI (colibri_cache_*).  Plain C++: nothing here
 * touches the GPU, so the planner runs and is tested without one.
 */
#include "expert_cache.h"

#include <algorithm>
#include <new>

namespace coli {

ExpertCache::ExpertCache(int32_t n_experts, int32_t n_slots)
    : E_(n_experts), n_slots_(n_slots), slot_of_(n_experts, -1), expert_in_(n_slots, -1),
      pinned_(n_slots, 0), last_use_(n_slots, 0), usage_(n_experts, 0), inflight_(n_slots, 0),
      ready_(n_slots, -1),
      first_(n_experts, -1), used_(n_experts, 0), excl_(n_slots, 0)
{
    order_.reserve(n_experts);
    ring_.reserve(n_slots);
    pass_of_.assign(n_experts, 0);
}

void ExpertCache::victims(const std::vector<uint8_t>& excluded, std::vector<int32_t>& out) const
{
    out.clear();
    for (int32_t s = 0; s < n_slots_; ++s)
        if (!pinned_[s] && !excluded[s])
            out.push_back(s);
    std::stable_sort(out.begin(), out.end(), [&](int32_t a, int32_t b) {
        const bool ea = expert_in_[a] < 0, eb = expert_in_[b] < 0;
        if (ea != eb)
            return ea;
        if (ea)
            return false;
        return last_use_[a] < last_use_[b];
    });
}

void ExpertCache::place(int32_t expert, int32_t slot)
{
    const int32_t old = expert_in_[slot];
    if (old >= 0)
        slot_of_[old] = -1;
    expert_in_[slot] = expert;
    slot_of_[expert] = slot;
    last_use_[slot] = tick_;
}

int ExpertCache::pin(const int32_t* experts, int32_t n, coli_cache_load* loads, int32_t* n_load)
{
    if (n < 0 || !n_load || (n > 0 && (!experts || !loads)))
        return COLI_E_INVAL;
    int32_t fresh = 0;
    int st = COLI_OK;
    for (int32_t i = 0; i < n && st == COLI_OK; ++i) {
        const int32_t e = experts[i];
        if (e < 0 || e >= E_ || used_[e]) {
            st = COLI_E_INVAL; /* out of range or repeated */
            break;
        }
        used_[e] = 1;
        if (slot_of_[e] < 0 || !pinned_[slot_of_[e]])
            ++fresh;
    }
    for (int32_t i = 0; i < n; ++i)
        if (experts && experts[i] >= 0 && experts[i] < E_)
            used_[experts[i]] = 0;
    if (st)
        return st;
    const int32_t total = n_pinned_ + fresh;
    if (!(total <= n_slots_ - 1 || (total == E_ && n_slots_ == E_)))
        return COLI_E_UNSUPPORTED; /* a slot has to stay free for misses */
    ++tick_;
    *n_load = 0;
    for (int32_t i = 0; i < n; ++i) {
        const int32_t e = experts[i];
        int32_t s = slot_of_[e];
        if (s < 0) {
            victims(excl_, ring_);
            s = ring_[0];
            place(e, s);
            loads[(*n_load)++] = coli_cache_load{e, s, 1, -1};
            ++st_.pin_loads;
        }
        if (!pinned_[s]) {
            pinned_[s] = 1;
            ++n_pinned_;
        }
        last_use_[s] = tick_;
    }
    return COLI_OK;
}

void ExpertCache::unpin()
{
    std::fill(pinned_.begin(), pinned_.end(), 0);
    n_pinned_ = 0;
}

void ExpertCache::reset()
{
    std::fill(slot_of_.begin(), slot_of_.end(), -1);
    std::fill(expert_in_.begin(), expert_in_.end(), -1);
    std::fill(last_use_.begin(), last_use_.end(), 0);
    std::fill(inflight_.begin(), inflight_.end(), 0);
    unpin();
}

int ExpertCache::plan(const int32_t* ids, int32_t P, int32_t* pair_code, coli_cache_load* loads,
                      int32_t* pass_pairs, coli_cache_plan* out)
{
    if (P < 0 || !out || !loads || !pass_pairs || (P > 0 && (!ids || !pair_code)))
        return COLI_E_INVAL;
    for (int32_t p = 0; p < P; ++p)
        if (ids[p] >= E_)
            return COLI_E_INVAL;
    ++tick_;

    /* distinct experts in order of first appearance */
    order_.clear();
    for (int32_t p = 0; p < P; ++p) {
        const int32_t e = ids[p];
        if (e >= 0 && !used_[e]) {
            used_[e] = 1;
            order_.push_back(e);
        }
    }

    /* hits run in pass 0 from the slot they hold */
    int32_t n_hit = 0, n_miss = 0, n_late = 0;
    for (const int32_t e : order_) {
        const int32_t s = slot_of_[e];
        if (s >= 0) {
            used_[e] = 2; /* hit */
            excl_[s] = 1;
            last_use_[s] = tick_;
            pass_of_[e] = 0;
            first_[e] = s;
            ++n_hit;
        } else {
            ++n_miss;
        }
    }

    /* victim ring: free slots in LRU order, then unpinned hit slots (ready
     * once pass 0 has finished).  When the misses fit the free slots, a hit
     * whose slot a prefetch may still be filling (a late hit) runs in pass 1,
     * which follows every load, and its slot stays out of the ring. */
    victims(excl_, ring_);
    const int32_t n_free = (int32_t)ring_.size();
    if (n_miss <= n_free) {
        for (const int32_t e : order_)
            if (used_[e] == 2 && inflight_[first_[e]]) {
                excl_[first_[e]] = 2;
                pass_of_[e] = 1;
                ++n_late;
            }
    }
    for (int32_t s = 0; s < n_slots_; ++s)
        if (excl_[s] == 1 && !pinned_[s])
            ring_.push_back(s);
    const int32_t R = (int32_t)ring_.size();
    for (int32_t i = 0; i < R; ++i)
        ready_[i] = i < n_free ? -1 : 0;
    for (const int32_t e : order_)
        if (used_[e] == 2)
            excl_[first_[e]] = 0;

    int st = COLI_OK;
    int32_t n_pass = 1;
    if (n_miss > 0 && R == 0) {
        st = COLI_E_UNSUPPORTED; /* every slot pinned: excluded by pin()'s limit */
    } else if (n_miss > 0) {
        /* c <= R/2 (or R == 1): two consecutive chunks take disjoint slots,
         * so a chunk's loads wait at most for the pass before the previous one */
        const int32_t c = n_miss <= R ? n_miss : std::max(1, R / 2);
        int32_t i = 0;
        for (const int32_t e : order_) {
            if (used_[e] == 2)
                continue; /* hit */
            const int32_t pass = 1 + i / c;
            const int32_t r = i % R;
            const int32_t s = ring_[r];
            loads[i] = coli_cache_load{e, s, pass, ready_[r]};
            ready_[r] = pass;
            place(e, s);
            pass_of_[e] = pass;
            first_[e] = s;
            ++i;
        }
        n_pass = 1 + (n_miss + c - 1) / c;
    }
    if (n_late > 0 && n_pass < 2)
        n_pass = 2;

    if (st == COLI_OK) {
        std::fill(inflight_.begin(), inflight_.end(), 0);
        std::fill(pass_pairs, pass_pairs + n_pass, 0);
        int64_t kept = 0;
        for (int32_t p = 0; p < P; ++p) {
            const int32_t e = ids[p];
            if (e < 0) {
                pair_code[p] = -1;
                continue;
            }
            pair_code[p] = (pass_of_[e] << COLI_PLAN_SLOT_BITS) | first_[e];
            ++pass_pairs[pass_of_[e]];
            ++usage_[e];
            ++kept;
        }
        out->n_pass = n_pass;
        out->n_load = n_miss;
        out->n_hit = n_hit;
        out->n_miss = n_miss;
        ++st_.plans;
        st_.pairs += (uint64_t)kept;
        st_.hits += (uint64_t)n_hit;
        st_.misses += (uint64_t)n_miss;
        st_.passes += (uint64_t)n_pass;
    }
    for (const int32_t e : order_) {
        used_[e] = 0;
        first_[e] = -1;
    }
    return st;
}

int ExpertCache::prefetch(const int32_t* ids, int32_t P, coli_cache_load* loads, coli_cache_plan* out)
{
    if (P < 0 || !out || !loads || (P > 0 && !ids))
        return COLI_E_INVAL;
    for (int32_t p = 0; p < P; ++p)
        if (ids[p] >= E_)
            return COLI_E_INVAL;
    ++tick_;
    order_.clear();
    for (int32_t p = 0; p < P; ++p) {
        const int32_t e = ids[p];
        if (e >= 0 && !used_[e]) {
            used_[e] = 1;
            order_.push_back(e);
        }
    }
    int32_t n_hit = 0;
    for (const int32_t e : order_) {
        const int32_t s = slot_of_[e];
        if (s >= 0) {
            used_[e] = 2;
            excl_[s] = 1;
            last_use_[s] = tick_;
            ++n_hit;
        }
    }
    /* only the free slots: no slot of a predicted expert is given up */
    victims(excl_, ring_);
    for (const int32_t e : order_)
        if (used_[e] == 2)
            excl_[slot_of_[e]] = 0;
    const int32_t R = (int32_t)ring_.size();
    int32_t n_load = 0;
    for (const int32_t e : order_) {
        if (used_[e] == 2 || n_load >= R)
            continue;
        loads[n_load] = coli_cache_load{e, ring_[n_load], 1, -1};
        place(e, ring_[n_load]);
        inflight_[ring_[n_load]] = 1;
        ++n_load;
    }
    for (const int32_t e : order_)
        used_[e] = 0;
    out->n_pass = n_load ? 2 : 1;
    out->n_load = n_load;
    out->n_hit = n_hit;
    out->n_miss = n_load;
    ++st_.prefetches;
    st_.prefetch_loads += (uint64_t)n_load;
    return COLI_OK;
}

void ExpertCache::stats(coli_cache_stats* st) const
{
    *st = st_;
    st->resident = 0;
    for (const int32_t e : expert_in_)
        st->resident += e >= 0 ? 1 : 0;
    st->pinned = n_pinned_;
}

} // namespace coli

extern "C" {

int colibri_cache_create(int32_t n_experts, int32_t n_slots, coli_expert_cache** out)
{
    if (!out)
        return COLI_E_INVAL;
    *out = nullptr;
    if (n_experts < 1 || n_slots < 1 || n_slots > n_experts)
        return COLI_E_INVAL;
    if (n_experts > COLI_MAX_EXPERTS)
        return COLI_E_UNSUPPORTED;
    try {
        *out = new coli_expert_cache(n_experts, n_slots);
    } catch (const std::bad_alloc&) {
        return COLI_E_INVAL;
    }
    return COLI_OK;
}

void colibri_cache_destroy(coli_expert_cache* c)
{
    delete c;
}

int colibri_cache_pin(coli_expert_cache* c, const int32_t* experts, int32_t n, coli_cache_load* loads,
                      int32_t* n_load)
{
    if (!c)
        return COLI_E_INVAL;
    return c->pin(experts, n, loads, n_load);
}

void colibri_cache_unpin(coli_expert_cache* c)
{
    if (c)
        c->unpin();
}

int colibri_cache_plan(coli_expert_cache* c, const int32_t* ids, int32_t P, int32_t* pair_code,
                       coli_cache_load* loads, int32_t* pass_pairs, coli_cache_plan* plan)
{
    if (!c)
        return COLI_E_INVAL;
    if ((int64_t)P > COLI_MAX_PAIRS)
        return COLI_E_UNSUPPORTED;
    return c->plan(ids, P, pair_code, loads, pass_pairs, plan);
}

int colibri_cache_prefetch(coli_expert_cache* c, const int32_t* ids, int32_t P, coli_cache_load* loads,
                           coli_cache_plan* plan)
{
    if (!c)
        return COLI_E_INVAL;
    if ((int64_t)P > COLI_MAX_PAIRS)
        return COLI_E_UNSUPPORTED;
    return c->prefetch(ids, P, loads, plan);
}

int colibri_cache_stats(const coli_expert_cache* c, coli_cache_stats* st)
{
    if (!c || !st)
        return COLI_E_INVAL;
    c->stats(st);
    return COLI_OK;
}

int colibri_cache_state(const coli_expert_cache* c, int32_t* slot_of, uint64_t* usage)
{
    if (!c)
        return COLI_E_INVAL;
    if (slot_of)
        std::copy(c->slot_of().begin(), c->slot_of().end(), slot_of);
    if (usage)
        std::copy(c->usage().begin(), c->usage().end(), usage);
    return COLI_OK;
}

} // extern "C"
