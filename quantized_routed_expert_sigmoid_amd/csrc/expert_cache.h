/*
 * expert_cache.h -- the host-side slot cache of the tiered expert store
 * (plain C++, no HIP): which routed expert occupies which HBM slot, the
 * least-recently-used order, the pinned hot set, usage counts, and the plan
 * that turns one batch's routed ids into slot ids, expert loads and passes.
 *
 * The per-layer LRU cache with an optional pinned hot store follows "Show HN:
 * 如何在我的低配置电脑上运行 GLM-5.2", section "思路" (idea); the pin-the-
 * hottest-experts learned cache and usage record follow the same page's
 * learned-cache paragraph; the passes follow its deferred cold-expert
 * pipeline paragraph (resident experts compute while missing experts load;
 * their results are merged before the layer ends).
 */
#ifndef COLI_EXPERT_CACHE_H
#define COLI_EXPERT_CACHE_H

#include "../../include/colibri.h"

#include <stdint.h>
#include <vector>

namespace coli {

class ExpertCache {
public:
    ExpertCache(int32_t n_experts, int32_t n_slots);

    /* All-or-nothing; see colibri_cache_pin. */
    int pin(const int32_t* experts, int32_t n, coli_cache_load* loads, int32_t* n_load);
    void unpin();
    /* Forgets every slot's contents and pin (after a failed transfer). */
    void reset();

    /* See colibri_cache_plan.  The arrays are host memory of the documented
     * sizes. */
    int plan(const int32_t* ids, int32_t P, int32_t* pair_code, coli_cache_load* loads,
             int32_t* pass_pairs, coli_cache_plan* out);

    /* See colibri_cache_prefetch. */
    int prefetch(const int32_t* ids, int32_t P, coli_cache_load* loads, coli_cache_plan* out);

    void stats(coli_cache_stats* st) const;

    int32_t n_experts() const { return E_; }
    int32_t n_slots() const { return n_slots_; }
    const std::vector<int32_t>& slot_of() const { return slot_of_; }
    const std::vector<uint64_t>& usage() const { return usage_; }

private:
    /* Unpinned slots not in `excluded`, empty ones first (ascending), then by
     * last use (oldest first), ties to the lower slot. */
    void victims(const std::vector<uint8_t>& excluded, std::vector<int32_t>& out) const;
    void place(int32_t expert, int32_t slot);

    int32_t E_, n_slots_;
    std::vector<int32_t> slot_of_;   /* [E]: slot or -1 */
    std::vector<int32_t> expert_in_; /* [n_slots]: expert or -1 */
    std::vector<uint8_t> pinned_;    /* [n_slots] */
    std::vector<uint64_t> last_use_; /* [n_slots]: plan tick of the last use */
    std::vector<uint64_t> usage_;    /* [E]: routed pairs so far */
    std::vector<uint8_t> inflight_;  /* [n_slots]: loaded by a prefetch no plan has consumed */
    uint64_t tick_ = 0;
    int32_t n_pinned_ = 0;
    coli_cache_stats st_ = {};

    /* per-plan scratch, kept to avoid reallocation */
    std::vector<int32_t> order_, ring_, ready_, first_, pass_of_;
    std::vector<uint8_t> used_, excl_;
};

} // namespace coli

/* The C ABI's opaque cache type is the planner itself. */
struct coli_expert_cache : coli::ExpertCache {
    using coli::ExpertCache::ExpertCache;
};

#endif
