// Adapter-aware admission: forms each step's batch from the request queue
// by a score of wait time and adapter locality, under a row budget, a cap
// on distinct adapters per batch, optional rank-class grouping and (with a
// slot cache) adapter residency.  Host code only; it reaches the cache
// through its C ABI.  Semantics: include/lora_mi355x.h ("Serving many LoRA
// adapters" (blog.ecitis.org), sections "Adapter-aware scheduling" and
// "Paging adapters"; "Serving multiple LoRAs: segmented matrix multiplies
// and adapter scheduling", section "Scheduling the adapters").
#include <cmath>
#include <cstring>
#include <vector>

#include "../../include/lora_mi355x.h"

namespace {

struct Req {
    int64_t id;
    int32_t adapter;
    int32_t rows;
    double arrival;
    uint64_t seq;      // submission order (tie-break)
};

// Rank class: 1, 2, 3-4, 5-8, 9-16, 17-32, 33-64 -> 0 .. 6.
int rank_class(int32_t r) {
    int c = 0;
    while ((1 << c) < r) ++c;
    return c;
}

// Priority of a queued request: a fairness part that grows linearly with
// how long it has waited, plus a bonus for locality when its adapter is
// already active, in proportion to the rows it would add to that adapter's
// work.  No fused multiply-add, so the policy model computes the same double.
#pragma clang fp contract(off)
double priority(double w_fair, double w_local, double wait, bool adapter_active, int32_t rows) {
    const double fairness = w_fair * wait;
    const double locality_bonus = adapter_active ? w_local * (double)rows : 0.0;
    return fairness + locality_bonus;
}

}  // namespace

struct lora_sched_s {
    lora_sched_config_t cfg;
    int32_t n_adapters;
    std::vector<int32_t> ranks;        // empty when not given
    lora_cache_t cache;
    std::vector<Req> queue;            // submission order
    uint64_t next_seq = 0;
    std::vector<uint8_t> active_prev;  // adapters of the previous batch
    std::vector<int32_t> prev_list;
    std::vector<int32_t> held_admitted;  // holds kept until the next step
    // per-step scratch (sized once)
    std::vector<uint8_t> in_batch;
    std::vector<int8_t> resident;      // -1 unknown, 0 no, 1 yes (this step)
    std::vector<int32_t> touched;
    std::vector<uint8_t> done;
};

extern "C" {

lora_status_t lora_sched_create(lora_sched_t* out, const lora_sched_config_t* cfg, int32_t n_adapters,
                                const int32_t* ranks, lora_cache_t cache) {
    if (!out) return LORA_E_INVALID;
    *out = nullptr;
    if (!cfg || n_adapters < 1 || cfg->max_adapters < 1 || cfg->max_rows < 1 ||
        !(cfg->w_fair >= 0.0) || !(cfg->w_local >= 0.0) || !std::isfinite(cfg->w_fair) ||
        !std::isfinite(cfg->w_local))
        return LORA_E_INVALID;
    if (cfg->rank_groups && !ranks) return LORA_E_INVALID;
    if (ranks)
        for (int32_t u = 0; u < n_adapters; ++u)
            if (ranks[u] < 1 || ranks[u] > 64) return LORA_E_INVALID;
    lora_sched_s* s = new lora_sched_s;
    s->cfg = *cfg;
    s->n_adapters = n_adapters;
    if (ranks) s->ranks.assign(ranks, ranks + n_adapters);
    s->cache = cache;
    s->active_prev.assign(n_adapters, 0);
    s->in_batch.assign(n_adapters, 0);
    s->resident.assign(n_adapters, -1);
    *out = s;
    return LORA_OK;
}

lora_status_t lora_sched_destroy(lora_sched_t s) {
    if (!s) return LORA_OK;
    if (s->cache) {
        for (int32_t a : s->held_admitted) (void)lora_cache_hold(s->cache, a, -1);
        for (const Req& r : s->queue)
            if (r.adapter >= 0) (void)lora_cache_hold(s->cache, r.adapter, -1);
    }
    delete s;
    return LORA_OK;
}

lora_status_t lora_sched_submit(lora_sched_t s, int64_t request, int32_t adapter, int32_t rows,
                                double arrival) {
    if (!s || adapter < -1 || adapter >= s->n_adapters || rows < 1 || !std::isfinite(arrival))
        return LORA_E_INVALID;
    if (s->cache && adapter >= 0) {
        const lora_status_t st = lora_cache_hold(s->cache, adapter, 1);
        if (st != LORA_OK) return st;
    }
    s->queue.push_back(Req{request, adapter, rows, arrival, s->next_seq++});
    return LORA_OK;
}

int32_t lora_sched_queued(lora_sched_t s) { return s ? (int32_t)s->queue.size() : -1; }

lora_status_t lora_sched_step(lora_sched_t s, double now, int32_t capacity, int64_t* requests,
                              int32_t* adapters, int32_t* rows, double* waits,
                              lora_sched_step_t* info) {
    if (!s || !info || !std::isfinite(now) || capacity < 0 ||
        (capacity > 0 && (!requests || !adapters || !rows)))
        return LORA_E_INVALID;
    std::memset(info, 0, sizeof(*info));
    // The previous batch has been handed to the cache (mapped) by now: its
    // requests no longer need their adapters held.
    if (s->cache)
        for (int32_t a : s->held_admitted) {
            const lora_status_t st = lora_cache_hold(s->cache, a, -1);
            if (st != LORA_OK) return st;
        }
    s->held_admitted.clear();

    const lora_sched_config_t& c = s->cfg;
    const size_t n = s->queue.size();
    s->done.assign(n, 0);
    int32_t distinct = 0, batch_rows = 0, admitted = 0, batch_class = -1;
    std::vector<int32_t> batch_adapters;
    lora_status_t err = LORA_OK;   // a cache error ends the fill; the step is still closed consistently
    for (;;) {
        if (admitted >= capacity || batch_rows >= c.max_rows) break;
        // best pending request by score, then arrival, then submission
        int64_t best = -1;
        double best_score = 0.0;
        for (size_t i = 0; i < n; ++i) {
            if (s->done[i]) continue;
            const Req& r = s->queue[i];
            const bool local = r.adapter >= 0 && (s->active_prev[r.adapter] || s->in_batch[r.adapter]);
            const double sc = priority(c.w_fair, c.w_local, now - r.arrival, local, r.rows);
            if (best < 0 || sc > best_score ||
                (sc == best_score && (r.arrival < s->queue[best].arrival ||
                                      (r.arrival == s->queue[best].arrival &&
                                       r.seq < s->queue[best].seq)))) {
                best = (int64_t)i;
                best_score = sc;
            }
        }
        if (best < 0) break;
        s->done[best] = 1;   // decided for this step (admitted or skipped)
        const Req& r = s->queue[best];
        const int32_t a = r.adapter;
        if (a >= 0 && s->cache) {
            if (s->resident[a] < 0) {
                lora_cache_state_t st;
                const lora_status_t e = lora_cache_request(s->cache, a, &st);
                if (e != LORA_OK) {
                    err = e;
                    s->done[best] = 0;   // not decided: it stays queued
                    break;
                }
                s->resident[a] = st == LORA_CACHE_RESIDENT ? 1 : 0;
                s->touched.push_back(a);
            }
            if (!s->resident[a]) {
                ++info->deferred_not_resident;
                continue;
            }
        }
        if (batch_rows + r.rows > c.max_rows) {
            ++info->skipped_rows;
            continue;
        }
        if (a >= 0 && !s->in_batch[a] && distinct >= c.max_adapters) {
            ++info->skipped_cap;
            continue;
        }
        if (a >= 0 && c.rank_groups) {
            const int k = rank_class(s->ranks[a]);
            if (batch_class >= 0 && k != batch_class) {
                ++info->skipped_rank_group;
                continue;
            }
            batch_class = k;
        }
        // admit
        if (a >= 0 && !s->in_batch[a]) {
            s->in_batch[a] = 1;
            batch_adapters.push_back(a);
            ++distinct;
        }
        if (a >= 0 && s->cache) s->held_admitted.push_back(a);   // its submit hold, kept one step
        requests[admitted] = r.id;
        adapters[admitted] = a;
        rows[admitted] = r.rows;
        const double wt = now - r.arrival;
        if (waits) waits[admitted] = wt;
        if (wt > info->max_wait_admitted || admitted == 0) info->max_wait_admitted = wt;
        ++admitted;
        batch_rows += r.rows;
        s->done[best] = 2;
    }
    // compact the queue (admitted requests leave it, order kept)
    size_t k = 0;
    for (size_t i = 0; i < n; ++i) {
        if (s->done[i] == 2) continue;
        const double wt = now - s->queue[i].arrival;
        if (k == 0 || wt > info->max_wait_queued) info->max_wait_queued = wt;
        s->queue[k++] = s->queue[i];
    }
    s->queue.resize(k);
    // the batch becomes the active set of the next step
    for (int32_t a : s->prev_list) s->active_prev[a] = 0;
    s->prev_list.clear();
    for (int32_t a : batch_adapters) {
        s->in_batch[a] = 0;
        s->active_prev[a] = 1;
        s->prev_list.push_back(a);
    }
    for (int32_t a : s->touched) s->resident[a] = -1;
    s->touched.clear();
    info->admitted = admitted;
    info->rows = batch_rows;
    info->distinct_adapters = distinct;
    info->queued = (int32_t)k;
    return err;
}

}  // extern "C"
