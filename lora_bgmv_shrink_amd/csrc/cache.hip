// Adapter slot cache: GPU slots over adapters kept in host memory, loaded
// on demand by asynchronous copies on a side stream, evicted LRU.  The
// policy follows "Multi-LoRA batching and adapter paging", section "Adapter
// paging" (hit: schedule now; miss: evict a cold adapter and copy it in;
// cap concurrent loads; pinned adapters stay) and "Serving many LoRA
// adapters" (blog.ecitis.org), section "Paging adapters" (a fetch never
// blocks the step: the request is deferred while the load runs; LRU over
// adapter ids; no eviction of an adapter with queued requests).  Semantics
// of every entry point: include/lora_mi355x.h.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

#include "lora_internal.hpp"
#include "pool.hpp"

using namespace lora;

namespace {

constexpr int kMaxRank = 64;
constexpr int64_t kBlockAlignElems = 128;   // 256 B in bf16, 512 B in fp32

enum SlotState : int8_t { SLOT_EMPTY = 0, SLOT_LOADING = 1, SLOT_READY = 2 };

struct Slot {
    int32_t adapter = -1;
    SlotState state = SLOT_EMPTY;
    bool bound = false;           // mapped by a batch that is not released yet
    bool used = false;            // use_done holds the end of a released batch
    hipStream_t waited = nullptr; // the stream last made to wait for the load
    bool waited_any = false;
    uint64_t last_use = 0;        // LRU clock
    hipEvent_t load_done = nullptr;
    hipEvent_t use_done = nullptr;
};

struct Entry {
    bool registered = false;
    bool pinned = false;
    int32_t holds = 0;
    int32_t rank = 0;
    float scale = 0.f;
    const void* blob = nullptr;
    int32_t slot = -1;            // slot holding it (loading or ready), -1 if none
};

// Compact blob of one adapter of rank r: [A_0][B_0][A_1][B_1]..., each block
// rounded up to kBlockAlignElems elements.  Part p's A starts at the returned
// a_off(p), its B at b_off(p).
__host__ __device__ inline int64_t block_elems(int64_t rows, int64_t cols) {
    return (rows * cols + kBlockAlignElems - 1) / kBlockAlignElems * kBlockAlignElems;
}

// After a load into `slot`: the slot's rank and scale (one entry shared by
// every part's pool) and every part's block offsets.  One workgroup of 256
// threads walks the parts 256 at a time: thread t sizes part p0 + t, an
// exclusive prefix sum (wave shuffles, then the four wave totals) places it,
// and the chunk total carries into the next chunk.
constexpr int kTableThreads = 256;

__global__ void __launch_bounds__(kTableThreads)
k_cache_slot_tables(int32_t* __restrict__ ranks, float* __restrict__ scales,
                    int64_t* __restrict__ a_off, int64_t* __restrict__ b_off,
                    const int32_t* __restrict__ d_in, const int32_t* __restrict__ d_out,
                    int32_t n_parts, int32_t n_slots, int32_t slot, int32_t rank, float scale,
                    int64_t slot_base) {
    __shared__ int64_t wave_sum[kTableThreads / 64];
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int w = t >> 6;
    int64_t carry = slot_base;
    for (int32_t p0 = 0; p0 < n_parts; p0 += kTableThreads) {
        const int32_t p = p0 + t;
        int64_t ea = 0, eb = 0;
        if (p < n_parts) {
            ea = block_elems(d_in[p], rank);
            eb = block_elems(rank, d_out[p]);
        }
        int64_t v = ea + eb;   // inclusive scan within the wave
        for (int o = 1; o < 64; o <<= 1) {
            const int64_t u = __shfl_up(v, o, 64);
            if (lane >= o) v += u;
        }
        if (lane == 63) wave_sum[w] = v;
        __syncthreads();
        int64_t before = 0, total = 0;
        for (int k = 0; k < kTableThreads / 64; ++k) {
            before += k < w ? wave_sum[k] : 0;
            total += wave_sum[k];
        }
        if (p < n_parts) {
            const int64_t o = carry + before + v - (ea + eb);
            a_off[(int64_t)p * n_slots + slot] = o;
            b_off[(int64_t)p * n_slots + slot] = o + ea;
        }
        carry += total;
        __syncthreads();   // wave_sum is rewritten by the next chunk
    }
    if (t == 0) {
        ranks[slot] = rank;
        scales[slot] = scale;
    }
}

}  // namespace

struct lora_cache_s {
    lora_dtype_t dtype;
    int32_t eb;
    int32_t n_parts, r_max, n_adapters, n_slots, max_loads, flags;
    bool host_only;
    std::vector<int32_t> d_in, d_out;
    int64_t cap_elems;             // blob elements at rank r_max = slot stride
    std::vector<Slot> slots;
    std::vector<Entry> entries;
    std::vector<int32_t> loading;  // slots with a load in flight
    std::vector<int32_t> bound;    // slots mapped since the last release
    uint64_t clock = 0;
    lora_cache_stats_t st;
    // device side (absent when host_only)
    void* arena = nullptr;
    void* tables = nullptr;
    int32_t* t_ranks = nullptr;
    float* t_scales = nullptr;
    int64_t* t_aoff = nullptr;
    int64_t* t_boff = nullptr;
    int32_t* t_din = nullptr;
    int32_t* t_dout = nullptr;
    hipStream_t copy = nullptr;
    std::vector<lora_pool_s*> pools;
};

namespace {

int64_t blob_elems_for(const lora_cache_s* c, int32_t rank, int64_t* a_off, int64_t* b_off) {
    int64_t o = 0;
    for (int32_t p = 0; p < c->n_parts; ++p) {
        if (a_off) a_off[p] = o;
        o += block_elems(c->d_in[p], rank);
        if (b_off) b_off[p] = o;
        o += block_elems(rank, c->d_out[p]);
    }
    return o;
}

bool rank_taken(const lora_cache_s* c, int32_t rank) {
    if (rank < 1 || rank > c->r_max) return false;
    if (c->flags & LORA_CACHE_ANY_RANK) return true;
    const int ve = 16 / c->eb;
    return rank % ve == 0 && (512 * ve) % rank == 0;
}

// Notice completed loads.  A host-only cache has no copies: its loads
// complete when the caller polls or waits (explicit), never inside request
// or map, so a policy run is a pure function of the call sequence.  A device
// cache created with LORA_CACHE_EXPLICIT_POLL behaves the same way.
lora_status_t poll_loads(lora_cache_s* c, int32_t* n_done, bool explicit_poll) {
    int32_t done = 0;
    if ((c->host_only || (c->flags & LORA_CACHE_EXPLICIT_POLL)) && !explicit_poll) {
        if (n_done) *n_done = 0;
        return LORA_OK;
    }
    for (size_t i = 0; i < c->loading.size();) {
        Slot& s = c->slots[c->loading[i]];
        bool complete = c->host_only;
        if (!complete) {
            const hipError_t q = hipEventQuery(s.load_done);
            if (q == hipSuccess) complete = true;
            else if (q != hipErrorNotReady) return LORA_E_DEVICE;
        }
        if (complete) {
            s.state = SLOT_READY;
            c->loading[i] = c->loading.back();
            c->loading.pop_back();
            ++c->st.loads_completed;
            ++done;
        } else {
            ++i;
        }
    }
    if (n_done) *n_done = done;
    return LORA_OK;
}

// Empty slots first (lowest index), else the least recently used ready slot
// whose adapter is not pinned, held or bound (ties to the lowest index).
int32_t pick_victim(const lora_cache_s* c) {
    for (int32_t v = 0; v < c->n_slots; ++v)
        if (c->slots[v].state == SLOT_EMPTY) return v;
    int32_t best = -1;
    for (int32_t v = 0; v < c->n_slots; ++v) {
        const Slot& s = c->slots[v];
        if (s.state != SLOT_READY || s.bound) continue;
        const Entry& e = c->entries[s.adapter];
        if (e.pinned || e.holds > 0) continue;
        if (best < 0 || s.last_use < c->slots[best].last_use) best = v;
    }
    return best;
}

lora_status_t start_load(lora_cache_s* c, int32_t v, int32_t adapter) {
    Slot& s = c->slots[v];
    Entry& e = c->entries[adapter];
    if (s.adapter >= 0) {
        Entry& old = c->entries[s.adapter];
        c->st.bytes_resident -= blob_elems_for(c, old.rank, nullptr, nullptr) * c->eb;
        old.slot = -1;
        ++c->st.evictions;
        s.adapter = -1;
        s.state = SLOT_EMPTY;
    }
    const int64_t bytes = blob_elems_for(c, e.rank, nullptr, nullptr) * c->eb;
    if (!c->host_only) {
        // the copy overwrites the slot only after the last batch that read it
        if (s.used && hipStreamWaitEvent(c->copy, s.use_done, 0) != hipSuccess) return LORA_E_DEVICE;
        char* dst = (char*)c->arena + (size_t)v * (size_t)c->cap_elems * c->eb;
        if (hipMemcpyAsync(dst, e.blob, (size_t)bytes, hipMemcpyHostToDevice, c->copy) != hipSuccess)
            return LORA_E_DEVICE;
        hipLaunchKernelGGL(k_cache_slot_tables, dim3(1), dim3(kTableThreads), 0, c->copy, c->t_ranks,
                           c->t_scales, c->t_aoff, c->t_boff, c->t_din, c->t_dout, c->n_parts,
                           c->n_slots, v, e.rank, e.scale, (int64_t)v * c->cap_elems);
        if (hipGetLastError() != hipSuccess) return LORA_E_DEVICE;
        if (hipEventRecord(s.load_done, c->copy) != hipSuccess) return LORA_E_DEVICE;
        for (lora_pool_s* p : c->pools) p->ranks[v] = e.rank;
    }
    s.adapter = adapter;
    s.state = SLOT_LOADING;
    s.waited_any = false;
    s.last_use = ++c->clock;
    e.slot = v;
    c->loading.push_back(v);
    ++c->st.loads_started;
    c->st.bytes_loaded += bytes;
    c->st.bytes_resident += bytes;
    return LORA_OK;
}

bool adapter_ok(const lora_cache_s* c, int32_t a) { return a >= 0 && a < c->n_adapters; }

void free_device(lora_cache_s* c) {
    for (Slot& s : c->slots) {
        if (s.load_done) (void)hipEventDestroy(s.load_done);
        if (s.use_done) (void)hipEventDestroy(s.use_done);
    }
    for (lora_pool_s* p : c->pools) delete p;
    c->pools.clear();
    if (c->arena) (void)hipFree(c->arena);
    if (c->tables) (void)hipFree(c->tables);
    if (c->copy) (void)hipStreamDestroy(c->copy);
}

}  // namespace

extern "C" {

lora_status_t lora_cache_blob_layout(lora_cache_t c, int32_t rank, int64_t* a_off, int64_t* b_off,
                                     int64_t* blob_elems) {
    if (!c || !a_off || !b_off || !blob_elems || rank < 1 || rank > c->r_max) return LORA_E_INVALID;
    *blob_elems = blob_elems_for(c, rank, a_off, b_off);
    return LORA_OK;
}

lora_status_t lora_cache_create(lora_cache_t* out, lora_dtype_t dtype, int32_t n_parts,
                                const int32_t* d_in, const int32_t* d_out, int32_t r_max,
                                int32_t n_adapters, int32_t n_slots, int32_t max_loads_in_flight,
                                int32_t flags) {
    if (!out) return LORA_E_INVALID;
    *out = nullptr;
    int dt = 0;   // validated as an int: a C caller may pass any value
    std::memcpy(&dt, &dtype, sizeof dt);
    if ((dt != LORA_F32 && dt != LORA_BF16) || n_parts < 1 || !d_in || !d_out ||
        r_max < 1 || n_adapters < 1 || n_slots < 1 || max_loads_in_flight < 1 ||
        (flags & ~(LORA_CACHE_HOST_ONLY | LORA_CACHE_ANY_RANK | LORA_CACHE_EXPLICIT_POLL)) != 0)
        return LORA_E_INVALID;
    if (r_max > kMaxRank) return LORA_E_UNSUPPORTED;
    for (int32_t p = 0; p < n_parts; ++p)
        if (d_in[p] < 1 || d_out[p] < 1) return LORA_E_INVALID;

    lora_cache_s* c = new lora_cache_s;
    c->dtype = dtype;
    c->eb = dtype == LORA_BF16 ? 2 : 4;
    c->n_parts = n_parts;
    c->r_max = r_max;
    c->n_adapters = n_adapters;
    c->n_slots = n_slots;
    c->max_loads = max_loads_in_flight;
    c->flags = flags;
    c->host_only = (flags & LORA_CACHE_HOST_ONLY) != 0;
    c->d_in.assign(d_in, d_in + n_parts);
    c->d_out.assign(d_out, d_out + n_parts);
    c->cap_elems = blob_elems_for(c, r_max, nullptr, nullptr);
    c->slots.resize(n_slots);
    c->entries.resize(n_adapters);
    c->loading.reserve(max_loads_in_flight);
    c->bound.reserve(n_slots);
    std::memset(&c->st, 0, sizeof(c->st));
    c->st.n_slots = n_slots;
    if (c->host_only) {
        *out = c;
        return LORA_OK;
    }

    // One table allocation: ranks and scales (shared by every part), then
    // per part the A and B offsets of each slot, the part shapes, and one
    // error word per part.
    const size_t o_ranks = 0;
    const size_t o_scales = align_up(o_ranks + (size_t)n_slots * 4, 256);
    const size_t o_aoff = align_up(o_scales + (size_t)n_slots * 4, 256);
    const size_t o_boff = align_up(o_aoff + (size_t)n_parts * n_slots * 8, 256);
    const size_t o_din = align_up(o_boff + (size_t)n_parts * n_slots * 8, 256);
    const size_t o_dout = align_up(o_din + (size_t)n_parts * 4, 256);
    const size_t o_err = align_up(o_dout + (size_t)n_parts * 4, 256);
    const size_t total = align_up(o_err + (size_t)n_parts * 4, 256);
    std::vector<uint8_t> host(total, 0);
    {
        int32_t* rk = (int32_t*)(host.data() + o_ranks);
        int64_t* ao = (int64_t*)(host.data() + o_aoff);
        int64_t* bo = (int64_t*)(host.data() + o_boff);
        std::vector<int64_t> pa(n_parts), pb(n_parts);
        blob_elems_for(c, r_max, pa.data(), pb.data());
        for (int32_t v = 0; v < n_slots; ++v) {
            rk[v] = r_max;   // empty slots are never named by a mapped id
            for (int32_t p = 0; p < n_parts; ++p) {
                ao[(size_t)p * n_slots + v] = (int64_t)v * c->cap_elems + pa[p];
                bo[(size_t)p * n_slots + v] = (int64_t)v * c->cap_elems + pb[p];
            }
        }
        std::memcpy(host.data() + o_din, d_in, (size_t)n_parts * 4);
        std::memcpy(host.data() + o_dout, d_out, (size_t)n_parts * 4);
    }
    const size_t arena_bytes = (size_t)n_slots * (size_t)c->cap_elems * c->eb;
    bool ok = hipMalloc(&c->tables, total) == hipSuccess &&
              hipMemcpy(c->tables, host.data(), total, hipMemcpyHostToDevice) == hipSuccess &&
              hipMalloc(&c->arena, arena_bytes) == hipSuccess &&
              hipStreamCreateWithFlags(&c->copy, hipStreamNonBlocking) == hipSuccess;
    for (int32_t v = 0; ok && v < n_slots; ++v)
        ok = hipEventCreateWithFlags(&c->slots[v].load_done, hipEventDisableTiming) == hipSuccess &&
             hipEventCreateWithFlags(&c->slots[v].use_done, hipEventDisableTiming) == hipSuccess;
    if (!ok) {
        free_device(c);
        delete c;
        return LORA_E_DEVICE;
    }
    uint8_t* m = (uint8_t*)c->tables;
    c->t_ranks = (int32_t*)(m + o_ranks);
    c->t_scales = (float*)(m + o_scales);
    c->t_aoff = (int64_t*)(m + o_aoff);
    c->t_boff = (int64_t*)(m + o_boff);
    c->t_din = (int32_t*)(m + o_din);
    c->t_dout = (int32_t*)(m + o_dout);
    const bool stream_ok = (flags & LORA_CACHE_ANY_RANK) == 0;
    for (int32_t p = 0; p < n_parts; ++p) {
        lora_pool_s* q = new lora_pool_s;
        q->layout = LORA_LAYOUT_RAGGED;
        q->dtype = dtype;
        q->ranks.assign(n_slots, r_max);
        q->tables = nullptr;
        q->owned_by_cache = true;
        q->dev.A = c->arena;
        q->dev.B = c->arena;
        q->dev.ranks = c->t_ranks;
        q->dev.a_off = c->t_aoff + (size_t)p * n_slots;
        q->dev.b_off = c->t_boff + (size_t)p * n_slots;
        q->dev.scales = c->t_scales;
        q->dev.err = (int32_t*)(m + o_err) + p;
        q->dev.n_adapters = n_slots;
        q->dev.d_in = d_in[p];
        q->dev.d_out = d_out[p];
        q->dev.r_max = r_max;
        q->dev.vec_a = 1;   // blocks start 256-byte aligned
        q->dev.vec_b = ((int64_t)d_out[p] * c->eb) % 16 == 0 ? 1 : 0;
        q->dev.stream_ok = stream_ok ? 1 : 0;
        q->dev.vec_rank = stream_ok ? 1 : 0;   // taken ranks are whole 16-byte pieces
        c->pools.push_back(q);
    }
    *out = c;
    return LORA_OK;
}

lora_status_t lora_cache_destroy(lora_cache_t c) {
    if (!c) return LORA_OK;
    lora_status_t st = LORA_OK;
    if (!c->host_only) {
        if (hipStreamSynchronize(c->copy) != hipSuccess || hipDeviceSynchronize() != hipSuccess)
            st = LORA_E_DEVICE;
        free_device(c);
    }
    delete c;
    return st;
}

lora_status_t lora_cache_register(lora_cache_t c, int32_t adapter, int32_t rank, float scale,
                                  const void* blob) {
    if (!c || !adapter_ok(c, adapter) || !std::isfinite(scale)) return LORA_E_INVALID;
    if (!blob && !c->host_only) return LORA_E_INVALID;
    if (rank < 1 || rank > c->r_max) return LORA_E_UNSUPPORTED;
    if (!rank_taken(c, rank)) return LORA_E_UNSUPPORTED;
    Entry& e = c->entries[adapter];
    if (e.slot >= 0) return LORA_E_INVALID;
    e.registered = true;
    e.rank = rank;
    e.scale = scale;
    e.blob = blob;
    return LORA_OK;
}

lora_status_t lora_cache_pin(lora_cache_t c, int32_t adapter, int32_t pinned) {
    if (!c || !adapter_ok(c, adapter) || !c->entries[adapter].registered) return LORA_E_INVALID;
    c->entries[adapter].pinned = pinned != 0;
    return LORA_OK;
}

lora_status_t lora_cache_hold(lora_cache_t c, int32_t adapter, int32_t delta) {
    if (!c || !adapter_ok(c, adapter) || !c->entries[adapter].registered) return LORA_E_INVALID;
    Entry& e = c->entries[adapter];
    if ((int64_t)e.holds + delta < 0 || (int64_t)e.holds + delta > INT32_MAX) return LORA_E_INVALID;
    e.holds += delta;
    return LORA_OK;
}

lora_status_t lora_cache_poll(lora_cache_t c, int32_t* n_completed) {
    if (!c) return LORA_E_INVALID;
    return poll_loads(c, n_completed, true);
}

lora_status_t lora_cache_wait(lora_cache_t c) {
    if (!c) return LORA_E_INVALID;
    if (!c->host_only)
        for (int32_t v : c->loading)
            if (hipEventSynchronize(c->slots[v].load_done) != hipSuccess) return LORA_E_DEVICE;
    return poll_loads(c, nullptr, true);
}

lora_status_t lora_cache_request(lora_cache_t c, int32_t adapter, lora_cache_state_t* state) {
    if (!c || !state || !adapter_ok(c, adapter) || !c->entries[adapter].registered)
        return LORA_E_INVALID;
    lora_status_t st = poll_loads(c, nullptr, false);
    if (st != LORA_OK) return st;
    ++c->st.requests;
    Entry& e = c->entries[adapter];
    if (e.slot >= 0) {
        Slot& s = c->slots[e.slot];
        s.last_use = ++c->clock;
        if (s.state == SLOT_READY) {
            ++c->st.hits;
            *state = LORA_CACHE_RESIDENT;
        } else {
            ++c->st.pending;
            *state = LORA_CACHE_LOADING;
        }
        return LORA_OK;
    }
    if ((int32_t)c->loading.size() >= c->max_loads) {
        ++c->st.deferred_load_cap;
        *state = LORA_CACHE_DEFERRED;
        return LORA_OK;
    }
    const int32_t v = pick_victim(c);
    if (v < 0) {
        ++c->st.deferred_no_slot;
        *state = LORA_CACHE_DEFERRED;
        return LORA_OK;
    }
    st = start_load(c, v, adapter);
    if (st != LORA_OK) return st;
    *state = LORA_CACHE_LOADING;
    return LORA_OK;
}

lora_status_t lora_cache_map(lora_cache_t c, const int32_t* adapters, int32_t n, int32_t* slots,
                             hipStream_t stream) {
    if (!c || n < 0 || (n > 0 && (!adapters || !slots))) return LORA_E_INVALID;
    lora_status_t st = poll_loads(c, nullptr, false);
    if (st != LORA_OK) return st;
    for (int32_t i = 0; i < n; ++i) {
        const int32_t a = adapters[i];
        if (a == -1) continue;
        if (!adapter_ok(c, a) || !c->entries[a].registered) return LORA_E_INVALID;
        const int32_t v = c->entries[a].slot;
        if (v < 0 || c->slots[v].state != SLOT_READY) return LORA_E_NOT_RESIDENT;
    }
    for (int32_t i = 0; i < n; ++i) {
        const int32_t a = adapters[i];
        if (a == -1) {
            slots[i] = -1;
            continue;
        }
        const int32_t v = c->entries[a].slot;
        Slot& s = c->slots[v];
        slots[i] = v;
        s.last_use = ++c->clock;
        if (!s.bound) {
            s.bound = true;
            c->bound.push_back(v);
        }
        if (!c->host_only && (!s.waited_any || s.waited != stream)) {
            if (hipStreamWaitEvent(stream, s.load_done, 0) != hipSuccess) return LORA_E_DEVICE;
            s.waited = stream;
            s.waited_any = true;
        }
    }
    return LORA_OK;
}

lora_status_t lora_cache_release(lora_cache_t c, hipStream_t stream) {
    if (!c) return LORA_E_INVALID;
    for (int32_t v : c->bound) {
        Slot& s = c->slots[v];
        if (!c->host_only) {
            if (hipEventRecord(s.use_done, stream) != hipSuccess) return LORA_E_DEVICE;
            s.used = true;
        }
        s.bound = false;
    }
    c->bound.clear();
    return LORA_OK;
}

lora_pool_t lora_cache_pool(lora_cache_t c, int32_t part) {
    if (!c || c->host_only || part < 0 || part >= c->n_parts) return nullptr;
    return c->pools[part];
}

int32_t lora_cache_slot_of(lora_cache_t c, int32_t adapter) {
    if (!c || !adapter_ok(c, adapter)) return -1;
    return c->entries[adapter].slot;
}

lora_status_t lora_cache_stats(lora_cache_t c, lora_cache_stats_t* out) {
    if (!c || !out) return LORA_E_INVALID;
    lora_cache_stats_t s = c->st;
    s.slots_resident = 0;
    for (const Slot& v : c->slots) s.slots_resident += v.state == SLOT_READY ? 1 : 0;
    s.slots_loading = (int32_t)c->loading.size();
    s.slots_bound = (int32_t)c->bound.size();
    *out = s;
    return LORA_OK;
}

}  // extern "C"
