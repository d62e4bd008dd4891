// The delta cache: per-variant residency of (packed signs, α) sets in HBM
// slots, loads on demand, eviction of the least recently requested variant
// outside the pinned top by request rate, and one load per variant however
// many requests wait for it.
//
// Follows "BitDelta : servir 14 modèles Zen depuis un seul cluster GPU"
// (hanzo-blog, 2026-02-28), section "Infrastructure details" (cold start,
// eviction policy, request routing); the reading of the rate weighting is
// stated in include/bitdelta_cache.h.  Host code only: the device work is a
// copy per load, ordered with HIP events.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <vector>

#include "../../include/bitdelta_cache.h"
#include "bd_internal.h"

namespace {

enum SlotState { kEmpty = 0, kLoading = 1, kReady = 2 };

struct UseEvent {
    hipStream_t stream;
    hipEvent_t event;
};

struct Slot {
    int var = -1;
    int state = kEmpty;
    int refs = 0;
    hipEvent_t loaded = nullptr;     // recorded on the copy stream after the load
    std::vector<UseEvent> uses;      // last release per stream since the load
};

struct Variant {
    double rate = 0.0;               // decayed request count at time `t`
    double t = 0.0;
    bool seen = false;
    uint64_t last = 0;               // request tick of the last request (LRU order)
    int slot = -1;
    const void* src = nullptr;       // pinned host source (device mode)
};

}  // namespace

struct bd_cache {
    bd_cache_config cfg;
    char* base = nullptr;            // device slots, or nullptr in policy mode
    hipStream_t copy = nullptr;
    std::vector<Slot> slots;
    std::vector<Variant> vars;
    std::vector<hipEvent_t> spare;   // recycled use events
    uint64_t tick = 0;
    double now = -HUGE_VAL;          // time of the latest request; requests may not go back
    bd_cache_stats stats{};
};

namespace {

bool device_mode(const bd_cache* c) { return c->base != nullptr; }

double decayed(const Variant& v, const bd_cache* c, double now) {
    if (!v.seen) return 0.0;
    return v.rate * std::exp2(-(now - v.t) / c->cfg.half_life);
}

// The pinned set at `now`: the cfg.pinned variants with the highest decayed
// rate (ties: lower index), among variants that have been requested.
std::vector<char> pinned_set(const bd_cache* c, double now) {
    const int nv = c->cfg.num_variants;
    std::vector<char> pin(nv, 0);
    if (c->cfg.pinned <= 0) return pin;
    std::vector<std::pair<double, int>> r;
    r.reserve(nv);
    for (int i = 0; i < nv; ++i)
        if (c->vars[i].seen) r.emplace_back(decayed(c->vars[i], c, now), i);
    const size_t k = std::min<size_t>((size_t)c->cfg.pinned, r.size());
    std::partial_sort(r.begin(), r.begin() + k, r.end(), [](const auto& a, const auto& b) {
        return a.first > b.first || (a.first == b.first && a.second < b.second);
    });
    for (size_t i = 0; i < k; ++i) pin[r[i].second] = 1;
    return pin;
}

bd_status note_hip(hipError_t e) {
    bd::note_hip_error(e);
    return BD_ERR_HIP;
}

// Device mode: loads whose event has fired become ready (no blocking).
bd_status poll_loads(bd_cache* c) {
    if (!device_mode(c)) return BD_OK;
    for (Slot& s : c->slots) {
        if (s.state != kLoading) continue;
        const hipError_t e = hipEventQuery(s.loaded);
        if (e == hipSuccess) s.state = kReady;
        else if (e != hipErrorNotReady) return note_hip(e);
    }
    return BD_OK;
}

// The state machine of one request (both modes).  On LOAD the slot is
// assigned and marked loading; the caller issues the load.
void decide(bd_cache* c, int v, double now, bd_cache_grant* g) {
    Variant& var = c->vars[v];
    var.rate = decayed(var, c, now) + 1.0;
    var.t = now;
    var.seen = true;
    var.last = ++c->tick;
    c->now = now;
    ++c->stats.requests;
    g->evicted = -1;
    if (var.slot >= 0) {
        Slot& s = c->slots[var.slot];
        ++s.refs;
        g->slot = var.slot;
        g->action = s.state == kReady ? BD_CACHE_HIT : BD_CACHE_JOIN;
        ++(g->action == BD_CACHE_HIT ? c->stats.hits : c->stats.joins);
        return;
    }
    // a free slot, else the least recently requested unpinned idle variant
    int slot = -1;
    for (int i = 0; i < (int)c->slots.size() && slot < 0; ++i)
        if (c->slots[i].var < 0) slot = i;
    if (slot < 0) {
        const std::vector<char> pin = pinned_set(c, now);
        uint64_t oldest = UINT64_MAX;
        for (int i = 0; i < (int)c->slots.size(); ++i) {
            const Slot& s = c->slots[i];
            if (s.refs > 0 || pin[s.var]) continue;
            if (c->vars[s.var].last < oldest) {
                oldest = c->vars[s.var].last;
                slot = i;
            }
        }
    }
    if (slot < 0) {
        g->action = BD_CACHE_BUSY;
        g->slot = -1;
        ++c->stats.busy;
        return;
    }
    Slot& s = c->slots[slot];
    if (s.var >= 0) {
        g->evicted = s.var;
        c->vars[s.var].slot = -1;
        ++c->stats.evictions;
    }
    s.var = v;
    s.state = kLoading;
    s.refs = 1;
    var.slot = slot;
    g->slot = slot;
    g->action = BD_CACHE_LOAD;
    ++c->stats.loads;
    c->stats.bytes_loaded += (int64_t)c->cfg.slot_bytes;
}

// Device mode: enqueue the load of the slot's variant after the releases of
// the slot's previous contents, then record its event.  The release events
// are recycled only once the copy and its event are enqueued: until then the
// slot keeps them, so a failed attempt leaves nothing half moved.
bd_status issue_load(bd_cache* c, int slot) {
    Slot& s = c->slots[slot];
    for (const UseEvent& u : s.uses) {
        hipError_t e = hipStreamWaitEvent(c->copy, u.event, 0);
        if (e != hipSuccess) return note_hip(e);
    }
    char* dst = c->base + (size_t)slot * c->cfg.slot_bytes;
    hipError_t e = hipMemcpyAsync(dst, c->vars[s.var].src, c->cfg.slot_bytes, hipMemcpyHostToDevice, c->copy);
    if (e != hipSuccess) return note_hip(e);
    e = hipEventRecord(s.loaded, c->copy);
    if (e != hipSuccess) return note_hip(e);
    // the copy stream now orders every later load of this slot after them
    for (const UseEvent& u : s.uses) c->spare.push_back(u.event);
    s.uses.clear();
    return BD_OK;
}

// A LOAD grant whose data will not arrive: the slot goes back to empty and
// the variant to not resident, and the slot's references are dropped (the
// load's own and, in policy mode, those of requests that joined it).  The
// variant evicted to make room stays evicted; the load leaves the counters.
void undo_load(bd_cache* c, int v) {
    Variant& var = c->vars[v];
    Slot& s = c->slots[var.slot];
    s.var = -1;
    s.state = kEmpty;
    s.refs = 0;
    var.slot = -1;
    --c->stats.loads;
    c->stats.bytes_loaded -= (int64_t)c->cfg.slot_bytes;
}

// Device mode: a granted request's stream waits for the slot's load (free
// once the load has been seen complete).
bd_status wait_for_slot(bd_cache* c, int slot, hipStream_t stream) {
    Slot& s = c->slots[slot];
    if (s.state == kReady) return BD_OK;
    const hipError_t e = hipStreamWaitEvent(stream, s.loaded, 0);
    return e == hipSuccess ? BD_OK : note_hip(e);
}

bool valid_variant(const bd_cache* c, int v) { return v >= 0 && v < c->cfg.num_variants; }

// A request time: finite and not before the previous request's.
bool valid_now(const bd_cache* c, double now) { return std::isfinite(now) && now >= c->now; }

}  // namespace

extern "C" {

bd_status bd_cache_create(const bd_cache_config* cfg, void* device_base, void* copy_stream,
                          bd_cache** out) {
    if (!cfg || !out) return BD_ERR_NULL;
    *out = nullptr;
    if (cfg->num_variants < 1 || cfg->num_variants > BD_CACHE_MAX_VARIANTS || cfg->num_slots < 1 ||
        cfg->num_slots > cfg->num_variants || cfg->pinned < 0 || cfg->pinned >= cfg->num_slots ||
        !(cfg->half_life > 0.0) || !std::isfinite(cfg->half_life) || cfg->slot_bytes == 0)
        return BD_ERR_SHAPE;
    if (device_base && (reinterpret_cast<uintptr_t>(device_base) & 15) != 0) return BD_ERR_ALIGN;
    bd_cache* c = new bd_cache;
    c->cfg = *cfg;
    c->base = static_cast<char*>(device_base);
    c->copy = static_cast<hipStream_t>(copy_stream);
    c->slots.resize(cfg->num_slots);
    c->vars.resize(cfg->num_variants);
    if (device_base) {
        for (Slot& s : c->slots) {
            const hipError_t e = hipEventCreateWithFlags(&s.loaded, hipEventDisableTiming);
            if (e != hipSuccess) {
                bd_cache_destroy(c);
                return note_hip(e);
            }
        }
    }
    *out = c;
    return BD_OK;
}

bd_status bd_cache_destroy(bd_cache* c) {
    if (!c) return BD_OK;
    bd_status st = BD_OK;
    for (Slot& s : c->slots) {
        if (s.loaded) {
            if (s.state == kLoading) {
                const hipError_t e = hipEventSynchronize(s.loaded);
                if (e != hipSuccess) st = note_hip(e);
            }
            (void)hipEventDestroy(s.loaded);
        }
        for (const UseEvent& u : s.uses) (void)hipEventDestroy(u.event);
    }
    for (hipEvent_t e : c->spare) (void)hipEventDestroy(e);
    delete c;
    return st;
}

bd_status bd_cache_set_source(bd_cache* c, int32_t v, const void* src) {
    if (!c || !src) return BD_ERR_NULL;
    if (!device_mode(c) || !valid_variant(c, v)) return BD_ERR_SHAPE;
    c->vars[v].src = src;
    return BD_OK;
}

bd_status bd_cache_request(bd_cache* c, int32_t v, double now, bd_cache_grant* g) {
    if (!c || !g) return BD_ERR_NULL;
    if (device_mode(c) || !valid_variant(c, v) || !valid_now(c, now)) return BD_ERR_SHAPE;
    decide(c, v, now, g);
    return BD_OK;
}

bd_status bd_cache_complete(bd_cache* c, int32_t v) {
    if (!c) return BD_ERR_NULL;
    if (device_mode(c) || !valid_variant(c, v) || c->vars[v].slot < 0) return BD_ERR_SHAPE;
    c->slots[c->vars[v].slot].state = kReady;
    return BD_OK;
}

bd_status bd_cache_load_failed(bd_cache* c, int32_t v) {
    if (!c) return BD_ERR_NULL;
    if (device_mode(c) || !valid_variant(c, v) || c->vars[v].slot < 0 ||
        c->slots[c->vars[v].slot].state != kLoading)
        return BD_ERR_SHAPE;
    undo_load(c, v);
    return BD_OK;
}

bd_status bd_cache_release(bd_cache* c, int32_t v, void* stream) {
    if (!c) return BD_ERR_NULL;
    if (!valid_variant(c, v) || c->vars[v].slot < 0) return BD_ERR_SHAPE;
    Slot& s = c->slots[c->vars[v].slot];
    if (s.refs <= 0) return BD_ERR_SHAPE;
    if (device_mode(c)) {
        hipStream_t st = static_cast<hipStream_t>(stream);
        // one event per stream: a later release on a stream covers earlier ones
        UseEvent* u = nullptr;
        for (UseEvent& e : s.uses)
            if (e.stream == st) u = &e;
        if (!u) {
            hipEvent_t ev;
            if (!c->spare.empty()) {
                ev = c->spare.back();
                c->spare.pop_back();
            } else {
                const hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
                if (e != hipSuccess) return note_hip(e);
            }
            s.uses.push_back({st, ev});
            u = &s.uses.back();
        }
        const hipError_t e = hipEventRecord(u->event, st);
        if (e != hipSuccess) return note_hip(e);
    }
    --s.refs;
    return BD_OK;
}

bd_status bd_cache_acquire(bd_cache* c, int32_t v, double now, void* stream, void** slot_ptr,
                           bd_cache_grant* g) {
    if (!c || !slot_ptr || !g) return BD_ERR_NULL;
    *slot_ptr = nullptr;
    if (!device_mode(c) || !valid_variant(c, v) || !valid_now(c, now)) return BD_ERR_SHAPE;
    // a variant that would have to be loaded needs a source
    if (c->vars[v].slot < 0 && !c->vars[v].src) return BD_ERR_NULL;
    bd_status st = poll_loads(c);
    if (st != BD_OK) return st;
    decide(c, v, now, g);
    if (g->action == BD_CACHE_BUSY) return BD_OK;
    if (g->action == BD_CACHE_LOAD) {
        st = issue_load(c, g->slot);
        if (st != BD_OK) {
            undo_load(c, v);  // the slot is not left claimed by a load that never started
            return st;
        }
    }
    st = wait_for_slot(c, g->slot, static_cast<hipStream_t>(stream));
    if (st != BD_OK) {
        --c->slots[g->slot].refs;  // not granted: the request holds no reference
        return st;
    }
    *slot_ptr = c->base + (size_t)g->slot * c->cfg.slot_bytes;
    return BD_OK;
}

bd_status bd_cache_acquire_batch(bd_cache* c, const int32_t* req, int32_t n, double now, void* stream,
                                 int32_t* local_ids, void** slot_ptrs, int32_t* variants_out,
                                 int32_t* num_distinct, int32_t* busy_variant) {
    if (!c || !num_distinct || !busy_variant || (n > 0 && (!req || !local_ids || !slot_ptrs || !variants_out)))
        return BD_ERR_NULL;
    *num_distinct = 0;
    *busy_variant = -1;
    if (n < 0 || !device_mode(c) || !valid_now(c, now)) return BD_ERR_SHAPE;
    for (int i = 0; i < n; ++i)
        if (!valid_variant(c, req[i])) return BD_ERR_SHAPE;
    // distinct variants in order of first appearance
    std::vector<int> local(c->cfg.num_variants, -1);
    int G = 0;
    for (int i = 0; i < n; ++i) {
        int& l = local[req[i]];
        if (l < 0) {
            l = G;
            variants_out[G++] = req[i];
        }
        local_ids[i] = l;
    }
    for (int g = 0; g < G; ++g) {
        bd_cache_grant gr;
        bd_status st = bd_cache_acquire(c, variants_out[g], now, stream, &slot_ptrs[g], &gr);
        if (st == BD_OK && gr.action == BD_CACHE_BUSY) {
            *busy_variant = variants_out[g];
            st = BD_OK;
        }
        if (st != BD_OK || *busy_variant >= 0) {
            for (int h = 0; h < g; ++h) {
                const bd_status r = bd_cache_release(c, variants_out[h], stream);
                if (r != BD_OK && st == BD_OK) st = r;
            }
            return st;
        }
    }
    *num_distinct = G;
    return BD_OK;
}

bd_status bd_cache_release_batch(bd_cache* c, const int32_t* variants, int32_t num_distinct, void* stream) {
    if (!c || (num_distinct > 0 && !variants)) return BD_ERR_NULL;
    if (num_distinct < 0) return BD_ERR_SHAPE;
    bd_status st = BD_OK;
    for (int g = 0; g < num_distinct; ++g) {
        const bd_status r = bd_cache_release(c, variants[g], stream);
        if (r != BD_OK && st == BD_OK) st = r;
    }
    return st;
}

bd_status bd_cache_query(bd_cache* c, int32_t v, int32_t* slot, int32_t* state, int32_t* refs) {
    if (!c || !slot || !state || !refs) return BD_ERR_NULL;
    if (!valid_variant(c, v)) return BD_ERR_SHAPE;
    const bd_status st = poll_loads(c);
    if (st != BD_OK) return st;
    const int s = c->vars[v].slot;
    *slot = s;
    *state = s < 0 ? -1 : (c->slots[s].state == kReady ? 1 : 0);
    *refs = s < 0 ? 0 : c->slots[s].refs;
    return BD_OK;
}

bd_status bd_cache_get_stats(const bd_cache* c, bd_cache_stats* out) {
    if (!c || !out) return BD_ERR_NULL;
    *out = c->stats;
    return BD_OK;
}

}  // extern "C"
