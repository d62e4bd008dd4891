/*
 * bitdelta_cache.h -- the delta cache of libbitdelta.so: which variants'
 * (packed signs, α) sets are resident in HBM, loading them on demand and
 * evicting the least recently used unpinned one.
 *
 * Source: "BitDelta : servir 14 modèles Zen depuis un seul cluster GPU"
 * (hanzo-blog, 2026-02-28), section "Infrastructure details":
 *   - cold start: a variant whose delta is not cached pays one delta load
 *     (about 200 ms for a 70B variant's 8.75 GB) on its first request, and
 *     then stays cached until evicted;
 *   - eviction: LRU weighted by request rate; the variants with the most
 *     traffic are pinned (in practice the top 6 are always resident) and the
 *     others share the rest of the cache under LRU;
 *   - routing: requests in flight are tracked per variant, and requests for
 *     a variant whose delta is loading queue behind that one load instead of
 *     each starting its own.
 * Section "Serving architecture": one shared base, a delta cache with one
 * (α, sign(Δ)) entry per variant, and a router in front of it.
 *
 * Reading of "weighted by request rate" (the post gives no formula): each
 * variant keeps an exponentially decayed request count, r <- r·2^(-dt/H) + 1
 * per request (H the half-life, in the caller's time unit).  At an eviction,
 * the `pinned` variants with the highest decayed rates at that moment (ties:
 * the lower variant index) are not candidates; among the others that are
 * resident and not in use, the least recently requested one is evicted.
 *
 * Model of the cache
 * ------------------
 * The cache has `num_slots` equal slots of `slot_bytes`, each holding one
 * variant's whole delta set (the caller decides its layout, e.g. all layers'
 * sign planes and α of that variant).  A request for variant v:
 *   HIT   v is resident and its load has completed;
 *   JOIN  v's load is still in flight: the request waits for that load;
 *   LOAD  v was not resident: a slot (free, else the victim's) is assigned
 *         and a load of v into it starts;
 *   BUSY  v is not resident and every slot holds a pinned or in-use variant:
 *         nothing changes (apart from v's request rate); retry later.
 * A granted request holds a reference on the slot until it is released; a
 * slot with references is never evicted.
 *
 * Two modes share this state machine:
 *   - device mode (bd_cache_create with a device base): the cache issues the
 *     loads itself, as copies from pinned host memory (the caller's stand-in
 *     for NVMe) on a copy stream, and orders them with HIP events: a
 *     requester's stream waits for the slot's load, and a load into an
 *     evicted slot waits for the work that released the previous variant;
 *     no call blocks the host.
 *   - policy mode (device base NULL): no HIP calls at all; the caller moves
 *     the data and reports a load's completion with bd_cache_complete.
 *
 * Conventions: as in bitdelta.h.  Pointers marked DEVICE are HIP device
 * memory of the current device; streams are hipStream_t as void*.  The
 * cache allocates host memory and HIP events only, never device memory.
 * A cache object is not thread safe: one thread (a router) drives it.
 * `now` must be finite and must not decrease from one request to the next;
 * a request that breaks this is refused with BD_ERR_SHAPE and changes
 * nothing.  A request that fails with BD_ERR_HIP in bd_cache_acquire holds
 * no reference, and a load it could not enqueue leaves its slot empty and
 * the variant not resident (the variant evicted for it stays evicted); the
 * cache stays usable.
 */
#ifndef BITDELTA_CACHE_H
#define BITDELTA_CACHE_H

#include <stddef.h>
#include <stdint.h>

#include "bitdelta.h"

#ifdef __cplusplus
extern "C" {
#endif

#define BD_CACHE_MAX_VARIANTS 1024

typedef struct bd_cache bd_cache;

typedef enum bd_cache_action {
    BD_CACHE_HIT = 0,
    BD_CACHE_JOIN = 1,
    BD_CACHE_LOAD = 2,
    BD_CACHE_BUSY = 3
} bd_cache_action;

typedef struct bd_cache_config {
    int32_t num_variants; /* variants 0 .. num_variants-1, 1 .. BD_CACHE_MAX_VARIANTS */
    int32_t num_slots;    /* resident delta sets, 1 .. num_variants                    */
    int32_t pinned;       /* top variants by request rate never evicted, 0 .. slots-1  */
    double half_life;     /* request-rate decay half-life (> 0), caller's time unit   */
    size_t slot_bytes;    /* bytes of one variant's delta set (> 0)                    */
} bd_cache_config;

typedef struct bd_cache_grant {
    int32_t action;       /* bd_cache_action                                          */
    int32_t slot;         /* slot of the variant (-1 when BUSY)                       */
    int32_t evicted;      /* variant evicted to make room (-1 if none)                */
} bd_cache_grant;

typedef struct bd_cache_stats {
    int64_t requests, hits, joins, loads, busy, evictions;
    int64_t bytes_loaded;
} bd_cache_stats;

/* Create a cache.  device_base: DEVICE memory of num_slots * slot_bytes
 * bytes (slot i at device_base + i * slot_bytes, 16-byte aligned), owned by
 * the caller and alive as long as the cache; NULL selects policy mode.
 * copy_stream: the stream loads run on (device mode; NULL = default stream).
 * Errors: BD_ERR_NULL (cfg or out NULL), BD_ERR_SHAPE (a config field out of
 * range), BD_ERR_ALIGN (device_base not 16-byte aligned), BD_ERR_HIP. */
bd_status bd_cache_create(const bd_cache_config* cfg, void* device_base, void* copy_stream,
                          bd_cache** out);
/* Destroy: waits for the cache's own loads to finish (device mode), then
 * frees its host state and events.  NULL is a no-op. */
bd_status bd_cache_destroy(bd_cache* cache);

/* Device mode: where variant v's delta set is loaded from, a HOST pointer to
 * slot_bytes bytes of pinned host memory (hipHostMalloc or a pinned torch
 * tensor), owned by the caller, read by every later load of v.
 * Errors: BD_ERR_NULL, BD_ERR_SHAPE (v out of range, or policy mode). */
bd_status bd_cache_set_source(bd_cache* cache, int32_t variant, const void* host_src);

/* Policy mode: one request for v at time `now` (non-decreasing across
 * calls).  Fills *grant; on HIT, JOIN and LOAD the request holds a reference
 * until bd_cache_release.  After a LOAD the caller moves the data into the
 * slot and calls bd_cache_complete (a JOIN is the caller's cue to wait for
 * that same load).  Returns BD_OK for every action, BUSY included;
 * BD_ERR_SHAPE for v out of range, a `now` before the previous request's
 * (or not finite), or device mode. */
bd_status bd_cache_request(bd_cache* cache, int32_t variant, double now, bd_cache_grant* grant);
/* Policy mode: v's load has completed (later requests are HITs). */
bd_status bd_cache_complete(bd_cache* cache, int32_t variant);
/* Policy mode: v's load (a LOAD grant not yet completed) failed.  The slot
 * becomes empty, v is not resident, and every reference on the slot is
 * dropped: the request that got LOAD and those that JOINed it are all
 * failed and must not be released (each may request v again).  The variant
 * evicted for the load stays evicted; stats no longer count the load.
 * Errors: BD_ERR_SHAPE (v out of range, not loading, or device mode). */
bd_status bd_cache_load_failed(bd_cache* cache, int32_t variant);
/* Either mode: drop one reference of v (device mode: after the work that
 * reads the slot has been enqueued on `stream`, which the next load into
 * the slot will wait for; policy mode: `stream` is ignored).
 * Errors: BD_ERR_SHAPE (v out of range, not resident, or no reference). */
bd_status bd_cache_release(bd_cache* cache, int32_t variant, void* stream);

/* Device mode: one request for v at `now`; on HIT, JOIN and LOAD sets
 * *slot_ptr to the slot's DEVICE address and makes `stream` wait for the
 * slot's load (LOAD first enqueues that load, after the releases of the
 * evicted variant).  *grant as above; on BUSY *slot_ptr is NULL.
 * Errors: BD_ERR_NULL (no source set for a variant that must be loaded,
 * or a NULL output), BD_ERR_SHAPE (v out of range, `now` as for
 * bd_cache_request, or policy mode), BD_ERR_HIP. */
bd_status bd_cache_acquire(bd_cache* cache, int32_t variant, double now, void* stream,
                           void** slot_ptr, bd_cache_grant* grant);

/* Device mode, the router's batch: requests[i] (HOST int32, n of them) are
 * variant ids.  Each distinct variant is acquired once, in order of first
 * appearance; local_ids[i] (HOST int32 [n]) gets the index of requests[i]'s
 * variant in that order, slot_ptrs[g] (HOST array of >= n pointers) its
 * slot's DEVICE address, variants_out[g] (HOST int32, >= n) the variant,
 * and *num_distinct the count -- the arguments bd_linear_grouped takes,
 * once the caller adds its layout's offsets.  If some variant is BUSY, the
 * batch's other acquisitions are released again, *num_distinct is 0,
 * *busy_variant names it and BD_OK is returned; otherwise *busy_variant is
 * -1.  Release with bd_cache_release_batch.
 * Errors: as bd_cache_acquire, plus BD_ERR_SHAPE for n < 0. */
bd_status bd_cache_acquire_batch(bd_cache* cache, const int32_t* requests, int32_t n, double now,
                                 void* stream, int32_t* local_ids, void** slot_ptrs,
                                 int32_t* variants_out, int32_t* num_distinct,
                                 int32_t* busy_variant);
/* Release every variant of a batch (variants[0 .. num_distinct-1]) on
 * `stream`. */
bd_status bd_cache_release_batch(bd_cache* cache, const int32_t* variants, int32_t num_distinct,
                                 void* stream);

/* State of variant v: *slot = its slot or -1; *state = -1 not resident,
 * 0 loading, 1 resident; *refs = references held.  Device mode first
 * notes loads that have completed (without blocking). */
bd_status bd_cache_query(bd_cache* cache, int32_t variant, int32_t* slot, int32_t* state,
                         int32_t* refs);
/* Counters since creation. */
bd_status bd_cache_get_stats(const bd_cache* cache, bd_cache_stats* out);

#ifdef __cplusplus
}
#endif

#endif /* BITDELTA_CACHE_H */
