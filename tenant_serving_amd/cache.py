"""Python binding of the delta cache (include/bitdelta_cache.h), same names.

Argument marshalling only: the residency, eviction and load ordering run in
libbitdelta's C++ cache (bd_cache_*).  The delta cache of "BitDelta : servir
14 modèles Zen depuis un seul cluster GPU" (hanzo-blog, 2026-02-28),
"Infrastructure details": cold-start loads, LRU eviction with the busiest
variants pinned, and requests for a loading variant queued behind its one
load.
"""

from __future__ import annotations

import ctypes

import torch

from .bitdelta import _check, library

BD_CACHE_HIT, BD_CACHE_JOIN, BD_CACHE_LOAD, BD_CACHE_BUSY = 0, 1, 2, 3
ACTIONS = {0: "hit", 1: "join", 2: "load", 3: "busy"}


class CacheConfig(ctypes.Structure):
    _fields_ = [("num_variants", ctypes.c_int32), ("num_slots", ctypes.c_int32),
                ("pinned", ctypes.c_int32), ("half_life", ctypes.c_double),
                ("slot_bytes", ctypes.c_size_t)]


class CacheGrant(ctypes.Structure):
    _fields_ = [("action", ctypes.c_int32), ("slot", ctypes.c_int32), ("evicted", ctypes.c_int32)]


class CacheStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in
                ("requests", "hits", "joins", "loads", "busy", "evictions", "bytes_loaded")]


def declare(lib):
    p, i32, d = ctypes.c_void_p, ctypes.c_int32, ctypes.c_double
    P = ctypes.POINTER
    lib.bd_cache_create.argtypes = [P(CacheConfig), p, p, P(p)]
    lib.bd_cache_destroy.argtypes = [p]
    lib.bd_cache_set_source.argtypes = [p, i32, p]
    lib.bd_cache_request.argtypes = [p, i32, d, P(CacheGrant)]
    lib.bd_cache_complete.argtypes = [p, i32]
    lib.bd_cache_load_failed.argtypes = [p, i32]
    lib.bd_cache_release.argtypes = [p, i32, p]
    lib.bd_cache_acquire.argtypes = [p, i32, d, p, P(p), P(CacheGrant)]
    lib.bd_cache_acquire_batch.argtypes = [p, P(i32), i32, d, p, P(i32), P(p), P(i32), P(i32), P(i32)]
    lib.bd_cache_release_batch.argtypes = [p, P(i32), i32, p]
    lib.bd_cache_query.argtypes = [p, i32, P(i32), P(i32), P(i32)]
    lib.bd_cache_get_stats.argtypes = [p, P(CacheStats)]
    for n in ("create", "destroy", "set_source", "request", "complete", "release", "acquire",
              "acquire_batch", "release_batch", "query", "get_stats"):
        getattr(lib, "bd_cache_" + n).restype = ctypes.c_int
    return lib


class Busy(RuntimeError):
    """Every slot holds a pinned or in-use variant: `variant` cannot load now."""

    def __init__(self, variant):
        self.variant = variant
        super().__init__("delta cache busy: variant %d cannot be loaded now" % variant)


def _stream_handle(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return ctypes.c_void_p(stream.cuda_stream)


class bd_cache:
    """One delta cache.  With ``device_slots`` (a CUDA uint8 tensor of at least
    num_slots * slot_bytes bytes) it loads variants itself from pinned host
    tensors given to ``bd_cache_set_source`` on ``copy_stream``; without, it
    is the bare policy (``bd_cache_request`` / ``bd_cache_complete``)."""

    def __init__(self, num_variants, num_slots, pinned, half_life, slot_bytes,
                 device_slots: torch.Tensor | None = None, copy_stream=None):
        self.lib = declare(library())
        self.cfg = CacheConfig(num_variants, num_slots, pinned, float(half_life), int(slot_bytes))
        base = ctypes.c_void_p(0)
        cs = ctypes.c_void_p(0)
        if device_slots is not None:
            if device_slots.device.type != "cuda" or device_slots.dtype != torch.uint8:
                raise ValueError("device_slots must be a CUDA uint8 tensor")
            if device_slots.numel() < num_slots * slot_bytes or not device_slots.is_contiguous():
                raise ValueError("device_slots must hold num_slots * slot_bytes contiguous bytes")
            base = ctypes.c_void_p(device_slots.data_ptr())
            cs = _stream_handle(copy_stream) if copy_stream is not None else ctypes.c_void_p(0)
        self.device_slots = device_slots
        self.copy_stream = copy_stream
        self.sources = {}
        h = ctypes.c_void_p(0)
        _check(self.lib, "bd_cache_create", self.lib.bd_cache_create(ctypes.byref(self.cfg), base, cs,
                                                                     ctypes.byref(h)))
        self.handle = h

    def close(self):
        if self.handle:
            st = self.lib.bd_cache_destroy(self.handle)
            self.handle = ctypes.c_void_p(0)
            _check(self.lib, "bd_cache_destroy", st)

    def __del__(self):
        try:
            if getattr(self, "handle", None):
                self.lib.bd_cache_destroy(self.handle)
        except Exception:
            pass

    def bd_cache_set_source(self, variant: int, host: torch.Tensor):
        if host.device.type != "cpu" or not host.is_pinned() or not host.is_contiguous():
            raise ValueError("a variant's source must be a contiguous pinned host tensor")
        if host.numel() * host.element_size() < self.cfg.slot_bytes:
            raise ValueError("a variant's source must hold slot_bytes bytes")
        self.sources[variant] = host
        _check(self.lib, "bd_cache_set_source",
               self.lib.bd_cache_set_source(self.handle, variant, ctypes.c_void_p(host.data_ptr())))

    def bd_cache_request(self, variant: int, now: float):
        g = CacheGrant()
        _check(self.lib, "bd_cache_request", self.lib.bd_cache_request(self.handle, variant, now, ctypes.byref(g)))
        return ACTIONS[g.action], g.slot, g.evicted

    def bd_cache_complete(self, variant: int):
        _check(self.lib, "bd_cache_complete", self.lib.bd_cache_complete(self.handle, variant))

    def bd_cache_load_failed(self, variant: int):
        """Policy mode: the load of `variant` failed; its slot is freed and
        the requests that waited on it hold no reference any more."""
        _check(self.lib, "bd_cache_load_failed", self.lib.bd_cache_load_failed(self.handle, variant))

    def bd_cache_release(self, variant: int, stream=None):
        s = _stream_handle(stream) if self.device_slots is not None else ctypes.c_void_p(0)
        _check(self.lib, "bd_cache_release", self.lib.bd_cache_release(self.handle, variant, s))

    def bd_cache_acquire(self, variant: int, now: float, stream=None):
        """-> (slot view: uint8 tensor of slot_bytes on the device, or None when
        busy; action; slot; evicted variant)."""
        g = CacheGrant()
        ptr = ctypes.c_void_p(0)
        _check(self.lib, "bd_cache_acquire",
               self.lib.bd_cache_acquire(self.handle, variant, now, _stream_handle(stream),
                                         ctypes.byref(ptr), ctypes.byref(g)))
        return self.slot_view(g.slot), ACTIONS[g.action], g.slot, g.evicted

    def slot_view(self, slot: int):
        if slot < 0:
            return None
        b = self.cfg.slot_bytes
        return self.device_slots[slot * b:(slot + 1) * b]

    def bd_cache_acquire_batch(self, requests, now: float, stream=None):
        """Per-request variant ids -> (local ids [n], slot views per distinct
        variant, the distinct variants); raises Busy if one cannot load now."""
        n = len(requests)
        req = (ctypes.c_int32 * max(n, 1))(*requests)
        local = (ctypes.c_int32 * max(n, 1))()
        ptrs = (ctypes.c_void_p * max(n, 1))()
        var = (ctypes.c_int32 * max(n, 1))()
        G = ctypes.c_int32(0)
        busy = ctypes.c_int32(-1)
        _check(self.lib, "bd_cache_acquire_batch",
               self.lib.bd_cache_acquire_batch(self.handle, req, n, now, _stream_handle(stream), local, ptrs,
                                               var, ctypes.byref(G), ctypes.byref(busy)))
        if busy.value >= 0:
            raise Busy(busy.value)
        base = self.device_slots.data_ptr()
        b = self.cfg.slot_bytes
        views = [self.slot_view((ptrs[g] - base) // b) for g in range(G.value)]
        return list(local[:n]), views, list(var[:G.value])

    def bd_cache_release_batch(self, variants, stream=None):
        n = len(variants)
        arr = (ctypes.c_int32 * max(n, 1))(*variants)
        _check(self.lib, "bd_cache_release_batch",
               self.lib.bd_cache_release_batch(self.handle, arr, n, _stream_handle(stream)))

    def bd_cache_query(self, variant: int):
        """-> (slot or -1, state: -1 absent / 0 loading / 1 resident, refs)."""
        s, st, r = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check(self.lib, "bd_cache_query",
               self.lib.bd_cache_query(self.handle, variant, ctypes.byref(s), ctypes.byref(st), ctypes.byref(r)))
        return s.value, st.value, r.value

    def bd_cache_get_stats(self):
        out = CacheStats()
        _check(self.lib, "bd_cache_get_stats", self.lib.bd_cache_get_stats(self.handle, ctypes.byref(out)))
        return {n: getattr(out, n) for n, _ in CacheStats._fields_}
