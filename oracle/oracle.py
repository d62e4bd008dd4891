"""Python wrapper of the BitDelta CPU oracle -- TEST INFRASTRUCTURE ONLY.

Only the tests, the GPU smoke check and the benchmark's CPU-baseline leg may
import this module.  The product path never does.

The arithmetic lives in ``bitdelta_oracle.c`` (plain C, fp64 accumulation,
OpenMP over output rows); this file compiles it with gcc, loads it with
ctypes and converts numpy / torch-CPU arrays.  Definitions follow the post
"BitDelta : servir 14 modèles Zen depuis un seul cluster GPU" (hanzo-blog,
2026-02-28), sections "Mathematical foundation" (sign code, scale factor),
"Serving architecture" (reconstruction, conceptual fused linear, one base
shared by many variants) and "Infrastructure details" (packed storage, fp32
scale per output dimension).
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "bitdelta_oracle.c")
LIBRARY = os.path.join(HERE, "liboracle.so")

PER_MATRIX = 0
PER_ROW = 1

_lock = threading.Lock()
_lib = None

GCC_FLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
             "-std=c11", "-Wall", "-Wextra"]


def compile_library(source: str = SOURCE, output: str = LIBRARY, extra=()) -> str:
    """Compile the oracle (or a copy of its source) with gcc."""
    tmp = output + ".tmp%d" % os.getpid()
    cmd = ["gcc", *GCC_FLAGS, *extra, source, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(tmp, output)
    return output


def build(force: bool = True) -> str:
    if force or not os.path.exists(LIBRARY):
        compile_library()
    return LIBRARY


def _declare(lib):
    i64, i32, p = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    sig = {
        "orc_pack_signs": [p, i64, i64, p],
        "orc_delta_from_pair": [p, p, i64, p],
        "orc_unpack_signs": [p, i64, i64, p],
        "orc_alpha": [p, i64, i64, ctypes.c_int, p],
        "orc_bf16_rne_array": [p, i64, p],
        "orc_bf16_rne_f64_array": [p, i64, p],
        "orc_weff": [p, p, p, ctypes.c_int, i64, i64, p],
        "orc_linear": [p, p, p, p, ctypes.c_int, i64, i64, i64, p],
        "orc_linear_sampled": [p, p, p, p, ctypes.c_int, i64, i64, i64, p, p, i64, p],
        "orc_linear_grouped": [p, p, p, p, p, ctypes.c_int, i32, i64, i64, i64, p],
        "orc_linear_grouped_sampled": [p, p, p, p, p, ctypes.c_int, i32, i64, i64, i64, p, p,
                                       i64, p],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.orc_num_threads.argtypes = []
    lib.orc_num_threads.restype = ctypes.c_int
    lib.orc_bf16_rne.argtypes = [ctypes.c_uint32]
    lib.orc_bf16_rne.restype = ctypes.c_uint16
    lib.orc_bf16_rne_f64.argtypes = [ctypes.c_double]
    lib.orc_bf16_rne_f64.restype = ctypes.c_uint16
    return lib


def load(path: str | None = None):
    """Load the oracle library, compiling it first if it is not built."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            if not os.path.exists(LIBRARY):
                build(force=True)
            _lib = _declare(ctypes.CDLL(LIBRARY))
    return _lib


# ----------------------------------------------------------------------------
# array conversion helpers (accept numpy arrays or CPU torch tensors)

def _np(a):
    if hasattr(a, "detach"):
        t = a.detach()
        if t.device.type != "cpu":
            raise ValueError("oracle inputs must be host arrays")
        import torch
        if t.dtype == torch.bfloat16:
            return t.contiguous().view(torch.int16).numpy().view(np.uint16)
        return t.contiguous().numpy()
    return np.ascontiguousarray(a)


def _bf16(a):
    a = _np(a)
    if a.dtype != np.uint16:
        raise TypeError("expected bf16 bit patterns (uint16 or torch.bfloat16), got %s" % a.dtype)
    return np.ascontiguousarray(a)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise ValueError("oracle %s rejected its arguments (code %d)" % (what, rc))


def num_threads(lib=None) -> int:
    return int((lib or load()).orc_num_threads())


# ----------------------------------------------------------------------------
# the oracle's operations

def pack_signs(delta, lib=None):
    lib = lib or load()
    d = np.ascontiguousarray(_np(delta), dtype=np.float32)
    n, k = d.shape
    out = np.empty((n, k // 8), dtype=np.uint8)
    _check(lib.orc_pack_signs(_ptr(d), n, k, _ptr(out)), "pack_signs")
    return out


def unpack_signs(signs, d_in, lib=None):
    lib = lib or load()
    s = np.ascontiguousarray(_np(signs), dtype=np.uint8)
    n = s.shape[0]
    out = np.empty((n, d_in), dtype=np.float32)
    _check(lib.orc_unpack_signs(_ptr(s), n, d_in, _ptr(out)), "unpack_signs")
    return out


def alpha(delta, per_row: bool, lib=None):
    lib = lib or load()
    d = np.ascontiguousarray(_np(delta), dtype=np.float32)
    n, k = d.shape
    out = np.empty((n if per_row else 1,), dtype=np.float32)
    _check(lib.orc_alpha(_ptr(d), n, k, int(per_row), _ptr(out)), "alpha")
    return out


def compress(delta, per_row: bool, lib=None):
    """(packed signs uint8 [d_out, d_in/8], alpha fp32 [d_out] or [1])."""
    return pack_signs(delta, lib), alpha(delta, per_row, lib)


def delta_from_pair(w_ft, w_base, lib=None):
    """Δ = W_ft − W_base ("Mathematical foundation"), both bf16 widened to
    fp32 and subtracted in fp32; returns fp32 [d_out, d_in]."""
    lib = lib or load()
    ft, base = _bf16(w_ft), _bf16(w_base)
    if ft.shape != base.shape:
        raise ValueError("w_ft and w_base shapes differ")
    out = np.empty(ft.shape, dtype=np.float32)
    _check(lib.orc_delta_from_pair(_ptr(ft), _ptr(base), ft.size, _ptr(out)), "orc_delta_from_pair")
    return out


def compress_pair(w_ft, w_base, per_row: bool, lib=None):
    """Compression from a (fine-tuned, base) bf16 pair: the fp32 Δ of
    delta_from_pair, then signs and α as in compress()."""
    delta = delta_from_pair(w_ft, w_base, lib)
    return compress(delta, per_row, lib)


def bf16_rne(bits_u32, lib=None):
    lib = lib or load()
    a = np.ascontiguousarray(bits_u32, dtype=np.uint32)
    out = np.empty(a.shape, dtype=np.uint16)
    _check(lib.orc_bf16_rne_array(_ptr(a), a.size, _ptr(out)), "bf16_rne")
    return out


def bf16_rne_f64(values, lib=None):
    """fp64 values -> bf16 bit patterns (uint16), one rounding to nearest even."""
    lib = lib or load()
    a = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(a.shape, dtype=np.uint16)
    _check(lib.orc_bf16_rne_f64_array(_ptr(a), a.size, _ptr(out)), "bf16_rne_f64")
    return out


def weff(w_base, signs, alpha_, per_row: bool, lib=None):
    """Reconstructed bf16 weight as uint16 bit patterns [d_out, d_in]."""
    lib = lib or load()
    w = _bf16(w_base)
    s = np.ascontiguousarray(_np(signs), dtype=np.uint8)
    a = np.ascontiguousarray(_np(alpha_), dtype=np.float32)
    n, k = w.shape
    out = np.empty((n, k), dtype=np.uint16)
    _check(lib.orc_weff(_ptr(w), _ptr(s), _ptr(a), int(per_row), n, k, _ptr(out)), "weff")
    return out


def linear(x, w_base, signs, alpha_, per_row: bool, lib=None):
    """fp64 y [M, d_out]; x may carry leading dimensions [..., d_in]."""
    lib = lib or load()
    xa = _bf16(x)
    lead = xa.shape[:-1]
    xa = xa.reshape(-1, xa.shape[-1])
    w = _bf16(w_base)
    s = np.ascontiguousarray(_np(signs), dtype=np.uint8)
    a = np.ascontiguousarray(_np(alpha_), dtype=np.float32)
    m, k = xa.shape
    n = w.shape[0]
    if w.shape[1] != k:
        raise ValueError("d_in mismatch")
    y = np.empty((m, n), dtype=np.float64)
    _check(lib.orc_linear(_ptr(xa), _ptr(w), _ptr(s), _ptr(a), int(per_row), m, n, k, _ptr(y)),
           "linear")
    return y.reshape(*lead, n)


def linear_bf16(x, w_base, signs, alpha_, per_row: bool, lib=None):
    """The fused linear with a bf16 result, as the conceptual listing's
    F.linear on bf16 operands returns: the fp64 y of linear() rounded once to
    bf16 (bit patterns, uint16 [..., d_out])."""
    return bf16_rne_f64(linear(x, w_base, signs, alpha_, per_row, lib), lib)


def linear_sampled(x, w_base, signs, alpha_, per_row: bool, ms, ns, lib=None):
    lib = lib or load()
    xa = _bf16(x)
    w = _bf16(w_base)
    s = np.ascontiguousarray(_np(signs), dtype=np.uint8)
    a = np.ascontiguousarray(_np(alpha_), dtype=np.float32)
    mi = np.ascontiguousarray(ms, dtype=np.int64)
    ni = np.ascontiguousarray(ns, dtype=np.int64)
    out = np.empty(mi.shape, dtype=np.float64)
    m, k = xa.shape
    _check(lib.orc_linear_sampled(_ptr(xa), _ptr(w), _ptr(s), _ptr(a), int(per_row), m,
                                  w.shape[0], k, _ptr(mi), _ptr(ni), mi.size, _ptr(out)),
           "linear_sampled")
    return out


def _ptr_arrays(signs_list, alpha_list):
    s = [np.ascontiguousarray(_np(v), dtype=np.uint8) for v in signs_list]
    a = [np.ascontiguousarray(_np(v), dtype=np.float32) for v in alpha_list]
    sp = (ctypes.c_void_p * len(s))(*[v.ctypes.data for v in s])
    ap = (ctypes.c_void_p * len(a))(*[v.ctypes.data for v in a])
    return s, a, sp, ap


def linear_grouped(x, ids, w_base, signs_list, alpha_list, per_row: bool, lib=None):
    lib = lib or load()
    xa = _bf16(x)
    w = _bf16(w_base)
    ia = np.ascontiguousarray(_np(ids), dtype=np.int32)
    keep_s, keep_a, sp, ap = _ptr_arrays(signs_list, alpha_list)
    m, k = xa.shape
    n = w.shape[0]
    y = np.empty((m, n), dtype=np.float64)
    _check(lib.orc_linear_grouped(_ptr(xa), _ptr(ia), _ptr(w), sp, ap, int(per_row),
                                  len(keep_s), m, n, k, _ptr(y)), "linear_grouped")
    return y


def linear_grouped_sampled(x, ids, w_base, signs_list, alpha_list, per_row: bool, ms, ns,
                           lib=None):
    lib = lib or load()
    xa = _bf16(x)
    w = _bf16(w_base)
    ia = np.ascontiguousarray(_np(ids), dtype=np.int32)
    keep_s, keep_a, sp, ap = _ptr_arrays(signs_list, alpha_list)
    mi = np.ascontiguousarray(ms, dtype=np.int64)
    ni = np.ascontiguousarray(ns, dtype=np.int64)
    out = np.empty(mi.shape, dtype=np.float64)
    m, k = xa.shape
    _check(lib.orc_linear_grouped_sampled(_ptr(xa), _ptr(ia), _ptr(w), sp, ap, int(per_row),
                                          len(keep_s), m, w.shape[0], k, _ptr(mi), _ptr(ni),
                                          mi.size, _ptr(out)), "linear_grouped_sampled")
    return out
