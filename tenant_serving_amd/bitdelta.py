"""Python binding of libbitdelta (ctypes), same names as the C ABI.

Argument marshalling only: shape/dtype/device checks, output and workspace
allocation with torch, and the current HIP stream.  Every step of the
computation runs in the library's HIP kernels; there is no fallback.  If the
library is not built, or the tensors are not on a gfx950 GPU, calls raise.

The operations are those of "BitDelta : servir 14 modèles Zen depuis un seul
cluster GPU" (hanzo-blog, 2026-02-28): compression of a fine-tuning delta to
packed signs and α ("Mathematical foundation", "Infrastructure details"), the
fused reconstruct-and-multiply linear ("Serving architecture", conceptual
fused_bitdelta_linear listing), and one batch mixing several variants over
one shared base ("Serving architecture" diagram).
"""

from __future__ import annotations

import ctypes
import os
import threading

import torch

LIBRARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbitdelta.so")

BD_ALPHA_PER_MATRIX = 0
BD_ALPHA_PER_ROW = 1
BD_MAX_VARIANTS = 64
BD_NOALLOC_SCRATCH_BYTES = 64 << 20
ABI_VERSION = 4

_EXPORTS = (
    "bd_abi_version", "bd_status_string", "bd_last_hip_error",
    "bd_compress_workspace_bytes", "bd_compress", "bd_compress_pair",
    "bd_linear_workspace_bytes", "bd_linear_path", "bd_linear", "bd_linear_bf16",
    "bd_linear_grouped_workspace_bytes", "bd_linear_grouped",
    "bd_linear_grouped_plan_bytes", "bd_linear_grouped_plan", "bd_linear_grouped_planned",
    "bd_linear_grouped_noalloc",
)

_lock = threading.Lock()
_lib = None


class BitDeltaError(RuntimeError):
    """A libbitdelta call returned a non-OK status."""

    def __init__(self, func, status, message, hip_error=0):
        self.status = status
        self.hip_error = hip_error
        extra = " (hipError %d)" % hip_error if status == 6 else ""
        super().__init__("%s failed: status %d: %s%s" % (func, status, message, extra))


def _declare(lib):
    i64, i32, p, sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
    lib.bd_abi_version.argtypes = []
    lib.bd_abi_version.restype = i32
    lib.bd_status_string.argtypes = [ctypes.c_int]
    lib.bd_status_string.restype = ctypes.c_char_p
    lib.bd_last_hip_error.argtypes = []
    lib.bd_last_hip_error.restype = i32
    lib.bd_compress_workspace_bytes.argtypes = [i64, i64, i32]
    lib.bd_compress_workspace_bytes.restype = sz
    lib.bd_compress.argtypes = [p, i64, i64, i32, p, p, p, sz, p]
    lib.bd_compress.restype = ctypes.c_int
    lib.bd_compress_pair.argtypes = [p, p, i64, i64, i32, p, p, p, sz, p]
    lib.bd_compress_pair.restype = ctypes.c_int
    lib.bd_linear_workspace_bytes.argtypes = [i64, i64, i64]
    lib.bd_linear_workspace_bytes.restype = sz
    lib.bd_linear_path.argtypes = [i64, i64, i64]
    lib.bd_linear_path.restype = ctypes.c_char_p
    lib.bd_linear.argtypes = [p, p, p, p, i32, p, i64, i64, i64, p, sz, p]
    lib.bd_linear.restype = ctypes.c_int
    lib.bd_linear_bf16.argtypes = [p, p, p, p, i32, p, i64, i64, i64, p, sz, p]
    lib.bd_linear_bf16.restype = ctypes.c_int
    lib.bd_linear_grouped_workspace_bytes.argtypes = [i64, i64, i64, i32]
    lib.bd_linear_grouped_workspace_bytes.restype = sz
    lib.bd_linear_grouped.argtypes = [p, p, p, p, p, i32, i32, p, i64, i64, i64, p, sz, p]
    lib.bd_linear_grouped.restype = ctypes.c_int
    lib.bd_linear_grouped_plan_bytes.argtypes = [i64, i32]
    lib.bd_linear_grouped_plan_bytes.restype = sz
    lib.bd_linear_grouped_plan.argtypes = [p, i64, i32, p, sz, p]
    lib.bd_linear_grouped_plan.restype = ctypes.c_int
    lib.bd_linear_grouped_planned.argtypes = [p, p, p, p, p, i32, i32, p, i64, i64, i64, p, sz, p]
    lib.bd_linear_grouped_planned.restype = ctypes.c_int
    lib.bd_linear_grouped_noalloc.argtypes = [p, p, p, p, p, i32, i32, p, i64, i64, i64, p]
    lib.bd_linear_grouped_noalloc.restype = ctypes.c_int
    return lib


def library(path: str | None = None):
    """Load libbitdelta.so (raises if it has not been built)."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            if not os.path.exists(LIBRARY):
                raise ImportError("libbitdelta.so is not built (run __graft_entry__.build() or "
                                  "python tenant_serving_amd/build.py): " + LIBRARY)
            lib = _declare(ctypes.CDLL(LIBRARY))
            if lib.bd_abi_version() != ABI_VERSION:
                raise ImportError("libbitdelta ABI version %d, binding expects %d"
                                  % (lib.bd_abi_version(), ABI_VERSION))
            _lib = lib
    return _lib


def _check(lib, func, status):
    if status != 0:
        msg = lib.bd_status_string(status).decode()
        raise BitDeltaError(func, status, msg, lib.bd_last_hip_error())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _require(name, t, dtype):
    """Type, dtype and contiguity (any device)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s (got %s)" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _on_gpu(device, **tensors):
    """Every tensor on the same GPU; there is no CPU path."""
    if device.type != "cuda":
        raise ValueError("tensors must be on a GPU (got %s); there is no CPU path" % device)
    for name, t in tensors.items():
        if t.device != device:
            raise ValueError("%s is on %s, expected %s" % (name, t.device, device))


def _require_gpu(name, t, dtype):
    _require(name, t, dtype)
    _on_gpu(t.device, **{name: t})


def _mode(alpha: torch.Tensor, d_out: int, mode):
    """The α mode: explicit, or inferred from alpha's size; alpha must hold
    exactly the elements the mode reads (d_out per row, 1 per matrix)."""
    if mode is None:
        if alpha.numel() == d_out:
            return BD_ALPHA_PER_ROW
        if alpha.numel() == 1:
            return BD_ALPHA_PER_MATRIX
        raise ValueError("alpha must have 1 or d_out=%d elements (got %d)" % (d_out, alpha.numel()))
    mode = int(mode)
    if mode == BD_ALPHA_PER_ROW and alpha.numel() != d_out:
        raise ValueError("per-row alpha must have d_out=%d elements (got %d)" % (d_out, alpha.numel()))
    if mode == BD_ALPHA_PER_MATRIX and alpha.numel() != 1:
        raise ValueError("per-matrix alpha must have 1 element (got %d)" % alpha.numel())
    return mode  # other values: the library answers BD_ERR_MODE


def _workspace(nbytes: int, device):
    if nbytes == 0:
        return None
    return torch.empty((nbytes + 7) // 8, dtype=torch.float64, device=device)


def bd_compress(delta: torch.Tensor, mode: int = BD_ALPHA_PER_ROW):
    """Δ [d_out, d_in] fp32 -> (signs uint8 [d_out, d_in/8], alpha fp32 [d_out] or [1])."""
    lib = library()
    _require_gpu("delta", delta, torch.float32)
    if delta.dim() != 2:
        raise ValueError("delta must be 2-D [d_out, d_in]")
    d_out, d_in = delta.shape
    signs = torch.empty((d_out, max(d_in // 8, 0)), dtype=torch.uint8, device=delta.device)
    alpha = torch.empty((d_out if mode == BD_ALPHA_PER_ROW else 1,), dtype=torch.float32,
                        device=delta.device)
    nbytes = lib.bd_compress_workspace_bytes(d_out, d_in, int(mode))
    ws = _workspace(nbytes, delta.device)
    st = lib.bd_compress(_ptr(delta), d_out, d_in, int(mode), _ptr(signs), _ptr(alpha), _ptr(ws),
                         nbytes, _stream(delta))
    _check(lib, "bd_compress", st)
    return signs, alpha


def bd_compress_pair(w_ft: torch.Tensor, w_base: torch.Tensor, mode: int = BD_ALPHA_PER_ROW):
    """(W_ft, W_base) bf16 [d_out, d_in] -> (signs uint8 [d_out, d_in/8], alpha fp32 [d_out] or [1]),
    with Δ = W_ft − W_base formed on the device and never stored."""
    lib = library()
    _require_gpu("w_ft", w_ft, torch.bfloat16)
    _require_gpu("w_base", w_base, torch.bfloat16)
    if w_ft.dim() != 2 or w_ft.shape != w_base.shape:
        raise ValueError("w_ft and w_base must be 2-D [d_out, d_in] of the same shape")
    if w_ft.device != w_base.device:
        raise ValueError("w_ft and w_base are on different devices")
    d_out, d_in = w_ft.shape
    signs = torch.empty((d_out, max(d_in // 8, 0)), dtype=torch.uint8, device=w_ft.device)
    alpha = torch.empty((d_out if mode == BD_ALPHA_PER_ROW else 1,), dtype=torch.float32,
                        device=w_ft.device)
    nbytes = lib.bd_compress_workspace_bytes(d_out, d_in, int(mode))
    ws = _workspace(nbytes, w_ft.device)
    st = lib.bd_compress_pair(_ptr(w_ft), _ptr(w_base), d_out, d_in, int(mode), _ptr(signs),
                              _ptr(alpha), _ptr(ws), nbytes, _stream(w_ft))
    _check(lib, "bd_compress_pair", st)
    return signs, alpha


def bd_linear_path(M: int, d_out: int, d_in: int) -> str:
    """Name of the kernel instance bd_linear uses for this shape."""
    return library().bd_linear_path(int(M), int(d_out), int(d_in)).decode()


def _linear(func, out_dtype, x, w_base, signs, alpha, mode, out):
    lib = library()
    _require("x", x, torch.bfloat16)
    _require("w_base", w_base, torch.bfloat16)
    _require("signs", signs, torch.uint8)
    _require("alpha", alpha, torch.float32)
    if w_base.dim() != 2:
        raise ValueError("w_base must be 2-D [d_out, d_in]")
    d_out, d_in = w_base.shape
    if x.dim() < 1 or x.shape[-1] != d_in:
        raise ValueError("x's last dim must be d_in=%d (got shape %s)" % (d_in, tuple(x.shape)))
    if tuple(signs.shape) != (d_out, d_in // 8):
        raise ValueError("signs must be [d_out, d_in/8] = [%d, %d]" % (d_out, d_in // 8))
    m = _mode(alpha, d_out, mode)
    lead = x.shape[:-1]
    M = 1
    for s in lead:
        M *= int(s)
    if out is not None:
        _require("out", out, out_dtype)
        if tuple(out.shape) != (*lead, d_out):
            raise ValueError("out must have shape %s (got %s)" % ((*lead, d_out), tuple(out.shape)))
        _on_gpu(x.device, w_base=w_base, signs=signs, alpha=alpha, out=out)
    else:
        _on_gpu(x.device, w_base=w_base, signs=signs, alpha=alpha)
        out = torch.empty((*lead, d_out), dtype=out_dtype, device=x.device)
    nbytes = lib.bd_linear_workspace_bytes(M, d_out, d_in)
    ws = _workspace(nbytes, x.device)
    st = getattr(lib, func)(_ptr(x), _ptr(w_base), _ptr(signs), _ptr(alpha), m, _ptr(out), M, d_out,
                            d_in, _ptr(ws), nbytes, _stream(x))
    _check(lib, func, st)
    return out


def bd_linear(x: torch.Tensor, w_base: torch.Tensor, signs: torch.Tensor, alpha: torch.Tensor,
              mode: int | None = None, out: torch.Tensor | None = None):
    """y = x · (W_base + α·sign(Δ))ᵀ in fp32; x is bf16 [..., d_in], y [..., d_out]."""
    return _linear("bd_linear", torch.float32, x, w_base, signs, alpha, mode, out)


def bd_linear_bf16(x: torch.Tensor, w_base: torch.Tensor, signs: torch.Tensor, alpha: torch.Tensor,
                   mode: int | None = None, out: torch.Tensor | None = None):
    """bd_linear with a bf16 result (each fp32 result rounded to nearest even),
    as the listing's F.linear on bf16 operands returns; y is bf16 [..., d_out]."""
    return _linear("bd_linear_bf16", torch.bfloat16, x, w_base, signs, alpha, mode, out)


def bd_linear_grouped_plan(variant_ids: torch.Tensor, num_variants: int, workspace: torch.Tensor):
    """Bucket the batch's tokens by variant once into `workspace` (a CUDA
    tensor big enough for every grouped call that will use the plan, e.g.
    bd_linear_grouped_workspace_bytes of the largest one); later calls pass
    plan=workspace and skip the bucketing."""
    lib = library()
    _require_gpu("variant_ids", variant_ids, torch.int32)
    if workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous CUDA tensor")
    nbytes = workspace.numel() * workspace.element_size()
    st = lib.bd_linear_grouped_plan(_ptr(variant_ids), variant_ids.numel(), int(num_variants),
                                    _ptr(workspace), nbytes, _stream(variant_ids))
    _check(lib, "bd_linear_grouped_plan", st)
    return workspace


def bd_linear_grouped(x: torch.Tensor, variant_ids: torch.Tensor, w_base: torch.Tensor,
                      signs_list, alpha_list, mode: int | None = None,
                      out: torch.Tensor | None = None, plan: torch.Tensor | None = None):
    """y[m] = x[m] · W_eff(variant_ids[m])ᵀ for a batch mixing variants over one base.
    With plan (the workspace of bd_linear_grouped_plan for these ids), the
    call uses that bucketing instead of doing its own."""
    lib = library()
    _require("x", x, torch.bfloat16)
    _require("variant_ids", variant_ids, torch.int32)
    _require("w_base", w_base, torch.bfloat16)
    if x.dim() != 2 or w_base.dim() != 2:
        raise ValueError("x must be 2-D [M, d_in] and w_base 2-D [d_out, d_in]")
    d_out, d_in = w_base.shape
    M = x.shape[0]
    if x.shape[1] != d_in or tuple(variant_ids.shape) != (M,):
        raise ValueError("shape mismatch between x, variant_ids and w_base")
    G = len(signs_list)
    if G != len(alpha_list) or not 1 <= G <= BD_MAX_VARIANTS:
        raise ValueError("need 1..%d variants with one alpha each" % BD_MAX_VARIANTS)
    for s in signs_list:
        _require("signs", s, torch.uint8)
        if tuple(s.shape) != (d_out, d_in // 8):
            raise ValueError("every signs tensor must be [d_out, d_in/8] = [%d, %d]" % (d_out, d_in // 8))
    for a in alpha_list:
        _require("alpha", a, torch.float32)
    # one mode for all variants; every alpha must hold what that mode reads
    m = _mode(alpha_list[0], d_out, mode)
    for a in alpha_list[1:]:
        _mode(a, d_out, m)
    if out is not None:
        _require("out", out, torch.float32)
        if tuple(out.shape) != (M, d_out):
            raise ValueError("out must have shape %s (got %s)" % ((M, d_out), tuple(out.shape)))
    if plan is not None and not plan.is_contiguous():
        raise ValueError("plan must be a contiguous tensor")
    extra = {"out": out} if out is not None else {}
    if plan is not None:
        extra["plan"] = plan
    _on_gpu(x.device, variant_ids=variant_ids, w_base=w_base,
            **{"signs[%d]" % i: t for i, t in enumerate(signs_list)},
            **{"alpha[%d]" % i: t for i, t in enumerate(alpha_list)}, **extra)
    if out is None:
        out = torch.empty((M, d_out), dtype=torch.float32, device=x.device)
    sp = (ctypes.c_void_p * G)(*[s.data_ptr() for s in signs_list])
    ap = (ctypes.c_void_p * G)(*[a.data_ptr() for a in alpha_list])
    if plan is None:
        nbytes = lib.bd_linear_grouped_workspace_bytes(M, d_out, d_in, G)
        ws = _workspace(nbytes, x.device)
        st = lib.bd_linear_grouped(_ptr(x), _ptr(variant_ids), _ptr(w_base), sp, ap, m, G, _ptr(out),
                                   M, d_out, d_in, _ptr(ws), nbytes, _stream(x))
        _check(lib, "bd_linear_grouped", st)
    else:
        nbytes = plan.numel() * plan.element_size()
        st = lib.bd_linear_grouped_planned(_ptr(x), _ptr(variant_ids), _ptr(w_base), sp, ap, m, G,
                                           _ptr(out), M, d_out, d_in, _ptr(plan), nbytes, _stream(x))
        _check(lib, "bd_linear_grouped_planned", st)
    return out


def bd_linear_grouped_noalloc(x: torch.Tensor, variant_ids: torch.Tensor, w_base: torch.Tensor,
                              signs_list, alpha_list, out: torch.Tensor, mode: int | None = None):
    """bd_linear_grouped for callers that cannot allocate: the library's own
    fixed per-GPU scratch is the workspace, and `out` (fp32 [M, d_out]) must
    be given.  Shapes whose workspace exceeds BD_NOALLOC_SCRATCH_BYTES are
    refused; calls that overlap on one GPU race on the scratch."""
    lib = library()
    if out is None:
        raise ValueError("out is required: this call allocates nothing")
    _require("x", x, torch.bfloat16)
    _require("variant_ids", variant_ids, torch.int32)
    _require("w_base", w_base, torch.bfloat16)
    if x.dim() != 2 or w_base.dim() != 2:
        raise ValueError("x must be 2-D [M, d_in] and w_base 2-D [d_out, d_in]")
    d_out, d_in = w_base.shape
    M = x.shape[0]
    if x.shape[1] != d_in or tuple(variant_ids.shape) != (M,):
        raise ValueError("shape mismatch between x, variant_ids and w_base")
    G = len(signs_list)
    if G != len(alpha_list) or not 1 <= G <= BD_MAX_VARIANTS:
        raise ValueError("need 1..%d variants with one alpha each" % BD_MAX_VARIANTS)
    for s in signs_list:
        _require("signs", s, torch.uint8)
        if tuple(s.shape) != (d_out, d_in // 8):
            raise ValueError("every signs tensor must be [d_out, d_in/8] = [%d, %d]" % (d_out, d_in // 8))
    for a in alpha_list:
        _require("alpha", a, torch.float32)
    m = _mode(alpha_list[0], d_out, mode)
    for a in alpha_list[1:]:
        _mode(a, d_out, m)
    _require("out", out, torch.float32)
    if tuple(out.shape) != (M, d_out):
        raise ValueError("out must have shape %s (got %s)" % ((M, d_out), tuple(out.shape)))
    _on_gpu(x.device, variant_ids=variant_ids, w_base=w_base, out=out,
            **{"signs[%d]" % i: t for i, t in enumerate(signs_list)},
            **{"alpha[%d]" % i: t for i, t in enumerate(alpha_list)})
    sp = (ctypes.c_void_p * G)(*[t.data_ptr() for t in signs_list])
    ap = (ctypes.c_void_p * G)(*[t.data_ptr() for t in alpha_list])
    st = lib.bd_linear_grouped_noalloc(_ptr(x), _ptr(variant_ids), _ptr(w_base), sp, ap, m, G, _ptr(out),
                                       M, d_out, d_in, _stream(x))
    _check(lib, "bd_linear_grouped_noalloc", st)
    return out
