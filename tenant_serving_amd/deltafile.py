"""On-disk delta sets and the delta cache's slot layout.

"BitDelta : servir 14 modèles Zen depuis un seul cluster GPU" (hanzo-blog,
2026-02-28), "Infrastructure details": a variant's delta is stored as packed
sign matrices, 8 signs per byte (a 4096x4096 weight becomes 4096x512 bytes),
plus fp32 scale factors, one per output dimension.  Here one variant's delta
set is one safetensors file: for every weight matrix ``<name>``, the tensor
``<name>.signs`` (uint8 [d_out, d_in/8], least significant bit first along
d_in, bit 1 = +1) and ``<name>.alpha`` (float32 [d_out], or [1] for one
scale per matrix); the header's metadata names the format and the variant.
safetensors holds raw little-endian tensors and a JSON header, and loading it
executes nothing from the file.

The cache keeps a variant's whole set in one slot; ``slot_layout`` fixes
where each matrix's signs and α sit in it (256-byte aligned, in the order
given), and ``read_into`` fills a host buffer (pinned, for the cache's
loads) with that layout straight from the file.
"""

from __future__ import annotations

import json

import torch
from safetensors import safe_open
from safetensors.torch import save_file

FORMAT = "bitdelta-signs-lsb-first/v1"


def _align(n: int, a: int = 256) -> int:
    return (n + a - 1) // a * a


def save_delta_set(path: str, entries, variant: str = "", per_row: bool = True):
    """entries: {name: (signs uint8 [d_out, d_in/8], alpha float32 [d_out] or [1])}
    (any device); writes one safetensors file."""
    tensors = {}
    shapes = {}
    for name, (s, a) in entries.items():
        if s.dtype != torch.uint8 or s.dim() != 2:
            raise ValueError("%s: signs must be uint8 [d_out, d_in/8]" % name)
        if a.dtype != torch.float32 or a.dim() != 1 or a.numel() != (s.shape[0] if per_row else 1):
            raise ValueError("%s: alpha must be float32 [%s]" % (name, "d_out" if per_row else "1"))
        tensors[name + ".signs"] = s.detach().contiguous().cpu()
        tensors[name + ".alpha"] = a.detach().contiguous().cpu()
        shapes[name] = [int(s.shape[0]), int(s.shape[1]) * 8]
    meta = {"format": FORMAT, "variant": variant, "alpha": "per_row" if per_row else "per_matrix",
            "matrices": json.dumps(shapes)}
    save_file(tensors, path, metadata=meta)


def read_meta(path: str):
    """The header's metadata: format, variant, alpha mode and {name: [d_out, d_in]}."""
    with safe_open(path, framework="pt") as f:
        meta = dict(f.metadata() or {})
    if meta.get("format") != FORMAT:
        raise ValueError("%s is not a BitDelta delta set (format %r)" % (path, meta.get("format")))
    meta["matrices"] = {k: tuple(v) for k, v in json.loads(meta["matrices"]).items()}
    return meta


def load_delta_set(path: str):
    """-> ({name: (signs, alpha)} on the CPU, metadata)."""
    meta = read_meta(path)
    out = {}
    with safe_open(path, framework="pt") as f:
        for name in meta["matrices"]:
            out[name] = (f.get_tensor(name + ".signs"), f.get_tensor(name + ".alpha"))
    return out, meta


def slot_layout(matrices, per_row: bool = True):
    """matrices: [(name, d_out, d_in)] in slot order -> ({name: (signs offset,
    alpha offset)}, slot bytes); every piece starts on a 256-byte boundary."""
    layout = {}
    off = 0
    for name, d_out, d_in in matrices:
        if d_in % 8:
            raise ValueError("%s: d_in must be a multiple of 8" % name)
        so = off
        off = _align(off + d_out * d_in // 8)
        ao = off
        off = _align(off + 4 * (d_out if per_row else 1))
        layout[name] = (so, ao)
    return layout, off


def read_into(path: str, buf: torch.Tensor, layout, shapes, per_row: bool = True):
    """Copy every matrix of the file into ``buf`` (a contiguous host uint8
    tensor, pinned for the cache) at its slot-layout offsets.

    ``shapes`` ({name: (d_out, d_in)}) and ``per_row`` are what the slot was
    laid out for.  The file must match them exactly: its α mode, and for each
    matrix uint8 signs of [d_out, d_in/8] and float32 α of [d_out] (per row)
    or [1] (per matrix); and the layout's pieces must lie inside ``buf``
    without overlapping.  Anything else is refused before a byte is copied,
    so a reused buffer never keeps part of another variant's set."""
    if buf.device.type != "cpu" or buf.dtype != torch.uint8 or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous host uint8 tensor")
    if set(shapes) != set(layout):
        raise ValueError("shapes and layout name different matrices")
    spans = []
    for name, (so, ao) in layout.items():
        d_out, d_in = shapes[name]
        spans.append((so, so + d_out * d_in // 8, name))
        spans.append((ao, ao + 4 * (d_out if per_row else 1), name))
    spans.sort()
    for (a0, a1, n0), (b0, b1, n1) in zip(spans, spans[1:]):
        if a1 > b0:
            raise ValueError("layout pieces of %s and %s overlap" % (n0, n1))
    if spans and (spans[0][0] < 0 or spans[-1][1] > buf.numel()):
        raise ValueError("the layout does not fit the buffer")
    meta = read_meta(path)
    if meta.get("alpha") != ("per_row" if per_row else "per_matrix"):
        raise ValueError("%s holds %s alpha, the slot expects %s" % (
            path, meta.get("alpha"), "per_row" if per_row else "per_matrix"))
    with safe_open(path, framework="pt") as f:
        # every check from the header first (shapes and dtypes, no data read)
        for name, (so, ao) in layout.items():
            d_out, d_in = shapes[name]
            if tuple(meta["matrices"].get(name, ())) != (d_out, d_in):
                raise ValueError("%s: the file's matrix is %s, the slot's [%d, %d]" % (
                    name, meta["matrices"].get(name), d_out, d_in))
            sg = f.get_slice(name + ".signs")
            if sg.get_dtype() != "U8" or tuple(sg.get_shape()) != (d_out, d_in // 8):
                raise ValueError("%s: signs must be uint8 [%d, %d] (file: %s %s)" % (
                    name, d_out, d_in // 8, sg.get_dtype(), tuple(sg.get_shape())))
            na = d_out if per_row else 1
            a = f.get_slice(name + ".alpha")
            if a.get_dtype() != "F32" or tuple(a.get_shape()) != (na,):
                raise ValueError("%s: alpha must be float32 [%d] (file: %s %s)" % (
                    name, na, a.get_dtype(), tuple(a.get_shape())))
        # then the copies, one matrix at a time
        for name, (so, ao) in layout.items():
            sg = f.get_tensor(name + ".signs")
            a = f.get_tensor(name + ".alpha")
            buf[so:so + sg.numel()].copy_(sg.contiguous().view(-1))
            buf[ao:ao + 4 * a.numel()].copy_(a.contiguous().view(torch.uint8))


def slot_views(slot: torch.Tensor, layout, shapes, per_row: bool = True):
    """{name: (signs view [d_out, d_in/8], alpha view)} of a slot (device or
    host uint8 tensor) under ``layout``; shapes: {name: (d_out, d_in)}."""
    out = {}
    for name, (so, ao) in layout.items():
        d_out, d_in = shapes[name]
        s = slot[so:so + d_out * d_in // 8].view(d_out, d_in // 8)
        na = d_out if per_row else 1
        a = slot[ao:ao + 4 * na].view(torch.float32)
        out[name] = (s, a)
    return out
