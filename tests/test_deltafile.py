"""The on-disk delta set (safetensors) and the cache's slot layout, on the
host: a file written and read back gives the same bytes, the layout packs
every matrix on 256-byte boundaries without overlap, and reading a file
into a slot buffer puts each matrix where the layout says."""

import numpy as np
import pytest
import torch

from tenant_serving_amd import deltafile, synth

SHAPES = [("l0.q", 64, 128), ("l0.k", 16, 128), ("l0.down", 64, 264)]


def _entries(per_row=True, seed=3):
    g = torch.Generator().manual_seed(seed)
    out = {}
    for name, n, k in SHAPES:
        s = torch.randint(0, 256, (n, k // 8), generator=g, dtype=torch.uint8)
        a = torch.rand(n if per_row else 1, generator=g) * 1e-3
        out[name] = (s, a)
    return out


@pytest.mark.parametrize("per_row", [True, False])
def test_round_trip(tmp_path, per_row):
    e = _entries(per_row)
    p = str(tmp_path / "v.safetensors")
    deltafile.save_delta_set(p, e, variant="zen-test", per_row=per_row)
    got, meta = deltafile.load_delta_set(p)
    assert meta["variant"] == "zen-test" and meta["alpha"] == ("per_row" if per_row else "per_matrix")
    assert meta["matrices"] == {n: (d, k) for n, d, k in SHAPES}
    for name, (s, a) in e.items():
        assert torch.equal(got[name][0], s)
        assert torch.equal(got[name][1].view(torch.int32), a.view(torch.int32))


def test_rejects_other_files(tmp_path):
    from safetensors.torch import save_file
    p = str(tmp_path / "x.safetensors")
    save_file({"w": torch.zeros(2)}, p, metadata={"format": "other"})
    with pytest.raises(ValueError):
        deltafile.read_meta(p)
    with pytest.raises(ValueError):
        deltafile.save_delta_set(p, {"m": (torch.zeros(4, 2, dtype=torch.uint8), torch.zeros(3))})


def test_slot_layout_is_aligned_and_disjoint():
    layout, total = deltafile.slot_layout(SHAPES)
    spans = []
    for name, n, k in SHAPES:
        so, ao = layout[name]
        assert so % 256 == 0 and ao % 256 == 0
        spans += [(so, so + n * k // 8), (ao, ao + 4 * n)]
    spans.sort()
    for (a0, a1), (b0, b1) in zip(spans, spans[1:]):
        assert a1 <= b0
    assert spans[-1][1] <= total and total % 256 == 0
    # the full 70B layer order: one variant of 80 layers is 8.58 GB
    layer = [("%d.%s" % (i, n), d, k) for i in range(80) for n, d, k in synth.LLAMA70B_LAYER]
    _, big = deltafile.slot_layout(layer)
    assert 8.58e9 < big < 8.59e9


def test_read_into_places_every_matrix(tmp_path):
    e = _entries()
    p = str(tmp_path / "v.safetensors")
    deltafile.save_delta_set(p, e)
    layout, total = deltafile.slot_layout(SHAPES)
    buf = torch.full((total,), 0xAB, dtype=torch.uint8)
    deltafile.read_into(p, buf, layout, {n: (d, k) for n, d, k in SHAPES})
    views = deltafile.slot_views(buf, layout, {n: (d, k) for n, d, k in SHAPES})
    for name, (s, a) in e.items():
        assert torch.equal(views[name][0], s)
        assert torch.equal(views[name][1], a)
    # padding between pieces is untouched
    used = np.zeros(total, bool)
    for name, n, k in SHAPES:
        so, ao = layout[name]
        used[so:so + n * k // 8] = True
        used[ao:ao + 4 * n] = True
    assert (buf.numpy()[~used] == 0xAB).all()


def test_read_into_refuses_a_layout_made_for_smaller_matrices(tmp_path):
    e = _entries()
    p = str(tmp_path / "v.safetensors")
    deltafile.save_delta_set(p, e)
    small = [(name, n // 2, k) for name, n, k in SHAPES]
    layout, total = deltafile.slot_layout(small)
    buf = torch.zeros(4 * total, dtype=torch.uint8)
    with pytest.raises(ValueError):
        deltafile.read_into(p, buf, layout, {n: (d, k) for n, d, k in small})


def _refused_untouched(p, buf, layout, shapes, per_row=True):
    before = buf.clone()
    with pytest.raises(ValueError):
        deltafile.read_into(p, buf, layout, shapes, per_row)
    assert torch.equal(buf, before), "a refused file must not write into the buffer"


def test_read_into_refuses_mismatched_files(tmp_path):
    """A file with fewer rows, the other α mode, other dtypes, or a layout that
    does not fit is refused before anything is copied (a reused pinned buffer
    must not end up holding part of the previous variant's set)."""
    shapes = {n: (d, k) for n, d, k in SHAPES}
    layout, total = deltafile.slot_layout(SHAPES)
    buf = torch.full((total,), 0x5A, dtype=torch.uint8)
    # fewer rows in one matrix (the metadata and the tensors agree with each other)
    e = _entries()
    s, a = e["l0.k"]
    e["l0.k"] = (s[:-1].contiguous(), a[:-1].contiguous())
    p = str(tmp_path / "short.safetensors")
    deltafile.save_delta_set(p, e)
    _refused_untouched(p, buf, layout, shapes)
    # a per-matrix file read into a per-row slot, and the other way round
    p = str(tmp_path / "pm.safetensors")
    deltafile.save_delta_set(p, _entries(per_row=False), per_row=False)
    _refused_untouched(p, buf, layout, shapes)
    p = str(tmp_path / "pr.safetensors")
    deltafile.save_delta_set(p, _entries())
    pm_layout, pm_total = deltafile.slot_layout(SHAPES, per_row=False)
    _refused_untouched(p, torch.zeros(pm_total, dtype=torch.uint8), pm_layout, shapes, per_row=False)
    # tensors of the wrong dtype under a well-formed header
    from safetensors.torch import save_file
    import json
    t = {}
    for name, n, k in SHAPES:
        t[name + ".signs"] = torch.zeros((n, k // 8), dtype=torch.uint8)
        t[name + ".alpha"] = torch.zeros((n,), dtype=torch.float64 if name == "l0.q" else torch.float32)
    p = str(tmp_path / "dtype.safetensors")
    save_file(t, p, metadata={"format": deltafile.FORMAT, "variant": "", "alpha": "per_row",
                              "matrices": json.dumps({n: [d, k] for n, d, k in SHAPES})})
    _refused_untouched(p, buf, layout, shapes)
    # the right file, but a buffer too small for the layout, or overlapping pieces
    p = str(tmp_path / "ok.safetensors")
    deltafile.save_delta_set(p, _entries())
    _refused_untouched(p, torch.zeros(total - 256, dtype=torch.uint8), layout, shapes)
    bad = dict(layout)
    bad["l0.k"] = (layout["l0.q"][0] + 256, layout["l0.k"][1])
    _refused_untouched(p, buf, bad, shapes)
    # and it is accepted as laid out
    deltafile.read_into(p, buf, layout, shapes)
