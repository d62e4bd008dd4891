"""The grouped linear without allocation (bd_linear_grouped_noalloc), through
the C ABI, against the existing bd_linear_grouped on the same inputs: two
calls in a row, the second smaller than the first, so the second runs on
scratch that still holds the first call's plan and partial sums.

The entry point is for callers that cannot allocate device memory; its
workspace is a fixed array inside the library, one per GPU."""

import ctypes
import gc
import sys

import numpy as np
import pytest
import torch

import oracle
from tenant_serving_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tenant_serving_amd as bd
    return bd.library()  # raises if the HIP library is missing


def _case(N, K, M, G, seed, lib):
    gen = synth.generator(seed, DEV)
    w = synth.base_weight(gen, N, K, DEV)
    scales = synth.variant_scales(gen, G, DEV)
    sl, al = [], []
    for b in scales:
        d = synth.laplace_delta(gen, N, K, b, DEV)
        s = torch.empty((N, K // 8), dtype=torch.uint8, device=DEV)
        a = torch.empty((N,), dtype=torch.float32, device=DEV)
        st = lib.bd_compress(ctypes.c_void_p(d.data_ptr()), N, K, 1, ctypes.c_void_p(s.data_ptr()),
                             ctypes.c_void_p(a.data_ptr()), None, 0, None)
        assert st == 0
        sl.append(s)
        al.append(a)
    x = synth.activations(gen, M, K, DEV)
    ids = synth.variant_ids(gen, M, G, DEV)
    return w, sl, al, x, ids


def _ptrs(ts):
    return (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])


def _grouped(lib, x, ids, w, sl, al, y, ws):
    M, K = x.shape
    N = w.shape[0]
    st = lib.bd_linear_grouped(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(ids.data_ptr()),
                               ctypes.c_void_p(w.data_ptr()), _ptrs(sl), _ptrs(al), 1, len(sl),
                               ctypes.c_void_p(y.data_ptr()), M, N, K, ctypes.c_void_p(ws.data_ptr()),
                               ws.numel(), None)
    assert st == 0, st


def _noalloc(lib, x, ids, w, sl, al, y):
    M, K = x.shape
    N = w.shape[0]
    return lib.bd_linear_grouped_noalloc(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(ids.data_ptr()),
                                         ctypes.c_void_p(w.data_ptr()), _ptrs(sl), _ptrs(al), 1, len(sl),
                                         ctypes.c_void_p(y.data_ptr()), M, N, K, None)


def _gate(got, ref, what):
    got = got.cpu().double().numpy()
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    rms = np.sqrt((ref ** 2).mean(axis=1, keepdims=True))
    worst = (np.abs(got - ref) / rms).max()
    assert rel <= 1e-3 and worst <= 5e-3, "%s: rel %.3g, max/row-RMS %.3g" % (what, rel, worst)


# first call: k/v-like rows with K split into ranges (plan + partial sums in
# the scratch); second, smaller: fewer tokens, rows and variants, and a d_in
# that takes the register-staged kernel
CALLS = [(1024, 8192, 64, 14, 501), (300, 1032, 20, 3, 502)]


def test_noalloc_equals_grouped_on_two_calls_in_a_row(lib):
    outs = []
    for N, K, M, G, seed in CALLS:
        _say("noalloc call", N, K, M, G)
        w, sl, al, x, ids = _case(N, K, M, G, seed, lib)
        ws = torch.empty(lib.bd_linear_grouped_workspace_bytes(M, N, K, G), dtype=torch.uint8, device=DEV)
        y_ref = torch.empty((M, N), dtype=torch.float32, device=DEV)
        _grouped(lib, x, ids, w, sl, al, y_ref, ws)
        y = torch.full((M, N), float("nan"), device=DEV)
        torch.cuda.synchronize()
        # no collection inside the window: a cycle of an earlier test's
        # tensors freed there would show as a change too
        gc.collect()
        gc.disable()
        try:
            before = torch.cuda.memory_allocated()
            assert _noalloc(lib, x, ids, w, sl, al, y) == 0
            torch.cuda.synchronize()
            assert torch.cuda.memory_allocated() == before
        finally:
            gc.enable()
        # the same kernels on the same plan: bit for bit the existing entry point's result
        assert torch.equal(y.view(torch.int32), y_ref.view(torch.int32)), (N, K, M, G)
        ref = oracle.linear_grouped(x.cpu(), ids.cpu(), w.cpu(), [t.cpu() for t in sl],
                                    [t.cpu() for t in al], True)
        _gate(y, ref, "noalloc %s" % ((N, K, M, G),))
        outs.append((x, ids, w, sl, al, y.clone()))
    # the first call again after the smaller one: the same result
    x, ids, w, sl, al, y0 = outs[0]
    y = torch.empty_like(y0)
    assert _noalloc(lib, x, ids, w, sl, al, y) == 0
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int32), y0.view(torch.int32))


def test_noalloc_refuses_oversized_shapes_and_keeps_going(lib):
    N, K, M, G, seed = CALLS[1]
    w, sl, al, x, ids = _case(N, K, M, G, seed, lib)
    big_M = 293  # 28672 rows x 8192: more than the 64 MiB scratch holds
    xb = torch.zeros((big_M, 8192), dtype=torch.bfloat16, device=DEV)
    idb = torch.zeros((big_M,), dtype=torch.int32, device=DEV)
    wb = torch.zeros((28672, 8192), dtype=torch.bfloat16, device=DEV)
    sb = [torch.zeros((28672, 1024), dtype=torch.uint8, device=DEV)]
    ab = [torch.zeros((28672,), dtype=torch.float32, device=DEV)]
    yb = torch.full((big_M, 28672), 7.0, device=DEV)
    assert _noalloc(lib, xb, idb, wb, sb, ab, yb) == 4
    torch.cuda.synchronize()
    assert torch.all(yb == 7.0)  # refused before anything ran
    del xb, wb, sb, yb
    y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    assert _noalloc(lib, x, ids, w, sl, al, y) == 0
    ref = oracle.linear_grouped(x.cpu(), ids.cpu(), w.cpu(), [t.cpu() for t in sl],
                                [t.cpu() for t in al], True)
    torch.cuda.synchronize()
    _gate(y, ref, "after a refusal")


def test_noalloc_binding(lib):
    import tenant_serving_amd as bd
    N, K, M, G, seed = CALLS[1]
    w, sl, al, x, ids = _case(N, K, M, G, seed, lib)
    with pytest.raises(ValueError):
        bd.bd_linear_grouped_noalloc(x, ids, w, sl, al, None)
    y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    bd.bd_linear_grouped_noalloc(x, ids, w, sl, al, y)
    y_ref = bd.bd_linear_grouped(x, ids, w, sl, al)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int32), y_ref.view(torch.int32))
