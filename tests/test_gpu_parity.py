"""GPU parity: every HIP path against the CPU oracle, on the same seeded inputs.

Gates (floating point): sign bits bit-exact; α within 1e-6 relative; y within
1e-3 relative Frobenius error and, per token row, max |y - y_ref| <=
5e-3 · RMS(y_ref row).  Where every summation order is exact (one-hot x, the
integer lattice) y must equal the oracle exactly.

Post: "BitDelta : servir 14 modèles Zen depuis un seul cluster GPU"
(hanzo-blog, 2026-02-28).
"""

import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle
from tenant_serving_amd import synth

pytestmark = pytest.mark.gpu

REL_FRO = 1e-3
ROW_MAX = 5e-3


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def bd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tenant_serving_amd as m
    m.library()  # raises if the HIP library is missing: no silent fallback
    return m


DEV = "cuda:0"


def gate(got, ref, what=""):
    got = got.detach().cpu().double().numpy().reshape(ref.shape)
    assert np.all(np.isfinite(got)), what + ": non-finite outputs"
    diff = got - ref
    nref = np.linalg.norm(ref)
    rel = np.linalg.norm(diff) / nref if nref > 0 else np.linalg.norm(diff)
    ref2 = ref.reshape(-1, ref.shape[-1])
    d2 = diff.reshape(-1, ref.shape[-1])
    rms = np.sqrt((ref2 ** 2).mean(axis=1))
    worst = 0.0
    for r in range(ref2.shape[0]):
        mx = np.abs(d2[r]).max()
        if rms[r] == 0:
            assert mx == 0, what + ": row %d should be exactly zero" % r
        else:
            worst = max(worst, mx / rms[r])
    assert rel <= REL_FRO, "%s: relative Frobenius error %.3g" % (what, rel)
    assert worst <= ROW_MAX, "%s: max/row-RMS error %.3g" % (what, worst)
    return rel, worst


def mode_of(per_row):
    return 1 if per_row else 0


# ----------------------------------------------------------------------------
# compression

@pytest.mark.parametrize("shape", [(1, 8), (3, 24), (256, 512), (300, 1000), (17, 4104),
                                   (1024, 8192), (5, 28672)])
@pytest.mark.parametrize("per_row", [False, True])
def test_compress_parity(bd, shape, per_row):
    _say("compress", shape, per_row)
    gen = synth.generator(40 + shape[0], DEV)
    d = synth.laplace_delta(gen, *shape, 1e-3, DEV)
    s, a = bd.bd_compress(d, mode_of(per_row))
    torch.cuda.synchronize()
    s_ref, a_ref = oracle.compress(d.cpu(), per_row)
    assert np.array_equal(s.cpu().numpy(), s_ref)
    a = a.cpu().numpy()
    assert a.shape == a_ref.shape
    assert np.all(np.abs(a.astype(np.float64) - a_ref) <= 1e-6 * np.abs(a_ref))


def test_compress_special_values_and_exact_c(bd):
    d = torch.tensor([[0.0, -0.0, float("nan"), -1e-45, 1e-45, -float("inf"), float("inf"), -3.0]],
                     device=DEV)
    s, _ = bd.bd_compress(d, 1)
    # bits b0..b7 = 1 1 1 0 1 0 1 0 (zeros and NaN encode +1, denormals keep their sign)
    assert int(s.item()) == int(oracle.pack_signs(d.cpu())[0, 0]) == 0x57
    c = 2.0 ** -10
    gen = synth.generator(41, DEV)
    dc = torch.where(torch.rand((96, 512), generator=gen, device=DEV) < 0.5, -c, c)
    for mode in (0, 1):
        _, a = bd.bd_compress(dc, mode)
        assert torch.all(a == c)
    z = torch.zeros((7, 64), device=DEV)
    for mode in (0, 1):
        _, a = bd.bd_compress(z, mode)
        assert torch.all(a == 0)


def test_compress_deterministic(bd):
    gen = synth.generator(42, DEV)
    d = synth.laplace_delta(gen, 2048, 8192, 1e-3, DEV)
    for mode in (0, 1):
        s1, a1 = bd.bd_compress(d, mode)
        s2, a2 = bd.bd_compress(d, mode)
        assert torch.equal(s1, s2) and torch.equal(a1.view(torch.int32), a2.view(torch.int32))


# compression from a (fine-tuned, base) bf16 pair: Δ formed on the device

def _ft_base(seed, n, k, scale):
    gen = synth.generator(seed, DEV)
    base = synth.base_weight(gen, n, k, DEV)
    ft = (base.float() + scale * torch.randn((n, k), generator=gen, device=DEV)).to(torch.bfloat16)
    return ft, base


@pytest.mark.parametrize("shape", [(1, 8), (3, 24), (256, 512), (300, 1000), (17, 4104),
                                   (1024, 8192), (5, 28672)])
@pytest.mark.parametrize("per_row", [False, True])
def test_compress_pair_parity(bd, shape, per_row):
    _say("compress_pair", shape, per_row)
    ft, base = _ft_base(90 + shape[0], *shape, 1e-3)
    s, a = bd.bd_compress_pair(ft, base, mode_of(per_row))
    torch.cuda.synchronize()
    s_ref, a_ref = oracle.compress_pair(ft.cpu(), base.cpu(), per_row)
    assert np.array_equal(s.cpu().numpy(), s_ref)
    a = a.cpu().numpy()
    assert a.shape == a_ref.shape
    assert np.all(np.abs(a.astype(np.float64) - a_ref) <= 1e-6 * np.abs(a_ref))


def test_compress_pair_equals_compress_of_the_difference(bd):
    # the same outputs as bd_compress on the fp32 difference formed by torch,
    # including equal pairs, ±0 pairs and a wide exponent gap
    ft, base = _ft_base(95, 64, 1024, 2e-3)
    ft[0, :4] = base[0, :4]
    ft[1, 0], base[1, 0] = -0.0, 0.0
    ft[1, 1], base[1, 1] = 0.0, -0.0
    ft[2, 0], base[2, 0] = 1024.0, 2.0 ** -20
    d = ft.float() - base.float()
    for mode in (0, 1):
        s1, a1 = bd.bd_compress_pair(ft, base, mode)
        s2, a2 = bd.bd_compress(d, mode)
        assert torch.equal(s1, s2)
        assert torch.allclose(a1, a2, rtol=1e-6, atol=0)
    z, _ = bd.bd_compress_pair(base, base, 1)
    assert torch.all(z == 0xFF)


# ----------------------------------------------------------------------------
# fused linear, all dispatch paths (M <= 4 VALU, <= 64 MFMA skinny, else tiled)

SMALL_SHAPES = [(256, 512), (300, 520), (1040, 1032), (4104, 520), (8200, 264)]
MS = [1, 2, 3, 4, 5, 8, 16, 17, 33, 48, 64, 65, 128, 300]


@pytest.mark.parametrize("shape", SMALL_SHAPES)
@pytest.mark.parametrize("M", MS)
def test_linear_parity(bd, shape, M):
    N, K = shape
    _say("linear", M, shape)
    for per_row in (False, True):
        w, d, x = synth.projection(N, K, M, seed=100 + M, device=DEV)
        s, a = bd.bd_compress(d, mode_of(per_row))
        y = bd.bd_linear(x, w, s, a, mode_of(per_row))
        torch.cuda.synchronize()
        ref = oracle.linear(x.cpu(), w.cpu(), s.cpu(), a.cpu(), per_row)
        gate(y, ref, "M=%d %s per_row=%s" % (M, shape, per_row))


@pytest.mark.parametrize("M", [1, 4, 16, 64, 128])
def test_linear_one_hot_reads_out_weff(bd, M):
    # x = unit vectors: y[m, n] = W_eff[n, k_m] exactly (a single nonzero term).
    N, K = 200, 1032
    _say("one-hot", M, bd.bd_linear_path(M, N, K))
    expect_path = {1: "gemv_kernel", 4: "shot_kernel", 16: "shot_kernel", 64: "skinny_kernel",
                   128: "prefill_kernel"}[M]
    assert bd.bd_linear_path(M, N, K).startswith(expect_path), bd.bd_linear_path(M, N, K)
    w, d, _ = synth.projection(N, K, 1, seed=7, device=DEV)
    ks = torch.randperm(K, generator=torch.Generator().manual_seed(M))[:M]
    x = torch.zeros((M, K), dtype=torch.bfloat16)
    x[torch.arange(M), ks] = 1.0
    x = x.to(DEV)
    for per_row in (False, True):
        s, a = bd.bd_compress(d, mode_of(per_row))
        y = bd.bd_linear(x, w, s, a, mode_of(per_row))
        torch.cuda.synchronize()
        weff = oracle.weff(w.cpu(), s.cpu(), a.cpu(), per_row)
        wf = torch.from_numpy(weff.view(np.int16)).view(torch.bfloat16).float().numpy()
        expect = wf[:, ks.numpy()].T
        got = y.cpu().numpy()
        bad = np.argwhere(got != expect)
        assert bad.size == 0, "W_eff mismatch at %s: got %r expect %r" % (
            bad[:5].tolist(), got[tuple(bad[0])], expect[tuple(bad[0])])


# The x-stationary streaming path (2..16 tokens, 8192+ rows, where row
# streaming would need more than 1.5 workgroups per CU, or 2..3 tokens with x
# beyond 128 KiB): several K ranges, a range with fewer chunks than waves, a
# ragged last chunk, and row groups past the end of the matrix.
STREAM_SHAPES = [(16392, 4360), (8192, 2048), (8208, 520)]
XSTAT_SHAPES = [(16392, 8200), (16400, 2048), (16392, 1032)]


@pytest.mark.parametrize("shape,M", [(sh, m) for sh in XSTAT_SHAPES for m in (5, 7, 16)]
                         + [((8200, 32776), 2), ((8200, 21848), 3), ((12296, 21848), 4), ((12296, 16392), 4)])
def test_linear_streaming_path(bd, shape, M):
    N, K = shape
    _say("stream", M, shape)
    assert bd.bd_linear_path(M, N, K).startswith("xstat_kernel"), bd.bd_linear_path(M, N, K)
    for per_row in (False, True):
        w, d, x = synth.projection(N, K, M, seed=300 + M, device=DEV)
        s, a = bd.bd_compress(d, mode_of(per_row))
        y = bd.bd_linear(x, w, s, a, mode_of(per_row))
        torch.cuda.synchronize()
        ref = oracle.linear(x.cpu(), w.cpu(), s.cpu(), a.cpu(), per_row)
        gate(y, ref, "stream M=%d %s per_row=%s" % (M, shape, per_row))


# four tokens on 8192 or more rows of up to 16K weights: the row-quad MFMA
# kernel (one x phase and two, a ragged last chunk, rows that do not fill the
# last quad, whole quads per wave and quads split over sub-ranges)
@pytest.mark.parametrize("shape", [(8200, 1032), (8195, 8200), (16392, 4360), (8192, 16384), (8196, 520)])
def test_linear_quad_path(bd, shape):
    N, K = shape
    M = 4
    _say("quad", M, shape)
    assert bd.bd_linear_path(M, N, K).startswith("quad_kernel"), bd.bd_linear_path(M, N, K)
    for per_row in (False, True):
        w, d, x = synth.projection(N, K, M, seed=340 + N % 97, device=DEV)
        s, a = bd.bd_compress(d, mode_of(per_row))
        y = bd.bd_linear(x, w, s, a, mode_of(per_row))
        torch.cuda.synchronize()
        ref = oracle.linear(x.cpu(), w.cpu(), s.cpu(), a.cpu(), per_row)
        gate(y, ref, "quad %s per_row=%s" % (shape, per_row))
        # deterministic
        y2 = bd.bd_linear(x, w, s, a, mode_of(per_row))
        assert torch.equal(y.view(torch.int32), y2.view(torch.int32))


# two or three tokens with x within 128 KiB: x resident in LDS (both
# workgroup shapes, the largest x of each, ragged K, and rows that do not fill
# the last round of waves)
@pytest.mark.parametrize("shape,M", [(sh, m) for sh in STREAM_SHAPES for m in (2, 3)]
                         + [((8192, 16384), 2), ((8200, 10920), 3), ((12296, 1032), 3), ((8200, 16904), 2),
                            ((8200, 10928), 3), ((8192, 28672), 2), ((8200, 21840), 3), ((2048, 1032), 2),
                            ((4104, 520), 4), ((6152, 8200), 3), ((4096, 16384), 4), ((8184, 4104), 4)])
def test_linear_x_resident_path(bd, shape, M):
    N, K = shape
    _say("x resident", M, shape)
    assert bd.bd_linear_path(M, N, K).startswith("xres_kernel"), bd.bd_linear_path(M, N, K)
    for per_row in (False, True):
        w, d, x = synth.projection(N, K, M, seed=310 + M, device=DEV)
        s, a = bd.bd_compress(d, mode_of(per_row))
        y = bd.bd_linear(x, w, s, a, mode_of(per_row))
        torch.cuda.synchronize()
        ref = oracle.linear(x.cpu(), w.cpu(), s.cpu(), a.cpu(), per_row)
        gate(y, ref, "x resident M=%d %s per_row=%s" % (M, shape, per_row))


# a few tokens whose x exceeds 128 KiB on fewer than 8192 rows: the GEMV with
# x through the caches
@pytest.mark.parametrize("shape,M", [((4104, 16904), 4), ((4104, 21848), 3), ((6000, 32776), 2)])
def test_linear_gemv_long_rows(bd, shape, M):
    N, K = shape
    _say("gemv long rows", M, shape)
    assert bd.bd_linear_path(M, N, K).startswith("gemv_kernel"), bd.bd_linear_path(M, N, K)
    w, d, x = synth.projection(N, K, M, seed=320 + M, device=DEV)
    s, a = bd.bd_compress(d, 1)
    y = bd.bd_linear(x, w, s, a, 1)
    torch.cuda.synchronize()
    ref = oracle.linear(x.cpu(), w.cpu(), s.cpu(), a.cpu(), True)
    gate(y, ref, "gemv long rows M=%d %s" % (M, shape))


# Exact read-out of W_eff through the streaming kernels, one token per K
# range edge: the x-resident VALU kernel at two and three tokens (x within
# 128 KiB) and at four on 4096..8191 rows; the row-quad kernel at four on
# 8192 or more rows (two x phases); the x-stationary MFMA kernel at 16
# tokens, and at two and three tokens where x exceeds 128 KiB.
@pytest.mark.parametrize("N,K,M,path", [
    (16392, 4360, 2, "xres_kernel"), (16392, 4360, 3, "xres_kernel"), (6152, 8200, 4, "xres_kernel"),
    (8195, 8200, 4, "quad_kernel"), (16392, 4360, 4, "quad_kernel"),
    (16392, 4360, 16, "xstat_kernel"), (8200, 32776, 2, "xstat_kernel"), (8200, 21848, 3, "xstat_kernel"),
])
def test_linear_streaming_one_hot(bd, N, K, M, path):
    _say("stream one-hot", N, K, M, path)
    assert bd.bd_linear_path(M, N, K).startswith(path), bd.bd_linear_path(M, N, K)
    w, d, _ = synth.projection(N, K, 1, seed=8, device=DEV)
    pick = [0, K - 1, 511, 512, 2047, 2048, 4351, 4352, 1000, 3000, 4100, 17, 2600, 3600, 4200, K - 9]
    ks = torch.tensor([k % K for k in pick])[:M]
    x = torch.zeros((M, K), dtype=torch.bfloat16)
    x[torch.arange(M), ks] = 1.0
    x = x.to(DEV)
    s, a = bd.bd_compress(d, 1)
    y = bd.bd_linear(x, w, s, a, 1)
    torch.cuda.synchronize()
    weff = oracle.weff(w.cpu(), s.cpu(), a.cpu(), True)
    wf = torch.from_numpy(weff.view(np.int16)).view(torch.bfloat16).float().numpy()
    expect = wf[:, ks.numpy()].T
    got = y.cpu().numpy()
    bad = np.argwhere(got != expect)
    assert bad.size == 0, "W_eff mismatch at %s" % bad[:5].tolist()


# Exact read-out of W_eff through the row-streaming kernel (4 to 32 tokens on
# 4096 or more rows; 16-row workgroups on 4096 rows): one token per column at
# the 512-wide chunk edges, the last 16-byte group of a ragged K, a K shorter
# than one chunk, partial m-tiles and a ragged row count.
@pytest.mark.parametrize("N,K,M", [(8195, 8200, 16), (4100, 4360, 16), (8200, 264, 32), (4104, 1032, 17),
                                   (6152, 8200, 20), (6152, 8200, 5), (8195, 4096, 8), (4096, 4360, 16),
                                   (4096, 1032, 32), (16392, 1032, 17), (32776, 520, 8)])
def test_linear_rowstream_one_hot(bd, N, K, M):
    path = bd.bd_linear_path(M, N, K)
    _say("rowstream one-hot", N, K, M, path)
    assert path.startswith("rowstream_kernel"), path
    w, d, _ = synth.projection(N, K, 1, seed=9, device=DEV)
    edges = [0, 7, 8, 511, 512, 1023, 1024, 4095, 4096, 4351, 4352, 8191, 8192, K - 9, K - 8, K - 1]
    rest = np.random.default_rng(3).integers(0, K, size=32).tolist()
    ks = torch.tensor(sorted({k for k in edges if 0 <= k < K}) + rest)[:M]
    x = torch.zeros((M, K), dtype=torch.bfloat16)
    x[torch.arange(M), ks] = 1.0
    x = x.to(DEV)
    s, a = bd.bd_compress(d, 1)
    y = bd.bd_linear(x, w, s, a, 1)
    torch.cuda.synchronize()
    weff = oracle.weff(w.cpu(), s.cpu(), a.cpu(), True)
    wf = torch.from_numpy(weff.view(np.int16)).view(torch.bfloat16).float().numpy()
    expect = wf[:, ks.numpy()].T
    got = y.cpu().numpy()
    bad = np.argwhere(got != expect)
    assert bad.size == 0, "W_eff mismatch at %s" % bad[:5].tolist()


# The band kernel (4..16 tokens, 8192 or more rows of 4097..8192 weights):
# the layer's q/o shape at 4 and 16 tokens, a ragged row count (the last band
# has 3 rows), a ragged K with idle waves (4360: 9 chunks, the last of 264;
# 4104: the last chunk one 16-byte group), odd token counts (5, 13: partial
# token tiles), 16 bands per workgroup at four tokens and 28 at eight (the
# largest slot use of each), and the fewer-row shapes it also takes: 2050
# rows (513 bands, a last band of 2 rows, two bands on one workgroup),
# 3072 x 7176 (15 chunks, the last one group), 4104 and 8188 rows.
BAND_CASES = [(8192, 8192, 4), (8192, 8192, 16), (8195, 4360, 8), (8200, 4104, 5), (12296, 5000, 13),
              (16384, 8192, 4), (28672, 8192, 8), (2050, 8192, 16), (3072, 7176, 7), (4104, 8192, 5),
              (8188, 7680, 8)]


@pytest.mark.parametrize("N,K,M", BAND_CASES)
def test_linear_band_path(bd, N, K, M):
    _say("band", N, K, M)
    assert bd.bd_linear_path(M, N, K) == "band_kernel", bd.bd_linear_path(M, N, K)
    w, d, x = synth.projection(N, K, M, seed=360 + M, device=DEV)
    rows = torch.from_numpy(np.unique(np.concatenate([
        np.arange(0, 8), np.arange(N - 8, N), np.random.default_rng(M).integers(0, N, size=240)])))
    for per_row in (False, True):
        s, a = bd.bd_compress(d, mode_of(per_row))
        y = bd.bd_linear(x, w, s, a, mode_of(per_row))
        y16 = bd.bd_linear_bf16(x, w, s, a, mode_of(per_row))
        y2 = bd.bd_linear(x, w, s, a, mode_of(per_row))
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), y2.view(torch.int32))  # fixed summation order
        assert np.array_equal(_bf16_bits(y16), _bf16_bits(y.to(torch.bfloat16)))
        # oracle on sampled rows (every token), the first and last bands included
        ac = a.cpu()
        ref = oracle.linear(x.cpu(), w[rows.to(DEV)].cpu(), s[rows.to(DEV)].cpu(),
                            ac[rows] if per_row else ac, per_row)
        gate(y[:, rows.to(DEV)], ref, "band %dx%d M=%d per_row=%s" % (N, K, M, per_row))


# Exact read-out of W_eff through the band kernel: one token per column at the
# chunk edges (every wave's chunk) and the last 16-byte group of a ragged K.
@pytest.mark.parametrize("N,K,M", [(8195, 4360, 8), (8192, 8192, 16), (12296, 5000, 13), (16384, 8192, 4),
                                   (8200, 4104, 5), (2050, 8192, 16), (3072, 7176, 7)])
def test_linear_band_one_hot(bd, N, K, M):
    path = bd.bd_linear_path(M, N, K)
    _say("band one-hot", N, K, M, path)
    assert path == "band_kernel", path
    w, d, _ = synth.projection(N, K, 1, seed=10, device=DEV)
    edges = [0, K - 1, 511, 512, 1023, 1024, 2047, 4095, 4096, 4103, K - 8, 7679, 7680, 8191, 3000, 5000]
    ks = torch.tensor([k for k in edges if 0 <= k < K][:M])
    while ks.numel() < M:
        ks = torch.cat([ks, ks[:M - ks.numel()] + 1])
    x = torch.zeros((M, K), dtype=torch.bfloat16)
    x[torch.arange(M), ks] = 1.0
    x = x.to(DEV)
    s, a = bd.bd_compress(d, 1)
    y = bd.bd_linear(x, w, s, a, 1)
    torch.cuda.synchronize()
    weff = oracle.weff(w.cpu(), s.cpu(), a.cpu(), True)
    wf = torch.from_numpy(weff.view(np.int16)).view(torch.bfloat16).float().numpy()
    expect = wf[:, ks.numpy()].T
    got = y.cpu().numpy()
    bad = np.argwhere(got != expect)
    assert bad.size == 0, "W_eff mismatch at %s" % bad[:5].tolist()


# The slice path (3..16 tokens on fewer than 4096 rows; 16-row workgroups over
# 2048-wide slices of K, summed in slice order by a second kernel): the
# layer's k/v shape at 16 tokens (4 slices), ragged row counts (2050, 1026:
# a last block of 2 rows; 2044, 4095), a ragged K whose last slice is partly
# idle (5000: the last slice 904 wide; 8200: the last slice one 16-byte group
# in one wave), one slice (K = 2048, written straight to y), 8 slices
# (16384), odd token counts, and 2048..4095 rows at 3 tokens.
SLICE_CASES = [(1024, 8192, 16), (2050, 5000, 3), (4095, 2048, 16), (3072, 4096, 7), (1026, 16384, 9),
               (2044, 8192, 16), (2048, 8200, 3)]


@pytest.mark.parametrize("N,K,M", SLICE_CASES)
def test_linear_slice_path(bd, N, K, M):
    _say("slice", N, K, M)
    assert bd.bd_linear_path(M, N, K) == "slice_kernel", bd.bd_linear_path(M, N, K)
    w, d, x = synth.projection(N, K, M, seed=420 + M, device=DEV)
    for per_row in (False, True):
        s, a = bd.bd_compress(d, mode_of(per_row))
        y = bd.bd_linear(x, w, s, a, mode_of(per_row))
        y16 = bd.bd_linear_bf16(x, w, s, a, mode_of(per_row))
        y2 = bd.bd_linear(x, w, s, a, mode_of(per_row))
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), y2.view(torch.int32))  # fixed summation order
        assert np.array_equal(_bf16_bits(y16), _bf16_bits(y.to(torch.bfloat16)))
        ref = oracle.linear(x.cpu(), w.cpu(), s.cpu(), a.cpu(), per_row)
        gate(y, ref, "slice %dx%d M=%d per_row=%s" % (N, K, M, per_row))


# Exact read-out of W_eff through the slice path: one token per column at the
# edges of the waves' 128-wide pieces and of the slices, and the last weight
# of a ragged K.
@pytest.mark.parametrize("N,K,M", [(1024, 8192, 16), (2050, 5000, 3), (4095, 2048, 16), (2048, 8200, 3),
                                   (1026, 16384, 9)])
def test_linear_slice_one_hot(bd, N, K, M):
    path = bd.bd_linear_path(M, N, K)
    _say("slice one-hot", N, K, M, path)
    assert path == "slice_kernel", path
    w, d, _ = synth.projection(N, K, 1, seed=11, device=DEV)
    edges = [K - 1, 0, 127, 128, 2047, 2048, 4095, 4096, K - 8, 1919, 1920, 6143, 8191, 8192, 3001, 16383]
    ks = torch.tensor([k for k in edges if 0 <= k < K][:M])
    while ks.numel() < M:
        ks = torch.cat([ks, (ks[:M - ks.numel()] + 1) % K])
    x = torch.zeros((M, K), dtype=torch.bfloat16)
    x[torch.arange(M), ks] = 1.0
    x = x.to(DEV)
    s, a = bd.bd_compress(d, 1)
    y = bd.bd_linear(x, w, s, a, 1)
    torch.cuda.synchronize()
    weff = oracle.weff(w.cpu(), s.cpu(), a.cpu(), True)
    wf = torch.from_numpy(weff.view(np.int16)).view(torch.bfloat16).float().numpy()
    expect = wf[:, ks.numpy()].T
    got = y.cpu().numpy()
    bad = np.argwhere(got != expect)
    assert bad.size == 0, "W_eff mismatch at %s" % bad[:5].tolist()


# Non-finite inputs through every decode path: a NaN in one token's x makes
# exactly that token's outputs NaN, and a NaN base weight exactly that row's
# (the MFMA kernels repeat token rows and B columns and drop the copies, so a
# NaN must not leak into a neighbour); everything else matches the oracle, and
# nothing is written around y.
@pytest.mark.parametrize("N,K,M,path", [
    (8192, 4360, 8, "band_kernel"), (8195, 4096, 8, "rowstream_kernel"), (16392, 4360, 4, "quad_kernel"),
    (16392, 8200, 5, "xstat_kernel"), (1024, 8192, 4, "shot_kernel"), (1024, 8192, 16, "slice_kernel"),
    (2050, 5000, 3, "slice_kernel"), (8192, 8192, 1, "gemv_kernel"),
    (4096, 8192, 1, "gemv8_kernel"), (1024, 8192, 1, "gemv_kernel<1,1,4>"), (8192, 8192, 2, "xres_kernel")])
def test_linear_nonfinite_token_and_row(bd, N, K, M, path):
    _say("non-finite", N, K, M, path)
    assert bd.bd_linear_path(M, N, K).startswith(path), bd.bd_linear_path(M, N, K)
    w, d, x = synth.projection(N, K, M, seed=380 + M, device=DEV)
    s, a = bd.bd_compress(d, 1)
    tbad, nbad = M - 1, N // 2 + 1  # the last token; a row inside a band, quad or row group
    x = x.clone()
    x[tbad, K // 3] = float("nan")
    w = w.clone()
    w[nbad, 7] = float("nan")
    buf = torch.full((M * N + 16,), 12345.0, device=DEV)
    out = buf[8:8 + M * N].view(M, N)
    bd.bd_linear(x, w, s, a, 1, out=out)
    torch.cuda.synchronize()
    assert torch.all(buf[:8] == 12345.0) and torch.all(buf[8 + M * N:] == 12345.0)
    y = out.cpu().double().numpy()
    bad = np.zeros((M, N), dtype=bool)
    bad[tbad, :] = True
    bad[:, nbad] = True
    assert np.all(np.isnan(y[bad])), "NaN expected in the poisoned token and row"
    assert np.all(np.isfinite(y[~bad])), "NaN leaked outside the poisoned token and row"
    rows = np.unique(np.concatenate([np.arange(0, 4), np.arange(N - 4, N), [nbad - 1, nbad + 1],
                                     np.random.default_rng(N).integers(0, N, size=120)]))
    rows = rows[rows != nbad]
    toks = [t for t in range(M) if t != tbad]
    if toks:
        rt = torch.from_numpy(rows)
        ref = oracle.linear(x[toks].cpu(), w[rt.to(DEV)].cpu(), s[rt.to(DEV)].cpu(), a.cpu()[rt], True)
        gate(torch.from_numpy(y[np.ix_(toks, rows)]), ref, "non-finite %s" % path)


# The one-token GEMV's workgroup shapes: one row per workgroup below 2048
# rows, 8-wave workgroups splitting K 8 ways on 4096..8191 rows of
# 8192..16384 weights, two rows per 4-wave workgroup otherwise; ragged row
# counts and K, per-matrix and per-row α, and an exact one-hot read-out.
@pytest.mark.parametrize("N,K,path", [(1025, 5000, "gemv_kernel<1,1,4>"), (1024, 16384, "gemv_kernel<1,1,4>"),
                                      (4100, 8200, "gemv8_kernel<1,2,2>"), (6152, 14336, "gemv8_kernel<1,2,2>"),
                                      (4104, 4096, "gemv_kernel<1,2,4>"), (2050, 8192, "gemv_kernel<1,2,4>")])
def test_linear_gemv_forms(bd, N, K, path):
    _say("gemv form", N, K, path)
    assert bd.bd_linear_path(1, N, K) == path, bd.bd_linear_path(1, N, K)
    w, d, x = synth.projection(N, K, 1, seed=390 + N % 89, device=DEV)
    for per_row in (False, True):
        s, a = bd.bd_compress(d, mode_of(per_row))
        y = bd.bd_linear(x, w, s, a, mode_of(per_row))
        y2 = bd.bd_linear(x, w, s, a, mode_of(per_row))
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), y2.view(torch.int32))
        ref = oracle.linear(x.cpu(), w.cpu(), s.cpu(), a.cpu(), per_row)
        gate(y, ref, "gemv form %dx%d per_row=%s" % (N, K, per_row))
    # one-hot: y[0, n] = W_eff[n, k] exactly, k at the last 16-byte group
    k = K - 1
    xo = torch.zeros((1, K), dtype=torch.bfloat16)
    xo[0, k] = 1.0
    s, a = bd.bd_compress(d, 1)
    yo = bd.bd_linear(xo.to(DEV), w, s, a, 1)
    torch.cuda.synchronize()
    weff = oracle.weff(w.cpu(), s.cpu(), a.cpu(), True)
    wf = torch.from_numpy(weff.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(yo.cpu().numpy()[0], wf[:, k])


def _lattice(N, K, M, seed, device):
    rng = np.random.default_rng(seed)
    wm = rng.integers(-64, 65, size=(N, K))
    w = torch.from_numpy((wm * 2.0 ** -8).astype(np.float32)).to(torch.bfloat16)
    x = torch.from_numpy(rng.integers(-2, 3, size=(M, K)).astype(np.float32)).to(torch.bfloat16)
    aint = rng.integers(1, 9, size=(N, 1))
    d = torch.from_numpy((np.where(rng.random((N, K)) < 0.5, -1.0, 1.0) * aint * 2.0 ** -8)
                         .astype(np.float32))
    return w.to(device), x.to(device), d.to(device)


@pytest.mark.parametrize("M,N,K", [(m, n, k) for m in (1, 3, 4, 16, 40, 256)
                                   for n, k in ((96, 1032), (96, 28672), (8200, 1032))]
                         + [(4, 8192, 8192), (13, 8195, 4360)])
def test_linear_exact_lattice(bd, M, N, K):
    # Every partial sum is an integer multiple of 2^-8 below 2^16: exact in
    # fp32 in any order, so y must equal the oracle exactly.
    _say("lattice", M, N, K)
    w, x, d = _lattice(N, K, M, 1000 + M, DEV)
    s, a = bd.bd_compress(d, 1)
    torch.cuda.synchronize()
    assert np.all(np.rint(a.cpu().numpy() * 256) == a.cpu().numpy() * 256)
    y = bd.bd_linear(x, w, s, a, 1)
    torch.cuda.synchronize()
    ref = oracle.linear(x.cpu(), w.cpu(), s.cpu(), a.cpu(), True)
    assert np.array_equal(y.cpu().double().numpy(), ref)


# ----------------------------------------------------------------------------
# bf16 output (the listing's F.linear on bf16 operands returns bf16): every
# path rounds its fp32 result once to bf16 as it stores it

def _bf16_bits(t):
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def _bf16_value(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _bf16_gate(got_bits, ref64, what):
    """The bf16 result against the oracle's one rounding of its fp64 result.
    They agree except where the fp32 accumulation falls on the other side of
    a bf16 rounding boundary: rare (about the fp32 error over one bf16 step,
    under 1e-3 at these sizes, a few percent at d_in = 2^23), and then the
    bf16 value is still within half a bf16 step (of its own magnitude) plus
    the fp32 tolerance (5e-3 x row RMS) of the exact result.  (The rounding
    mode itself is pinned by the bitwise bf16(y32) comparisons.)"""
    ref64 = ref64.reshape(got_bits.shape)
    ref_bits = oracle.bf16_rne_f64(ref64)
    diff = got_bits != ref_bits
    assert diff.mean() <= 0.02, "%s: %.3g of outputs differ" % (what, diff.mean())
    if diff.any():
        got = _bf16_value(got_bits)
        rms = np.sqrt((ref64 ** 2).mean(axis=-1, keepdims=True)) * np.ones_like(ref64)
        half_step = np.abs(got) * 2.0 ** -8
        err = np.abs(got - ref64)
        assert np.all(err[diff] <= half_step[diff] + ROW_MAX * rms[diff]), what + ": beyond the fp32 tolerance"


@pytest.mark.parametrize("shape", [(256, 512), (1040, 1032), (4104, 520), (8200, 264)])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 16, 20, 33, 64, 65, 300])
def test_linear_bf16_output(bd, shape, M):
    N, K = shape
    _say("linear bf16", M, shape, bd.bd_linear_path(M, N, K))
    w, d, x = synth.projection(N, K, M, seed=700 + M, device=DEV)
    for per_row in (False, True):
        s, a = bd.bd_compress(d, mode_of(per_row))
        y32 = bd.bd_linear(x, w, s, a, mode_of(per_row))
        y16 = bd.bd_linear_bf16(x, w, s, a, mode_of(per_row))
        torch.cuda.synchronize()
        assert y16.dtype == torch.bfloat16 and y16.shape == (M, N)
        # the same kernel and summation order: bit for bit bf16(y32)
        assert np.array_equal(_bf16_bits(y16), _bf16_bits(y32.to(torch.bfloat16)))
        ref = oracle.linear(x.cpu(), w.cpu(), s.cpu(), a.cpu(), per_row)
        gate(y32, ref, "fp32 M=%d %s per_row=%s" % (M, shape, per_row))
        _bf16_gate(_bf16_bits(y16), ref, "bf16 M=%d %s per_row=%s" % (M, shape, per_row))


@pytest.mark.parametrize("M,N,K", [(1, 96, 28672), (4, 8200, 1032), (16, 8200, 1032), (40, 96, 1032),
                                   (256, 2000, 1032), (2048, 1024, 1024)])
def test_linear_bf16_output_exact_lattice(bd, M, N, K):
    # y is exact in fp32 on the lattice, so its bf16 rounding is the oracle's bit for bit
    _say("lattice bf16", M, N, K, bd.bd_linear_path(M, N, K))
    w, x, d = _lattice(N, K, M, 1100 + M, DEV)
    s, a = bd.bd_compress(d, 1)
    y16 = bd.bd_linear_bf16(x, w, s, a, 1)
    torch.cuda.synchronize()
    ref = oracle.linear_bf16(x.cpu(), w.cpu(), s.cpu(), a.cpu(), True)
    assert np.array_equal(_bf16_bits(y16), ref)


def test_linear_bf16_output_split_tiles_and_guards(bd):
    # the tiled path's K-split tiles (their sum kernel stores bf16 too), and
    # nothing written outside y
    M, N, K = 1800, 9000, 2056
    w, d, x = synth.projection(N, K, M, seed=703, device=DEV)
    s, a = bd.bd_compress(d, 1)
    buf = torch.full((M * N + 16,), float("nan"), dtype=torch.bfloat16, device=DEV)
    out = buf[8:8 + M * N].view(M, N)
    bd.bd_linear_bf16(x, w, s, a, 1, out=out)
    y32 = bd.bd_linear(x, w, s, a, 1)
    torch.cuda.synchronize()
    assert torch.isnan(buf[:8]).all() and torch.isnan(buf[8 + M * N:]).all()
    assert np.array_equal(_bf16_bits(out), _bf16_bits(y32.to(torch.bfloat16)))
    rows = np.array([0, 255, 256, 1000, 1791, 1799])
    ref = oracle.linear(x[rows].cpu(), w.cpu(), s.cpu(), a.cpu(), True)
    gate(y32[rows], ref, "fp32 split tiles")
    _bf16_gate(_bf16_bits(out[rows]), ref, "bf16 split tiles")


@pytest.mark.parametrize("M", [1, 16, 256])
def test_linear_alpha_zero_is_matmul(bd, M):
    N, K = 128, 1024
    w, _, x = synth.projection(N, K, M, seed=9, device=DEV)
    s = torch.randint(0, 256, (N, K // 8), dtype=torch.uint8, device=DEV)
    a = torch.zeros(N, device=DEV)
    y = bd.bd_linear(x, w, s, a, 1)
    ref = x.double().cpu().numpy() @ w.double().cpu().numpy().T
    gate(y, ref, "alpha=0")


def test_linear_deterministic_leading_dims_stream_and_guards(bd):
    N, K = 1040, 1032
    w, d, x = synth.projection(N, K, 24, seed=11, device=DEV)
    s, a = bd.bd_compress(d, 1)
    for M in (1, 4, 16, 24):
        y1 = bd.bd_linear(x[:M].contiguous(), w, s, a)
        y2 = bd.bd_linear(x[:M].contiguous(), w, s, a)
        assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))
    y3 = bd.bd_linear(x.view(2, 3, 4, K), w, s, a)
    assert y3.shape == (2, 3, 4, N)
    assert torch.equal(y3.reshape(24, N), bd.bd_linear(x, w, s, a))
    # guard bands around y stay untouched; a side stream orders correctly
    for M in (1, 16, 24):
        buf = torch.full((M * N + 8,), float("nan"), device=DEV)
        out = buf[4:4 + M * N].view(M, N)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            bd.bd_linear(x[:M].contiguous(), w, s, a, out=out)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        assert torch.isnan(buf[:4]).all() and torch.isnan(buf[4 + M * N:]).all()
        ref = oracle.linear(x[:M].cpu(), w.cpu(), s.cpu(), a.cpu(), True)
        gate(out, ref, "guarded M=%d" % M)


def test_boundary_errors_on_gpu(bd):
    N, K = 64, 64
    w, d, x = synth.projection(N, K, 2, seed=12, device=DEV)
    s, a = bd.bd_compress(d, 1)
    flat = torch.zeros(2 * K + 1, dtype=torch.bfloat16, device=DEV)
    xm = flat[1:].view(2, K)  # contiguous but 2 bytes off 16-byte alignment
    with pytest.raises(bd.BitDeltaError) as e:
        bd.bd_linear(xm, w, s, a)
    assert e.value.status == 3
    with pytest.raises(bd.BitDeltaError) as e:
        bd.bd_linear(x, w, s, a, mode=5)
    assert e.value.status == 5
    y = bd.bd_linear(x[:0], w, s, a)
    assert y.shape == (0, N)
    lib = bd.library()
    ws = torch.empty(16, dtype=torch.uint8, device=DEV)
    st = lib.bd_compress(ctypes.c_void_p(d.data_ptr()), N, K, 0, ctypes.c_void_p(s.data_ptr()),
                         ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(ws.data_ptr()), 16, None)
    assert st == 4


# ----------------------------------------------------------------------------
# grouped multi-variant linear

def _variants(N, K, G, seed, per_row, bd):
    gen = synth.generator(seed, DEV)
    w = synth.base_weight(gen, N, K, DEV)
    scales = synth.variant_scales(gen, G, DEV)
    comp = [bd.bd_compress(synth.laplace_delta(gen, N, K, b, DEV), mode_of(per_row)) for b in scales]
    return w, [c[0] for c in comp], [c[1] for c in comp]


# d_in % 64 == 0 takes the staged kernel (odd and even stage counts, one and
# two stages, 1/2/4/8 x-load slots by token count, K ranges on few rows, passes
# with fewer segments than waves); other d_in the fallback
@pytest.mark.parametrize("N,K,M,G", [(256, 512, 4, 1), (300, 520, 64, 3), (1040, 1056, 256, 14),
                                     (1040, 1088, 256, 14), (1040, 1032, 256, 14), (136, 1024, 300, 64),
                                     (136, 1032, 300, 64), (200, 4096, 37, 5), (200, 4104, 37, 5),
                                     (520, 2048, 700, 3), (96, 64, 40, 3), (96, 128, 120, 3),
                                     (72, 192, 513, 2), (1024, 8192, 16, 14), (520, 1984, 9, 9),
                                     (136, 128, 1500, 5)])
@pytest.mark.parametrize("per_row", [False, True])
def test_grouped_parity(bd, N, K, M, G, per_row):
    _say("grouped", N, K, M, G, per_row)
    w, sl, al = _variants(N, K, G, 50 + G, per_row, bd)
    gen = synth.generator(60 + M, DEV)
    x = synth.activations(gen, M, K, DEV)
    ids = synth.variant_ids(gen, M, G, DEV)
    y = bd.bd_linear_grouped(x, ids, w, sl, al, mode_of(per_row))
    torch.cuda.synchronize()
    ref = oracle.linear_grouped(x.cpu(), ids.cpu(), w.cpu(), [t.cpu() for t in sl],
                                [t.cpu() for t in al], per_row)
    gate(y, ref, "grouped")
    y2 = bd.bd_linear_grouped(x, ids, w, sl, al, mode_of(per_row))
    assert torch.equal(y.view(torch.int32), y2.view(torch.int32))


# Up to 4 tokens on 4096 or more rows take the decode path (rows streamed
# once, a rebuild per present variant, x one K range at a time in LDS): one
# token and several, K shorter than one chunk and ragged, one K range and
# several (the range partials added by the reduction), ragged row counts, one
# variant for all tokens and every token its own variant; fewer rows keep the
# staged kernel.
GDEC_CASES = [(4096, 8192, 4, 14), (8200, 1032, 4, 5), (4100, 28680, 3, 64), (4100, 264, 1, 3),
              (4104, 4096, 2, 2), (4096, 520, 4, 4), (4100, 2048, 4, 1), (4160, 28672, 4, 4),
              (28672, 1024, 3, 14), (4097, 1032, 1, 5), (8192, 8192, 1, 14), (1024, 8192, 4, 14)]


@pytest.mark.parametrize("N,K,M,G", GDEC_CASES)
@pytest.mark.parametrize("per_row", [False, True])
def test_grouped_decode_path(bd, N, K, M, G, per_row):
    _say("grouped decode", N, K, M, G, per_row)
    w, sl, al = _variants(N, K, G, 150 + G, per_row, bd)
    gen = synth.generator(160 + M, DEV)
    x = synth.activations(gen, M, K, DEV)
    if G == M:
        ids = torch.randperm(G, generator=torch.Generator().manual_seed(M)).to(torch.int32).to(DEV)
    else:
        ids = synth.variant_ids(gen, M, G, DEV)
    y = bd.bd_linear_grouped(x, ids, w, sl, al, mode_of(per_row))
    torch.cuda.synchronize()
    ref = oracle.linear_grouped(x.cpu(), ids.cpu(), w.cpu(), [t.cpu() for t in sl],
                                [t.cpu() for t in al], per_row)
    gate(y, ref, "grouped decode")
    y2 = bd.bd_linear_grouped(x, ids, w, sl, al, mode_of(per_row))
    assert torch.equal(y.view(torch.int32), y2.view(torch.int32))


@pytest.mark.parametrize("K", [1032, 28672])
def test_grouped_decode_special_cases(bd, K):
    # K = 1032: one K range (y written directly); 28672: four ranges (partials)
    N, M, G = 4104, 4, 4
    w, sl, al = _variants(N, K, G, 170, True, bd)
    gen = synth.generator(171, DEV)
    x = synth.activations(gen, M, K, DEV)
    for g in range(G):  # all tokens on one variant == the single-variant linear
        ids = torch.full((M,), g, dtype=torch.int32, device=DEV)
        y = bd.bd_linear_grouped(x, ids, w, sl, al)
        ref = oracle.linear(x.cpu(), w.cpu(), sl[g].cpu(), al[g].cpu(), True)
        gate(y, ref, "one variant")
    ids = torch.tensor([2, 0, 2, 1], dtype=torch.int32, device=DEV)
    y = bd.bd_linear_grouped(x, ids, w, sl, al)
    bad = ids.clone()
    bad[[0, 3]] = torch.tensor([-1, 1 << 30], dtype=torch.int32, device=DEV)
    yb = bd.bd_linear_grouped(x, bad, w, sl, al)
    torch.cuda.synchronize()
    assert torch.isnan(yb[[0, 3]]).all()
    assert torch.equal(yb[[1, 2]].view(torch.int32), y[[1, 2]].view(torch.int32))
    none = torch.full((M,), -1, dtype=torch.int32, device=DEV)  # no valid token at all
    assert torch.isnan(bd.bd_linear_grouped(x, none, w, sl, al)).all()
    perm = torch.tensor([3, 1, 0, 2], device=DEV)
    yp = bd.bd_linear_grouped(x[perm].contiguous(), ids[perm].contiguous(), w, sl, al)
    torch.cuda.synchronize()
    assert torch.equal(yp.view(torch.int32), y[perm].view(torch.int32))  # a token's sums do not depend on the others


@pytest.mark.parametrize("K,M", [(4104, 4), (28672, 2)])
def test_grouped_decode_exact_lattice(bd, K, M):
    N, G = 4096, 6
    rng = np.random.default_rng(7)
    wm = rng.integers(-64, 65, size=(N, K))
    w = torch.from_numpy((wm * 2.0 ** -8).astype(np.float32)).to(torch.bfloat16).to(DEV)
    x = torch.from_numpy(rng.integers(-2, 3, size=(M, K)).astype(np.float32)).to(torch.bfloat16).to(DEV)
    sl, al = [], []
    for g in range(G):
        aint = rng.integers(1, 9, size=(N, 1))
        d = np.where(rng.random((N, K)) < 0.5, -1.0, 1.0) * aint * 2.0 ** -8
        s, a = bd.bd_compress(torch.from_numpy(d.astype(np.float32)).to(DEV), 1)
        sl.append(s)
        al.append(a)
    ids = torch.from_numpy(rng.integers(0, G, size=M).astype(np.int32)).to(DEV)
    y = bd.bd_linear_grouped(x, ids, w, sl, al)
    torch.cuda.synchronize()
    ref = oracle.linear_grouped(x.cpu(), ids.cpu(), w.cpu(), [t.cpu() for t in sl],
                                [t.cpu() for t in al], True)
    assert np.array_equal(y.cpu().double().numpy(), ref)


def test_grouped_misaligned_sign_plane_takes_the_fallback(bd):
    # A sign plane that is not 8-byte aligned (a view 4 bytes into a larger
    # buffer) cannot feed the staged kernel's 8-byte sign loads: the launch
    # falls back to the register-staged kernel and the result is unchanged.
    N, K, M, G = 96, 1024, 50, 3
    w, sl, al = _variants(N, K, G, 77, True, bd)
    gen = synth.generator(78, DEV)
    x = synth.activations(gen, M, K, DEV)
    ids = synth.variant_ids(gen, M, G, DEV)
    y = bd.bd_linear_grouped(x, ids, w, sl, al)
    raw = torch.empty(N * (K // 8) + 4, dtype=torch.uint8, device=DEV)
    moved = raw[4:].view(N, K // 8)
    moved.copy_(sl[1])
    assert moved.data_ptr() % 8 == 4
    y2 = bd.bd_linear_grouped(x, ids, w, [sl[0], moved, sl[2]], al)
    torch.cuda.synchronize()
    ref = oracle.linear_grouped(x.cpu(), ids.cpu(), w.cpu(), [t.cpu() for t in sl],
                                [t.cpu() for t in al], True)
    gate(y, ref, "aligned planes")
    gate(y2, ref, "misaligned plane")


@pytest.mark.parametrize("K", [1032, 1024])
def test_grouped_special_cases(bd, K):
    N, M, G = 272, 100, 4
    w, sl, al = _variants(N, K, G, 70, True, bd)
    gen = synth.generator(71, DEV)
    x = synth.activations(gen, M, K, DEV)
    # all tokens on one variant == the single-variant linear (within fp32 order)
    for g in range(G):
        ids = torch.full((M,), g, dtype=torch.int32, device=DEV)
        y = bd.bd_linear_grouped(x, ids, w, sl, al)
        ref = oracle.linear(x.cpu(), w.cpu(), sl[g].cpu(), al[g].cpu(), True)
        gate(y, ref, "one variant")
        gate(bd.bd_linear(x, w, sl[g], al[g]), y.cpu().double().numpy(), "vs bd_linear")
    # out-of-range ids: NaN rows, others unaffected
    ids = synth.variant_ids(gen, M, G, DEV)
    y = bd.bd_linear_grouped(x, ids, w, sl, al)
    bad = ids.clone()
    bad[[3, 50, 99]] = torch.tensor([-1, 4, 1 << 30], dtype=torch.int32, device=DEV)
    yb = bd.bd_linear_grouped(x, bad, w, sl, al)
    torch.cuda.synchronize()
    assert torch.isnan(yb[[3, 50, 99]]).all()
    keep = [i for i in range(M) if i not in (3, 50, 99)]
    gate(yb[keep], y[keep].cpu().double().numpy(), "invalid ids")
    # permuting tokens permutes rows
    perm = torch.randperm(M, generator=torch.Generator().manual_seed(3)).to(DEV)
    yp = bd.bd_linear_grouped(x[perm].contiguous(), ids[perm].contiguous(), w, sl, al)
    gate(yp, y[perm].cpu().double().numpy(), "permuted")


@pytest.mark.parametrize("K", [4104, 4096])
def test_grouped_exact_lattice(bd, K):
    N, M, G = 96, 200, 6
    rng = np.random.default_rng(5)
    wm = rng.integers(-64, 65, size=(N, K))
    w = torch.from_numpy((wm * 2.0 ** -8).astype(np.float32)).to(torch.bfloat16).to(DEV)
    x = torch.from_numpy(rng.integers(-2, 3, size=(M, K)).astype(np.float32)).to(torch.bfloat16).to(DEV)
    sl, al = [], []
    for g in range(G):
        aint = rng.integers(1, 9, size=(N, 1))
        d = np.where(rng.random((N, K)) < 0.5, -1.0, 1.0) * aint * 2.0 ** -8
        s, a = bd.bd_compress(torch.from_numpy(d.astype(np.float32)).to(DEV), 1)
        sl.append(s)
        al.append(a)
    ids = torch.from_numpy(rng.integers(0, G, size=M).astype(np.int32)).to(DEV)
    y = bd.bd_linear_grouped(x, ids, w, sl, al)
    torch.cuda.synchronize()
    ref = oracle.linear_grouped(x.cpu(), ids.cpu(), w.cpu(), [t.cpu() for t in sl],
                                [t.cpu() for t in al], True)
    assert np.array_equal(y.cpu().double().numpy(), ref)


# ----------------------------------------------------------------------------
# full workload sizes, in the launch configuration the benchmark times.  The
# oracle computes whole output rows (every column, so every output tile of
# those rows), and the gates take the row RMS from the oracle's rows.

@pytest.mark.parametrize("name,N,K", synth.LLAMA70B_LAYER)
def test_full_decode_layer_projection(bd, name, N, K):
    _say("full decode", name, N, K)
    w, d, x = synth.projection(N, K, 16, seed=synth.SEEDS["decode"], device=DEV)
    s, a = bd.bd_compress(d, 1)
    torch.cuda.synchronize()
    dc = d.cpu()
    del d
    s_ref, a_ref = oracle.compress(dc, True)
    assert np.array_equal(s.cpu().numpy(), s_ref)
    assert np.all(np.abs(a.cpu().numpy() - a_ref) <= 1e-6 * a_ref)
    # every output of the 16 tokens; the first M rows are the reference of
    # the M-token call (x[:M] is a prefix of x)
    ref16 = oracle.linear(x.cpu(), w.cpu(), s_ref, a_ref, True)
    for M in (1, 2, 3, 4, 16):
        xm = x[:M].contiguous()
        y = bd.bd_linear(xm, w, s, a, 1)
        torch.cuda.synchronize()
        gate(y, ref16[:M], "%s M=%d (%s)" % (name, M, bd.bd_linear_path(M, N, K)))


def test_linear_rows_beyond_the_tiled_path(bd):
    # d_in = 2^23: too long for the tiled path's 32-bit tile offsets, so 66
    # tokens run as a 64-token and a 2-token block of the skinny path
    N, K, M = 4, 1 << 23, 66
    _say("long rows", M, N, K, bd.library().bd_linear_path(M, N, K).decode())
    w, d, x = synth.projection(N, K, M, seed=71, device=DEV)
    s, a = bd.bd_compress(d, 1)
    del d
    y = bd.bd_linear(x, w, s, a, 1)
    y64 = bd.bd_linear(x[:64].contiguous(), w, s, a, 1)
    torch.cuda.synchronize()
    assert torch.equal(y[:64], y64)
    ms, ns = np.repeat(np.arange(M), N), np.tile(np.arange(N), M)
    ref = oracle.linear_sampled(x.cpu(), w.cpu(), s.cpu(), a.cpu(), True, ms, ns)
    gate(y, ref.reshape(M, N), "long rows")
    # the bf16 result through the same 64-token blocks
    y16 = bd.bd_linear_bf16(x, w, s, a, 1)
    torch.cuda.synchronize()
    assert np.array_equal(_bf16_bits(y16), _bf16_bits(y.to(torch.bfloat16)))
    _bf16_gate(_bf16_bits(y16), ref.reshape(M, N), "long rows bf16")


def _prefill_plan(M, N, K):
    """The tiled path's work split as the library sizes its workspace: whole
    tiles run over all of K, the tiles of a last partial round of 256
    workgroups are split over K.  Returns (tiles, split parts) from the
    workspace size (parts x one 256x256 fp32 tile)."""
    nbytes = bd_lib().bd_linear_workspace_bytes(M, N, K)
    tiles = -(-M // 256) * -(-N // 256)
    return tiles, nbytes // (256 * 256 * 4)


def bd_lib():
    import tenant_serving_amd as m
    return m.library()


# one row at each edge of every 256-token tile, plus a few inside
PREFILL_ROWS = sorted({256 * t + e for t in range(8) for e in (0, 255)} | {1, 77, 1000, 1500})


@pytest.mark.parametrize("name,N,K", synth.LLAMA70B_LAYER)
def test_full_prefill_projection(bd, name, N, K):
    M = 2048
    tiles, parts = _prefill_plan(M, N, K)
    _say("full prefill", name, N, K, "tiles", tiles, "split parts", parts)
    assert bd.bd_linear_path(M, N, K) == "prefill_kernel"
    if name in ("gate", "up"):
        # 896 tiles: 768 whole ones and 128 split over K in the same grid
        assert tiles == 896 and parts == 256, (tiles, parts)
    w, d, x = synth.projection(N, K, M, seed=synth.SEEDS["prefill"], device=DEV)
    s, a = bd.bd_compress(d, 0)
    del d
    y = bd.bd_linear(x, w, s, a, 0)
    torch.cuda.synchronize()
    rows = np.array(PREFILL_ROWS)
    ref = oracle.linear(x[rows].cpu(), w.cpu(), s.cpu(), a.cpu(), False)
    gate(y[rows], ref, "prefill %s rows %s" % (name, PREFILL_ROWS))


# The tiled path's mixed plans at sizes the oracle computes in full: more than
# 256 tiles, a count that is not a multiple of 8 (plain tile order) or is one
# (XCD order plus a remainder strip), whole tiles beside tiles split 4 and 8
# ways over K, ragged M, N and K.
@pytest.mark.parametrize("M,N,K,per_row,expect", [
    (2304, 7424, 1024, False, (261, 20)),   # 256 whole + 5 tiles x 4 parts
    (2048, 8448, 1024, True, (264, 32)),    # 256 whole (XCD order) + 8 x 4
    (1800, 9000, 2056, True, (288, 256)),   # 256 whole + 32 x 8; ragged M, N, K
])
def test_prefill_mixed_plan_in_full(bd, M, N, K, per_row, expect):
    _say("prefill mixed plan", M, N, K)
    assert bd.bd_linear_path(M, N, K) == "prefill_kernel"
    assert _prefill_plan(M, N, K) == expect, _prefill_plan(M, N, K)
    w, d, x = synth.projection(N, K, M, seed=330 + M, device=DEV)
    s, a = bd.bd_compress(d, mode_of(per_row))
    del d
    y = bd.bd_linear(x, w, s, a, mode_of(per_row))
    torch.cuda.synchronize()
    ref = oracle.linear(x.cpu(), w.cpu(), s.cpu(), a.cpu(), per_row)
    gate(y, ref, "prefill mixed plan %s" % ((M, N, K),))


def _token_rows(M, count, seed):
    """Token rows whose every output the oracle computes: the first, the last
    and random others (all of them when M <= count)."""
    if M <= count:
        return np.arange(M)
    rng = np.random.default_rng(seed)
    return np.array(sorted({0, M - 1} | set(rng.choice(M, count - 2, replace=False).tolist())))


def test_full_grouped(bd):
    _say("full grouped")
    N, K, M, G = 8192, 28672, 256, 14
    gen = synth.generator(synth.SEEDS["grouped"], DEV)
    w = synth.base_weight(gen, N, K, DEV)
    scales = synth.variant_scales(gen, G, DEV)
    sl, al = [], []
    for b in scales:
        d = synth.laplace_delta(gen, N, K, b, DEV)
        s, a = bd.bd_compress(d, 1)
        sl.append(s)
        al.append(a)
        del d
    x = synth.activations(gen, M, K, DEV)
    ids = synth.variant_ids(gen, M, G, DEV)
    y = bd.bd_linear_grouped(x, ids, w, sl, al, 1)
    torch.cuda.synchronize()
    toks = _token_rows(M, 16, 6)
    ref = oracle.linear_grouped(x[toks].cpu(), ids[toks].cpu(), w.cpu(), [t.cpu() for t in sl],
                                [t.cpu() for t in al], True)
    gate(y[toks], ref, "grouped full, tokens %s" % toks.tolist())


def test_full_share_layer_calls(bd):
    """The call pattern of the full single-GPU share on one layer: 14 variants
    resident, 16 requests on variants drawn from them; the 512-token mixed
    prefill and the 16-token mixed decode through every projection, with only
    the variants present passed to the grouped call (ids remapped)."""
    _say("full share, one layer")
    G, R, P = 14, 16, 32
    gen = synth.generator(synth.SEEDS["full"], DEV)
    scales = synth.variant_scales(gen, G, DEV)
    req = synth.request_mix(gen, R, G, DEV).cpu().tolist()
    present = sorted(set(req))
    local = {v: i for i, v in enumerate(present)}
    dec_ids = torch.tensor([local[v] for v in req], dtype=torch.int32, device=DEV)
    pre_ids = dec_ids.repeat_interleave(P).contiguous()
    xs = {K: synth.activations(gen, R * P, K, DEV) for K in (8192, 28672)}
    for li, (name, N, K) in enumerate(synth.LLAMA70B_LAYER):
        w = synth.base_weight(gen, N, K, DEV)
        sl, al = [], []
        for g in range(G):
            d = synth.laplace_delta(gen, N, K, scales[g], DEV)
            s, a = bd.bd_compress(d, 1)
            sl.append(s)
            al.append(a)
            del d
        sp = [sl[g] for g in present]
        ap = [al[g] for g in present]
        wc = w.cpu()
        spc = [t.cpu() for t in sp]
        apc = [t.cpu() for t in ap]
        for M, ids in ((R * P, pre_ids), (R, dec_ids)):
            x = xs[K][:M].contiguous()
            y = bd.bd_linear_grouped(x, ids, w, sp, ap, 1)
            torch.cuda.synchronize()
            toks = _token_rows(M, 12, 70 + li)
            ref = oracle.linear_grouped(x[toks].cpu(), ids[toks].cpu(), wc, spc, apc, True)
            gate(y[toks], ref, "full share %s M=%d" % (name, M))
        del w, sl, al
        torch.cuda.empty_cache()


# ----------------------------------------------------------------------------
# delta cache in device mode: loads from pinned host memory, grouped linear on
# the slots, eviction ordered behind the work that used the evicted variant

def _variant_blobs(N, K, G, seed, bd):
    """Per variant: one pinned host blob = signs [N, K/8] then α fp32 [N]."""
    gen = synth.generator(seed, DEV)
    w = synth.base_weight(gen, N, K, DEV)
    scales = synth.variant_scales(gen, G, DEV)
    sb = N * K // 8
    blobs, sl, al = [], [], []
    for b in scales:
        s, a = bd.bd_compress(synth.laplace_delta(gen, N, K, b, DEV), 1)
        h = torch.empty(sb + 4 * N, dtype=torch.uint8, pin_memory=True)
        h[:sb].copy_(s.view(-1).cpu())
        h[sb:].copy_(a.cpu().view(torch.uint8))
        blobs.append(h)
        sl.append(s)
        al.append(a)
    return w, blobs, sl, al, sb


def _slot_tensors(view, N, K, sb):
    return view[:sb].view(N, K // 8), view[sb:sb + 4 * N].view(torch.float32)


def test_cache_device_mode_grouped_through_slots(bd):
    from tenant_serving_amd.cache import bd_cache
    _say("cache device mode")
    N, K, G, slots = 1024, 2048, 6, 3
    w, blobs, sl, al, sb = _variant_blobs(N, K, G, 91, bd)
    slot_bytes = (sb + 4 * N + 255) // 256 * 256
    dev_slots = torch.empty(slots * slot_bytes, dtype=torch.uint8, device=DEV)
    copy = torch.cuda.Stream()
    c = bd_cache(G, slots, 1, 100.0, slot_bytes, dev_slots, copy)
    pol = bd_cache(G, slots, 1, 100.0, slot_bytes)        # the same policy, host only
    for v in range(G):
        c.bd_cache_set_source(v, blobs[v])
    gen = synth.generator(92, DEV)
    x = synth.activations(gen, 24, K, DEV)
    stream = torch.cuda.current_stream()
    rng = np.random.default_rng(93)
    # at most slots - pinned distinct variants per batch, so none is busy
    batches = [[0, 1, 0], [2], [0, 2, 2], [3, 4], [1, 1, 2], [5, 0], [2, 3], [4], [0, 5]]
    now = 0.0
    for bi, req in enumerate(batches):
        now += 1.0
        toks = rng.integers(0, len(req), size=24)
        requests = [req[t] for t in toks]
        # the policy alone decides the same slots, loads and evictions
        expect = {}
        for v in dict.fromkeys(requests):
            a, s, e = pol.bd_cache_request(v, now)
            expect[v] = s
            if a == "load":
                pol.bd_cache_complete(v)
        local, views, variants = c.bd_cache_acquire_batch(requests, now, stream)
        assert variants == list(expect)
        for v in variants:
            assert c.bd_cache_query(v)[0] == expect[v]
        ids = torch.tensor(local, dtype=torch.int32, device=DEV)
        st = [_slot_tensors(vw, N, K, sb) for vw in views]
        y = bd.bd_linear_grouped(x, ids, w, [t[0] for t in st], [t[1] for t in st], 1)
        c.bd_cache_release_batch(variants, stream)
        for v in variants:
            pol.bd_cache_release(v)
        # the same call on the original tensors: bit-identical
        y_ref = bd.bd_linear_grouped(x, ids, w, [sl[v] for v in variants], [al[v] for v in variants], 1)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), y_ref.view(torch.int32)), "batch %d" % bi
    stats = c.bd_cache_get_stats()
    pstats = pol.bd_cache_get_stats()
    assert stats["loads"] == pstats["loads"] and stats["evictions"] == pstats["evictions"]
    assert stats["evictions"] > 0
    c.close()


def test_cache_device_mode_one_load_per_variant(bd):
    from tenant_serving_amd.cache import bd_cache
    _say("cache join")
    N, K, G = 1024, 2048, 2
    _, blobs, sl, al, sb = _variant_blobs(N, K, G, 94, bd)
    slot_bytes = (sb + 4 * N + 255) // 256 * 256
    dev_slots = torch.zeros(2 * slot_bytes, dtype=torch.uint8, device=DEV)
    c = bd_cache(G, 2, 0, 10.0, slot_bytes, dev_slots, torch.cuda.Stream())
    for v in range(G):
        c.bd_cache_set_source(v, blobs[v])
    s1 = torch.cuda.Stream()
    s2 = torch.cuda.Stream()
    v1, a1, _, _ = c.bd_cache_acquire(1, 0.0, s1)
    v2, a2, _, _ = c.bd_cache_acquire(1, 0.0, s2)
    assert a1 == "load" and a2 in ("join", "hit")
    assert v1.data_ptr() == v2.data_ptr()
    # work on both streams sees the loaded bytes
    with torch.cuda.stream(s1):
        g1 = v1.clone()
    with torch.cuda.stream(s2):
        g2 = v2.clone()
    c.bd_cache_release(1, s1)
    c.bd_cache_release(1, s2)
    torch.cuda.synchronize()
    assert torch.equal(g1[:sb].cpu(), blobs[1][:sb]) and torch.equal(g2[:sb].cpu(), blobs[1][:sb])
    assert c.bd_cache_get_stats()["loads"] == 1
    assert c.bd_cache_query(1)[1:] == (1, 0)
    c.close()


def test_cache_serves_delta_files(bd, tmp_path):
    """Variants saved as delta-set files, read into pinned slot-layout buffers,
    loaded by the cache, multiplied through their slots: identical to the
    same call on the tensors compress produced."""
    from tenant_serving_amd import deltafile
    from tenant_serving_amd.cache import bd_cache
    _say("cache from delta files")
    mats = [("0.q", 512, 1024), ("0.down", 256, 2048)]
    G = 3
    gen = synth.generator(95, DEV)
    base = {n: synth.base_weight(gen, d, k, DEV) for n, d, k in mats}
    layout, slot_bytes = deltafile.slot_layout(mats)
    direct, blobs = [], []
    for g in range(G):
        e = {n: bd.bd_compress(synth.laplace_delta(gen, d, k, 1e-3 * (g + 1), DEV), 1) for n, d, k in mats}
        p = str(tmp_path / ("v%d.safetensors" % g))
        deltafile.save_delta_set(p, e, variant="v%d" % g)
        blob = torch.empty(slot_bytes, dtype=torch.uint8, pin_memory=True)
        deltafile.read_into(p, blob, layout, {n: (d, k) for n, d, k in mats})
        direct.append(e)
        blobs.append(blob)
    c = bd_cache(G, 2, 0, 10.0, slot_bytes, torch.empty(2 * slot_bytes, dtype=torch.uint8, device=DEV),
                 torch.cuda.Stream())
    for g in range(G):
        c.bd_cache_set_source(g, blobs[g])
    shapes = {n: (d, k) for n, d, k in mats}
    stream = torch.cuda.current_stream()
    for bi, req in enumerate([[0, 2, 2, 0, 0, 2], [1, 1, 0, 1, 0, 0], [2, 1, 2, 2, 1, 1]]):
        local, views, variants = c.bd_cache_acquire_batch(req, float(bi), stream)
        ids = torch.tensor(local, dtype=torch.int32, device=DEV)
        sv = [deltafile.slot_views(v, layout, shapes) for v in views]
        for n, d, k in mats:
            x = synth.activations(synth.generator(96 + bi, DEV), len(req), k, DEV)
            y = bd.bd_linear_grouped(x, ids, base[n], [s[n][0] for s in sv], [s[n][1] for s in sv], 1)
            y_ref = bd.bd_linear_grouped(x, ids, base[n], [direct[v][n][0] for v in variants],
                                         [direct[v][n][1] for v in variants], 1)
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.int32), y_ref.view(torch.int32)), (bi, n)
        c.bd_cache_release_batch(variants, stream)
    assert c.bd_cache_get_stats()["evictions"] >= 1
    c.close()


# ----------------------------------------------------------------------------
# MonoSoup merge (a tool beside the serving path): randomized truncated SVD on
# the GPU against the oracle's exact one

@pytest.mark.parametrize("m,n", [(1024, 1024), (768, 1280)])
@pytest.mark.parametrize("noise", [0.0, 1e-3])
def test_monosoup_merge_matches_oracle(m, n, noise):
    from oracle import monosoup as oms
    from tenant_serving_amd import monosoup
    _say("monosoup", m, n, noise)
    k, r = 3, 32
    g = torch.Generator().manual_seed(97 + m + int(noise * 1e4))
    base = torch.randn((m, n), generator=g) * 0.02
    deltas = []
    for _ in range(k):
        u, _ = torch.linalg.qr(torch.randn((m, r), generator=g, dtype=torch.float64))
        v, _ = torch.linalg.qr(torch.randn((n, r), generator=g, dtype=torch.float64))
        s = 1.0 + torch.rand(r, generator=g, dtype=torch.float64)
        d = (u * s) @ v.t() * 1e-2 + noise * 1e-2 * torch.randn((m, n), generator=g, dtype=torch.float64)
        deltas.append(d.float())
    ckpts = [(base + d).to(DEV) for d in deltas]
    got = monosoup.merge(base.to(DEV), checkpoints=ckpts, rank=r, seed=5)
    torch.cuda.synchronize()
    want = oms.merge(base.double().numpy(), [(base + d).double().numpy() - base.double().numpy()
                                             for d in deltas], r)
    dg = got.cpu().double().numpy() - base.double().numpy()
    dw = want - base.double().numpy()
    rel = np.linalg.norm(dg - dw) / np.linalg.norm(dw)
    assert rel <= 1e-4, rel


def test_cache_busy_batch_releases_what_it_took(bd):
    """A batch with more distinct variants than unpinned slots raises Busy,
    and the variants it had already acquired are released again."""
    from tenant_serving_amd.cache import Busy, bd_cache
    _say("cache busy batch")
    N, K, G = 256, 1024, 4
    _, blobs, _, _, sb = _variant_blobs(N, K, G, 98, bd)
    slot_bytes = (sb + 4 * N + 255) // 256 * 256
    c = bd_cache(G, 2, 0, 10.0, slot_bytes, torch.empty(2 * slot_bytes, dtype=torch.uint8, device=DEV),
                 torch.cuda.Stream())
    for v in range(G):
        c.bd_cache_set_source(v, blobs[v])
    stream = torch.cuda.current_stream()
    with pytest.raises(Busy) as ei:
        c.bd_cache_acquire_batch([0, 1, 2, 0], 0.0, stream)
    assert ei.value.variant == 2
    for v in (0, 1):
        assert c.bd_cache_query(v)[2] == 0          # no reference left behind
    # a batch that fits goes through and evicts the least recent variant
    local, views, variants = c.bd_cache_acquire_batch([2, 2, 1], 1.0, stream)
    assert variants == [2, 1] and local == [0, 0, 1]
    c.bd_cache_release_batch(variants, stream)
    torch.cuda.synchronize()
    assert c.bd_cache_query(0)[0] == -1
    assert torch.equal(views[0][:sb].cpu(), blobs[2][:sb])
    c.close()


def test_grouped_planned_equals_grouped(bd):
    """One bucketing plan serves grouped calls of several shapes (staged,
    K ranges, fallback) over the same ids: bit-identical to the unplanned
    call.  A plan made for another batch size runs no passes (wrong rows,
    nothing outside the arguments touched)."""
    _say("grouped planned")
    M, G = 40, 5
    gen = synth.generator(99, DEV)
    ids = synth.variant_ids(gen, M, G, DEV)
    shapes = [(256, 1024), (1040, 2048), (96, 1032), (2048, 512)]
    ws_bytes = max(bd.library().bd_linear_grouped_workspace_bytes(M, N, K, G) for N, K in shapes)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    bd.bd_linear_grouped_plan(ids, G, ws)
    for N, K in shapes:
        w, sl, al = _variants(N, K, G, 100 + N, True, bd)
        x = synth.activations(gen, M, K, DEV)
        y1 = bd.bd_linear_grouped(x, ids, w, sl, al, 1)
        y2 = bd.bd_linear_grouped(x, ids, w, sl, al, 1, plan=ws)
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int32), y2.view(torch.int32)), (N, K)
    # a plan for 40 tokens used by a 24-token call: the kernels run no passes
    # (one K range here, so nothing at all is written to y)
    N, K = 256, 512
    w, sl, al = _variants(N, K, G, 150, True, bd)
    x = synth.activations(gen, 24, K, DEV)
    y = torch.full((24, N), 7.0, device=DEV)
    bd.bd_linear_grouped(x, ids[:24].contiguous(), w, sl, al, 1, out=y, plan=ws)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)


# ----------------------------------------------------------------------------
# the C ABI from a plain C program (no Python, no torch in the process)

def test_c_client_through_the_abi(bd, tmp_path):
    import os
    import subprocess
    from tests.c_client import build as c_client
    if not os.path.exists(c_client.BINARY):
        pytest.fail("the C client is not built (build() compiles it)")
    N, K, M, G = 300, 1032, 40, 3
    _say("C client", N, K, M, G)
    w, deltas, _, x, ids = synth.grouped(N, K, M, G, seed=77)
    np.concatenate([d.numpy().ravel() for d in deltas]).astype(np.float32).tofile(tmp_path / "delta.f32")
    w.view(torch.int16).numpy().tofile(tmp_path / "w.bf16")
    x.view(torch.int16).numpy().tofile(tmp_path / "x.bf16")
    ids.numpy().astype(np.int32).tofile(tmp_path / "ids.i32")
    from tenant_serving_amd.build import LIBRARY
    r = subprocess.run([c_client.BINARY, LIBRARY, str(tmp_path), str(N), str(K), str(M), str(G)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    signs = np.fromfile(tmp_path / "signs.u8", dtype=np.uint8).reshape(G, N, K // 8)
    alpha = np.fromfile(tmp_path / "alpha.f32", dtype=np.float32).reshape(G, N)
    refs = [oracle.compress(d, True) for d in deltas]
    for g, (s_ref, a_ref) in enumerate(refs):
        assert np.array_equal(signs[g], s_ref), "variant %d: sign bits" % g
        assert np.all(np.abs(alpha[g] - a_ref) <= 1e-6 * np.abs(a_ref)), "variant %d: alpha" % g
    y = torch.from_numpy(np.fromfile(tmp_path / "y.f32", dtype=np.float32).reshape(M, N))
    gate(y, oracle.linear(x, w, refs[0][0], refs[0][1], True), "C client, bd_linear")
    yg = torch.from_numpy(np.fromfile(tmp_path / "yg.f32", dtype=np.float32).reshape(M, N))
    ref = oracle.linear_grouped(x, ids, w, [s for s, _ in refs], [a for _, a in refs], True)
    gate(yg, ref, "C client, bd_linear_grouped")
