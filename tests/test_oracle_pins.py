"""Pins of the CPU oracle against what the post and mathematics fix.

No test here compares the oracle with itself: each checks it against a
worked example from the post (or derived by hand from its definitions and the
stated readings), a library routine that computes a special case, a closed
form, an invariant, a statistical law with a stated bound, or the exact
rational brute force in ``brute_force.py``.

Post: "BitDelta : servir 14 modèles Zen depuis un seul cluster GPU"
(hanzo-blog, 2026-02-28).
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests import brute_force as bf
from tenant_serving_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16_bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


# ----------------------------------------------------------------------------
# sign code ("Mathematical foundation"; "Infrastructure details")

def _golden_sign_rows():
    rows = []
    with open(os.path.join(GOLDEN, "sign_bytes.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            rows.append(([float(p) for p in parts[:8]], int(parts[8], 16)))
    return rows


def test_sign_bytes_worked_examples():
    rows = _golden_sign_rows()
    assert len(rows) == 6
    d = np.array([r[0] for r in rows], dtype=np.float32)
    got = oracle.pack_signs(d)
    assert got.shape == (len(rows), 1)
    assert [int(v) for v in got[:, 0]] == [r[1] for r in rows]


def test_sign_packing_equals_numpy_packbits_little():
    # numpy's packbits with little bit order is LSB-first packing of booleans.
    rng = np.random.default_rng(11)
    for n, k in [(1, 8), (3, 16), (17, 104), (64, 512)]:
        d = rng.standard_normal((n, k)).astype(np.float32)
        d[rng.random((n, k)) < 0.05] = 0.0
        d[rng.random((n, k)) < 0.05] = -0.0
        expect = np.packbits(~(d < 0), axis=1, bitorder="little")
        assert np.array_equal(oracle.pack_signs(d), expect)


def test_sign_pack_unpack_round_trip():
    rng = np.random.default_rng(12)
    b = rng.integers(0, 256, size=(9, 40), dtype=np.uint8)
    pm = oracle.unpack_signs(b, 320)
    assert set(np.unique(pm)) <= {-1.0, 1.0}
    # unpack agrees with numpy's LSB-first unpack
    ref = np.unpackbits(b, axis=1, bitorder="little").astype(np.float32) * 2 - 1
    assert np.array_equal(pm, ref)
    assert np.array_equal(oracle.pack_signs(pm), b)


def test_packed_shape_matches_post_example():
    # "Infrastructure details": a 4096x4096 weight packs to 4096x512 bytes.
    d = np.zeros((4096, 4096), dtype=np.float32)
    s = oracle.pack_signs(d)
    assert s.shape == (4096, 512) and s.dtype == np.uint8
    assert int(s.min()) == 0xFF
    with open(os.path.join(GOLDEN, "memory_accounting.txt")) as f:
        kv = dict(l.split() for l in f if l.strip() and not l.startswith("#"))
    assert int(float(kv["packed_example_cols_out"])) == s.shape[1]
    # 1 bit per element is 1/32 of an fp32 delta
    assert d.nbytes // s.nbytes == int(kv["sign_storage_ratio_vs_fp32"])


def test_signed_zero_and_nan_encode_plus_one():
    d = np.array([[0.0, -0.0, np.nan, -np.nan, -1e-45, 1e-45, -np.inf, np.inf]],
                 dtype=np.float32)
    byte = int(oracle.pack_signs(d)[0, 0])
    bits = [(byte >> b) & 1 for b in range(8)]
    assert bits == [1, 1, 1, 1, 0, 1, 0, 1]


def test_laplace_sign_balance():
    # Laplace(0, b) is symmetric: the fraction of +1 bits is 1/2 within 5 sigma.
    gen = synth.generator(101)
    d = synth.laplace_delta(gen, 512, 1024, 1e-3)
    s = oracle.pack_signs(d)
    ones = int(np.unpackbits(s).sum())
    n = d.numel()
    assert abs(ones / n - 0.5) <= 5 * 0.5 / math.sqrt(n)


# ----------------------------------------------------------------------------
# scale factor α ("Mathematical foundation"; "Infrastructure details")

def test_alpha_minimises_reconstruction_error():
    # mean|Δ| is the least-squares optimum of ||Δ - α·sign(Δ)||^2 (closed form:
    # derivative 2(nα - Σ|Δ|) = 0); check the objective around it.
    rng = np.random.default_rng(3)
    d = rng.laplace(0.0, 1e-3, size=(64, 96)).astype(np.float32)
    a = float(oracle.alpha(d, per_row=False)[0])
    s = oracle.unpack_signs(oracle.pack_signs(d), 96).astype(np.float64)
    dd = d.astype(np.float64)

    def f(x):
        return float(((dd - x * s) ** 2).sum())

    for eps in (1e-2, 1e-4):
        assert f(a) <= f(a * (1 + eps)) and f(a) <= f(a * (1 - eps))
    grad = 2 * (d.size * a - np.abs(dd).sum())
    assert abs(grad) <= 1e-6 * np.abs(dd).sum()


def test_alpha_per_row_minimises_each_row():
    rng = np.random.default_rng(4)
    d = rng.laplace(0.0, 2e-3, size=(8, 64)).astype(np.float32)
    a = oracle.alpha(d, per_row=True)
    for n in range(8):
        exact = bf.alpha_exact([float(v) for v in d[n]])
        assert a[n] == np.float32(float(exact))


def test_alpha_exact_against_rational_mean():
    rng = np.random.default_rng(5)
    d = (rng.standard_normal((16, 40)) * 1e-3).astype(np.float32)
    exact = bf.alpha_exact([float(v) for v in d.ravel()])
    a = oracle.alpha(d, per_row=False)[0]
    assert a == np.float32(float(exact))


def test_alpha_exact_for_plus_minus_c_and_exact_reconstruction():
    # Δ = ±c with c = 2^-10: α = c exactly, so α·sign(Δ) = Δ and the
    # reconstruction equals bf16(W_base + Δ) = bf16(W_ft) computed by torch.
    c = 2.0 ** -10
    gen = synth.generator(7)
    w = synth.base_weight(gen, 96, 256)
    sg = torch.where(torch.rand((96, 256), generator=gen) < 0.5, -1.0, 1.0)
    d = (sg * c).to(torch.float32)
    for per_row in (False, True):
        s, a = oracle.compress(d, per_row)
        assert np.all(a == np.float32(c))
        weff = oracle.weff(w, s, a, per_row)
        ref = _bf16_bits((w.float() + d).to(torch.bfloat16))
        assert np.array_equal(weff, ref)


def test_alpha_laplace_scale():
    # For Laplace(0, b), E|Δ| = b and Var|Δ| = b^2: α/b - 1 within 5/sqrt(n).
    gen = synth.generator(8)
    b = 1e-3
    d = synth.laplace_delta(gen, 1024, 2048, b)
    a = float(oracle.alpha(d, per_row=False)[0])
    assert abs(a / b - 1) <= 5 / math.sqrt(d.numel())
    ar = oracle.alpha(d, per_row=True).astype(np.float64)
    assert np.all(np.abs(ar / b - 1) <= 5 / math.sqrt(2048))


def test_alpha_zero_delta_and_identical_rows():
    z = np.zeros((5, 16), dtype=np.float32)
    assert oracle.alpha(z, False)[0] == 0.0 and np.all(oracle.alpha(z, True) == 0.0)
    z[:, 3] = -0.0
    assert oracle.alpha(z, False)[0] == 0.0
    rng = np.random.default_rng(9)
    row = rng.laplace(0, 1e-3, size=(1, 48)).astype(np.float32)
    d = np.repeat(row, 7, axis=0)
    assert np.all(oracle.alpha(d, True) == oracle.alpha(d, False)[0])


# ----------------------------------------------------------------------------
# Δ from a (fine-tuned, base) pair ("Mathematical foundation": Δ = W_ft − W_base)

def _pair(seed, n, k, scale=1e-3):
    """A bf16 base ~ N(0, 0.02) and a fine-tuned copy: base + N(0, scale), in bf16."""
    gen = synth.generator(seed)
    base = synth.base_weight(gen, n, k)
    ft = (base.float() + scale * torch.randn((n, k), generator=gen)).to(torch.bfloat16)
    return ft, base


def test_pair_delta_against_exact_rational_difference():
    # Every fp32 Δ equals the exact difference rounded once to fp32; pairs of
    # widely different magnitude (exponent gaps beyond 15) force real rounding.
    ft, base = _pair(30, 12, 64)
    fb, bb = _bf16_bits(ft), _bf16_bits(base)
    fb[0, :8] = [0x4480, 0x3F80, 0x0001, 0x7F00, 0x8000, 0x0000, 0xC2F7, 0x3C01]
    bb[0, :8] = [0x3380, 0x2D80, 0x8001, 0x0001, 0x0000, 0x8000, 0x42F7, 0xBF81]
    d = oracle.delta_from_pair(fb, bb)
    for n in range(fb.shape[0]):
        for k in range(fb.shape[1]):
            want = bf.delta_pair(int(fb[n, k]), int(bb[n, k]))
            assert Fraction(float(d[n, k])) == want, (n, k)


def test_pair_signs_follow_the_comparison():
    # bit = !(Δ < 0) and Δ < 0 exactly when W_ft < W_base: the sign code is
    # decided by comparing the two weights, with equal weights (and ±0 pairs)
    # encoding +1.
    ft, base = _pair(31, 40, 256)
    fb, bb = _bf16_bits(ft), _bf16_bits(base)
    fb[1, :4] = bb[1, :4]                      # equal pairs
    fb[2, :2], bb[2, :2] = 0x8000, 0x0000      # -0 vs +0
    fb[2, 2:4], bb[2, 2:4] = 0x0000, 0x8000    # +0 vs -0
    s, _ = oracle.compress_pair(fb, bb, per_row=True)
    f32 = lambda b: (b.astype(np.uint32) << 16).view(np.float32)
    bits = ~(f32(fb) < f32(bb))
    assert np.array_equal(s, np.packbits(bits, axis=1, bitorder="little"))


def test_pair_alpha_against_exact_rational_mean():
    ft, base = _pair(32, 6, 48)
    fb, bb = _bf16_bits(ft), _bf16_bits(base)
    for per_row in (True, False):
        _, a = oracle.compress_pair(fb, bb, per_row)
        rows = [[abs(bf.bf16_value(int(f)) - bf.bf16_value(int(b))) for f, b in zip(fr, br)]
                for fr, br in zip(fb, bb)]
        if per_row:
            want = [bf.round_f32(sum(r, Fraction(0)) / len(r)) for r in rows]
        else:
            flat = [v for r in rows for v in r]
            want = [bf.round_f32(sum(flat, Fraction(0)) / len(flat))]
        assert [Fraction(float(v)) for v in a] == want


def test_pair_identical_and_one_ulp_offsets():
    # W_ft == W_base: Δ = 0, α = 0, every sign +1.  W_ft one bf16 ulp above
    # (below) a base strictly inside (0.25, 0.5): Δ = ±2^-9 exactly, α = 2^-9.
    gen = torch.Generator().manual_seed(33)
    base = (0.26 + 0.22 * torch.rand((8, 64), generator=gen)).to(torch.bfloat16)  # inside (0.25, 0.5)
    s, a = oracle.compress_pair(base, base, per_row=False)
    assert a[0] == 0.0 and np.all(s == 0xFF)
    bb = _bf16_bits(base)
    for step, byte in ((1, 0xFF), (-1, 0x00)):
        fb = (bb.astype(np.int32) + step).astype(np.uint16)
        s, a = oracle.compress_pair(fb, bb, per_row=True)
        assert np.all(a == np.float32(2.0 ** -9)) and np.all(s == byte)


def test_pair_equals_numpy_fp32_difference():
    # numpy's float32 subtraction of the widened weights, fed to the fp32-Δ
    # compression, gives the same signs and α.
    ft, base = _pair(34, 64, 512)
    fb, bb = _bf16_bits(ft), _bf16_bits(base)
    f32 = lambda b: (b.astype(np.uint32) << 16).view(np.float32)
    d = f32(fb) - f32(bb)
    for per_row in (True, False):
        s1, a1 = oracle.compress_pair(fb, bb, per_row)
        s2, a2 = oracle.compress(d, per_row)
        assert np.array_equal(s1, s2) and np.array_equal(a1, a2)


# ----------------------------------------------------------------------------
# bf16 rounding (the reconstructed weight is rounded once to bf16)

def test_bf16_rne_matches_torch_on_structured_patterns():
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x3FFF, 0x7FFE, 0x7FFF, 0x8000, 0x8001, 0xBFFF,
                     0xC000, 0xFFFE, 0xFFFF], dtype=np.uint32)
    rng = np.random.default_rng(13)
    lows = np.concatenate([lows, rng.integers(0, 1 << 16, size=13, dtype=np.uint32)])
    u = (hi[:, None] | lows[None, :]).ravel()
    got = oracle.bf16_rne(u)
    ref = torch.from_numpy(u.view(np.float32).copy()).to(torch.bfloat16)
    ref = ref.view(torch.int16).numpy().view(np.uint16)
    finite = (u & 0x7FFFFFFF) <= 0x7F800000
    assert np.array_equal(got[finite], ref[finite])
    # NaN stays NaN
    nan_out = got[~finite]
    assert np.all(((nan_out & 0x7F80) == 0x7F80) & ((nan_out & 0x7F) != 0))


def test_bf16_rne_against_rational_rounding():
    rng = np.random.default_rng(14)
    u = rng.integers(0, 0x7F800000, size=400, dtype=np.uint32)
    u[::2] |= np.uint32(0x80000000)
    u[:6] = [0x3F808000, 0x3F818000, 0x00008000, 0x00018000, 0x7F7FFFFF, 0x7F7F8000]
    got = oracle.bf16_rne(u)
    for bits, g in zip(u.tolist(), got.tolist()):
        r = bf.round_bf16(bf.f32_value(bits))
        if isinstance(r, float):
            assert (g & 0x7FFF) == 0x7F80 and math.copysign(1, r) == (-1 if g >> 15 else 1)
        else:
            assert bf.bf16_value(g) == r


def _f64_cases(seed=21, count=600):
    """Doubles across bf16's range: random values, exact ties between bf16
    neighbours and values one double-ulp either side of them, ties hidden by
    an fp32 rounding (a value just above a bf16 tie whose fp32 rounding lands
    on the tie), subnormals, the overflow boundary, zeros and non-finites."""
    rng = np.random.default_rng(seed)
    ex = rng.integers(-140, 128, size=count)
    v = list((1.0 + rng.random(count)) * np.exp2(ex.astype(np.float64)) * np.where(rng.random(count) < 0.5, -1, 1))
    b = rng.integers(0x0001, 0x7F7F, size=200).astype(np.uint32) << 16
    lo = b.view(np.float32).astype(np.float64)
    hi = (b + 0x10000).view(np.float32).astype(np.float64)
    mid = (lo + hi) / 2                                    # exact in fp64
    v += list(mid) + list(np.nextafter(mid, 0)) + list(np.nextafter(mid, np.inf)) + list(-mid)
    for t in (1.0, 1.5, 3.0 * 2.0 ** -100, 2.0 ** 100):
        v += [t * (1 + 2.0 ** -8 + 2.0 ** -30), t * (1 + 2.0 ** -8), t * (1 + 3 * 2.0 ** -8),
              t * (1 + 2.0 ** -8 - 2.0 ** -30)]
    v += [2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -134, 2.0 ** -135, 2.0 ** -149, 5e-324,
          (2 - 2.0 ** -7) * 2.0 ** 127, (2 - 2.0 ** -8) * 2.0 ** 127, np.nextafter((2 - 2.0 ** -8) * 2.0 ** 127, 0),
          1e39, -1e39, 0.0, -0.0, np.inf, -np.inf]
    return np.array(v, dtype=np.float64)


def test_bf16_rne_f64_against_rational_rounding():
    # the bf16 output of the fused linear: one rounding of the fp64 result,
    # checked against exact rational rounding (ties to even) of each double
    v = _f64_cases()
    got = oracle.bf16_rne_f64(v)
    for val, g in zip(v.tolist(), got.tolist()):
        if math.isinf(val):
            assert g == (0xFF80 if val < 0 else 0x7F80)
            continue
        r = bf.round_bf16(Fraction(val))
        if isinstance(r, float):
            assert (g & 0x7FFF) == 0x7F80 and (g >> 15) == (1 if r < 0 else 0), val
        else:
            assert bf.bf16_value(g) == r, (val, hex(g))
            if r == 0:
                assert (g >> 15) == (1 if math.copysign(1.0, val) < 0 else 0)
    nan = oracle.bf16_rne_f64(np.array([np.nan, -np.nan]))
    assert np.all(((nan & 0x7F80) == 0x7F80) & ((nan & 0x7F) != 0))


def test_bf16_rne_f64_one_rounding_not_two():
    # 1 + 2^-8 + 2^-30 lies above the tie between 1 and 1 + 2^-7: rounded once
    # it goes up; rounded to fp32 first it would land on the tie and go to 1.
    got = oracle.bf16_rne_f64(np.array([1 + 2.0 ** -8 + 2.0 ** -30, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8]))
    assert got.tolist() == [0x3F81, 0x3F80, 0x3F82]


def test_bf16_rne_f64_matches_torch_where_fp32_is_exact():
    # for doubles that are fp32 values the single rounding is torch's fp32 -> bf16
    rng = np.random.default_rng(22)
    u = rng.integers(0, 0x7F800000, size=20000, dtype=np.uint32)
    u[::2] |= np.uint32(0x80000000)
    f = u.view(np.float32)
    got = oracle.bf16_rne_f64(f.astype(np.float64))
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


# ----------------------------------------------------------------------------
# reconstruction W_eff = W_base + α·sign(Δ) ("Serving architecture")

def test_weff_alpha_zero_is_base():
    gen = synth.generator(15)
    w = synth.base_weight(gen, 32, 64)
    s = np.random.default_rng(0).integers(0, 256, size=(32, 8), dtype=np.uint8)
    for per_row, a in ((False, np.zeros(1, np.float32)), (True, np.zeros(32, np.float32))):
        assert np.array_equal(oracle.weff(w, s, a, per_row), _bf16_bits(w))


def test_weff_against_brute_force():
    gen = synth.generator(16)
    w = synth.base_weight(gen, 6, 24)
    d = synth.laplace_delta(gen, 6, 24, 3e-3)
    for per_row in (False, True):
        s, a = oracle.compress(d, per_row)
        got = oracle.weff(w, s, a, per_row)
        wb = _bf16_bits(w)
        for n in range(6):
            for k in range(24):
                bit = (int(s[n, k // 8]) >> (k % 8)) & 1
                assert bit == bf.sign_bit(float(d[n, k]))
                ref = bf.weff(int(wb[n, k]), bit, float(a[n] if per_row else a[0]))
                assert bf.bf16_value(int(got[n, k])) == ref


def test_weff_sign_selects_plus_or_minus_alpha():
    # one element per case, chosen so the fp32 sum is exact and the bf16
    # rounding is visible: w = 1.0, α = 2^-8 -> 1 + 2^-8 is a bf16 tie -> 1.0;
    # α = 3·2^-8 -> 1.01171875 is the tie between 1.0078125 (odd last bit)
    # and 1.015625 (even) -> 1.015625.  Below 1.0 the bf16 step is 2^-8, so
    # 1 - a·2^-8 is exact.
    w = torch.tensor([[1.0] * 8], dtype=torch.bfloat16)
    s = np.array([[0b10101010]], dtype=np.uint8)
    for a_val, plus, minus in ((2.0 ** -8, 1.0, 1.0 - 2.0 ** -8),
                               (3 * 2.0 ** -8, 1.015625, 1.0 - 3 * 2.0 ** -8)):
        a = np.array([a_val], dtype=np.float32)
        got = oracle.weff(w, s, a, False)
        vals = torch.from_numpy(got.view(np.int16)).view(torch.bfloat16).float().numpy()
        assert list(vals[0, 1::2]) == [plus] * 4
        assert list(vals[0, 0::2]) == [np.float32(minus)] * 4


# ----------------------------------------------------------------------------
# fused linear y = x·W_effᵀ ("Serving architecture" listing)

def test_linear_alpha_zero_is_plain_matmul():
    gen = synth.generator(17)
    w = synth.base_weight(gen, 40, 128)
    x = synth.activations(gen, 5, 128)
    s = np.full((40, 16), 0x5A, dtype=np.uint8)
    y = oracle.linear(x, w, s, np.zeros(1, np.float32), False)
    ref = x.double().numpy() @ w.double().numpy().T
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_linear_equals_matmul_with_reconstructed_weight():
    gen = synth.generator(18)
    w = synth.base_weight(gen, 48, 256)
    d = synth.laplace_delta(gen, 48, 256)
    x = synth.activations(gen, 3, 256)
    for per_row in (False, True):
        s, a = oracle.compress(d, per_row)
        weff = oracle.weff(w, s, a, per_row)
        wt = torch.from_numpy(weff.view(np.int16)).view(torch.bfloat16).double().numpy()
        ref = x.double().numpy() @ wt.T
        assert np.allclose(oracle.linear(x, w, s, a, per_row), ref, rtol=1e-12, atol=1e-13)


def _lattice(seed, m, n, k, g=1):
    """Inputs on which every summation order is exact (see test below)."""
    rng = np.random.default_rng(seed)
    wm = rng.integers(-64, 65, size=(n, k))
    w = torch.from_numpy((wm * 2.0 ** -8).astype(np.float32)).to(torch.bfloat16)
    x = torch.from_numpy(rng.integers(-2, 3, size=(m, k)).astype(np.float32)).to(torch.bfloat16)
    deltas = []
    for _ in range(g):
        a_int = rng.integers(1, 9, size=(n, 1))
        sg = np.where(rng.random((n, k)) < 0.5, -1.0, 1.0)
        deltas.append(torch.from_numpy((sg * a_int * 2.0 ** -8).astype(np.float32)))
    return w, x, deltas, wm


def test_linear_exact_lattice():
    # W_base = m·2^-8 (|m| <= 64), α = a·2^-8 (1 <= a <= 8, per row), x in
    # {-2..2}: W_eff = (m ± a)·2^-8 exactly and y is an exact integer multiple
    # of 2^-8; compare with Python integer arithmetic.
    m, n, k = 3, 10, 200
    w, x, (d,), wm = _lattice(19, m, n, k)
    s, a = oracle.compress(d, per_row=True)
    y = oracle.linear(x, w, s, a, True)
    sgn = np.where(d.numpy() < 0, -1, 1)
    aint = np.rint(a.astype(np.float64) * 256).astype(np.int64)
    assert np.all(aint * 2.0 ** -8 == a)
    weff_int = wm + sgn * aint[:, None]
    xi = x.float().numpy().astype(np.int64)
    yint = xi @ weff_int.T
    assert np.array_equal(y, yint * 2.0 ** -8)


def test_linear_bf16_on_the_lattice():
    # the bf16 result of the fused linear: the exact integer result (Python
    # integers, as above) rounded by exact rational rounding
    m, n, k = 4, 12, 304
    w, x, (d,), wm = _lattice(23, m, n, k)
    s, a = oracle.compress(d, per_row=True)
    got = oracle.linear_bf16(x, w, s, a, True)
    sgn = np.where(d.numpy() < 0, -1, 1)
    aint = np.rint(a.astype(np.float64) * 256).astype(np.int64)
    yint = x.float().numpy().astype(np.int64) @ (wm + sgn * aint[:, None]).T
    assert got.shape == (m, n) and got.dtype == np.uint16
    for i in range(m):
        for j in range(n):
            assert bf.bf16_value(int(got[i, j])) == bf.round_bf16(Fraction(int(yint[i, j]), 256))
    # rounding the result is not the identity here: most lattice sums need
    # more than bf16's 8 significant bits
    assert np.mean(yint % 2 != 0) > 0.3


def test_linear_against_brute_force():
    gen = synth.generator(20)
    w = synth.base_weight(gen, 3, 16)
    d = synth.laplace_delta(gen, 3, 16, 2e-3)
    x = synth.activations(gen, 2, 16)
    for per_row in (False, True):
        s, a = oracle.compress(d, per_row)
        y = oracle.linear(x, w, s, a, per_row)
        xb = _bf16_bits(x).tolist()
        yx, weffs = bf.linear(xb, _bf16_bits(w).tolist(), s.tolist(), [float(v) for v in a],
                              per_row)
        for mi in range(2):
            xs = [bf.bf16_value(v) for v in xb[mi]]
            for ni in range(3):
                # products are exact in fp64; sequential summation of K terms
                # errs by at most (K-1)·2^-53·Σ|terms|
                mag = sum((abs(xs[kk] * weffs[ni][kk]) for kk in range(16)), Fraction(0))
                bound = 15 * Fraction(1, 2 ** 53) * mag
                assert abs(Fraction(y[mi, ni]) - yx[mi][ni]) <= bound


def test_linear_leading_dims_and_sampled():
    gen = synth.generator(21)
    w = synth.base_weight(gen, 24, 64)
    d = synth.laplace_delta(gen, 24, 64)
    x = synth.activations(gen, 6, 64)
    s, a = oracle.compress(d, True)
    y = oracle.linear(x, w, s, a, True)
    y3 = oracle.linear(x.view(2, 3, 64), w, s, a, True)
    assert y3.shape == (2, 3, 24) and np.array_equal(y3.reshape(6, 24), y)
    ms = np.array([0, 5, 3, 3]); ns = np.array([0, 23, 7, 8])
    assert np.array_equal(oracle.linear_sampled(x, w, s, a, True, ms, ns), y[ms, ns])


# ----------------------------------------------------------------------------
# several variants over one base ("Serving architecture" diagram)

def test_grouped_reduces_to_single_variant_linear():
    gen = synth.generator(22)
    w = synth.base_weight(gen, 20, 64)
    deltas = [synth.laplace_delta(gen, 20, 64, b) for b in (5e-4, 1e-3, 2e-3)]
    x = synth.activations(gen, 9, 64)
    comp = [oracle.compress(d, True) for d in deltas]
    ids = np.array([2, 0, 1, 1, 2, 0, 0, 2, 1], dtype=np.int32)
    y = oracle.linear_grouped(x, ids, w, [c[0] for c in comp], [c[1] for c in comp], True)
    for g in range(3):
        yg = oracle.linear(x, w, comp[g][0], comp[g][1], True)
        assert np.array_equal(y[ids == g], yg[ids == g])
    # permutation of tokens permutes rows
    perm = np.random.default_rng(1).permutation(9)
    yp = oracle.linear_grouped(x[perm], ids[perm], w, [c[0] for c in comp],
                               [c[1] for c in comp], True)
    assert np.array_equal(yp, y[perm])
    # out-of-range ids give NaN rows, other rows untouched
    bad = ids.copy(); bad[4] = 3; bad[6] = -1
    yb = oracle.linear_grouped(x, bad, w, [c[0] for c in comp], [c[1] for c in comp], True)
    assert np.all(np.isnan(yb[[4, 6]]))
    keep = [i for i in range(9) if i not in (4, 6)]
    assert np.array_equal(yb[keep], y[keep])
    ms = np.array([0, 8, 4]); ns = np.array([19, 0, 5])
    got = oracle.linear_grouped_sampled(x, ids, w, [c[0] for c in comp],
                                        [c[1] for c in comp], True, ms, ns)
    assert np.array_equal(got, y[ms, ns])


def test_grouped_exact_lattice():
    m, n, k, g = 12, 8, 96, 4
    w, x, deltas, wm = _lattice(23, m, n, k, g)
    ids = np.random.default_rng(2).integers(0, g, size=m).astype(np.int32)
    comp = [oracle.compress(d, True) for d in deltas]
    y = oracle.linear_grouped(x, ids, w, [c[0] for c in comp], [c[1] for c in comp], True)
    xi = x.float().numpy().astype(np.int64)
    for t in range(m):
        d = deltas[ids[t]].numpy()
        aint = np.rint(comp[ids[t]][1].astype(np.float64) * 256).astype(np.int64)
        weff_int = wm + np.where(d < 0, -1, 1) * aint[:, None]
        assert np.array_equal(y[t], (weff_int @ xi[t]) * 2.0 ** -8)


def test_memory_accounting_of_post():
    # "Mathematical foundation": 70B params in bf16 = 140 GB; one sign bit per
    # parameter = 8.75 GB; 14 variants: 1.96 TB naive vs ~262 GB, ~87% less.
    with open(os.path.join(GOLDEN, "memory_accounting.txt")) as f:
        kv = {a: float(b) for a, b in (l.split() for l in f if l.strip() and not l.startswith("#"))}
    p = kv["params_70b"]
    assert p * 2 == kv["bf16_base_bytes"]
    assert p / 8 == kv["delta_bytes_per_variant"]
    assert kv["variants"] * kv["bf16_base_bytes"] == kv["naive_total_bytes"]
    total = kv["bf16_base_bytes"] + kv["variants"] * kv["delta_bytes_per_variant"]
    assert abs(total - kv["bitdelta_total_bytes_approx"]) / total < 0.01
    assert round(100 * (1 - total / kv["naive_total_bytes"])) == kv["reduction_percent_approx"]
