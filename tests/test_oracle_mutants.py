"""Planted-mistake check of the oracle's pins.

Each mutant is a copy of the oracle's C source with one plausible mistake
(wrong bit order, wrong sign(0), a dropped term, a wrong index, a missing
absolute value or rounding, ...).  The copy is compiled on the CPU and run
through a battery of pins drawn from what the post and mathematics fix; every
mutant must fail at least one pin, and the unmodified source must pass all of
them.  Nothing here touches the GPU.
"""

import math
from fractions import Fraction
import os
import tempfile

import numpy as np
import pytest
import torch

import oracle
from tests import brute_force as bf
from tenant_serving_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# (name, original text, replacement).  Each original must occur in the source.
MUTANTS = [
    ("msb_first_pack", "byte |= (unsigned)sign_bit(delta[n * d_in + 8 * j + b]) << b;",
     "byte |= (unsigned)sign_bit(delta[n * d_in + 8 * j + b]) << (7 - b);"),
    ("sign_zero_negative", "static int sign_bit(float d) { return !(d < 0.0f); }",
     "static int sign_bit(float d) { return d > 0.0f; }"),
    ("alpha_without_abs", "double a = fabs((double)v[i]);", "double a = (double)v[i];"),
    ("alpha_row_sum_not_mean", "alpha[n] = (float)(abs_sum(delta + n * d_in, d_in) / (double)d_in);",
     "alpha[n] = (float)(abs_sum(delta + n * d_in, d_in));"),
    ("alpha_matrix_wrong_count", "alpha[0] = (float)(total / ((double)d_out * (double)d_in));",
     "alpha[0] = (float)(total / (double)d_in);"),
    ("per_row_alpha_wrong_row", "float a = per_row ? alpha[n] : alpha[0];",
     "float a = per_row ? alpha[0] : alpha[0];"),
    ("sign_inverted", "float s = bit ? a : -a;", "float s = bit ? -a : a;"),
    ("weff_truncated_not_rounded", "return orc_bf16_rne(f32_to_bits(t));",
     "return (uint16_t)(f32_to_bits(t) >> 16);"),
    ("bf16_ties_away", "return (uint16_t)((u + 0x7fffu + lsb) >> 16);",
     "return (uint16_t)((u + 0x8000u) >> 16);"),
    ("unpack_msb_first", "int bit = (signs[n * nbytes + k / 8] >> (k % 8)) & 1;\n        out[k]",
     "int bit = (signs[n * nbytes + k / 8] >> (7 - k % 8)) & 1;\n        out[k]"),
    ("dot_drops_first_term", "for (int64_t k = 0; k < d_in; ++k) acc +=",
     "for (int64_t k = 1; k < d_in; ++k) acc +="),
    ("linear_wrong_token_row", "for (int64_t m = 0; m < M; ++m) y[m * d_out + n] = dot_f64(x + m * d_in, row, d_in);",
     "for (int64_t m = 0; m < M; ++m) y[m * d_out + n] = dot_f64(x + 0 * d_in, row, d_in);"),
    ("grouped_uses_variant_zero", "weff_row(w_base, signs[g], alpha[g], per_row, n, d_in, row);\n                    for",
     "weff_row(w_base, signs[0], alpha[0], per_row, n, d_in, row);\n                    for"),
    ("weff_alpha_added_twice", "float t = w + s;", "float t = w + s + s;"),
    ("out_bf16_ties_away", "double r = nearbyint(a / q) * q;", "double r = round(a / q) * q;"),
    ("out_bf16_truncated", "double r = nearbyint(a / q) * q;", "double r = trunc(a / q) * q;"),
    ("out_bf16_via_fp32", "double a = fabs(v);", "double a = fabs((double)(float)v);"),
    ("out_bf16_subnormal_spacing", "if (ex < -126) ex = -126;", "if (ex < -149) ex = -149;"),
    ("pair_delta_reversed", "delta[i] = ft - base;", "delta[i] = base - ft;"),
    ("pair_delta_from_base_only", "delta[i] = ft - base;", "delta[i] = ft;"),
]


def _bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _pins(lib):
    """Run the pin battery against one compiled oracle; return failing names."""
    fails = []

    def check(name, fn):
        try:
            ok = bool(fn())
        except Exception:  # a mutant may also crash a pin
            ok = False
        if not ok:
            fails.append(name)

    rows = []
    with open(os.path.join(GOLDEN, "sign_bytes.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                p = line.split()
                rows.append(([float(v) for v in p[:8]], int(p[8], 16)))
    d_g = np.array([r[0] for r in rows], dtype=np.float32)
    check("golden_bytes", lambda: [int(v) for v in oracle.pack_signs(d_g, lib)[:, 0]]
          == [r[1] for r in rows])

    rng = np.random.default_rng(31)
    d = rng.laplace(0, 1e-3, size=(12, 64)).astype(np.float32)
    check("packbits", lambda: np.array_equal(oracle.pack_signs(d, lib),
                                            np.packbits(~(d < 0), axis=1, bitorder="little")))
    check("alpha_matrix_rational", lambda: oracle.alpha(d, False, lib)[0]
          == np.float32(float(bf.alpha_exact([float(v) for v in d.ravel()]))))
    check("alpha_rows_rational", lambda: all(
        oracle.alpha(d, True, lib)[n] == np.float32(float(bf.alpha_exact([float(v) for v in d[n]])))
        for n in range(12)))

    c = 2.0 ** -10
    gen = synth.generator(32)
    w = synth.base_weight(gen, 16, 64)
    dc = torch.where(torch.rand((16, 64), generator=gen) < 0.5, -c, c).float()

    def exact_recon():
        for per_row in (False, True):
            s, a = oracle.compress(dc, per_row, lib)
            if not np.array_equal(oracle.weff(w, s, a, per_row, lib),
                                  _bits((w.float() + dc).to(torch.bfloat16))):
                return False
        return True
    check("plus_minus_c_exact", exact_recon)

    def weff_brute():
        g2 = synth.generator(33)
        wb = synth.base_weight(g2, 4, 16)
        dd = synth.laplace_delta(g2, 4, 16, 3e-3)
        for per_row in (False, True):
            s, a = oracle.compress(dd, per_row, lib)
            got = oracle.weff(wb, s, a, per_row, lib)
            wbits = _bits(wb)
            for n in range(4):
                for k in range(16):
                    bit = bf.sign_bit(float(dd[n, k]))
                    ref = bf.weff(int(wbits[n, k]), bit, float(a[n] if per_row else a[0]))
                    if bf.bf16_value(int(got[n, k])) != ref:
                        return False
        return True
    check("weff_brute_force", weff_brute)

    def matmul_alpha0():
        g3 = synth.generator(34)
        wb = synth.base_weight(g3, 8, 32)
        x = synth.activations(g3, 3, 32)
        s = np.full((8, 4), 0x3C, dtype=np.uint8)
        y = oracle.linear(x, wb, s, np.zeros(1, np.float32), False, lib)
        return np.allclose(y, x.double().numpy() @ wb.double().numpy().T, rtol=1e-12, atol=1e-12)
    check("alpha0_matmul", matmul_alpha0)

    def lattice():
        r = np.random.default_rng(35)
        n, k, m = 6, 48, 4
        wm = r.integers(-64, 65, size=(n, k))
        wb = torch.from_numpy((wm * 2.0 ** -8).astype(np.float32)).to(torch.bfloat16)
        x = torch.from_numpy(r.integers(-2, 3, size=(m, k)).astype(np.float32)).to(torch.bfloat16)
        aint = r.integers(1, 9, size=(n, 1))
        sg = np.where(r.random((n, k)) < 0.5, -1, 1)
        dd = torch.from_numpy((sg * aint * 2.0 ** -8).astype(np.float32))
        s, a = oracle.compress(dd, True, lib)
        y = oracle.linear(x, wb, s, a, True, lib)
        ref = (x.float().numpy().astype(np.int64) @ (wm + sg * aint).T) * 2.0 ** -8
        return np.array_equal(y, ref)
    check("exact_lattice", lattice)

    def grouped():
        g4 = synth.generator(36)
        wb = synth.base_weight(g4, 8, 32)
        ds = [synth.laplace_delta(g4, 8, 32, b) for b in (5e-4, 2e-3)]
        x = synth.activations(g4, 5, 32)
        comp = [oracle.compress(v, True, lib) for v in ds]
        ids = np.array([1, 0, 1, 1, 0], dtype=np.int32)
        y = oracle.linear_grouped(x, ids, wb, [q[0] for q in comp], [q[1] for q in comp], True, lib)
        # each token's row equals the dot with the torch-built reconstruction
        for t in range(5):
            dt = ds[ids[t]]
            a = comp[ids[t]][1]
            sgn = torch.where(dt < 0, -1.0, 1.0)
            weff = (wb.float() + sgn * torch.from_numpy(a)[:, None]).to(torch.bfloat16)
            ref = weff.double().numpy() @ x[t].double().numpy()
            if not np.allclose(y[t], ref, rtol=1e-12, atol=1e-12):
                return False
        return True
    check("grouped_per_token", grouped)

    def pair_exact():
        # Δ = W_ft − W_base against the exact difference rounded to fp32
        g5 = synth.generator(37)
        base = synth.base_weight(g5, 4, 32)
        ft = (base.float() + 1e-3 * torch.randn((4, 32), generator=g5)).to(torch.bfloat16)
        fb, bb = _bits(ft), _bits(base)
        d = oracle.delta_from_pair(fb, bb, lib)
        return all(Fraction(float(d[n, k])) == bf.delta_pair(int(fb[n, k]), int(bb[n, k]))
                   for n in range(4) for k in range(32))
    check("pair_exact_difference", pair_exact)

    def out_bf16_rational():
        # the bf16 output rounding against exact rational rounding
        from tests.test_oracle_pins import _f64_cases
        v = _f64_cases(seed=38, count=200)
        v = v[np.isfinite(v)]
        got = oracle.bf16_rne_f64(v, lib)
        for val, g in zip(v.tolist(), got.tolist()):
            r = bf.round_bf16(Fraction(val))
            if isinstance(r, float):
                if (g & 0x7FFF) != 0x7F80:
                    return False
            elif bf.bf16_value(g) != r:
                return False
        return True
    check("out_bf16_rational", out_bf16_rational)
    return fails


@pytest.fixture(scope="module")
def source():
    with open(oracle.oracle.SOURCE) as f:
        return f.read()


def test_unmodified_oracle_passes_battery(source, tmp_path):
    src = tmp_path / "control.c"
    src.write_text(source)
    lib = oracle.load(oracle.oracle.compile_library(str(src), str(tmp_path / "control.so")))
    assert _pins(lib) == []


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(source, tmp_path, name, old, new):
    assert source.count(old) == 1, "mutation site not unique: " + name
    src = tmp_path / (name + ".c")
    src.write_text(source.replace(old, new))
    lib = oracle.load(oracle.oracle.compile_library(str(src), str(tmp_path / (name + ".so"))))
    fails = _pins(lib)
    assert fails, "planted mistake %s passed every pin" % name
