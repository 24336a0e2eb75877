"""Pins of the oracle's INT2 quantizer and packed layout.

Brute force (every code is a nearest level), closed forms (min -> 0,
max -> 3, constant group -> 0), hand-made worked examples stored under
tests/golden/, the half-step reconstruction bound, and layout bijectivity.
"""
import os

import numpy as np
import pytest

from int2_kv_cache_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "int2_quantizer_cases.txt")


def _f16(x):
    return synth.to_fp16_bits(np.asarray(x, np.float32))


def _groups(rng, n):
    """Random fp16 groups of 32 with a mix of scales, ties and constants."""
    out = []
    for i in range(n):
        kind = i % 4
        if kind == 0:
            x = rng.standard_normal(32) * np.exp2(rng.integers(-8, 8))
        elif kind == 1:
            x = rng.integers(-3, 4, 32).astype(np.float64) * 0.25   # many ties
        elif kind == 2:
            x = rng.standard_normal(32) * 0.03 + rng.standard_normal() * 0.01
        else:
            x = np.full(32, rng.standard_normal())
        out.append(_f16(x))
    return out


def test_codes_are_nearest_levels_brute_force(orc):
    rng = np.random.default_rng(11)
    for g in _groups(rng, 400):
        d, z, codes = orc.quant_group32(g)
        x = g.view(np.float16).astype(np.float64)
        if d == 0:
            assert not codes.any()
            continue
        levels = np.float64(z) + np.arange(4) * np.float64(d)
        dist = np.abs(x[:, None] - levels[None, :])
        best = dist.min(axis=1)
        mine = dist[np.arange(32), codes]
        # a tie may go either way; fp32 rounding of (x-z)/d allows ~1 ulp
        assert np.all(mine <= best + 4e-7 * (np.abs(x) + abs(float(d))) + 1e-30)


def test_extremes_map_to_0_and_3(orc):
    rng = np.random.default_rng(12)
    for g in _groups(rng, 200):
        d, z, codes = orc.quant_group32(g)
        x = g.view(np.float16).astype(np.float32)
        assert np.float32(z) == x.min()
        if d > 0:
            assert np.all(codes[x == x.min()] == 0)
            assert np.all(codes[x == x.max()] == 3)
            assert np.float32(d) == (x.max() - x.min()) / np.float32(3.0)


def test_constant_group_is_all_zero(orc):
    d, z, codes = orc.quant_group32(_f16(np.full(32, -2.75)))
    assert d == 0 and z == np.float32(-2.75) and not codes.any()


def _golden_cases():
    cases = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            xs, cs = line.split("->")
            cases.append(([float(v) for v in xs.split()], [int(v) for v in cs.split()]))
    return cases


@pytest.mark.parametrize("xs,want", _golden_cases())
def test_worked_examples(orc, xs, want):
    """Hand-derived cases (tests/golden/int2_quantizer_cases.txt): values on
    the four levels z + j*delta, and exact half-way points (ties to even)."""
    x = np.zeros(32, np.float64)
    x[:len(xs)] = xs
    x[len(xs):] = xs[0]
    d, z, codes = orc.quant_group32(_f16(x))
    assert list(codes[:len(want)]) == want


def test_reconstruction_within_half_step(orc):
    """|x - (z16 + delta16*code)| <= delta/2 plus the fp16 rounding of the
    stored step and zero point (the half-step bound of min-max rounding)."""
    rng = np.random.default_rng(13)
    for g in _groups(rng, 200):
        d, z, codes = orc.quant_group32(g)
        x = g.view(np.float16).astype(np.float64)
        d16 = np.float64(np.float16(d))
        z16 = np.float64(np.float16(z))
        rec = z16 + d16 * codes
        bound = d / 2 + abs(z - z16) + 3 * abs(d - d16) + 1e-6 * abs(d) + 1e-30
        assert np.all(np.abs(x - rec) <= bound)


def test_layout_is_a_bijection(orc):
    L = orc.lib()
    kpos = {(L.orc_kcode_byte(t, c), L.orc_kcode_shift(t, c)) for t in range(32) for c in range(128)}
    vpos = {(L.orc_vcode_byte(t, c), L.orc_vcode_shift(t, c)) for t in range(32) for c in range(128)}
    assert len(kpos) == len(vpos) == 4096
    assert all(0 <= b < 1024 and s in (0, 2, 4, 6) for b, s in kpos)
    assert all(1024 <= b < 2048 and s in (0, 2, 4, 6) for b, s in vpos)


def test_quant_pack_roundtrip(orc):
    """Codes read back from packed records equal the group quantizer's codes,
    and params land where the layout says."""
    rng = np.random.default_rng(14)
    hkv, nb = 2, 2
    khat = _f16(rng.standard_normal((32 * nb, hkv, 128)) * 0.05)
    v16 = _f16(rng.standard_normal((32 * nb, hkv, 128)))
    knorm = _f16(np.abs(rng.standard_normal(32 * nb)) + 0.5)
    rec, norm = orc.quant_pack(khat, knorm, v16)
    assert np.array_equal(norm.ravel(), knorm)
    for j in range(nb):
        for h in range(hkv):
            r = rec[j, h]
            for c in range(0, 128, 7):
                d, z, codes = orc.quant_group32(khat[32 * j:32 * j + 32, h, c])
                got = [orc.kcode_get(r, t, c) for t in range(32)]
                assert got == list(codes)
                assert r[2048 + 2 * c:2050 + 2 * c].view(np.uint16)[0] == _f16(d)[()]
                assert r[2304 + 2 * c:2306 + 2 * c].view(np.uint16)[0] == _f16(z)[()]
            for t in range(0, 32, 5):
                for g in range(4):
                    d, z, codes = orc.quant_group32(v16[32 * j + t, h, 32 * g:32 * g + 32])
                    got = [orc.vcode_get(r, t, 32 * g + i) for i in range(32)]
                    assert got == list(codes)
                    off = 2560 + 4 * (32 * g + t)
                    assert r[off:off + 4].view(np.uint16)[0] == _f16(d)[()]
                    assert r[off:off + 4].view(np.uint16)[1] == _f16(z)[()]


def test_signed_zero_minimum_is_canonical(orc):
    """A group whose minimum is zero stores zero point +0 whichever signed zero
    comes first (a parallel min must give the same bytes as a scan)."""
    for first in (-0.0, 0.0):
        x = np.full(32, 1.0)
        x[0] = first
        x[1] = -first
        d, z, codes = orc.quant_group32(_f16(x))
        assert _f16(z)[()] == 0 and codes[0] == 0 and codes[1] == 0
