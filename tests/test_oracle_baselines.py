"""Pins of the 4-bit comparison types (Int4, FP4) and their stored forms
(reading R19): decode tables from the bit layouts' own definitions, codes
against a brute-force exact nearest level, constructed ties, exactness of the
fp64 decision, round-trip idempotence, and the quantization error on
N(0, 0.02) weights against independently computed figures."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import baselines, nf4

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "mse_4bit_types.json")))


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def test_int4_table_is_twos_complement_over_seven():
    t = baselines.type_table("int4")
    for c in range(16):
        k = int(np.array([c << 4], dtype=np.uint8).view(np.int8)[0]) >> 4   # sign-extend the nibble
        assert t[c] == np.float32(k / 7.0)
    assert set(np.round(t[[c for c in range(16) if c != 8]] * 7).astype(int)) == set(range(-7, 8))


def test_fp4_table_is_e2m1_over_six():
    # OCP MX E2M1 element values for codes 0..7 (sign bit clear)
    e2m1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    t = baselines.type_table("fp4")
    for c in range(16):
        v = np.float32(e2m1[c & 7] / 6.0)
        assert t[c] == (-v if c & 8 else v)
        assert np.signbit(t[c]) == bool(c & 8)
    assert np.array_equal(np.sort(np.unique(np.abs(t))), np.sort(np.unique(np.float32(np.array(e2m1) / 6))))


def test_levels_and_midpoints_are_exact():
    for kind in baselines.TYPES:
        levels, code_of_level, zero = baselines.type_levels(kind)
        assert levels.size == (16 if kind == "nf4" else 15)
        assert levels[0] == -1.0 and levels[-1] == 1.0
        assert baselines.type_table(kind)[zero] == 0.0
        assert np.array_equal(baselines.type_table(kind)[code_of_level], levels)
        for m, lo, hi in zip(baselines.type_midpoints(kind), levels[:-1], levels[1:]):
            assert Fraction(m) == (Fraction(float(lo)) + Fraction(float(hi))) / 2   # exact midpoint
            mant, _ = np.frexp(abs(m))
            bits = 0 if m == 0 else len(bin(Fraction(float(mant)).limit_denominator(1 << 60).denominator)) - 3
            assert bits <= 29          # 24-bit absmax times m fits the 53-bit fp64 significand


def _brute_codes(w, kind, blocksize=64):
    """Exact nearest level of w/absmax by rational arithmetic (ties to the
    lower level), mapped to the type's code."""
    levels, code_of_level, zero = baselines.type_levels(kind)
    L = [Fraction(float(x)) for x in levels]
    out = []
    for b0 in range(0, w.size, blocksize):
        blk = w[b0:b0 + blocksize]
        a = max(abs(Fraction(float(x))) for x in blk)
        for x in blk:
            if a == 0:
                out.append(zero)
                continue
            u = Fraction(float(x)) / a
            d = [abs(u - l) for l in L]
            best = min(range(len(L)), key=lambda i: (d[i], i))
            out.append(int(code_of_level[best]))
    return np.array(out, dtype=np.uint8)


@pytest.mark.parametrize("kind", ["int4", "fp4", "nf4"])
@pytest.mark.parametrize("seed", [0, 1])
def test_codes_match_brute_force(kind, seed):
    rng = _rng(100 + seed)
    w = (rng.normal(0, 0.02, 256) * rng.choice([1.0, 1e-3, 10.0], 256)).astype(np.float32)
    w[:64] = 0.0                      # an all-zero block
    w[70] = -w[71]                    # some exact ties of opposite sign
    codes, absmax = baselines.quantize_4bit(w, kind)
    assert np.array_equal(nf4.unpack_codes(codes, w.size), _brute_codes(w, kind))
    assert np.array_equal(absmax, nf4.block_absmax(w))


@pytest.mark.parametrize("kind", ["int4", "fp4"])
def test_constructed_ties_go_to_lower_level(kind):
    levels, code_of_level, _ = baselines.type_levels(kind)
    mids = baselines.type_midpoints(kind)
    a = np.float32(0.5)  # a power of two: a * m is an fp32 value when m has <= 24 bits
    w, want = [a], [int(code_of_level[-1])]
    for j, m in enumerate(mids):
        x = np.float32(float(a) * m)
        if float(x) == float(a) * m:      # representable midpoint: an exact tie
            w.append(x)
            want.append(int(code_of_level[j]))
    w = np.array(w + [0.0] * (64 - len(w)), dtype=np.float32)
    codes = nf4.unpack_codes(baselines.quantize_4bit(w, kind)[0], 64)
    assert len(want) >= 3          # a itself plus at least two exact ties
    assert list(codes[:len(want)]) == want


@pytest.mark.parametrize("kind", baselines.TYPES)
def test_roundtrip_idempotent(kind):
    w = _rng(7).normal(0, 0.02, 64 * 600).astype(np.float32)
    codes, q8, s2, _ = baselines.quantize_all_4bit(w, kind)
    wd = baselines.dequantize_4bit(codes, q8, s2, w.size, kind, "f32")
    c2, q2, s22, _ = baselines.quantize_all_4bit(wd, kind)
    assert np.array_equal(codes, c2) and np.array_equal(q8, q2) and np.array_equal(s2, s22)


def test_nf4_stored_type_is_the_nf4_quantizer():
    w = _rng(8).normal(0, 0.02, 64 * 100).astype(np.float32)
    a = baselines.quantize_4bit(w, "nf4")
    b = nf4.quantize_nf4(w)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.fixture(scope="module")
def weights_2p20():
    return _rng(20).normal(0, GOLD["sigma"], GOLD["n"]).astype(np.float32)


@pytest.mark.parametrize("kind", ["nf4", "nf4_dq", "int4_k8", "fp4", "int4_k7"])
def test_mse_matches_independent_figures(weights_2p20, kind):
    got = baselines.mse(weights_2p20, kind)
    want = GOLD["mse"][kind]
    assert abs(got - want) <= GOLD["rel_tol"] * want, (kind, got, want)


def test_mse_order_nf4_best(weights_2p20):
    m = {k: baselines.mse(weights_2p20, k) for k in GOLD["mse"]}
    assert m["nf4"] < m["int4_k8"] < m["fp4"] < m["int4_k7"]


@pytest.mark.parametrize("kind,cmp", [("int4", "int4_k7"), ("fp4", "fp4")])
def test_stored_types_keep_the_comparison_error(weights_2p20, kind, cmp):
    """fp32 rounding of the levels changes the round-trip error by < 1e-4."""
    w = weights_2p20[: 1 << 18]
    codes, absmax = baselines.quantize_4bit(w, kind)
    wd = nf4.dequantize_fp32_absmax(codes, absmax, w.size, cb=baselines.type_table(kind)).astype(np.float64)
    d = wd - w.astype(np.float64)
    assert abs(np.mean(d * d) / baselines.mse(w, cmp) - 1) < 1e-4
