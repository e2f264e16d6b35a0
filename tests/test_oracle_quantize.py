"""Pins for blockwise NF4 quantization and double quantization (readings
R2-R6) against brute force in exact rational arithmetic."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import nf4


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _brute_codes(w, blocksize=64):
    """Exact argmin over the 16 codes with Fractions; ties to the lower code."""
    c = [Fraction(float(v)) for v in nf4.codebook()]
    out = []
    for b0 in range(0, len(w), blocksize):
        blk = w[b0:b0 + blocksize]
        a = max(abs(Fraction(float(x))) for x in blk)
        for x in blk:
            if a == 0:
                out.append(7)
                continue
            u = Fraction(float(x)) / a
            d = [abs(u - cj) for cj in c]
            out.append(min(range(16), key=lambda j: (d[j], j)))
    return np.array(out, dtype=np.uint8)


def _f32_nearest(fr: Fraction) -> np.float32:
    """Correctly rounded Fraction -> fp32 (ties to even), by neighbour search."""
    f = np.float32(float(fr))
    best = None
    for cand in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        d = abs(Fraction(float(cand)) - fr)
        key = (d, int(np.array(cand, dtype=np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, cand)
    return np.float32(best[1])


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_codes_match_brute_force_argmin(seed):
    w = _rng(seed).normal(0, 0.02, 64 * 5 + 22).astype(np.float32)  # ragged tail block
    packed, absmax = nf4.quantize_nf4(w)
    got = nf4.unpack_codes(packed, w.size)
    assert np.array_equal(got, _brute_codes(w))
    for b in range(absmax.size):
        assert absmax[b] == np.abs(w[64 * b:64 * b + 64]).max()


def test_ties_go_to_lower_code_and_specials():
    c = nf4.codebook()
    m = nf4.midpoints()
    rep = [j for j in range(15) if float(np.float32(m[j])) == m[j]]
    assert rep, "some midpoints must be fp32-representable for the tie test"
    blk = np.zeros(64, dtype=np.float32)
    blk[0] = 1.0                      # absmax = 1 -> code 15
    blk[1] = -1.0                     # -absmax -> code 0
    blk[2] = 0.0                      # zero -> code 7
    for i, j in enumerate(rep):
        blk[3 + 2 * i] = np.float32(m[j])                                   # tie -> j
        blk[4 + 2 * i] = np.nextafter(np.float32(m[j]), np.float32(2.0))    # just above -> j+1
    codes = nf4.unpack_codes(nf4.quantize_nf4(blk)[0], 64)
    assert codes[0] == 15 and codes[1] == 0 and codes[2] == 7
    for i, j in enumerate(rep):
        assert codes[3 + 2 * i] == j
        assert codes[4 + 2 * i] == j + 1
    assert np.array_equal(codes, _brute_codes(blk))
    assert c[codes[3]] <= m[rep[0]]


def test_zero_block_maps_to_zero_code():
    w = np.zeros(128, dtype=np.float32)
    w[64:] = _rng(3).normal(0, 1, 64)
    codes = nf4.unpack_codes(nf4.quantize_nf4(w)[0], 128)
    assert np.all(codes[:64] == 7)
    assert codes[64:].min() == 0 or codes[64:].max() == 15


def test_every_nonzero_block_hits_an_extreme_code():
    w = _rng(4).normal(0, 0.02, 64 * 200).astype(np.float32)
    codes = nf4.unpack_codes(nf4.quantize_nf4(w)[0], w.size).reshape(-1, 64)
    assert np.all((codes == 0).any(1) | (codes == 15).any(1))


def test_packing_low_nibble_first_and_odd_n():
    assert list(nf4.pack_codes(np.array([1, 2, 3, 4, 15, 0]))) == [0x21, 0x43, 0x0F]
    with pytest.raises(ValueError):
        nf4.quantize_nf4(np.ones(63, dtype=np.float32))


def test_double_quant_matches_exact_rational_rounding():
    rng = _rng(5)
    head = (np.abs(rng.normal(0, 0.02, 256 * 3)) + 1e-3).astype(np.float32)
    # a whole group with s2 = 255 whose members are k + 1/2: exact ties -> even k
    ties = np.array([255.0] + [k + 0.5 for k in range(254)] + [3.0], dtype=np.float32)
    tail = (np.abs(rng.normal(0, 0.02, 77)) + 1e-3).astype(np.float32)   # ragged last group
    absmax = np.concatenate([head, ties, tail]).astype(np.float32)
    q8, s2 = nf4.double_quant(absmax)
    assert s2.size == -(-absmax.size // 256)
    for g in range(s2.size):
        assert s2[g] == absmax[256 * g:256 * g + 256].max()
    for b in range(absmax.size):
        sg = Fraction(float(s2[b // 256]))
        want = round(255 * Fraction(float(absmax[b])) / sg)   # Python rounds halves to even
        assert q8[b] == want, (b, absmax[b], s2[b // 256], q8[b], want)
    t0 = 256 * 3
    assert s2[3] == 255.0
    for k in range(254):
        assert q8[t0 + 1 + k] == (k if k % 2 == 0 else k + 1)


def test_double_quant_zero_group():
    q8, s2 = nf4.double_quant(np.zeros(300, dtype=np.float32))
    assert np.all(q8 == 0) and np.all(s2 == 0)


def test_dequant_scale_is_correctly_rounded():
    rng = _rng(6)
    absmax = np.abs(rng.normal(0, 0.02, 256 * 2)).astype(np.float32)
    q8, s2 = nf4.double_quant(absmax)
    scale = nf4.dequant_scales(q8, s2)
    for b in range(0, absmax.size, 7):
        exact = Fraction(int(q8[b])) * Fraction(float(s2[b // 256])) / 255
        assert scale[b] == _f32_nearest(exact)


def test_dequantize_brute_force():
    rng = _rng(7)
    w = rng.normal(0, 0.02, 64 * 9).astype(np.float32)
    codes, q8, s2, _ = nf4.quantize_all(w)
    d32 = nf4.dequantize(codes, q8, s2, w.size, "f32")
    d16 = nf4.dequantize(codes, q8, s2, w.size, "bf16")
    c = nf4.codebook()
    idx = nf4.unpack_codes(codes, w.size)
    for i in range(0, w.size, 5):
        b = i // 64
        s = _f32_nearest(Fraction(int(q8[b])) * Fraction(float(s2[b // 256])) / 255)
        prod = _f32_nearest(Fraction(float(c[idx[i]])) * Fraction(float(s)))
        assert d32[i] == prod
        # bf16: nearest-even with 8 significant bits
        fr = Fraction(float(prod))
        cands = sorted(set(float(np.float32(v)) for v in _bf16_neighbours(prod)))
        best = min(cands, key=lambda v: (abs(Fraction(v) - fr), _bf16_lsb(v)))
        assert d16[i] == np.float32(best)


def _bf16_neighbours(x):
    u = int(np.array(x, dtype=np.float32).view(np.uint32))
    lo = u & 0xFFFF0000
    for v in (lo, lo + 0x10000):
        yield np.array(v & 0xFFFFFFFF, dtype=np.uint32).view(np.float32)


def _bf16_lsb(v):
    return (int(np.array(v, dtype=np.float32).view(np.uint32)) >> 16) & 1


def test_roundtrip_idempotent_fp32():
    """quantize -> dequantize (fp32) -> quantize reproduces codes, q8 and s2."""
    w = _rng(8).normal(0, 0.02, 1 << 16).astype(np.float32)
    codes, q8, s2, _ = nf4.quantize_all(w)
    wd = nf4.dequantize(codes, q8, s2, w.size, "f32")
    codes2, q82, s22, _ = nf4.quantize_all(wd)
    assert np.array_equal(codes, codes2) and np.array_equal(q8, q82) and np.array_equal(s2, s22)


def test_roundtrip_via_bf16_keeps_codes():
    w = _rng(9).normal(0, 0.02, 1 << 16).astype(np.float32)
    codes, q8, s2, _ = nf4.quantize_all(w)
    wd = nf4.dequantize(codes, q8, s2, w.size, "bf16")
    codes2, q82, _, _ = nf4.quantize_all(wd)
    assert np.array_equal(codes, codes2)
    assert np.abs(q8.astype(int) - q82.astype(int)).max() <= 1


def test_bf16_rounding_ties_to_even():
    x = np.array([1.00390625, 1.01171875, 1.0 + 2 ** -8 + 2 ** -20, -3.0], dtype=np.float32)
    bits = nf4.f32_to_bf16_bits(x)
    assert list(bits) == [0x3F80, 0x3F82, 0x3F81, 0xC040]
