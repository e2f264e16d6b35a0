"""NF4 encoding oracle: codebook, blockwise quantization, double quantization,
dequantization.  TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix:
  * NF4 is a 4-bit data type that is information-theoretically optimal for
    normally distributed weights ("QLoRA: Efficient Finetuning of Quantized
    LLMs", fugumt.com paper page, Abstract item (a); the news write-up's
    innovations list).
  * Double quantization quantizes the quantization constants themselves and
    saves about 0.37 bit per parameter (Abstract item (b); innovations list).
  * Weights are computed in bf16 (QLoRA project page, configuration example:
    4-bit load, 'nf4', double quantization on, bf16 compute dtype).

Readings taken where the pages are silent:
  R1  Codebook: 7 negative values, an exact zero and 8 positive values, each
      the standard-normal quantile at probabilities equally spaced on
      [1/2, p_max] (8 steps on the positive side, 7 on the negative side),
      with p_max = 1 - (1/30 + 1/32)/2, divided by Q(p_max) so that the
      extremes are exactly -1 and +1, sorted and rounded to fp32.
  R2  Blocks: the weight is flattened row-major; block b holds elements
      [64b, 64b+64); absmax_b is the exact fp32 maximum of |w| in the block.
  R3  Code choice: the code nearest to w/absmax_b in exact arithmetic;
      ties (w exactly on a midpoint) go to the lower code; absmax_b == 0 maps
      every element of the block to the zero code 7.
  R4  Packing: byte i = code(2i) | code(2i+1) << 4 (low nibble first).
  R5  Double quantization: group g holds absmax values [256g, 256g+256);
      s2_g is their exact fp32 maximum; q8_b is the integer nearest to
      255 * absmax_b / s2_g (ties to even), or 0 when s2_g == 0.
  R6  Dequantization: c1'_b = fp32(q8_b * s2_g / 255) rounded once to nearest;
      the fp32 weight is fp32(c[code] * c1'_b) (one fp32 multiply); the bf16
      compute weight is that value rounded to nearest-even bf16.
"""

from __future__ import annotations

import statistics

import numpy as np

BLOCK = 64     # elements per first-level absmax block (R2)
BLOCK2 = 256   # first-level constants per second-level group (R5)
ZERO_CODE = 7  # index of the exact zero in the sorted codebook (R1)

# p_max of R1, evaluated in fp64 exactly as written.
P_MAX = 1.0 - (1.0 / 30.0 + 1.0 / 32.0) / 2.0


def _quantile_positions():
    """Probabilities of R1, in fp64: (positive side, negative side)."""
    step_pos = (P_MAX - 0.5) / 8.0
    step_neg = (P_MAX - 0.5) / 7.0
    pos = [P_MAX - j * step_pos for j in range(8)]
    neg = [P_MAX - j * step_neg for j in range(7)]
    return pos, neg


def codebook(inv_cdf=None) -> np.ndarray:
    """The 16 NF4 values (R1), ascending, as float32.

    ``inv_cdf`` is the standard-normal quantile function; the default is the
    Python standard library's ``NormalDist().inv_cdf``.  Tests pass a second,
    independent implementation and require the same fp32 bit patterns.
    """
    q = inv_cdf if inv_cdf is not None else statistics.NormalDist().inv_cdf
    pos, neg = _quantile_positions()
    top = q(P_MAX)
    values = [q(p) / top for p in pos] + [-q(p) / top for p in neg] + [0.0]
    values.sort()
    return np.array(values, dtype=np.float64).astype(np.float32)


def midpoints(cb: np.ndarray | None = None) -> np.ndarray:
    """Decision boundaries m_j = (c_j + c_{j+1}) / 2, j = 0..14, in fp64.

    The sum of two fp32 values of magnitude <= 1 is exact in fp64 and halving
    is exact, so every m_j is the exact real midpoint.
    """
    c = (codebook() if cb is None else cb).astype(np.float64)
    return (c[:-1] + c[1:]) / 2.0


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to nearest-even bfloat16; return the uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return (u & np.uint64(0xFFFF)).astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x) -> np.ndarray:
    """float32 -> nearest-even bfloat16 value, returned as float32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """R4: two 4-bit codes per byte, element 2i in the low nibble."""
    codes = np.asarray(codes, dtype=np.uint8).ravel()
    if codes.size % 2:
        raise ValueError("number of codes must be even")
    return (codes[0::2] | (codes[1::2] << np.uint8(4))).astype(np.uint8)


def unpack_codes(packed: np.ndarray, n: int) -> np.ndarray:
    """Inverse of pack_codes: returns n codes as uint8."""
    packed = np.asarray(packed, dtype=np.uint8).ravel()
    out = np.empty(packed.size * 2, dtype=np.uint8)
    out[0::2] = packed & np.uint8(0x0F)
    out[1::2] = packed >> np.uint8(4)
    return out[:n]


def block_absmax(w: np.ndarray, blocksize: int = BLOCK) -> np.ndarray:
    """R2: exact fp32 max |w| per block of ``blocksize`` (tail block partial)."""
    w = np.ascontiguousarray(w, dtype=np.float32).ravel()
    nb = -(-w.size // blocksize)
    padded = np.zeros(nb * blocksize, dtype=np.float32)  # |0| never raises a max
    padded[: w.size] = np.abs(w)
    return padded.reshape(nb, blocksize).max(axis=1)


def nearest_codes(w: np.ndarray, absmax_per_elem: np.ndarray, cb=None) -> np.ndarray:
    """R3: code = #{j : w > absmax * m_j}, decided exactly in fp64.

    absmax (24-bit significand) times m_j (at most 26 significant bits: the
    sum of two fp32 values one binade apart, halved) fits the 53-bit fp64
    significand, so every product and comparison is exact and "nearest, ties
    to the lower code" is decided without rounding.
    """
    m = midpoints(cb)
    w64 = np.asarray(w, dtype=np.float32).astype(np.float64)
    a64 = np.asarray(absmax_per_elem, dtype=np.float32).astype(np.float64)
    code = np.zeros(w64.shape, dtype=np.int64)
    for j in range(m.size):
        code += w64 > a64 * m[j]
    code[a64 == 0.0] = ZERO_CODE
    return code.astype(np.uint8)


def quantize_nf4(w, blocksize: int = BLOCK, cb=None):
    """Blockwise NF4 quantization (R2-R4).

    w: float32 array of n elements (any shape; flattened row-major), n even.
    Returns (packed codes uint8[n/2], absmax float32[ceil(n/64)]).
    """
    w = np.ascontiguousarray(w, dtype=np.float32).ravel()
    if w.size % 2:
        raise ValueError("n must be even")
    absmax = block_absmax(w, blocksize)
    per_elem = np.repeat(absmax, blocksize)[: w.size]
    codes = nearest_codes(w, per_elem, cb)
    return pack_codes(codes), absmax


def double_quant(absmax, blocksize2: int = BLOCK2):
    """R5: 8-bit quantization of the absmax constants with one fp32 scale per
    group of 256.

    Returns (q8 uint8[nb], s2 float32[ceil(nb/256)]).

    The nearest integer k to v = 255*c/s2 is found exactly: a first guess
    k0 = floor(fl(v)) is within one of the answer, and the choice between k0
    and k0+1 compares 510*c with (2*k0+1)*s2, both exact in fp64 (at most
    9 + 24 significant bits).  Equality is a tie and goes to the even integer.
    """
    c = np.ascontiguousarray(absmax, dtype=np.float32).ravel()
    s2 = block_absmax(c, blocksize2)  # constants are >= 0, so |c| = c
    s2_e = np.repeat(s2, blocksize2)[: c.size].astype(np.float64)
    c64 = c.astype(np.float64)
    q = np.zeros(c.size, dtype=np.int64)
    nz = s2_e > 0.0
    k0 = np.floor(255.0 * c64[nz] / s2_e[nz]).astype(np.int64)
    lhs = 510.0 * c64[nz]
    rhs = (2.0 * k0 + 1.0) * s2_e[nz]
    up = (lhs > rhs) | ((lhs == rhs) & (k0 % 2 == 1))
    q[nz] = k0 + up
    if q.min(initial=0) < 0 or q.max(initial=0) > 255:
        raise AssertionError("q8 out of range")
    return q.astype(np.uint8), s2


def dequant_scales(q8, s2, blocksize2: int = BLOCK2) -> np.ndarray:
    """R6: c1'_b = fp32(q8_b * s2_g / 255), rounded once.

    q8*s2 is exact in fp64 (8 + 24 bits); the fp64 quotient by 255 is then
    rounded to fp32.  That double rounding cannot differ from a single
    rounding: a quotient P/255 with a 32-bit P is never an fp32 halfway point
    and lies at least 2**-40 (relative) away from one, far more than the
    2**-53 fp64 error.
    """
    q8 = np.asarray(q8, dtype=np.uint8).ravel().astype(np.float64)
    s2_e = np.repeat(np.asarray(s2, dtype=np.float32), blocksize2)[: q8.size].astype(np.float64)
    return (q8 * s2_e / 255.0).astype(np.float32)


def dequantize(codes, q8, s2, n: int, dtype: str = "bf16", cb=None,
               blocksize: int = BLOCK, blocksize2: int = BLOCK2) -> np.ndarray:
    """R6: dequantized weights as float32 (bf16-exact values when dtype='bf16')."""
    c = codebook() if cb is None else cb
    scale = dequant_scales(q8, s2, blocksize2)
    idx = unpack_codes(codes, n)
    per_elem = np.repeat(scale, blocksize)[:n]
    w32 = c[idx].astype(np.float32) * per_elem.astype(np.float32)  # one fp32 multiply
    if dtype == "f32":
        return w32
    if dtype == "bf16":
        return bf16_round(w32)
    raise ValueError(dtype)


def dequantize_fp32_absmax(codes, absmax, n: int, cb=None, blocksize: int = BLOCK) -> np.ndarray:
    """Dequantization with the un-quantized fp32 absmax (no double quant)."""
    c = codebook() if cb is None else cb
    idx = unpack_codes(codes, n)
    per_elem = np.repeat(np.asarray(absmax, dtype=np.float32), blocksize)[:n]
    return c[idx].astype(np.float32) * per_elem


def quantize_all(w, cb=None):
    """Quantize + double quant in one call: (codes, q8, s2, absmax)."""
    codes, absmax = quantize_nf4(w, cb=cb)
    q8, s2 = double_quant(absmax)
    return codes, q8, s2, absmax


def storage_bytes(n: int, double_quant_on: bool = True) -> int:
    """Bytes of the stored format for n weights (codes + constants)."""
    nb = -(-n // BLOCK)
    if not double_quant_on:
        return n // 2 + 4 * nb
    ng = -(-nb // BLOCK2)
    return n // 2 + nb + 4 * ng


def n_blocks(n: int) -> int:
    return -(-n // BLOCK)


def n_groups(nb: int) -> int:
    return -(-nb // BLOCK2)

