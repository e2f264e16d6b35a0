"""4-bit comparison data types (Int4, FP4) and quantization error, in fp64.
TEST INFRASTRUCTURE ONLY.

The pages state that NF4 gives better results than 4-bit integers and 4-bit
floats (news write-up, innovations list and the NF4-vs-FP4 section; project
page, core innovations).  Reading R11 fixes the comparison types:
  * Int4, symmetric absmax with the 15 levels k/7, k = -7..7 (and the 16-level
    two's-complement variant k/8, k = -8..7);
  * FP4 as E2M1 with magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6} / 6 and a sign;
all with the same block of 64 and nearest rounding (ties to the lower value).
"""

from __future__ import annotations

import numpy as np

from .nf4 import BLOCK, block_absmax, codebook, quantize_all, dequantize, dequantize_fp32_absmax, quantize_nf4


def _nearest_level(u: np.ndarray, levels: np.ndarray) -> np.ndarray:
    """Nearest value of the sorted ``levels`` to each u (ties to the lower)."""
    levels = np.asarray(levels, dtype=np.float64)
    mids = (levels[:-1] + levels[1:]) / 2.0
    idx = np.searchsorted(mids, u, side="left")
    return levels[idx]


def _blockwise(w, levels, blocksize=BLOCK):
    w = np.ascontiguousarray(w, dtype=np.float64).ravel()
    a = np.repeat(block_absmax(w.astype(np.float32), blocksize).astype(np.float64), blocksize)[: w.size]
    u = np.divide(w, a, out=np.zeros_like(w), where=a > 0)
    return _nearest_level(u, levels) * a


def int4_levels(variant: str = "k7") -> np.ndarray:
    if variant == "k7":
        return np.arange(-7, 8, dtype=np.float64) / 7.0
    if variant == "k8":
        return np.arange(-8, 8, dtype=np.float64) / 8.0
    raise ValueError(variant)


def fp4_levels() -> np.ndarray:
    mag = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]) / 6.0
    return np.unique(np.concatenate([-mag, mag]))


def roundtrip(w, kind: str) -> np.ndarray:
    """Quantize-dequantize w with one of the 4-bit types; fp64 result."""
    w32 = np.ascontiguousarray(w, dtype=np.float32).ravel()
    if kind == "nf4":
        codes, absmax = quantize_nf4(w32)
        return dequantize_fp32_absmax(codes, absmax, w32.size).astype(np.float64)
    if kind == "nf4_dq":
        codes, q8, s2, _ = quantize_all(w32)
        return dequantize(codes, q8, s2, w32.size, dtype="f32").astype(np.float64)
    if kind == "int4_k7":
        return _blockwise(w32, int4_levels("k7"))
    if kind == "int4_k8":
        return _blockwise(w32, int4_levels("k8"))
    if kind == "fp4":
        return _blockwise(w32, fp4_levels())
    raise ValueError(kind)


def mse(w, kind: str) -> float:
    w64 = np.ascontiguousarray(w, dtype=np.float32).ravel().astype(np.float64)
    d = roundtrip(w, kind) - w64
    return float(np.mean(d * d))


def nf4_levels() -> np.ndarray:
    return codebook().astype(np.float64)


# ---------------------------------------------------------------------------
# The comparison types as stored 4-bit formats (the GPU path's Int4 and FP4).
#
# Reading R19: a stored 4-bit type is a 16-entry fp32 decode table, exactly
# like the NF4 codebook, so quantization, double quantization and the
# dequantize rule c[code] * c1' are the same for every type and only the
# table differs.  The comparison levels above are rounded to fp32 for it:
#   * int4: code = k mod 16 (4-bit two's complement), value fp32(k / 7),
#     k = -7..7; code 8 (k = -8) is never produced and decodes to fp32(-8/7);
#   * fp4:  OCP E2M1, code = sign << 3 | exponent << 1 | mantissa, value
#     (-1)^sign * fp32(magnitude / 6) with magnitudes 0, 0.5, 1, 1.5, 2, 3,
#     4, 6; code 8 (-0) is never produced (zero is stored as code 0).
# The code of a weight is the level nearest to w / absmax in exact
# arithmetic among the type's distinct levels (ties to the lower level),
# decided as for NF4 by counting the midpoints m_j with w > absmax * m_j;
# an all-zero block gets the code of the value 0.
# ---------------------------------------------------------------------------

TYPES = ("nf4", "int4", "fp4")


def _e2m1_magnitude(c3: int) -> float:
    """OCP E2M1 magnitude of the 3 low bits: exponent bits 2..1, mantissa bit 0,
    exponent bias 1, subnormal when the exponent field is 0."""
    e, m = (c3 >> 1) & 3, c3 & 1
    return m * 0.5 if e == 0 else (1.0 + 0.5 * m) * 2.0 ** (e - 1)


def type_table(kind: str) -> np.ndarray:
    """The 16 fp32 decode values of a stored 4-bit type, indexed by code."""
    if kind == "nf4":
        return codebook()
    if kind == "int4":
        return np.array([np.float32((c if c < 8 else c - 16) / 7.0) for c in range(16)], dtype=np.float32)
    if kind == "fp4":
        top = _e2m1_magnitude(7)
        vals = []
        for c in range(16):
            v = np.float32(_e2m1_magnitude(c & 7) / top)
            vals.append(-v if c & 8 else v)
        return np.array(vals, dtype=np.float32)
    raise ValueError(kind)


def type_levels(kind: str):
    """(sorted distinct fp32 levels, code of each level, code of the value 0)."""
    table = type_table(kind)
    codes = [c for c in range(16) if not (kind == "int4" and c == 8) and not (kind == "fp4" and c == 8)]
    order = sorted(codes, key=lambda c: float(table[c]))
    levels = np.array([table[c] for c in order], dtype=np.float32)
    if np.any(np.diff(levels.astype(np.float64)) <= 0):
        raise AssertionError("levels must be distinct")
    zero = [c for c in order if table[c] == 0.0]
    return levels, np.array(order, dtype=np.uint8), int(zero[0])


def type_midpoints(kind: str) -> np.ndarray:
    """Exact fp64 midpoints of neighbouring levels (sums of two fp32 values
    within a few binades are exact in fp64, and halving is exact)."""
    levels, _, _ = type_levels(kind)
    l64 = levels.astype(np.float64)
    return (l64[:-1] + l64[1:]) / 2.0


def quantize_4bit(w, kind: str, blocksize: int = BLOCK):
    """Blockwise quantization to a stored 4-bit type (R2, R4, R19):
    (packed codes uint8[n/2], absmax float32[ceil(n/64)])."""
    from .nf4 import pack_codes
    w = np.ascontiguousarray(w, dtype=np.float32).ravel()
    if w.size % 2:
        raise ValueError("n must be even")
    absmax = block_absmax(w, blocksize)
    a64 = np.repeat(absmax, blocksize)[: w.size].astype(np.float64)
    w64 = w.astype(np.float64)
    _, code_of_level, zero = type_levels(kind)
    idx = np.zeros(w.size, dtype=np.int64)
    for m in type_midpoints(kind):
        idx += w64 > a64 * m            # exact: <= 24 + 29 significant bits
    codes = code_of_level[idx]
    codes[a64 == 0.0] = zero
    return pack_codes(codes), absmax


def quantize_all_4bit(w, kind: str):
    """Quantize + double quant to a stored 4-bit type: (codes, q8, s2, absmax)."""
    from .nf4 import double_quant
    codes, absmax = quantize_4bit(w, kind)
    q8, s2 = double_quant(absmax)
    return codes, q8, s2, absmax


def dequantize_4bit(codes, q8, s2, n: int, kind: str, dtype: str = "bf16") -> np.ndarray:
    """R6 with the type's table."""
    return dequantize(codes, q8, s2, n, dtype=dtype, cb=type_table(kind))
