"""CPU oracle for fp8 (e4m3) expert weights with per-block scales.

TEST INFRASTRUCTURE ONLY, like moe_oracle: only the tests, the smoke check and the
bench's CPU leg may use it; it shares no code with the HIP library.

What it follows.  The course notes "Dropless and grouped GEMM" (topic-01-dropless),
section 12, describe fp8 expert weights that carry a scale per quantisation block,
and the choice between scaling after the matrix product and dequantising before it
(dequantise first when the quantisation block is narrower than the matrix unit's
contraction depth).  The notes name the format "fp8" and the block "128 elements of
the contraction dimension" without fixing the rest; the readings taken here (also
listed in the design notes):
  * the fp8 format is the OCP 8-bit floating point E4M3 ("e4m3fn"): 1 sign bit, 4
    exponent bits with bias 7, 3 mantissa bits, subnormals at exponent 0, no
    infinities, the all-ones exponent-and-mantissa pattern is NaN, largest finite
    value 448;
  * a scale covers a 128 (contraction) x 128 (output column) block of one expert's
    weight matrix; partial blocks at the edges have their own scale;
  * the scale is amax / 448 in fp32 (amax = largest magnitude in the block), 1 for an
    all-zero block; a code is w / scale computed in fp32, clamped to [-448, 448] and
    rounded to the nearest e4m3 value, ties to the even mantissa;
  * the dequantised weight is code value * scale, exactly (fp64 here).
The codes are integers decided by floating point, so the quantiser works in fp32 as
the device does; everything after dequantisation is the fp64 definition.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
BLOCK = 128


def e4m3_decode(codes):
    """Value of each e4m3 code (uint8 array) as float64; NaN for 0x7F / 0xFF."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    subnormal = np.ldexp(m / 8.0, -6)
    v = sign * np.where(e == 0, subnormal, normal)
    return np.where(((c & 0x7F) == 0x7F), np.nan, v)


def _positive_grid():
    """The 127 non-negative finite e4m3 values with their codes, ascending."""
    codes = np.arange(0x7F, dtype=np.int64)          # 0x00 .. 0x7E
    return e4m3_decode(codes), codes


def e4m3_encode(x):
    """Nearest e4m3 code of each value, ties to the even mantissa (even code), values
    beyond +-448 saturated.  The sign of zero is kept."""
    x = np.asarray(x, dtype=np.float64)
    vals, codes = _positive_grid()
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(vals, a, side="left")        # first grid value >= a
    hi = np.minimum(hi, len(vals) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - vals[lo]
    d_hi = vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (codes[hi] % 2 == 0))
    exact = vals[hi] == a
    out = np.where(exact | pick_hi, codes[hi], codes[lo])
    neg = np.signbit(x)
    return (out | np.where(neg, 0x80, 0)).astype(np.uint8)


def block_scales(w, block: int = BLOCK):
    """fp32 scale of every (k-block, n-block) of each expert matrix w [E, K, N]."""
    w = np.asarray(w, dtype=np.float32)
    E, K, N = w.shape
    kb, nb = -(-K // block), -(-N // block)
    s = np.ones((E, kb, nb), dtype=np.float32)
    for e in range(E):
        for i in range(kb):
            for j in range(nb):
                amax = np.float32(np.abs(w[e, i * block:(i + 1) * block,
                                            j * block:(j + 1) * block]).max())
                if amax > 0:
                    s[e, i, j] = amax / np.float32(E4M3_MAX)
    return s


def quantize(w, block: int = BLOCK):
    """(codes uint8 [E, K, N], scales fp32 [E, ceil(K/128), ceil(N/128)])."""
    w = np.asarray(w, dtype=np.float32)
    s = block_scales(w, block)
    full = np.repeat(np.repeat(s, block, axis=1), block, axis=2)[:, :w.shape[1], :w.shape[2]]
    r = np.clip(w / full, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))   # fp32 division
    return e4m3_encode(r), s


def dequantize(codes, scales, block: int = BLOCK):
    """fp64 weights: code value * its block's scale."""
    codes = np.asarray(codes, dtype=np.uint8)
    E, K, N = codes.shape
    full = np.repeat(np.repeat(np.asarray(scales, np.float64), block, axis=1), block,
                     axis=2)[:, :K, :N]
    table = e4m3_decode(np.arange(256))            # the value of every code
    return table[codes] * full
