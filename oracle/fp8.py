"""OCP FP8 E4M3 codec and 1 x 128 block quantisation, from their definitions.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Sources.  Block quantisation: Perplexity, "Lower latency and higher throughput
with multi-node DeepSeek deployment", section "Quantization" -- activations
get one scale per 128-element vector computed on the fly, weights are
quantised ahead of time; the SiLU kernel of the same section splits the
activation into 128-wide blocks and takes each block's absolute maximum.
The pages do not define the 8-bit format; the reading used here is the OCP
E4M3 ("fn") encoding: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
bits, subnormals below 2**-6, no infinities, 0x7F/0xFF are NaN, so the
largest finite magnitude is 448.  Encoding rounds to the nearest
representable value with ties to the even code and saturates at +-448.
The block scale is ``fp32(amax / 448)`` (1 for an all-zero block) and a value
v is encoded as ``e4m3(fp32(v / scale))``.

Pins (tests/test_oracle_pins.py, the fp8 section): torch's ``float8_e4m3fn`` cast, a brute
force nearest-code search, and hand-derived values.
"""

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 code (uint8 array) as fp64, from the bit fields."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    man = c & 0x7
    sub = man.astype(np.float64) * 2.0 ** -9                       # exponent field 0
    nrm = (1.0 + man / 8.0) * np.exp2(exp.astype(np.float64) - 7.0)  # exponent field 1..15
    val = np.where(exp == 0, sub, nrm)
    val = np.where((exp == 15) & (man == 7), np.nan, val)
    return sign * val


# All non-negative finite magnitudes, indexed by code 0x00..0x7E (increasing).
_MAGS = e4m3_decode(np.arange(0x7F, dtype=np.uint8))


def e4m3_encode(v) -> np.ndarray:
    """Round fp64 values to E4M3 codes: nearest magnitude, ties to the even
    code, saturating at 448.  The sign bit is kept for values that round to
    zero (so -tiny encodes as 0x80)."""
    v = np.asarray(v, dtype=np.float64)
    if np.isnan(v).any():
        raise ValueError("NaN has no saturating E4M3 encoding in this oracle")
    a = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.searchsorted(_MAGS, a, side="left")          # first magnitude >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _MAGS[lo]
    d_hi = _MAGS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == _MAGS[hi], hi, code)            # exact hits
    sign = np.where(np.signbit(v), 0x80, 0)
    return (code | sign).astype(np.uint8)


def quantize_rows_fp8(a, block: int = 128):
    """Quantise each row of ``a`` [m, K] in blocks of ``block`` columns.

    Returns (codes uint8 [m, K], scales fp64 [m, K // block] holding fp32
    values, dequantised values fp64 [m, K] = decode(code) * scale).
    """
    a = np.asarray(a, dtype=np.float64)
    m, kdim = a.shape
    if kdim % block:
        raise ValueError("row length must be a multiple of the block width")
    ab = a.reshape(m, kdim // block, block)
    amax = np.abs(ab).max(axis=2)
    scale = (amax / E4M3_MAX).astype(np.float32).astype(np.float64)
    scale = np.where(amax == 0.0, 1.0, scale)
    ratio = (ab / scale[:, :, None]).astype(np.float32).astype(np.float64)
    codes = e4m3_encode(ratio)
    deq = e4m3_decode(codes) * scale[:, :, None]
    return codes.reshape(m, kdim), scale, deq.reshape(m, kdim)


# Value of every code, from the bit fields above (a lookup table for speed).
_DECODE_TABLE = e4m3_decode(np.arange(256, dtype=np.uint8))


def dequantize_weight(codes, scales, block: int = 128, block_rows: int = 1) -> np.ndarray:
    """[N, K] E4M3 codes with fp32 scales -> fp64 values: code value times the
    scale of its block of ``block_rows`` x ``block`` (row r, column c use
    scales[r // block_rows, c // block]).  block_rows = 1 is one scale per row
    per block; 128 is the 128 x 128 weight tiles of [PPLX] "Quantization"."""
    codes = np.asarray(codes, dtype=np.uint8)
    n, kdim = codes.shape
    s = np.asarray(scales, dtype=np.float64).reshape(n // block_rows, kdim // block)
    s_rows = np.repeat(s, block_rows, axis=0)                        # [N, K // block]
    return (_DECODE_TABLE[codes].reshape(n, kdim // block, block) * s_rows[:, :, None]).reshape(n, kdim)
