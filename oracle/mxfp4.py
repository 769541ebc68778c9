"""CPU oracle: MXFP4 output encoding - TEST INFRASTRUCTURE.

The call's output may be an FP4 tensor with block scale factors instead of a
dense one (FlashInfer API page for trtllm_batch_context_with_kv_cache,
parameters ``out``, ``out_dtype`` (the FP4 string), ``o_sf_scale`` - a scale
applied to the output's scale factors - and ``o_sf_vec_size`` - the number of
elements one scale factor covers).  The pages name NVIDIA's FP4 format and
define nothing further; this library re-targets the output to the OCP
Microscaling (MX) FP4 format that gfx950 supports, and takes these readings:

* element format E2M1: 1 sign, 2 exponent bits (bias 1), 1 mantissa bit, no
  infinities or NaN; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6;
* scale format E8M0: byte b stands for 2^(b - 127), 255 for NaN;
* one scale per ``vec`` consecutive elements of a row along head_dim (the
  OCP format fixes 32; 16 is accepted as well);
* block scale 2^E with E = floor(log2(amax)) - 2, where 2 is the exponent of
  E2M1's largest normal value, and E clamped below at -127 (so an all-zero
  block gets byte 0);  an infinite amax gives the NaN scale byte;
* element code = the nearest E2M1 value to y / 2^E, ties to the even code,
  magnitudes above 6 saturated to 6, the sign bit copied from y (so -0
  encodes as the code for -0); a NaN element, which E2M1 cannot hold,
  converts like an infinity of its sign, to +-6 (the convention of a
  saturating conversion);
* ``o_sf_scale`` = g multiplies the output before blocking,
  y = fp32(fp32(o) * g): the scale factors of g*o are g times those of o,
  and a reader dequantizes as code * 2^E / g;
* two codes per byte, element 2i in the low nibble; scale bytes in a plain
  [tokens, heads, head_dim / vec] array.

The amax and the scale exponent are taken in fp32, the precision the kernel
decides them in: floor(log2(amax)) is read from the fp32 exponent field.
"""
from __future__ import annotations

import numpy as np

E2M1_MAX = 6.0


def e2m1_value(code: int) -> float:
    """Value of a 4-bit E2M1 code from its bit fields: sign bit 3, exponent
    bits 2..1 with bias 1, mantissa bit 0; exponent 0 is subnormal
    (m * 0.5)."""
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    mag = m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 2.0)
    return -mag if s else mag


E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)


def encode_e2m1(v: np.ndarray) -> np.ndarray:
    """Real values -> E2M1 codes (uint8 0..15): nearest representable
    magnitude, ties to the even code, saturated at 6 (NaN as well); the sign
    bit is the sign bit of v."""
    v = np.asarray(v, dtype=np.float64)
    grid = E2M1_TABLE[:8]                          # codes 0..7, ascending 0..6
    a = np.where(np.isnan(v), E2M1_MAX, np.minimum(np.abs(v), E2M1_MAX))
    hi = np.clip(np.searchsorted(grid, a, side="left"), 0, 7)
    lo = np.clip(hi - 1, 0, 7)
    d_lo = a - grid[lo]
    d_hi = grid[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(v), code | np.uint8(8), code).astype(np.uint8)


def e8m0_value(byte) -> np.ndarray:
    """E8M0 scale byte -> 2^(b - 127); 255 -> NaN."""
    b = np.asarray(byte, dtype=np.int64)
    return np.where(b == 255, np.nan, np.ldexp(1.0, (b - 127).astype(np.int32)))


def mx_scale_byte(amax) -> np.ndarray:
    """E8M0 byte of the block scale for block maxima ``amax`` (fp32 values):
    E = floor(log2(amax)) - 2 clamped to >= -127, stored as E + 127; 255 for
    an infinite or NaN amax."""
    a = np.asarray(amax, dtype=np.float32)
    bits = np.atleast_1d(a).view(np.uint32)
    expfield = ((bits >> 23) & 0xFF).astype(np.int64).reshape(a.shape)
    # a normal amax has floor(log2(amax)) = expfield - 127, so the byte
    # E + 127 is expfield - 2; zero and subnormal maxima fall to the clamp
    byte = np.maximum(expfield - 2, 0)
    return np.where(expfield == 255, 255, byte).astype(np.uint8)


def quantize_mxfp4(y: np.ndarray, vec: int):
    """fp32 rows ``y`` [..., D] -> (packed codes uint8 [..., D/2], scale bytes
    uint8 [..., D/vec]).  Blocks are ``vec`` consecutive elements of the last
    axis."""
    y = np.asarray(y, dtype=np.float32)
    d = y.shape[-1]
    assert d % vec == 0 and vec % 2 == 0
    blocks = y.reshape(y.shape[:-1] + (d // vec, vec))
    absb = np.abs(blocks)
    amax = np.where(np.isnan(absb), np.float32(0), absb).max(axis=-1).astype(np.float32)
    sbyte = mx_scale_byte(amax)
    e = sbyte.astype(np.int64) - 127
    scaled = blocks.astype(np.float64) * np.ldexp(1.0, (-e).astype(np.int32))[..., None]
    codes = encode_e2m1(scaled)
    codes = np.where((sbyte == 255)[..., None], np.uint8(0), codes).astype(np.uint8)
    codes = codes.reshape(y.shape)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return packed, sbyte


def unpack_e2m1(packed: np.ndarray) -> np.ndarray:
    """Packed bytes [..., D/2] -> codes [..., D] (low nibble first)."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def dequantize_mxfp4(packed: np.ndarray, sbytes: np.ndarray, vec: int, o_sf_scale: float = 1.0) -> np.ndarray:
    """code * 2^E / g for every element (float64)."""
    codes = unpack_e2m1(packed)
    vals = E2M1_TABLE[codes]
    d = vals.shape[-1]
    scale = e8m0_value(sbytes)                      # [..., D/vec]
    vals = vals.reshape(vals.shape[:-1] + (d // vec, vec)) * scale[..., None]
    return vals.reshape(codes.shape) / float(o_sf_scale)


def mxfp4_output(o: np.ndarray, vec: int, o_sf_scale: float = 1.0):
    """The call's MXFP4 output for attention output ``o`` (any float array,
    [..., D]): y = fp32(fp32(o) * fp32(g)), then ``quantize_mxfp4``."""
    y = (np.asarray(o, dtype=np.float64).astype(np.float32) * np.float32(o_sf_scale)).astype(np.float32)
    return quantize_mxfp4(y, vec)
