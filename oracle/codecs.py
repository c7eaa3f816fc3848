"""Scalar codecs of the mixed-format KV cache, written from their definitions.

TEST INFRASTRUCTURE.  This module belongs to the CPU oracle.  Only the test
suite, the smoke check and the benchmark's CPU-baseline leg may import it; the
library's decode path never does.

What the pages fix and what is read here
----------------------------------------
The Minima-KV summary (brainszone.ai, pt and fr editions), section
"Ancoras em FP8, arquivo em TQ3", says that recent and anchor pages stay in FP8
and older pages are converted to a denser packed format called TQ3.  It gives
neither the FP8 variant nor the TQ3 bit layout.  The readings used throughout
this repository are:

* FP8 is OCP E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits with bias 7, 3
  mantissa bits, no infinities, NaN = 0x7F / 0xFF, largest finite value 448.
  Encoding rounds to nearest, ties to even code, and saturates to +-448.
* TQ3 packs 32 consecutive head-dim elements into one group: an fp16 scale
  s = fp16(fp32(absmax / 3.5)) and 32 three-bit codes c in 0..7 that decode to
  (c - 3.5) * s.  The codes form a little-endian bit stream: code j of a row
  sits in bits 3j..3j+2, stream bit n is bit (n % 8) of byte n // 8, so each
  group is exactly 12 bytes and the groups of one token row concatenate.
* A code is chosen by exact thresholds: c = #{b in -3..3 : x >= b*s}.  Every
  b*s is an exact fp32 product (fp16 significand times an integer of at most
  two bits), so the choice involves no rounding.  It is the nearest level with
  ties going to the upper level; x = 0 gives c = 4.  A zero scale gives c = 4
  for every element, and the scale is clamped to 65504 before the fp16
  rounding so it never becomes infinite.

Every function works on numpy arrays.  Floating-point steps that decide an
integer code are done in fp32, the precision the GPU kernels use for the same
decision; decoding is exact in fp64.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
TQ3_GROUP = 32
TQ3_GROUP_BYTES = 12
FP16_MAX = 65504.0


# --------------------------------------------------------------------------
# FP8 E4M3 (OCP)
# --------------------------------------------------------------------------
def _e4m3_table() -> np.ndarray:
    """Value of every byte 0..255 under OCP E4M3, in fp64 (NaN for 0x7F/0xFF)."""
    out = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        exp = (code >> 3) & 0xF
        man = code & 0x7
        if exp == 0xF and man == 0x7:
            out[code] = np.nan
        elif exp == 0:
            out[code] = sign * man * 2.0 ** -9          # subnormal: m/8 * 2^(1-7)
        else:
            out[code] = sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)
    return out


E4M3_VALUES = _e4m3_table()
# Non-negative finite codes 0x00..0x7E are monotonic in value.
_E4M3_POS = E4M3_VALUES[:0x7F].copy()


def e4m3_decode(codes) -> np.ndarray:
    """Exact fp64 value of E4M3 bytes."""
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x) -> np.ndarray:
    """Round fp32 values to E4M3 codes: nearest, ties to even code, saturating.

    Standard rounding to a binary format with 4 significant bits: with
    mag = min(|x|, 448) and e' = max(floor(log2 mag), -6) (the subnormal
    exponent floor), the representable neighbours of mag are spaced by the
    quantum 2^(e'-3), so the rounded magnitude is rint(mag / quantum) * quantum
    (rint = round half to even; an even multiple is an even mantissa, i.e. an
    even code).  Writing r = rint(mag * 2^(3-e')), the code is 8*(e'+6) + r:
    r in 8..15 gives exponent field e'+7 and mantissa r-8, r = 16 carries into
    the next exponent, and for e' = -6 the same formula gives the subnormal
    codes r = 0..8.  All steps are exact in fp64.  Inputs must be finite.
    """
    x = np.asarray(x, dtype=np.float32)
    mag = np.minimum(np.abs(x).astype(np.float64), E4M3_MAX)
    _, E = np.frexp(mag)                       # mag = f * 2^E, f in [0.5, 1)
    e = np.where(mag > 0, np.maximum(E - 1, -6), -6)
    r = np.rint(np.ldexp(mag, 3 - e))           # exact scaling, round half to even
    code = (8 * (e + 6) + r).astype(np.uint8)
    return np.where(np.signbit(x), code | np.uint8(0x80), code).astype(np.uint8)


# --------------------------------------------------------------------------
# fp16 / bf16 helpers (numpy float16 is IEEE binary16 with RNE conversion)
# --------------------------------------------------------------------------
def fp16_bits_to_value(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def bf16_bits_to_value(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_encode(x32) -> np.ndarray:
    """fp32 -> bf16 bits, rounding to nearest with ties to the even bf16 value
    (IEEE 754 roundTiesToEven).  bf16 is the upper half of an fp32 pattern, so
    rounding keeps the upper 16 bits and adds one unit in their last place
    when the dropped lower 16 bits exceed half of that unit, or equal half and
    the kept part is odd.  A carry out of the significand moves into the
    exponent, which is again the correctly rounded result (up to infinity past
    the largest finite bf16).  Finite inputs only (the cache stores no NaN)."""
    u = np.asarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    upper = u >> np.uint64(16)
    lower = u & np.uint64(0xFFFF)
    up = (lower > 0x8000) | ((lower == 0x8000) & ((upper & np.uint64(1)) == 1))
    return (upper + up.astype(np.uint64)).astype(np.uint16)


# --------------------------------------------------------------------------
# TQ3
# --------------------------------------------------------------------------
def tq3_scale(absmax32) -> np.ndarray:
    """fp16 scale of a group from its fp32 absmax: fp16_RNE(min(fp32(a/3.5), 65504)).

    Returns the fp16 values (numpy float16)."""
    a = np.asarray(absmax32, dtype=np.float32)
    q = a / np.float32(3.5)                       # correctly rounded fp32 division
    q = np.minimum(q, np.float32(FP16_MAX))
    return q.astype(np.float16)


def tq3_codes(x32, scale16) -> np.ndarray:
    """Codes 0..7 of fp32 values x against fp16 scales (broadcast), by exact thresholds."""
    x = np.asarray(x32, dtype=np.float32).astype(np.float64)
    s = np.asarray(scale16, dtype=np.float16).astype(np.float64)
    c = np.zeros(np.broadcast(x, s).shape, dtype=np.int64)
    for b in range(-3, 4):
        c += (x >= b * s)          # b*s is exact in fp64 (and in fp32)
    c = np.where(s == 0.0, 4, c)
    return c.astype(np.uint8)


def tq3_encode_groups(x32):
    """Encode fp32 values of shape [..., 32] into (codes [..., 32], fp16 scale [...])."""
    x = np.asarray(x32, dtype=np.float32)
    assert x.shape[-1] == TQ3_GROUP
    amax = np.max(np.abs(x), axis=-1)
    s = tq3_scale(amax)
    codes = tq3_codes(x, s[..., None])
    return codes, s


def tq3_decode(codes, scale16) -> np.ndarray:
    """(c - 3.5) * s in fp64 (exact).  codes [..., 32], scale [...]."""
    c = np.asarray(codes, dtype=np.float64)
    s = np.asarray(scale16, dtype=np.float16).astype(np.float64)
    return (c - 3.5) * s[..., None]


def tq3_pack_row(codes) -> np.ndarray:
    """Pack codes [..., n] (n % 8 == 0) into the little-endian 3-bit stream [..., 3n/8] bytes."""
    c = np.asarray(codes, dtype=np.uint8)
    n = c.shape[-1]
    assert n % 8 == 0
    bits = np.zeros(c.shape[:-1] + (3 * n,), dtype=np.uint8)
    for k in range(3):
        bits[..., k::3] = (c >> k) & 1            # stream bit 3j+k = bit k of code j
    return np.packbits(bits, axis=-1, bitorder="little")


def tq3_unpack_row(stream, n) -> np.ndarray:
    """Inverse of tq3_pack_row: bytes [..., 3n/8] -> codes [..., n]."""
    s = np.asarray(stream, dtype=np.uint8)
    bits = np.unpackbits(s, axis=-1, bitorder="little")[..., : 3 * n]
    c = bits[..., 0::3] | (bits[..., 1::3] << 1) | (bits[..., 2::3] << 2)
    return c.astype(np.uint8)
