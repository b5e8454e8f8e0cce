"""Number formats used by the layer, decoded and encoded from their definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name the formats but do not define them: FP8 activations and
FP8 x FP4 mixed precision ("DeepSeek悄悄更新：Mega MoE、FP4 Indexer来了",
section "Mega MoE 是什么？"), FP8/FP4 quantisation per token and per block
("DeepSeek 模型更新解读 Tile Kernels 与 DeepEP V2 新特性", section "Tile
Kernels", quantisation bullet), BF16 in the combine ("... DeepEP V2 ...",
section "性能表现").  The encodings below are the OCP 8-bit floating point
specification (E4M3 "fn" variant: bias 7, no infinities, only S.1111.111 is
NaN, largest finite 448) and the OCP Microscaling (MX) v1.0 element and scale
formats (E2M1: bias 1, values 0, 0.5, 1, 1.5, 2, 3, 4, 6 with a sign bit;
E8M0: 2**(code - 127), code 255 is NaN).  BF16 is the top half of an IEEE
binary32.

E5M6, the third format of the quantisation bullet, is not defined on the pages
either; it is read (R15) as the IEEE-754-style binary format with 1 sign, 5
exponent (bias 15) and 6 fraction bits: subnormals at exponent 0, exponent 31
reserved for infinities and NaN (as in binary16), largest finite
(2 - 2**-6) * 2**15 = 65024.  Codes are 12 bits (sign in bit 11), stored two
to three bytes, little-endian: byte 0 = low 8 bits of the first code, byte 1
= its high 4 bits and the low 4 bits of the second, byte 2 = the second's high
8 bits.

Every table here is built from those definitions with integer arithmetic, not
from any library cast; ``tests/test_formats.py`` pins them exhaustively against
the closed forms and against PyTorch's own float8 casts.
"""

import numpy as np

E4M3_MAX = 448.0
E2M1_MAX = 6.0


def _e4m3_value(code: int) -> float:
    """Value of one OCP E4M3 (fn) byte: sign, 4 exponent bits (bias 7), 3 mantissa bits."""
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:                       # subnormal: 0.m * 2**(1 - bias)
        return sign * (man / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


def _e2m1_value(code: int) -> float:
    """Value of one OCP MX E2M1 nibble: sign, 2 exponent bits (bias 1), 1 mantissa bit."""
    sign = -1.0 if (code >> 3) & 1 else 1.0
    exp = (code >> 1) & 0x3
    man = code & 0x1
    if exp == 0:                       # subnormal: 0.m * 2**(1 - bias)
        return sign * (man / 2.0)
    return sign * (1.0 + man / 2.0) * 2.0 ** (exp - 1)


E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)
E2M1_TABLE = np.array([_e2m1_value(c) for c in range(16)], dtype=np.float64)


def e8m0_decode(codes) -> np.ndarray:
    """OCP MX E8M0 scale byte -> 2**(code - 127); code 255 is NaN."""
    c = np.asarray(codes, dtype=np.int64)
    out = np.ldexp(1.0, c - 127).astype(np.float64)
    return np.where(c == 255, np.nan, out)


def e4m3_decode(codes) -> np.ndarray:
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e2m1_unpack(packed: np.ndarray) -> np.ndarray:
    """Unpack E2M1 pairs along the last axis: element 2i is the low nibble of
    byte i, element 2i+1 its high nibble.  Returns float64 values."""
    p = np.asarray(packed, dtype=np.uint8)
    lo = E2M1_TABLE[p & 0xF]
    hi = E2M1_TABLE[p >> 4]
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.float64)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def bf16_decode(bits) -> np.ndarray:
    """BF16 bit patterns (uint16) -> float64, exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------- encoders
# Finite non-negative E4M3 magnitudes in code order 0x00..0x7E; they increase
# strictly with the code, so the nearest code is found by bisection.
_E4M3_POS = E4M3_TABLE[:0x7F]


def e4m3_encode(values) -> np.ndarray:
    """Round float64 values to E4M3 codes: round to nearest, ties to the even
    code (mantissa LSB 0), saturating to +-448.  The sign bit follows the
    input's sign (so -0.0 and tiny negatives give 0x80)."""
    v = np.asarray(values, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("non-finite value passed to e4m3_encode")
    mag = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.searchsorted(_E4M3_POS, mag, side="left")          # first code >= mag
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(mag == _E4M3_POS[hi], hi, code)             # exact hits
    sign = np.signbit(v).astype(np.uint8) << 7
    return (code.astype(np.uint8) | sign).astype(np.uint8)


E5M6_MAX = 65024.0


def _e5m6_value(code: int) -> float:
    """Value of one 12-bit E5M6 code: sign (bit 11), 5 exponent bits (bias 15), 6 fraction bits."""
    sign = -1.0 if (code >> 11) & 1 else 1.0
    exp = (code >> 6) & 0x1F
    man = code & 0x3F
    if exp == 0x1F:
        return sign * float("inf") if man == 0 else float("nan")
    if exp == 0:                       # subnormal: 0.m * 2**(1 - bias)
        return sign * (man / 64.0) * 2.0 ** (1 - 15)
    return sign * (1.0 + man / 64.0) * 2.0 ** (exp - 15)


E5M6_TABLE = np.array([_e5m6_value(c) for c in range(4096)], dtype=np.float64)
_E5M6_POS = E5M6_TABLE[:0x7C0]         # +0 .. +65024, increasing in code order


def e5m6_decode(codes) -> np.ndarray:
    """12-bit E5M6 codes -> float64 values."""
    return E5M6_TABLE[np.asarray(codes, dtype=np.int64) & 0xFFF]


def e5m6_encode(values) -> np.ndarray:
    """Round float64 values to E5M6 codes: round to nearest, ties to the even
    code (fraction LSB 0), saturating to +-65024.  The sign bit follows the
    input's sign."""
    v = np.asarray(values, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("non-finite value passed to e5m6_encode")
    mag = np.minimum(np.abs(v), E5M6_MAX)
    hi = np.searchsorted(_E5M6_POS, mag, side="left")          # first code >= mag
    hi = np.minimum(hi, 0x7BF)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - _E5M6_POS[lo]
    d_hi = _E5M6_POS[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(mag == _E5M6_POS[hi], hi, code)             # exact hits
    sign = np.signbit(v).astype(np.uint16) << 11
    return (code.astype(np.uint16) | sign).astype(np.uint16)


def e5m6_pack(codes) -> np.ndarray:
    """[..., 2n] 12-bit codes -> [..., 3n] bytes (two codes to three bytes)."""
    c = np.asarray(codes, dtype=np.uint32)
    a, b = c[..., 0::2], c[..., 1::2]
    out = np.stack([a & 0xFF, (a >> 8) | ((b & 0xF) << 4), b >> 4], axis=-1)
    return out.reshape(*c.shape[:-1], -1).astype(np.uint8)


def e5m6_unpack(packed) -> np.ndarray:
    """[..., 3n] bytes -> [..., 2n] 12-bit codes."""
    p = np.asarray(packed, dtype=np.uint32).reshape(*np.shape(packed)[:-1], -1, 3)
    a = p[..., 0] | ((p[..., 1] & 0xF) << 8)
    b = (p[..., 1] >> 4) | (p[..., 2] << 4)
    return np.stack([a, b], axis=-1).reshape(*np.shape(packed)[:-1], -1).astype(np.uint16)


def bf16_round(values) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (8 significant bits, ties
    to even), returned as float64.  Normal range only (|v| >= 2**-126)."""
    v = np.asarray(values, dtype=np.float64)
    m, e = np.frexp(v)                  # v = m * 2**e, 0.5 <= |m| < 1
    r = np.rint(m * 256.0)              # np.rint rounds half to even
    return np.ldexp(r, e - 8)


def f32_round(values) -> np.ndarray:
    """Round float64 to the nearest binary32 (IEEE round-to-nearest-even)."""
    return np.asarray(values, dtype=np.float64).astype(np.float32).astype(np.float64)
