"""Decoders for the number formats the verify pass reads (oracle side).

Each decoder spells out the format's bit layout; none calls a library
conversion, so that the tests can pin them against the library ones.

* FP8 e4m3 ("fn" variant, as in the OCP 8-bit floating point spec): 1 sign,
  4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 is
  subnormal (m/8 * 2^-6); S.1111.111 is NaN; there is no infinity.  The
  OCRia stack page (quantization section) moves weights as FP8 to halve the
  bytes per weight.
* e2m1 (FP4): 1 sign, 2 exponent bits with bias 1, 1 mantissa bit; field 0
  is subnormal (m * 0.5).  Magnitudes: 0, 0.5, 1, 1.5, 2, 3, 4, 6.
* e8m0: an unsigned power-of-two exponent, value 2^(b-127); 255 is NaN.
* bfloat16: the upper 16 bits of an IEEE binary32.
"""
import numpy as np


def decode_e4m3(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.ldexp(1.0, e - 7)
    subnormal = (m / 8.0) * np.ldexp(1.0, -6)
    v = sign * np.where(e == 0, subnormal, normal)
    return np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, v)


def decode_e2m1(nibbles) -> np.ndarray:
    c = np.asarray(nibbles, dtype=np.uint8).astype(np.int64) & 0xF
    sign = np.where((c >> 3) & 1, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = (c & 0x1).astype(np.float64)
    v = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.ldexp(1.0, e - 1))
    return sign * v


def decode_e8m0(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    return np.where(b == 255, np.nan, np.ldexp(1.0, b - 127))


def decode_bf16(bits) -> np.ndarray:
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def dequant_fp8_rows(codes, scales) -> np.ndarray:
    """w'[n, k] = e4m3(codes[n, k]) * scales[n], exact in float64."""
    return decode_e4m3(codes) * np.asarray(scales, dtype=np.float64)[:, None]


def dequant_mxfp4(codes, e8) -> np.ndarray:
    """codes [rows, cols/2] (low nibble = even column), e8 [rows, cols/32]."""
    codes = np.asarray(codes, dtype=np.uint8)
    rows, half = codes.shape
    vals = np.empty((rows, 2 * half), dtype=np.float64)
    vals[:, 0::2] = decode_e2m1(codes & 0xF)
    vals[:, 1::2] = decode_e2m1(codes >> 4)
    scale = np.repeat(decode_e8m0(e8), 32, axis=1)
    return vals * scale
