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
* MXFP8 (OCP microscaling, used here for activations in the FP8-activation
  mode): blocks of 32 consecutive elements share a power-of-two scale 2^X,
  X = floor(log2(amax)) - 8 (8 = the largest exponent of e4m3, so the block
  maximum lands in [256, 512) before the elements are rounded), stored as
  e8m0 = X + 127 clamped to [0, 254]; each element is rounded to the nearest
  e4m3 value (ties to the even code), saturating at +-448.  The rounding
  decisions are taken on float32 values, the precision the kernels hold the
  activations in.
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


# decode_e4m3 / decode_e2m1 evaluated once on every code: applying a format to
# a large array is then a table lookup with exactly the same values.
_E4M3_TABLE = decode_e4m3(np.arange(256))
_E2M1_TABLE = decode_e2m1(np.arange(16))


def dequant_fp8_rows(codes, scales) -> np.ndarray:
    """w'[n, k] = e4m3(codes[n, k]) * scales[n], exact in float64."""
    return _E4M3_TABLE[np.asarray(codes, dtype=np.uint8)] * np.asarray(scales, dtype=np.float64)[:, None]


def dequant_mxfp4(codes, e8) -> np.ndarray:
    """codes [rows, cols/2] (low nibble = even column), e8 [rows, cols/32]."""
    codes = np.asarray(codes, dtype=np.uint8)
    rows, half = codes.shape
    vals = np.empty((rows, 2 * half), dtype=np.float64)
    vals[:, 0::2] = _E2M1_TABLE[codes & 0xF]
    vals[:, 1::2] = _E2M1_TABLE[codes >> 4]
    scale = np.repeat(decode_e8m0(e8), 32, axis=1)
    return vals * scale


_E4M3_POS = _E4M3_TABLE[:127]  # codes 0 .. 126: 0, then increasing finite positive values up to 448


def round_e4m3(v) -> np.ndarray:
    """Nearest e4m3 value of each element of v (ties to the even code),
    saturating at +-448.  Exact: |v| is compared with the midpoints of
    neighbouring codes in float64."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), 448.0)
    hi = np.clip(np.searchsorted(_E4M3_POS, a, side="left"), 1, 126)  # first code with value >= a
    lo = hi - 1
    d_lo, d_hi = a - _E4M3_POS[lo], _E4M3_POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    return np.sign(v) * _E4M3_POS[code]


def mxfp8_quantize(x):
    """x [..., n] (n a multiple of 32) -> (values on the e4m3 grid [..., n],
    X [..., n/32] int): the block exponent and the elements before scaling."""
    x32 = np.asarray(x, dtype=np.float32)
    shp = x32.shape
    blk = x32.reshape(shp[:-1] + (shp[-1] // 32, 32)).astype(np.float64)
    amax = np.abs(blk).max(axis=-1)
    with np.errstate(divide="ignore"):
        X = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 8, -127)
    X = np.clip(X, -127, 127).astype(np.int64)
    el = round_e4m3(blk * np.ldexp(1.0, -X)[..., None])
    return el.reshape(shp), X


def mxfp8_roundtrip(x) -> np.ndarray:
    """x as MXFP8 holds it: each element's e4m3 value times its block's 2^X."""
    el, X = mxfp8_quantize(x)
    shp = el.shape
    blk = el.reshape(shp[:-1] + (shp[-1] // 32, 32)) * np.ldexp(1.0, X)[..., None]
    return blk.reshape(shp)
