"""Pins for the oracle's number-format decoders and the input encoders.

Decoders are checked against torch's own dtype conversions (an independent
library implementation of the same formats), against fixed values of the
formats, and by exhaustive brute force where torch has no conversion."""
import os

import numpy as np
import pytest
import torch

from oracle.codecs import decode_bf16, decode_e2m1, decode_e4m3, decode_e8m0, dequant_fp8_rows, dequant_mxfp4
from workload import encode_fp8_rows, encode_mxfp4, to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
ALL8 = np.arange(256, dtype=np.uint8)


def test_e4m3_matches_torch_all_codes():
    ref = torch.from_numpy(ALL8.copy()).view(torch.float8_e4m3fn).double().numpy()
    got = decode_e4m3(ALL8)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(got[ok]))


def test_e4m3_landmarks():
    v = decode_e4m3(np.array([0x38, 0x7E, 0x01, 0x08, 0x07, 0x80, 0xFE, 0x7F, 0xFF], np.uint8))
    assert v[0] == 1.0 and v[1] == 448.0 and v[2] == 2.0 ** -9 and v[3] == 2.0 ** -6
    assert v[4] == 7 * 2.0 ** -9 and v[5] == 0.0 and np.signbit(v[5]) and v[6] == -448.0
    assert np.isnan(v[7]) and np.isnan(v[8])
    finite = decode_e4m3(ALL8[:0x7F])  # positive codes 0x00..0x7E are increasing
    assert np.all(np.diff(finite) > 0)


def test_e8m0_matches_torch_all_codes():
    ref = torch.from_numpy(ALL8.copy()).view(torch.float8_e8m0fnu).double().numpy()
    got = decode_e8m0(ALL8)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    assert np.array_equal(ref[:255], got[:255])


def test_e2m1_matches_spec_table():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "e2m1_values.txt")) if l.strip() and l[0] != "#"]
    codes = np.array([int(r[0]) for r in rows], np.uint8)
    vals = np.array([float(r[1]) for r in rows])
    got = decode_e2m1(codes)
    assert np.array_equal(got, vals)
    assert np.array_equal(np.signbit(got), np.signbit(vals))


def test_bf16_matches_torch():
    bits = np.random.default_rng(1).integers(0, 2 ** 16, size=50000).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = decode_bf16(bits)
    ok = ~np.isnan(ref)
    assert np.array_equal(np.isnan(ref), np.isnan(got)) and np.array_equal(ref[ok], got[ok])


def _nearest_even(target, grid_vals, grid_codes, even_mask):
    """Brute force: nearest grid value, ties to the code with an even mantissa."""
    d = np.abs(target[:, None] - grid_vals[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    pick = np.where(cand & even_mask[None, :], 1, 0)
    out = np.where(pick.any(axis=1), np.argmax(pick, axis=1), np.argmax(cand, axis=1))
    return grid_codes[out]


def test_fp8_encoder_is_nearest_even_and_saturating():
    rng = np.random.default_rng(2)
    w = (rng.standard_normal((64, 300)) * 0.02).astype(np.float32)
    w[3] = 0.0
    w[5, 7] = 0.5  # one large outlier
    codes, s = encode_fp8_rows(w)
    assert s.dtype == np.float32 and s[3] == 1.0
    amax = np.abs(w).max(axis=1)
    nz = amax > 0
    assert np.array_equal(s[nz], (amax[nz] / np.float32(448)).astype(np.float32))
    # every row's absmax element lands on +-448 (up to fp32 rounding of w/s)
    dec = decode_e4m3(codes)
    assert np.all(np.abs(dec[nz]).max(axis=1) == 448.0)
    # brute force nearest-even over all finite positive codes
    pos = np.arange(0x7F, dtype=np.uint8)
    grid = decode_e4m3(pos)
    even = (pos & 1) == 0
    target = np.abs((w / s[:, None]).astype(np.float32).astype(np.float64)).reshape(-1)
    want = _nearest_even(np.minimum(target, 448.0), grid, pos, even)
    assert np.array_equal(codes.reshape(-1) & 0x7F, want)
    # idempotence: re-encoding the decoded weights gives the same codes
    codes2, s2 = encode_fp8_rows((dequant_fp8_rows(codes, s)).astype(np.float32))
    assert np.array_equal(dequant_fp8_rows(codes2, s2), dequant_fp8_rows(codes, s))


def test_mxfp4_encoder_is_nearest_even_with_shared_exponent():
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((16, 128)) * 0.02).astype(np.float32)
    w[2, :32] = 0.0
    codes, e8 = encode_mxfp4(w)
    assert codes.shape == (16, 64) and e8.shape == (16, 4)
    assert e8[2, 0] == 0 and np.all(codes[2, :16] == 0)
    blk = w.reshape(16, 4, 32)
    amax = np.abs(blk).max(axis=2)
    nz = amax > 0
    assert np.array_equal(e8[nz].astype(int), np.floor(np.log2(amax[nz])).astype(int) - 2 + 127)
    # nibble order: low nibble is the even element
    nib = np.empty((16, 128), np.uint8)
    nib[:, 0::2], nib[:, 1::2] = codes & 0xF, codes >> 4
    scale = decode_e8m0(np.repeat(e8, 32, axis=1))
    target = np.abs(w.astype(np.float64) / scale).reshape(-1)
    grid_codes = np.arange(8, dtype=np.uint8)
    want = _nearest_even(np.minimum(target, 6.0), decode_e2m1(grid_codes), grid_codes, (grid_codes & 1) == 0)
    assert np.array_equal(nib.reshape(-1) & 7, want)
    sign_ok = (np.signbit(w.reshape(-1)) == ((nib.reshape(-1) >> 3) == 1)) | (want == 0)
    assert np.all(sign_ok)
    # the dequantised block max is within the e2m1 spacing of the true max
    deq = dequant_mxfp4(codes, e8)
    assert np.all(np.abs(deq - w) <= np.abs(w) * 0.25 + scale * 0.25 + 1e-12)


def test_bf16_encoder_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5e-3, 3.0e38], np.float32)
    got = decode_bf16(to_bf16_bits(x))
    assert got[0] == 1.0 and got[1] == 1.0 and got[2] == 1.0 + 2 ** -6
    assert abs(got[3] - (-2.5e-3)) <= 2.5e-3 * 2 ** -8
    assert np.isfinite(got[4])


# ---------------------------------------------------------------- MXFP8 (FP8-activation mode)

def test_round_e4m3_brute_force_with_ties():
    from oracle.codecs import _E4M3_POS, round_e4m3
    vals = _E4M3_POS
    mids = (vals[:-1] + vals[1:]) / 2                      # exact ties
    rng = np.random.default_rng(1)
    x = np.concatenate([mids, -mids, rng.uniform(-500, 500, 4000), rng.uniform(-0.02, 0.02, 2000), [0.0, 448, 1e4]])
    got = round_e4m3(x)
    # brute force: nearest representable magnitude, ties to the even code, saturate
    a = np.minimum(np.abs(x), 448.0)
    d = np.abs(a[:, None] - vals[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    codes = np.array([np.flatnonzero(c)[0] if c.sum() == 1 else [k for k in np.flatnonzero(c) if k % 2 == 0][0]
                      for c in cand])
    assert np.array_equal(got, np.sign(x) * vals[codes])
    # ties went to even codes
    tie_codes = np.searchsorted(vals, np.abs(round_e4m3(mids)))
    assert np.all(tie_codes % 2 == 0)


def test_round_e4m3_matches_torch_in_range():
    from oracle.codecs import round_e4m3
    x = np.random.default_rng(2).standard_normal(50000) * 50
    x = np.clip(x, -448, 448)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(round_e4m3(x), ref)


def test_mxfp8_block_scale_saturation_and_idempotence():
    from oracle.codecs import mxfp8_quantize, mxfp8_roundtrip
    rng = np.random.default_rng(3)
    x = rng.standard_normal((7, 96)).astype(np.float32)
    x[1, :32] = 0.0                              # all-zero block
    x[2, 5] = 1000.0                             # block max 1000 = 1.95 * 2^9: X = 1, saturates at 448 * 2
    el, X = mxfp8_quantize(x)
    amax = np.abs(x.reshape(7, 3, 32)).max(-1).astype(np.float64)
    nz = amax > 0
    assert np.array_equal(X[nz], np.floor(np.log2(amax[nz])).astype(np.int64) - 8)
    assert X[1, 0] == -127 and np.all(el[1, :32] == 0)
    rt = mxfp8_roundtrip(x)
    assert rt[2, 5] == 448.0 * 2.0 ** X[2, 0] and X[2, 0] == 1
    assert np.array_equal(mxfp8_roundtrip(rt), rt)                       # idempotent
    # per element: within half a step of e4m3 (3 mantissa bits) of the block's scale, or saturated
    step = np.maximum(2.0 ** (np.floor(np.log2(np.maximum(np.abs(x), 1e-30))) - 3), 2.0 ** (X.repeat(32, 1) - 9))
    sat = np.abs(x) >= 464 * 2.0 ** X.repeat(32, 1)
    err = np.abs(rt - x.astype(np.float64))
    assert np.all((err <= step / 2 * (1 + 1e-12)) | sat)


def test_mxfp8_decisions_follow_float32():
    """Values that round to the same float32 quantise identically: the codes
    are decided on float32, the precision the kernels hold activations in."""
    from oracle.codecs import mxfp8_roundtrip
    x32 = np.random.default_rng(4).standard_normal((3, 64)).astype(np.float32)
    nudged = x32.astype(np.float64) * (1 + 1e-10)
    assert np.array_equal(mxfp8_roundtrip(x32), mxfp8_roundtrip(nudged))
