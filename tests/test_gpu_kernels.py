"""Per-kernel parity of the HIP library against the float64 oracle pieces,
called through the C ABI's test hooks (spec_debug_linear,
spec_debug_attention)."""
import numpy as np
import pytest
import torch

import oracle
from oracle.codecs import decode_bf16, decode_e4m3, dequant_fp8_rows, dequant_mxfp4
import workload as W
from block_draft_verification_amd import (WFMT_BF16, WFMT_FP8_E4M3_ROW, WFMT_MXFP4, debug_attention, debug_linear,
                                          debug_residual, debug_rmsnorm, debug_swiglu)

pytestmark = pytest.mark.gpu


def _x(M, K, seed, f16=True):
    """Activations as the linear kernel takes them: FP16 bits (FP8/MXFP4
    weights) or BF16 bits (BF16 weights)."""
    a = np.random.default_rng(seed).standard_normal((M, K)).astype(np.float32)
    return a.astype(np.float16).view(np.uint16) if f16 else W.to_bf16_bits(a)


def _dec(bits, f16=True):
    return bits.view(np.float16).astype(np.float64) if f16 else decode_bf16(bits)


def _check_linear(xb, wdeq, y, f16=True):
    x = _dec(xb, f16)
    ref = x @ wdeq.T
    bound = np.abs(x) @ np.abs(wdeq).T                 # fp32 accumulation of exact products
    err = np.abs(y.astype(np.float64) - ref)
    assert np.all(err <= 3e-5 * bound + 1e-30), f"max err/bound {np.max(err / (bound + 1e-30)):.3g}"


def _dev(a):
    a = np.ascontiguousarray(a)
    return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()


def _packed(w, s, wfmt, rows, cols):
    """Row-major weights on the device, as the library's hooks take them (each
    hook packs its own copy)."""
    return _dev(w), None if s is None else _dev(s)


@pytest.mark.parametrize("M,N,K", [(16, 1152, 896), (40, 896, 4864), (512, 9728, 896), (1, 64, 64)])
def test_linear_fp8(M, N, K):
    rng = np.random.default_rng(M + N + K)
    codes = rng.integers(0, 256, size=(N, K)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3F                # no NaN codes
    if K >= 254:                                        # every finite code appears in row 0
        codes[0, :254] = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    scales = (rng.random(N) * 1e-3 + 1e-4).astype(np.float32)
    xb = _x(M, K, 1)
    y = debug_linear(_dev(xb), *_packed(codes, scales, WFMT_FP8_E4M3_ROW, N, K), WFMT_FP8_E4M3_ROW, N).cpu().numpy()
    _check_linear(xb, dequant_fp8_rows(codes, scales), y)


def test_linear_fp8_every_code_decodes():
    """Row n of W holds a single code; x = ones: y[n] = K * e4m3(code_n)."""
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    N = 256
    codes = np.zeros((N, 64), np.uint8)
    codes[:len(finite)] = finite[:, None]
    scales = np.ones(N, np.float32)
    xb = np.ones((16, 64), np.float16).view(np.uint16)
    y = debug_linear(_dev(xb), *_packed(codes, scales, WFMT_FP8_E4M3_ROW, N, 64), WFMT_FP8_E4M3_ROW, N).cpu().numpy()
    assert np.array_equal(y[0, :len(finite)].astype(np.float64), 64 * decode_e4m3(finite))


@pytest.mark.parametrize("M,N,K", [(16, 9728, 896), (256, 896, 4864), (33, 128, 64)])
def test_linear_mxfp4(M, N, K):
    rng = np.random.default_rng(N + K)
    codes = rng.integers(0, 256, size=(N, K // 2)).astype(np.uint8)
    e8 = rng.integers(110, 135, size=(N, K // 32)).astype(np.uint8)
    xb = _x(M, K, 2)
    y = debug_linear(_dev(xb), *_packed(codes, e8, WFMT_MXFP4, N, K), WFMT_MXFP4, N).cpu().numpy()
    _check_linear(xb, dequant_mxfp4(codes, e8), y)


@pytest.mark.parametrize("M,N,K", [(16, 1024, 896), (512, 640, 4096)])
def test_linear_bf16(M, N, K):
    w = W.to_bf16_bits((np.random.default_rng(5).standard_normal((N, K)) * 0.02).astype(np.float32))
    xb = _x(M, K, 3, f16=False)
    y = debug_linear(_dev(xb), *_packed(w, None, WFMT_BF16, N, K), WFMT_BF16, N).cpu().numpy()
    _check_linear(xb, decode_bf16(w), y, f16=False)


@pytest.mark.parametrize("M,H", [(37, 896), (16, 4096), (1, 64)])
def test_rmsnorm_fp16(M, H):
    """x = h / sqrt(mean(h^2) + eps) * g rounded once to FP16: within one
    FP16 rounding (2^-11 relative, plus the subnormal step) of the float64
    value, the fp32 normalisation adding well under 2^-16."""
    rng = np.random.default_rng(M + H)
    h = (rng.standard_normal((M, H)) * np.exp2(rng.integers(-6, 7, size=(M, 1)))).astype(np.float32)
    g = (1 + 0.5 * rng.standard_normal(H)).astype(np.float32)
    x = debug_rmsnorm(torch.from_numpy(h).cuda(), torch.from_numpy(g).cuda(), 1e-6).cpu().numpy()
    ref = oracle.rms_norm(h, g, 1e-6)
    err = np.abs(_dec(x.view(np.uint16)) - ref)
    assert np.all(err <= (2.0 ** -11 + 2.0 ** -16) * np.abs(ref) + 2.0 ** -25)


@pytest.mark.parametrize("wfmt,M,H,I", [(WFMT_FP8_E4M3_ROW, 16, 896, 4864), (WFMT_MXFP4, 40, 896, 4864),
                                        (WFMT_FP8_E4M3_ROW, 128, 896, 4864), (WFMT_MXFP4, 256, 896, 4864),
                                        (WFMT_FP8_E4M3_ROW, 300, 896, 4864), (WFMT_FP8_E4M3_ROW, 512, 896, 4864)])
def test_swiglu_fp16(wfmt, M, H, I):
    """a = SiLU(x Wg^T) * (x Wu^T) rounded to FP16: the gate and up sums carry
    the fp32 accumulation bound (3e-5 of sum |x||w|, as for the plain
    linear), carried through SiLU(g) * u (|SiLU'| <= 1.1), then one FP16
    rounding."""
    rng = np.random.default_rng(I + M)
    if wfmt == WFMT_FP8_E4M3_ROW:
        w = rng.integers(0, 256, size=(2 * I, H)).astype(np.uint8)
        w[(w & 0x7F) == 0x7F] = 0x3F
        ws = (rng.random(2 * I) * 2e-3 + 1e-3).astype(np.float32)
        wd = dequant_fp8_rows(w, ws)
    else:
        w = rng.integers(0, 256, size=(2 * I, H // 2)).astype(np.uint8)
        ws = rng.integers(118, 124, size=(2 * I, H // 32)).astype(np.uint8)
        wd = dequant_mxfp4(w, ws)
    xb = _x(M, H, 9)
    x = _dec(xb)
    gate, up = x @ wd[:I].T, x @ wd[I:].T
    ref = oracle.silu(gate) * up
    bg, bu = 3e-5 * (np.abs(x) @ np.abs(wd[:I]).T), 3e-5 * (np.abs(x) @ np.abs(wd[I:]).T)
    a = debug_swiglu(_dev(xb), None, *_packed(w, ws, wfmt, 2 * I, H), wfmt, I).cpu().numpy()
    err = np.abs(_dec(a.view(np.uint16)) - ref)
    bound = 1.1 * np.abs(up) * bg + np.abs(oracle.silu(gate)) * bu + bg * bu
    assert np.all(err <= 2.0 ** -11 * (np.abs(ref) + bound) + bound + 2.0 ** -24), \
        f"max excess {np.max(err - 2.0 ** -11 * np.abs(ref) - bound):.3g}"


NAN_BF16 = 0x7FC0


def _attn_case(B, Hq, Hkv, D, lens, max_ctx, seed, poison=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B * 16, Hq * D)).astype(np.float16).view(np.uint16)
    K = W.to_bf16_bits(rng.standard_normal((B, Hkv, max_ctx, D)).astype(np.float32))
    V = W.to_bf16_bits(rng.standard_normal((B, Hkv, max_ctx, D)).astype(np.float32))
    if poison:  # slots past each block are never read
        for b, n in enumerate(lens):
            K[b, :, n + 16:] = NAN_BF16
            V[b, :, n + 16:] = NAN_BF16
    return q, K, V


def _attn_ref(q, K, V, lens, Hq, Hkv, D):
    out = []
    for b, n in enumerate(lens):
        qb = _dec(q[b * 16:(b + 1) * 16]).reshape(16, Hq, D)
        o = oracle.attention(qb, decode_bf16(K[b, :, :n + 16]), decode_bf16(V[b, :, :n + 16]), n, Hq // Hkv)
        out.append(o.reshape(16, Hq * D))
    return np.concatenate(out)


@pytest.mark.parametrize("B,maxlen,seed", [(70, 300, 1), (140, 100, 2)])
def test_attention_many_sequences(B, maxlen, seed):
    """The split plan over more than 64 sequences (its scans run in chunks of
    64) and over more (sequence, KV head) units than one resident round of
    workgroups (then every unit gets one workgroup)."""
    Hq, Hkv, D = 4, 2, 64
    lens = [int(x) for x in np.random.default_rng(seed).integers(0, maxlen, size=B)]
    max_ctx = maxlen + 16 + 64
    q, K, V = _attn_case(B, Hq, Hkv, D, lens, max_ctx, seed=seed)
    ln = torch.tensor(lens, dtype=torch.int32, device="cuda")
    o = debug_attention(_dev(q), _dev(K), _dev(V), ln, B, Hq, Hkv, D, 0).cpu().numpy()
    got = _dec(o.view(np.uint16))
    ref = _attn_ref(q, K, V, lens, Hq, Hkv, D)
    for h in range(Hq):
        blk = slice(h * D, (h + 1) * D)
        rel = np.linalg.norm(got[:, blk] - ref[:, blk], axis=1) / np.linalg.norm(ref[:, blk], axis=1)
        assert np.all(np.isfinite(got[:, blk])) and rel.max() < 1e-2, f"head {h}: rel {rel.max():.3g}"


# pad = cache rows beyond the longest sequence's block; 0: that block ends at
# the cache's last row (the cache is full), so the last tile is clamped there
@pytest.mark.parametrize("Hq,Hkv,D,lens,split,pad", [
    (14, 2, 64, [0, 37, 200], 0, 64),
    (14, 2, 64, [0, 37, 200], 64, 64),
    (4, 2, 64, [1000, 5], 0, 64),
    (4, 2, 64, [1000, 5], 0, 0),
    (32, 8, 128, [300, 64], 0, 64),
    (8, 1, 128, [700], 128, 64),
    (8, 1, 128, [700], 128, 0),
    (4, 2, 128, [300, 64, 0], 0, 64),
    (3, 3, 128, [129, 1000], 0, 0),
    (2, 2, 64, [63, 64, 65, 127], 64, 64),
    (2, 2, 64, [48, 3], 64, 0),
])
def test_attention(Hq, Hkv, D, lens, split, pad):
    B, max_ctx = len(lens), max(lens) + 16 + pad
    q, K, V = _attn_case(B, Hq, Hkv, D, lens, max_ctx, seed=sum(lens) + Hq)
    ln = torch.tensor(lens, dtype=torch.int32, device="cuda")
    o = debug_attention(_dev(q), _dev(K), _dev(V), ln, B, Hq, Hkv, D, split).cpu().numpy()
    got = _dec(o.view(np.uint16))
    ref = _attn_ref(q, K, V, lens, Hq, Hkv, D)
    for h in range(Hq):
        blk = slice(h * D, (h + 1) * D)
        rel = np.linalg.norm(got[:, blk] - ref[:, blk], axis=1) / np.linalg.norm(ref[:, blk], axis=1)
        assert np.all(np.isfinite(got[:, blk])) and rel.max() < 1e-2, f"head {h}: rel {rel.max():.3g}"
    # the same call twice gives the same bits (fixed-order split merge)
    o2 = debug_attention(_dev(q), _dev(K), _dev(V), ln, B, Hq, Hkv, D, split).cpu().numpy()
    assert np.array_equal(o, o2)


@pytest.mark.parametrize("wfmt,M,N,K,bf16", [(WFMT_FP8_E4M3_ROW, 16, 896, 4864, False),
                                             (WFMT_FP8_E4M3_ROW, 40, 896, 896, False),
                                             (WFMT_MXFP4, 512, 896, 4864, False),
                                             (WFMT_FP8_E4M3_ROW, 600, 896, 4864, False),
                                             (WFMT_FP8_E4M3_ROW, 512, 896, 896, True),
                                             (WFMT_FP8_E4M3_ROW, 37, 4096, 128, False)])
def test_residual_with_folded_norm(wfmt, M, N, K, bf16):
    """The residual projection as the pass runs O and down: h_out = h_in + x W^T
    within the fp32 accumulation bound; xg = h_out * g rounded once (FP16 or
    BF16) from the GPU's own h_out; ssp[m][j] = sum of h_out^2 over columns
    32j .. 32j+31, to fp32 summation accuracy.  The shapes cover the
    workgroup layouts a launch chooses by its row count (one to four k groups,
    32- and 64-row activation tiles), ragged row counts, and down's staggered
    k order from 512 rows (each M block starting at its own k step)."""
    rng = np.random.default_rng(M + N + K)
    if wfmt == WFMT_FP8_E4M3_ROW:
        w = rng.integers(0, 256, size=(N, K)).astype(np.uint8)
        w[(w & 0x7F) == 0x7F] = 0x3F
        ws = (rng.random(N) * 2e-3 + 1e-3).astype(np.float32)
        wd = dequant_fp8_rows(w, ws)
    else:
        w = rng.integers(0, 256, size=(N, K // 2)).astype(np.uint8)
        ws = rng.integers(118, 124, size=(N, K // 32)).astype(np.uint8)
        wd = dequant_mxfp4(w, ws)
    xb = _x(M, K, 17)
    h_in = rng.standard_normal((M, N)).astype(np.float32)
    g = (1 + 0.3 * rng.standard_normal(N)).astype(np.float32)
    h_out, xg, ssp = debug_residual(_dev(xb), _dev(w), _dev(ws), wfmt, torch.from_numpy(h_in).cuda(),
                                    torch.from_numpy(g).cuda(), xg_bf16=bf16)
    h_out, xg, ssp = h_out.cpu().numpy(), xg.cpu().numpy(), ssp.cpu().numpy()
    x = _dec(xb)
    ref = h_in.astype(np.float64) + x @ wd.T
    bound = 3e-5 * (np.abs(x) @ np.abs(wd).T) + 2.0 ** -23 * np.abs(ref)
    assert np.all(np.abs(h_out - ref) <= bound), f"h_out: max excess {np.max(np.abs(h_out - ref) - bound):.3g}"
    hg = h_out.astype(np.float64) * g
    if bf16:
        got = decode_bf16(xg.view(np.uint16))
        assert np.all(np.abs(got - hg) <= 2.0 ** -8 * np.abs(hg) + 1e-38), "xg (BF16: 8 significant bits)"
    else:
        got = xg.view(np.float16).astype(np.float64)
        assert np.all(np.abs(got - hg) <= 2.0 ** -11 * np.abs(hg) + 2.0 ** -25), "xg (FP16)"
    ss_ref = (h_out.astype(np.float64) ** 2).reshape(M, N // 32, 32).sum(-1)
    assert np.allclose(ssp[:, :N // 32], ss_ref, rtol=1e-5, atol=0), "partial sums of squares"
    assert np.all(np.isnan(ssp[:, N // 32:])), "entries past the real ones must stay untouched"
