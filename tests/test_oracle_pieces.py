"""Pins for the oracle's building blocks: RMSNorm, RoPE, SiLU, block-causal
GQA attention, greedy argmax and the acceptance rule.  Each is compared with a
float64 library routine, a different formulation, a closed form or a brute
force, never with a retyped copy of itself."""
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import accept, attention, greedy, rms_norm, rope, silu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_rms_norm_matches_torch_and_is_scale_invariant():
    rng = np.random.default_rng(0)
    h = rng.standard_normal((7, 96)) * 3
    g = 1 + 0.1 * rng.standard_normal(96)
    ref = F.rms_norm(torch.from_numpy(h), (96,), torch.from_numpy(g), eps=1e-6).numpy()
    assert np.allclose(rms_norm(h, g, 1e-6), ref, rtol=1e-13, atol=1e-13)
    assert np.allclose(rms_norm(5.0 * h, g, 0.0), rms_norm(h, g, 0.0), rtol=1e-13)
    x = rms_norm(h, np.ones(96), 0.0)
    assert np.allclose(np.mean(x * x, axis=1), 1.0, rtol=1e-13)


def test_silu_matches_torch():
    x = np.linspace(-30, 30, 2001)
    assert np.allclose(silu(x), F.silu(torch.from_numpy(x)).numpy(), rtol=1e-14, atol=1e-300)


def _rope_complex(x, pos, theta):
    """RoPE as complex multiplication: z_i = x_i + i x_{i+D/2} times e^{i pos w_i}."""
    D = x.shape[-1]
    half = D // 2
    w = theta ** (-(2.0 * np.arange(half)) / D)
    z = x[..., :half] + 1j * x[..., half:]
    r = z * np.exp(1j * pos[:, None, None] * w)
    return np.concatenate([r.real, r.imag], axis=-1)


def test_rope_identities():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 3, 64))
    pos = np.array([0, 1, 17, 2048, 4111])
    out = rope(x, pos, 1e4)
    assert np.array_equal(out[0], x[0])                       # position 0 is the identity
    assert np.allclose(out, _rope_complex(x, pos, 1e4), rtol=1e-12, atol=1e-12)
    n_in = x[..., :32] ** 2 + x[..., 32:] ** 2                 # each rotated pair keeps its norm
    n_out = out[..., :32] ** 2 + out[..., 32:] ** 2
    assert np.allclose(n_in, n_out, rtol=1e-12)
    q, k = rng.standard_normal((1, 1, 128)), rng.standard_normal((1, 1, 128))
    a = np.sum(rope(q, np.array([37]), 1e4) * rope(k, np.array([5]), 1e4))
    b = np.sum(rope(q, np.array([37 + 900]), 1e4) * rope(k, np.array([5 + 900]), 1e4))
    assert abs(a - b) < 1e-9 * (1 + abs(a))                    # q.k depends on the offset only


def _sdpa_block(q, K, V, n, G):
    """torch SDPA in float64 with an explicit block-causal mask."""
    T, Hq, D = q.shape
    L = n + T
    mask = torch.arange(L)[None, :] <= (n + torch.arange(T))[:, None]
    o = F.scaled_dot_product_attention(
        torch.from_numpy(q).permute(1, 0, 2)[None], torch.from_numpy(K[:, :L])[None],
        torch.from_numpy(V[:, :L])[None], attn_mask=mask, enable_gqa=True)
    return o[0].permute(1, 0, 2).numpy()


def _masked_bruteforce(q, K, V, n, G):
    """Full [T, n+T] score matrix, -inf above the block diagonal, softmax, @V."""
    T, Hq, D = q.shape
    L = n + T
    out = np.zeros_like(q)
    for h in range(Hq):
        s = q[:, h, :] @ K[h // G, :L].T / np.sqrt(D)
        s[np.arange(L)[None, :] > (n + np.arange(T))[:, None]] = -np.inf
        p = np.exp(s - s.max(axis=1, keepdims=True))
        out[:, h, :] = (p / p.sum(axis=1, keepdims=True)) @ V[h // G, :L]
    return out


@pytest.mark.parametrize("n,G,Hkv,D", [(0, 1, 2, 16), (5, 7, 2, 64), (40, 4, 3, 32), (300, 2, 1, 128)])
def test_attention_vs_sdpa_and_bruteforce(n, G, Hkv, D):
    rng = np.random.default_rng(n + G)
    T = 16
    q = rng.standard_normal((T, G * Hkv, D))
    K = rng.standard_normal((Hkv, n + T + 3, D))
    V = rng.standard_normal((Hkv, n + T + 3, D))
    K[:, n + T:] = np.nan                                       # slots past the block are never read
    V[:, n + T:] = np.nan
    got = attention(q, K, V, n, G)
    assert np.allclose(got, _sdpa_block(q, K, V, n, G), rtol=1e-12, atol=1e-12)
    assert np.allclose(got, _masked_bruteforce(q, K, V, n, G), rtol=1e-12, atol=1e-12)


def test_attention_special_cases():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((16, 4, 8))
    K = rng.standard_normal((2, 16, 8))
    V = rng.standard_normal((2, 16, 8))
    o = attention(q, K, V, 0, 2)
    assert np.allclose(o[0, 0], V[0, 0]) and np.allclose(o[0, 3], V[1, 0])  # first row sees one key
    Kc = np.repeat(K[:, :1], 16, axis=1)                        # identical keys -> mean of visible V
    o = attention(q, Kc, V, 0, 2)
    for j in range(16):
        assert np.allclose(o[j, 1], V[0, :j + 1].mean(axis=0), rtol=1e-12)
    # duplicating KV heads turns GQA into plain multi-head attention
    Kd, Vd = np.repeat(K, 2, axis=0), np.repeat(V, 2, axis=0)
    assert np.allclose(attention(q, K, V, 0, 2), attention(q, Kd, Vd, 0, 1), rtol=1e-13)


def test_greedy_ties_and_margin():
    lg = np.array([[0.0, 3.0, 3.0, 1.0], [5.0, -1.0, 4.5, 4.9]])
    g, m = greedy(lg)
    assert list(g) == [1, 0] and m[0] == 0.0 and abs(m[1] - 0.1) < 1e-12
    rng = np.random.default_rng(5)
    big = rng.standard_normal((9, 1000))
    g, m = greedy(big)
    for r in range(9):
        srt = np.sort(big[r])
        assert big[r, g[r]] == srt[-1] and m[r] == srt[-1] - srt[-2]


def test_accept_golden_examples():
    for line in open(os.path.join(GOLDEN, "accept_examples.txt")):
        if not line.strip() or line.startswith("#"):
            continue
        blk, g, tau, emitted = [p.split() for p in line.split("|")]
        blk, g = np.array([blk], int), np.array([g], int)
        t, b = accept(blk, g)
        assert t[0] == int(tau[0])
        assert list(blk[0, 1:t[0]]) + [b[0]] == [int(e) for e in emitted]


def test_accept_bruteforce():
    rng = np.random.default_rng(6)
    for _ in range(500):
        V = int(rng.integers(2, 5))                               # tiny vocab: many accidental matches
        blk = rng.integers(0, V, size=(3, 16))
        g = rng.integers(0, V, size=(3, 16))
        tau, bonus = accept(blk, g)
        for b in range(3):
            kept = 1
            while kept < 16 and blk[b, kept] == g[b, kept - 1]:
                kept += 1
            assert tau[b] == kept and bonus[b] == g[b, kept - 1]
