"""Whole-model pins for the oracle.

1. An independent float64 PyTorch formulation: the whole sequence (prompt and
   block) in ONE causal forward with library routines (F.linear, F.rms_norm,
   F.scaled_dot_product_attention with GQA, F.silu, RoPE as a complex
   rotation, weights decoded through torch's float8 dtype) must reproduce
   the oracle's KV-cached chunked prefill followed by a block verify.
2. The lossless invariant (OCRia stack page, speculative decoding section;
   HunyuanOCR-1.5 / DFlash write-up, inference loop): greedy speculative
   decoding emits exactly the autoregressive greedy stream, for random,
   adversarial and planted drafts, and commits the same KV rows.
3. The planting law: planted acceptance lengths follow min(Geometric(p), 16)
   whose mean is (1 - (1-p)^16) / p, and a planted block is accepted
   exactly up to its planted length.
"""
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import workload as W
from oracle import (OracleKV, OracleModel, accept, ar_decode, commit, forward, greedy,
                    greedy_continuation, prefill, spec_decode, verify_block)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch_dequant(codes, scales, fmt):
    if fmt == "fp8":
        w = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double()
        return w * torch.from_numpy(scales).double()[:, None]
    table = {}
    for l in open(os.path.join(GOLDEN, "e2m1_values.txt")):
        if l.strip() and l[0] != "#":
            c, v = l.split()
            table[int(c)] = float(v)
    lut = torch.tensor([table[i] for i in range(16)], dtype=torch.float64)
    c = torch.from_numpy(codes.astype(np.int64))
    vals = torch.stack([lut[c & 15], lut[c >> 4]], dim=-1).reshape(codes.shape[0], -1)
    sc = torch.from_numpy(np.ascontiguousarray(scales)).view(torch.float8_e8m0fnu).double()
    return vals * sc.repeat_interleave(32, dim=1)


def _torch_full_forward(m, wts, seq):
    """All rows of one sequence in one causal forward, no cache."""
    T = len(seq)
    D, Hq, Hkv = m.head_dim, m.n_q_heads, m.n_kv_heads
    emb = torch.from_numpy(wts["embed"].view(np.int16)).view(torch.bfloat16).double()
    h = emb[torch.from_numpy(np.asarray(seq, np.int64))]
    half = D // 2
    inv = m.rope_theta ** (-(torch.arange(half, dtype=torch.float64) * 2) / D)
    rot = torch.polar(torch.ones(T, half, dtype=torch.float64), torch.arange(T, dtype=torch.float64)[:, None] * inv)

    def rope_c(x):  # x [T, heads, D]
        z = torch.complex(x[..., :half], x[..., half:]) * rot[:, None, :]
        return torch.cat([z.real, z.imag], dim=-1)

    kcache, vcache = [], []
    for lw in wts["layers"]:
        qkv = _torch_dequant(lw["w_qkv"], lw["s_qkv"], "fp8")
        wq, wk, wv = qkv[:Hq * D], qkv[Hq * D:(Hq + Hkv) * D], qkv[(Hq + Hkv) * D:]
        x = F.rms_norm(h, (m.hidden,), torch.from_numpy(lw["attn_norm"]).double(), eps=m.rms_eps)
        q = rope_c(F.linear(x, wq).view(T, Hq, D))
        k = rope_c(F.linear(x, wk).view(T, Hkv, D))
        v = F.linear(x, wv).view(T, Hkv, D)
        kcache.append(k.transpose(0, 1).numpy())
        vcache.append(v.transpose(0, 1).numpy())
        o = F.scaled_dot_product_attention(q.transpose(0, 1)[None], k.transpose(0, 1)[None],
                                           v.transpose(0, 1)[None], is_causal=True, enable_gqa=True)
        h = h + F.linear(o[0].transpose(0, 1).reshape(T, Hq * D), _torch_dequant(lw["w_o"], lw["s_o"], "fp8"))
        gu = _torch_dequant(lw["w_gate_up"], lw["s_gate_up"], m.mlp_format)
        wd = _torch_dequant(lw["w_down"], lw["s_down"], m.mlp_format)
        x = F.rms_norm(h, (m.hidden,), torch.from_numpy(lw["mlp_norm"]).double(), eps=m.rms_eps)
        h = h + F.linear(F.silu(F.linear(x, gu[:m.intermediate])) * F.linear(x, gu[m.intermediate:]), wd)
    x = F.rms_norm(h, (m.hidden,), torch.from_numpy(wts["final_norm"]).double(), eps=m.rms_eps)
    table = wts["embed"] if wts["lm_head"] is None else wts["lm_head"]
    lm = torch.from_numpy(table.view(np.int16)).view(torch.bfloat16).double()
    return x.numpy(), (x @ lm.T).numpy(), kcache, vcache


@pytest.mark.parametrize("fmt,gains", [("fp8", "ones"), ("fp8", "random"), ("mxfp4", "random")])
def test_oracle_matches_independent_full_forward(fmt, gains):
    import dataclasses
    m = dataclasses.replace(W.TINY, mlp_format=fmt)
    if fmt == "mxfp4":
        m = dataclasses.replace(m, tied_lm_head=False)
    wts = W.model_weights(m, seed=3, gains=gains)
    prompt = W.child_rng(3, 99).integers(0, m.vocab, size=45)
    block = W.child_rng(3, 98).integers(0, m.vocab, size=16)
    model = OracleModel(m, wts)
    kv = OracleKV(m, 1, 64)
    prefill(model, kv, [prompt], chunk=20)
    r = verify_block(model, kv, block[None])
    hid, lg, kc, vc = _torch_full_forward(m, wts, np.concatenate([prompt, block]))
    assert np.allclose(r.hidden[0], hid[45:], rtol=1e-11, atol=1e-11)
    assert np.allclose(r.logits[0], lg[45:], rtol=1e-11, atol=1e-11)
    # cache slots hold K (rotated at absolute position p = slot) and V of every row
    assert kv.n[0] == 45
    for l in range(m.n_layers):
        assert np.allclose(kv.K[l][0][:, :61], kc[l], rtol=1e-11, atol=1e-11)
        assert np.allclose(kv.V[l][0][:, :61], vc[l], rtol=1e-11, atol=1e-11)


def _setup_tiny(seed=0, B=1, capacity=128 + 16 * 40):
    wl = W.WORKLOADS["tiny-b1-ctx128"]
    m = wl.model
    wts = W.model_weights(m, seed)
    model = OracleModel(m, wts)
    kv = OracleKV(m, B, capacity)
    prompts = [W.child_rng(seed, 50, b).integers(0, m.vocab, size=128) for b in range(B)]
    pend = prefill(model, kv, prompts, chunk=64)
    return m, model, kv, pend


def test_block_rows_equal_autoregressive_rows():
    m, model, kv, pend = _setup_tiny()
    kv2 = kv.copy()
    cont = greedy_continuation(model, kv, pend)          # 16 greedy tokens
    r = verify_block(model, kv, cont)                    # a block that is all greedy
    assert r.tau[0] == 16 and r.bonus[0] == ar_decode(model, kv2.copy(), pend, 16)[0, 15]
    assert np.array_equal(r.g[0, :15], cont[0, 1:])
    # row j of the block equals AR step j: hidden states and KV slots
    ar_hidden = []
    cur = pend
    for j in range(16):
        x = forward(model, kv2, np.array([[cont[0, j]]]))
        ar_hidden.append(x[0, 0])
        commit(kv2, [1])
    assert np.allclose(np.stack(ar_hidden), r.hidden[0], rtol=1e-12, atol=1e-12)
    for l in range(m.n_layers):
        assert np.allclose(kv.K[l][0][:, 128:144], kv2.K[l][0][:, 128:144], rtol=1e-12, atol=1e-12)
        assert np.allclose(kv.V[l][0][:, 128:144], kv2.V[l][0][:, 128:144], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("kind", ["random", "planted", "all_right", "last_wrong", "first_wrong"])
def test_spec_equals_autoregressive(kind):
    N = 256
    m, model, kv, pend = _setup_tiny(B=2)
    kv_ar = kv.copy()
    ref = ar_decode(model, kv_ar, pend, N + 16)
    g = W.child_rng(7, 1)
    Lg = W.child_rng(7, 2)

    def draft(b, p, emitted):
        k = len(emitted)
        truth = np.zeros(15, dtype=np.int64)                 # past the reference: anything
        seg = ref[b, k:k + 15]
        truth[:len(seg)] = seg
        if kind == "random":
            return g.integers(0, m.vocab, size=15)
        d = truth.copy()
        if kind == "planted":
            L = int(W.geometric_capped(Lg, 0.1))
            if L < 16:
                d[L - 1] = (truth[L - 1] + 1 + g.integers(0, m.vocab - 1)) % m.vocab
        elif kind == "last_wrong":
            d[14] = (d[14] + 1) % m.vocab
        elif kind == "first_wrong":
            d[0] = (d[0] + 1) % m.vocab
        return d

    out, taus = spec_decode(model, kv, pend, N, draft)
    assert np.array_equal(out, ref[:, :N])
    taus = np.stack(taus)
    if kind == "all_right":
        assert np.all(taus == 16)
    if kind == "last_wrong":
        assert np.all(taus == 15)
    if kind == "first_wrong":
        assert np.all(taus == 1)
    # committed KV equals the autoregressive cache on the common committed prefix
    n = int(min(kv.n.min(), kv_ar.n.min()))
    for l in range(m.n_layers):
        for b in range(2):
            assert np.allclose(kv.K[l][b][:, :n], kv_ar.K[l][b][:, :n], rtol=1e-11, atol=1e-11)
            assert np.allclose(kv.V[l][b][:, :n], kv_ar.V[l][b][:, :n], rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("p", [0.1, 0.2])
def test_planted_length_law(p):
    L = W.geometric_capped(np.random.default_rng(11), p, size=400_000)
    assert L.min() == 1 and L.max() == 16
    assert abs(L.mean() - (1 - (1 - p) ** 16) / p) < 0.03
    assert abs(np.mean(L == 16) - (1 - p) ** 15) < 0.005


def test_planted_block_is_accepted_to_its_length():
    rng = np.random.default_rng(12)
    for L in range(1, 17):
        for _ in range(20):
            cont = rng.integers(0, 5, size=16)                 # tiny vocab forces redraws
            t = W.plant_block(cont, L, 5, rng)
            g = np.concatenate([cont[1:], [rng.integers(0, 5)]])  # argmax row j = cont[j+1]
            tau, bonus = accept(t[None], g[None])
            assert tau[0] == L and t[0] == cont[0]


def test_workload_recipes():
    wl = W.WORKLOADS["0.5b-fp8-b32-ctx512to4096"]
    lens = W.context_lengths(wl)
    assert lens.min() >= 512 and lens.max() <= 4096 and len(lens) == 32
    assert np.array_equal(lens, W.context_lengths(wl))            # seeded
    mx = W.WORKLOADS["0.5b-mxfp4mlp-b16-ctx3072"]
    L = W.accept_lengths(mx)
    assert np.all(L[:8] == 16) and np.all(L[8:] <= 16)
    pr = W.prompts(mx)
    assert np.array_equal(pr[0][:8], pr[0][8:16]) and len(pr[0]) == 3072


@pytest.mark.slow
def test_spec_equals_autoregressive_05b():
    """The invariant on the 0.5B-class shape (24 layers, vocab 151936) with a
    short random prompt and planted drafts, 64 emitted tokens."""
    m = W.M05B
    wts = W.model_weights(m, 0)
    model = OracleModel(m, wts)
    kv = OracleKV(m, 1, 32 + 64 + 32)
    pend = prefill(model, kv, [W.child_rng(0, 60).integers(0, m.vocab, size=32)])
    kv_ar = kv.copy()
    ref = ar_decode(model, kv_ar, pend, 64 + 16)
    Lg, g = W.child_rng(0, 61), W.child_rng(0, 62)

    def draft(b, p, emitted):
        d = np.zeros(15, dtype=np.int64)
        seg = ref[b, len(emitted):len(emitted) + 15]
        d[:len(seg)] = seg
        L = int(W.geometric_capped(Lg, 0.1))
        if L < 16:
            d[L - 1] = (d[L - 1] + 1 + g.integers(0, m.vocab - 1)) % m.vocab
        return d

    out, taus = spec_decode(model, kv, pend, 64, draft)
    assert np.array_equal(out, ref[:, :64])


# ---------------------------------------------------------------- FP8-activation mode

def test_act_mx8_mode_changes_only_the_three_points(monkeypatch):
    """With the MXFP8 round trip replaced by the identity the mode's forward is
    the exact forward, bit for bit; the round trip runs at exactly three
    points per layer (normed x before attention, before the MLP, and the
    SwiGLU output)."""
    import oracle.codecs as C
    m = W.TINY
    wts = W.model_weights(m, 1, gains="random")
    calls = []
    monkeypatch.setattr(C, "mxfp8_roundtrip", lambda x: (calls.append(np.shape(x)), x)[1])
    exact, mode = OracleModel(m, wts), OracleModel(m, wts, act_mx8=True)
    toks = W.child_rng(1, 60).integers(0, m.vocab, size=(1, 24))
    a = forward(exact, OracleKV(m, 1, 64), toks)
    b = forward(mode, OracleKV(m, 1, 64), toks)
    assert np.array_equal(a, b)
    assert calls == [(24, m.hidden), (24, m.hidden), (24, m.intermediate)] * m.n_layers


def test_act_mx8_mode_spec_equals_autoregressive():
    """Block quantisation is row-local, so greedy speculative decoding stays
    lossless in the FP8-activation mode."""
    m = W.TINY
    wts = W.model_weights(m, 2)
    model = OracleModel(m, wts, act_mx8=True)
    kv = OracleKV(m, 1, 128 + 16 * 12)
    pend = prefill(model, kv, [W.child_rng(2, 61).integers(0, m.vocab, size=128)], chunk=64)
    kv_ar = kv.copy()
    ref = ar_decode(model, kv_ar, pend, 96 + 16)
    Lg = W.child_rng(2, 62)

    def draft(b, p, emitted):
        k = len(emitted)
        d = np.zeros(15, dtype=np.int64)
        seg = ref[b, k:k + 15]
        d[:len(seg)] = seg
        L = int(W.geometric_capped(Lg, 0.2))
        if L < 16:
            d[L - 1] = (d[L - 1] + 1) % m.vocab
        return d

    out, _ = spec_decode(model, kv, pend, 96, draft)
    assert np.array_equal(out, ref[:, :96])
    # and the mode does change the numbers (the quantisation is not a no-op)
    exact = OracleModel(m, wts)
    x0 = forward(exact, OracleKV(m, 1, 32), ref[:, :16])
    x1 = forward(model, OracleKV(m, 1, 32), ref[:, :16])
    assert not np.array_equal(x0, x1) and np.max(np.abs(x0 - x1)) < 0.5
