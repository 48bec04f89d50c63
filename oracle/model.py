"""Float64 reference of the target forward and the greedy block verify.

Readings of points the pages leave open (each also listed in the design
notes): pre-norm decoder with RMSNorm (eps 1e-6) before attention, before the
MLP and after the last layer; no biases; rotate-half RoPE with
inv_freq_i = theta^(-2i/D) applied to q and k at absolute 0-based positions
before caching; attention scale 1/sqrt(D); query head h reads KV head
floor(h / G); SwiGLU MLP = down(SiLU(gate(x)) * up(x)); tied embedding /
lm_head unless the model carries its own lm_head.

Row j of a block for sequence b sits at position n_b + j and sees keys
0 .. n_b + j: the committed cache plus the block rows up to itself.  That
is the mask under which one forward over the block equals 16 autoregressive
steps (HunyuanOCR-1.5 / DFlash write-up, inference loop, step 3).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import codecs
from .codecs import decode_bf16, dequant_fp8_rows, dequant_mxfp4

BLOCK = 16


# ------------------------------------------------------------------ pieces

def rms_norm(h, g, eps):
    """x = h / sqrt(mean(h^2) + eps) * g over the last axis."""
    h = np.asarray(h, dtype=np.float64)
    return h / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps) * np.asarray(g, dtype=np.float64)


def rope(x, pos, theta):
    """Rotate-half RoPE.  x: [..., n, heads, D], pos: [..., n].  The pair
    (x_i, x_{i+D/2}) is rotated by the angle pos * theta^(-2i/D)."""
    D = x.shape[-1]
    half = D // 2
    inv = theta ** (-(2.0 * np.arange(half)) / D)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv  # [..., n, half]
    cos = np.cos(ang)[..., None, :]
    sin = np.sin(ang)[..., None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def silu(x):
    return x / (1.0 + np.exp(-x))


def attention(q, K, V, n, G):
    """Block-causal GQA attention for one sequence.

    q: [T, Hq, D] rows at positions n .. n+T-1; K, V: [Hkv, >= n+T, D] with the
    block's own keys already stored at n .. n+T-1.  Row j attends to keys
    0 .. n+j with softmax(q.k / sqrt(D)) (max subtracted).  Returns [T, Hq, D]."""
    T, Hq, D = q.shape
    out = np.empty_like(q)
    scale = 1.0 / np.sqrt(D)
    for j in range(T):
        last = n + j
        for kvh in range(Hq // G):
            qs = q[j, kvh * G:(kvh + 1) * G, :]          # [G, D]
            s = qs @ K[kvh, :last + 1, :].T * scale       # [G, last+1]
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            out[j, kvh * G:(kvh + 1) * G, :] = (p @ V[kvh, :last + 1, :]) / p.sum(axis=1, keepdims=True)
    return out


# ------------------------------------------------------------------ model

class OracleModel:
    """Weights in the boundary's layout, decoded to float64 on first use."""

    def __init__(self, shape, weights: dict, cache: bool = True, act_mx8: bool = False):
        """act_mx8: the FP8-activation mode -- the normed activations that feed
        the QKV and gate/up projections and the SwiGLU output that feeds the
        down projection are held as MXFP8 (codecs.mxfp8_roundtrip); everything
        else is unchanged."""
        self.m = shape
        self.w = weights
        self.cache = cache
        self.act = codecs.mxfp8_roundtrip if act_mx8 else (lambda x: x)
        self._layers = {}
        self._embed = None
        self._lm = None

    def layer(self, l: int) -> dict:
        if l in self._layers:
            return self._layers[l]
        m, lw = self.m, self.w["layers"][l]
        qkv = dequant_fp8_rows(lw["w_qkv"], lw["s_qkv"])
        nq, nk = m.n_q_heads * m.head_dim, m.n_kv_heads * m.head_dim
        if m.mlp_format == "fp8":
            gu = dequant_fp8_rows(lw["w_gate_up"], lw["s_gate_up"])
            wd = dequant_fp8_rows(lw["w_down"], lw["s_down"])
        else:
            gu = dequant_mxfp4(lw["w_gate_up"], lw["s_gate_up"])
            wd = dequant_mxfp4(lw["w_down"], lw["s_down"])
        d = {"wq": qkv[:nq], "wk": qkv[nq:nq + nk], "wv": qkv[nq + nk:],
             "wo": dequant_fp8_rows(lw["w_o"], lw["s_o"]),
             "wg": gu[:m.intermediate], "wu": gu[m.intermediate:], "wd": wd,
             "attn_norm": np.asarray(lw["attn_norm"], np.float64),
             "mlp_norm": np.asarray(lw["mlp_norm"], np.float64)}
        if self.cache:
            self._layers[l] = d
        return d

    def embed(self, tokens) -> np.ndarray:
        tokens = np.asarray(tokens).reshape(-1)
        return decode_bf16(self.w["embed"][tokens])

    def logits(self, x, chunk: int = 16384) -> np.ndarray:
        """x: [rows, H] -> [rows, V], lm_head rows decoded chunk by chunk."""
        table = self.w["embed"] if self.w.get("lm_head") is None else self.w["lm_head"]
        if self.cache and self._lm is None:
            self._lm = decode_bf16(table)
        out = np.empty((x.shape[0], self.m.vocab), dtype=np.float64)
        for v0 in range(0, self.m.vocab, chunk):
            w = self._lm[v0:v0 + chunk] if self._lm is not None else decode_bf16(table[v0:v0 + chunk])
            out[:, v0:v0 + chunk] = x @ w.T
        return out


class OracleKV:
    """Per-layer, per-sequence K and V, float64 [Hkv, capacity_b, D], plus
    committed lengths n.  capacity may be one int or one per sequence."""

    def __init__(self, shape, batch: int, capacity):
        self.m = shape
        caps = np.broadcast_to(np.asarray(capacity, dtype=np.int64), (batch,))
        self.caps = caps.copy()
        shp = lambda c: (shape.n_kv_heads, int(c), shape.head_dim)
        self.K = [[np.zeros(shp(c)) for c in caps] for _ in range(shape.n_layers)]
        self.V = [[np.zeros(shp(c)) for c in caps] for _ in range(shape.n_layers)]
        self.n = np.zeros(batch, dtype=np.int64)

    @classmethod
    def from_bf16(cls, shape, K_layers, V_layers, lens, extra: int = 16):
        """Load BF16 caches ([B, Hkv, cap, D] uint16 per layer); only the
        committed prefix of each sequence is read; each sequence gets room
        for ``extra`` more rows."""
        lens = np.asarray(lens)
        kv = cls(shape, len(lens), lens + extra)
        for l in range(shape.n_layers):
            for b, n in enumerate(lens):
                kv.K[l][b][:, :n] = decode_bf16(K_layers[l][b, :, :n])
                kv.V[l][b][:, :n] = decode_bf16(V_layers[l][b, :, :n])
        kv.n[:] = lens
        return kv

    def copy(self):
        c = OracleKV.__new__(OracleKV)
        c.m, c.caps = self.m, self.caps.copy()
        c.K = [[k.copy() for k in layer] for layer in self.K]
        c.V = [[v.copy() for v in layer] for layer in self.V]
        c.n = self.n.copy()
        return c


def forward(model: OracleModel, kv: OracleKV, tokens, seqs=None) -> np.ndarray:
    """One forward over T rows per sequence.  tokens: [B', T] for the
    sequences ``seqs`` (default: all, in order).  Row j of sequence b is at
    position n_b + j; its K/V are written to cache slots n_b + j (the
    committed length is not changed).  Returns the final normed hidden
    state [B', T, H]."""
    m = model.m
    tokens = np.asarray(tokens)
    Bp, T = tokens.shape
    seqs = np.arange(Bp) if seqs is None else np.asarray(seqs)
    n = kv.n[seqs]
    assert np.all(n + T <= kv.caps[seqs]), "block does not fit the cache"
    D, Hq, Hkv = m.head_dim, m.n_q_heads, m.n_kv_heads
    pos = n[:, None] + np.arange(T)[None, :]
    h = model.embed(tokens).reshape(Bp * T, m.hidden)
    for l in range(m.n_layers):
        w = model.layer(l)
        x = model.act(rms_norm(h, w["attn_norm"], m.rms_eps))
        q = rope((x @ w["wq"].T).reshape(Bp, T, Hq, D), pos, m.rope_theta)
        k = rope((x @ w["wk"].T).reshape(Bp, T, Hkv, D), pos, m.rope_theta)
        v = (x @ w["wv"].T).reshape(Bp, T, Hkv, D)
        o = np.empty((Bp, T, Hq, D))
        for i, b in enumerate(seqs):
            nb = int(n[i])
            kv.K[l][b][:, nb:nb + T] = k[i].transpose(1, 0, 2)
            kv.V[l][b][:, nb:nb + T] = v[i].transpose(1, 0, 2)
            o[i] = attention(q[i], kv.K[l][b], kv.V[l][b], nb, m.group)
        h = h + o.reshape(Bp * T, Hq * D) @ w["wo"].T
        x = model.act(rms_norm(h, w["mlp_norm"], m.rms_eps))
        h = h + model.act(silu(x @ w["wg"].T) * (x @ w["wu"].T)) @ w["wd"].T
    x = rms_norm(h, model.w["final_norm"], m.rms_eps)
    return x.reshape(Bp, T, m.hidden)


def greedy(logits):
    """Argmax over the last axis (lowest id on ties) and the top-2 margin."""
    g = np.argmax(logits, axis=-1)
    top2 = np.partition(logits, -2, axis=-1)[..., -2:]
    return g.astype(np.int64), top2[..., 1] - top2[..., 0]


def accept(tokens, g):
    """Longest accepted prefix.  tokens, g: [B, 16]; tokens[:, 0] is the
    pending token (always kept).  tau = the first j >= 1 with
    tokens[j] != g[j-1], else 16; bonus = g[tau-1] (the correction when a
    draft was rejected, the extra token when all were kept)."""
    tokens, g = np.asarray(tokens), np.asarray(g)
    B, K = tokens.shape
    tau = np.full(B, K, dtype=np.int64)
    for b in range(B):
        for j in range(1, K):
            if tokens[b, j] != g[b, j - 1]:
                tau[b] = j
                break
    bonus = g[np.arange(B), tau - 1]
    return tau, bonus


def commit(kv: OracleKV, counts, seqs=None):
    seqs = np.arange(len(kv.n)) if seqs is None else np.asarray(seqs)
    kv.n[seqs] += np.asarray(counts, dtype=np.int64)


@dataclass
class VerifyResult:
    g: np.ndarray        # [B, 16] argmax per row
    margin: np.ndarray   # [B, 16] top1 - top2 logit
    tau: np.ndarray      # [B] accepted length, 1..16
    bonus: np.ndarray    # [B]
    hidden: np.ndarray   # [B, 16, H] final normed hidden
    logits: np.ndarray   # [B, 16, V]


def verify_block(model, kv, tokens, seqs=None) -> VerifyResult:
    """One verify pass: forward the block, argmax every row, accept.  K/V of
    all 16 rows land in slots n_b .. n_b+15; nothing is committed."""
    tokens = np.asarray(tokens)
    x = forward(model, kv, tokens, seqs)
    Bp, T, H = x.shape
    lg = model.logits(x.reshape(Bp * T, H)).reshape(Bp, T, -1)
    g, margin = greedy(lg)
    tau, bonus = accept(tokens, g)
    return VerifyResult(g, margin, tau, bonus, x, lg)


def prefill(model, kv, prompts, chunk: int = 256, return_hidden: bool = False):
    """Run each prompt through the model in chunks, committing every row.
    Returns the pending token per sequence: the argmax at its last prompt row;
    with return_hidden, also that row's final normed hidden state [B, H] and
    the top-2 logit margin there."""
    pend = np.empty(len(prompts), dtype=np.int64)
    hid = np.empty((len(prompts), model.m.hidden))
    margin = np.empty(len(prompts))
    for b, p in enumerate(prompts):
        p = np.asarray(p)
        for c0 in range(0, len(p), chunk):
            rows = p[c0:c0 + chunk][None, :]
            x = forward(model, kv, rows, seqs=[b])
            commit(kv, [rows.shape[1]], seqs=[b])
        g, mg = greedy(model.logits(x[0, -1:]))
        pend[b], margin[b], hid[b] = g[0], mg[0], x[0, -1]
    return (pend, hid, margin) if return_hidden else pend


def greedy_continuation(model, kv, pending, steps: int = BLOCK - 1):
    """pending plus ``steps`` autoregressive greedy tokens per sequence:
    cont[:, 0] = pending, cont[:, j] = argmax after cont[:, :j].  Works on
    uncommitted slots and leaves the committed lengths as they were."""
    n0 = kv.n.copy()
    cur = np.asarray(pending, dtype=np.int64)
    cont = [cur]
    for _ in range(steps):
        x = forward(model, kv, cur[:, None])
        cur = greedy(model.logits(x[:, 0]))[0]
        commit(kv, np.ones_like(cur))
        cont.append(cur)
    kv.n[:] = n0
    return np.stack(cont, axis=1)


def ar_decode(model, kv, pending, n_tokens: int, return_margin: bool = False):
    """Plain autoregressive greedy decoding: feed the pending token, emit the
    argmax, commit one row, repeat.  Returns [B, n_tokens] emitted tokens
    (and, with return_margin, the top-2 logit margin of each step)."""
    cur = np.asarray(pending, dtype=np.int64)
    out, margins = [], []
    for _ in range(n_tokens):
        x = forward(model, kv, cur[:, None])
        cur, mg = greedy(model.logits(x[:, 0]))
        commit(kv, np.ones_like(cur))
        out.append(cur)
        margins.append(mg)
    toks = np.stack(out, axis=1)
    return (toks, np.stack(margins, axis=1)) if return_margin else toks


def spec_decode(model, kv, pending, n_tokens: int, draft_fn):
    """Greedy speculative decoding with 16-token blocks (one sequence per
    call row).  draft_fn(b, pending_b, emitted_b) -> 15 draft ids.  Each
    round emits tokens[1..tau-1] followed by the bonus, commits tau rows and
    makes the bonus the next pending token.  Returns ([B, n_tokens] emitted,
    list of per-round tau arrays)."""
    cur = np.asarray(pending, dtype=np.int64).copy()
    B = len(cur)
    emitted = [[] for _ in range(B)]
    taus = []
    while min(len(e) for e in emitted) < n_tokens:
        blk = np.stack([np.concatenate([[cur[b]], draft_fn(b, cur[b], emitted[b])]) for b in range(B)])
        r = verify_block(model, kv, blk)
        commit(kv, r.tau)
        for b in range(B):
            emitted[b] += list(blk[b, 1:r.tau[b]]) + [int(r.bonus[b])]
        cur = r.bonus.copy()
        taus.append(r.tau)
    return np.stack([np.array(e[:n_tokens]) for e in emitted]), taus
