"""Seeded synthetic inputs for the block-draft verify pass.

This module is input preparation only.  It draws random numbers and packs them
into the byte layouts that the verify pass consumes:

* FP8-e4m3 (OCP "fn" variant) weight codes with one fp32 scale per output row,
* MXFP4 weight codes (e2m1 nibbles, low nibble = even input index) with one
  e8m0 exponent per 32 inputs,
* BF16 embedding / lm_head tables (stored as uint16 bit patterns),
* prompts, context lengths, planted acceptance lengths, draft blocks and
  synthetic BF16 KV caches.

Nothing here computes a step of the verify pass.  The CPU oracle and the HIP
path both consume these arrays and share nothing else.  Encodings are the
shapes of the synthetic workloads (weights drawn N(0, 0.02^2), then quantised
per output channel); the verify pass only ever decodes them.

Seeds: every purpose draws from its own child of ``SeedSequence(seed)`` keyed
by (purpose, ...) so that any piece can be regenerated alone and in parallel.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
import os

import numpy as np
import torch

BLOCK_K = 16  # tokens per verify block: the pending token plus 15 drafts

# purpose keys for child seeds
_P_WEIGHTS, _P_PROMPTS, _P_CTXLEN, _P_ACCEPT, _P_DRAFT, _P_KV, _P_PENDING, _P_GAINS = range(1, 9)


@dataclass(frozen=True)
class ModelShape:
    name: str
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    vocab: int
    tied_lm_head: bool = True
    mlp_format: str = "fp8"  # "fp8" (per-row e4m3) or "mxfp4" (e2m1 + e8m0 per 32)
    rms_eps: float = 1e-6
    rope_theta: float = 1e4

    @property
    def qkv_rows(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


TINY = ModelShape("tiny-L2-H256", 2, 256, 4, 2, 64, 704, 1024)
M05B = ModelShape("0.5b-L24-H896", 24, 896, 14, 2, 64, 4864, 151936)
M05B_MXFP4 = dataclasses.replace(M05B, name="0.5b-L24-H896-mxfp4mlp", mlp_format="mxfp4")
M8B = ModelShape("8b-L32-H4096", 32, 4096, 32, 8, 128, 14336, 128256, tied_lm_head=False)


@dataclass(frozen=True)
class Workload:
    """One synthetic verify workload.

    context: ("fixed", n) or ("uniform", lo, hi) (inclusive integers).
    planting: per-sequence acceptance law, a tuple of (rule, share) where rule is
      ("geom", p) -> L = min(Geometric_{>=1}(p), 16), or ("cycle8",) -> L = 16
      with a period-8 prompt; shares split the batch in order.
    kv_fill: "prefill" (KV computed from the prompt) or "synthetic"
      (BF16 N(0, (0.02*sqrt(H))^2) entries, uniform pending token).
    """
    name: str
    model: ModelShape
    batch: int
    context: tuple
    planting: tuple
    kv_fill: str
    seed: int = 0

    @property
    def rows(self) -> int:
        return self.batch * BLOCK_K

    @property
    def max_ctx(self) -> int:
        hi = self.context[1] if self.context[0] == "fixed" else self.context[2]
        return ((hi + BLOCK_K + 63) // 64) * 64


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny-b1-ctx128", TINY, 1, ("fixed", 128), ((("geom", 0.1), 1),), "prefill"),
        Workload("0.5b-fp8-b1-ctx2048", M05B, 1, ("fixed", 2048), ((("geom", 0.1), 1),), "prefill"),
        Workload("0.5b-fp8-b32-ctx512to4096", M05B, 32, ("uniform", 512, 4096),
                 ((("geom", 0.1), 32),), "synthetic"),
        Workload("8b-fp8-b8-ctx4096", M8B, 8, ("fixed", 4096), ((("geom", 0.1), 8),), "synthetic"),
        Workload("0.5b-mxfp4mlp-b16-ctx3072", M05B_MXFP4, 16, ("fixed", 3072),
                 ((("cycle8",), 8), (("geom", 0.2), 8)), "synthetic"),
    ]
}


def child_rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(key))))


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


# ---------------------------------------------------------------- encodings

FP8_MAX = 448.0


def encode_fp8_rows(w: np.ndarray):
    """Per-output-row FP8-e4m3fn: s = absmax/448 (fp32, 1 for an all-zero row),
    codes = round-to-nearest-even(w/s) saturated to +-448."""
    w = np.asarray(w, dtype=np.float32)
    amax = np.abs(w).max(axis=1)
    s = (amax / np.float32(FP8_MAX)).astype(np.float32)
    s[amax == 0] = 1.0
    r = np.clip(w / s[:, None], -FP8_MAX, FP8_MAX)
    codes = torch.from_numpy(np.ascontiguousarray(r)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, s


# e2m1 magnitudes in code order, and the rounding boundaries between them;
# a value exactly on a boundary goes to the neighbour with an even mantissa.
_E2M1_BOUNDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)
_E2M1_TIE_UP = np.array([False, True, False, True, False, True, False])


def encode_mxfp4(w: np.ndarray):
    """MXFP4 along the input dimension: blocks of 32, shared exponent
    X = floor(log2(amax)) - 2 stored as e8m0 = X + 127 (clamped to [0, 254]),
    elements RNE onto the e2m1 grid saturating at +-6.  All-zero block -> e8m0 0.
    Returns (codes uint8 [rows, cols/2], low nibble = even column; e8m0 uint8 [rows, cols/32])."""
    w = np.asarray(w, dtype=np.float32)
    rows, cols = w.shape
    assert cols % 32 == 0
    blk = w.reshape(rows, cols // 32, 32)
    amax = np.abs(blk).max(axis=2)
    with np.errstate(divide="ignore"):
        x = np.floor(np.log2(np.where(amax > 0, amax, 1.0))).astype(np.int32) - 2
    e8 = np.clip(x + 127, 0, 254).astype(np.int32)
    e8[amax == 0] = 0
    scale = np.ldexp(np.float64(1.0), (e8 - 127)).astype(np.float64)
    v = (blk.astype(np.float64) / scale[:, :, None]).reshape(rows, cols)
    mag = np.abs(v)
    code = np.zeros(mag.shape, dtype=np.uint8)
    for b, up in zip(_E2M1_BOUNDS, _E2M1_TIE_UP):
        code += (mag > b) if not up else (mag >= b)
    sign = ((v < 0) & (code > 0)).astype(np.uint8) << 3
    nib = code | sign
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    return packed, e8.astype(np.uint8)


def to_bf16_bits(w: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (round to nearest even) as uint16 bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


# ---------------------------------------------------------------- weights

_MAT_IDS = {"q": 0, "k": 1, "v": 2, "o": 3, "gate": 4, "up": 5, "down": 6}


def _draw(seed, key, shape, std=0.02):
    g = child_rng(seed, *key)
    out = np.empty(shape, dtype=np.float32)
    g.standard_normal(out=out, dtype=np.float32)
    out *= np.float32(std)
    return out


_CHUNK_ELEMS = 1 << 22  # 16 MB of fp32 per drawn row block


def _draw_rows(seed, key, rows, cols, std=0.02):
    """Yields (r0, block) fp32 row blocks of one [rows, cols] draw; the blocks
    concatenated equal _draw(seed, key, (rows, cols), std) exactly (one
    generator, consumed in order).  The block buffer is reused between
    yields, so large matrices never exist in fp32 in full."""
    g = child_rng(seed, *key)
    step = max(1, min(rows, _CHUNK_ELEMS // cols))
    buf = np.empty((step, cols), dtype=np.float32)
    for r0 in range(0, rows, step):
        v = buf[:min(step, rows - r0)]
        g.standard_normal(out=v, dtype=np.float32)
        v *= np.float32(std)
        yield r0, v


def _encode(fmt, w):
    return encode_fp8_rows(w) if fmt == "fp8" else encode_mxfp4(w)


def _encoded_matrix(fmt, seed, layer, parts, cols, ex):
    """Rows of several drawn matrices stacked in order ([(name, rows), ...]),
    encoded block by block into preallocated code / scale arrays."""
    rows = sum(r for _, r in parts)
    if fmt == "fp8":
        codes, scales = np.empty((rows, cols), np.uint8), np.empty(rows, np.float32)
    else:
        codes, scales = np.empty((rows, cols // 2), np.uint8), np.empty((rows, cols // 32), np.uint8)

    def one(name, off, r):
        for r0, v in _draw_rows(seed, (_P_WEIGHTS, layer, _MAT_IDS[name]), r, cols):
            c, sc = _encode(fmt, v)
            codes[off + r0:off + r0 + len(v)] = c
            scales[off + r0:off + r0 + len(v)] = sc

    futs, off = [], 0
    for name, r in parts:
        futs.append(ex.submit(one, name, off, r))
        off += r
    return codes, scales, futs


def layer_weights(m: ModelShape, seed: int, layer: int, gains: str = "ones") -> dict:
    """One decoder layer in the boundary's layout (see include/spec_verify.h).

    w_qkv rows are [q heads | k heads | v heads], each head_dim rows;
    w_gate_up rows are [gate (I rows) | up (I rows)]."""
    H, D, I = m.hidden, m.head_dim, m.intermediate
    out = {}
    with ThreadPoolExecutor(_threads()) as ex:
        futs = []
        for wk, sk, fmt, parts, cols in (
                ("w_qkv", "s_qkv", "fp8", [("q", m.n_q_heads * D), ("k", m.n_kv_heads * D), ("v", m.n_kv_heads * D)], H),
                ("w_o", "s_o", "fp8", [("o", H)], m.n_q_heads * D),
                ("w_gate_up", "s_gate_up", m.mlp_format, [("gate", I), ("up", I)], H),
                ("w_down", "s_down", m.mlp_format, [("down", H)], I)):
            out[wk], out[sk], f = _encoded_matrix(fmt, seed, layer, parts, cols, ex)
            futs += f
        for f in futs:
            f.result()
    out["attn_norm"], out["mlp_norm"] = norm_gains(m, seed, layer, gains)
    return out


def _bf16_table(seed, key, rows, cols):
    out = np.empty((rows, cols), np.uint16)
    for r0, v in _draw_rows(seed, key, rows, cols):
        out[r0:r0 + len(v)] = to_bf16_bits(v)
    return out


def norm_gains(m: ModelShape, seed: int, layer: int, gains: str):
    if gains == "ones":
        return np.ones(m.hidden, np.float32), np.ones(m.hidden, np.float32)
    g = child_rng(seed, _P_GAINS, layer)
    return ((1.0 + 0.1 * g.standard_normal((2, m.hidden))).astype(np.float32))


def embedding_weights(m: ModelShape, seed: int, gains: str = "ones") -> dict:
    """BF16 token embedding [V, H]; untied models also get a BF16 lm_head drawn
    the same way; final_norm gains [H]."""
    out = {"embed": _bf16_table(seed, (_P_WEIGHTS, 10_000, 0), m.vocab, m.hidden)}
    out["lm_head"] = None if m.tied_lm_head else _bf16_table(seed, (_P_WEIGHTS, 10_000, 1), m.vocab, m.hidden)
    if gains == "ones":
        out["final_norm"] = np.ones(m.hidden, np.float32)
    else:
        out["final_norm"] = (1.0 + 0.1 * child_rng(seed, _P_GAINS, 10_000).standard_normal(m.hidden)).astype(np.float32)
    return out


def model_weights(m: ModelShape, seed: int = 0, gains: str = "ones") -> dict:
    return {"layers": [layer_weights(m, seed, l, gains) for l in range(m.n_layers)],
            **embedding_weights(m, seed, gains)}


# ---------------------------------------------------------------- sequences

def context_lengths(wl: Workload) -> np.ndarray:
    if wl.context[0] == "fixed":
        return np.full(wl.batch, wl.context[1], dtype=np.int32)
    lo, hi = wl.context[1], wl.context[2]
    return child_rng(wl.seed, _P_CTXLEN).integers(lo, hi + 1, size=wl.batch).astype(np.int32)


def _rules(wl: Workload):
    rules = []
    for rule, share in wl.planting:
        rules += [rule] * share
    assert len(rules) == wl.batch
    return rules


def prompts(wl: Workload, lens=None) -> list:
    """Prompt token ids per sequence: uniform in [0, V), or a uniformly drawn
    8-token cycle tiled to the context length."""
    lens = context_lengths(wl) if lens is None else lens
    out = []
    for b, (rule, n) in enumerate(zip(_rules(wl), lens)):
        g = child_rng(wl.seed, _P_PROMPTS, b)
        if rule[0] == "cycle8":
            cyc = g.integers(0, wl.model.vocab, size=8)
            out.append(np.resize(cyc, int(n)).astype(np.int32))
        else:
            out.append(g.integers(0, wl.model.vocab, size=int(n)).astype(np.int32))
    return out


def geometric_capped(g: np.random.Generator, p: float, size=None, cap: int = BLOCK_K):
    """min(Geometric(p), cap) with support {1, 2, ...}."""
    return np.minimum(g.geometric(p, size=size), cap)


def accept_lengths(wl: Workload) -> np.ndarray:
    """Planted acceptance length L per sequence."""
    out = np.empty(wl.batch, dtype=np.int32)
    for b, rule in enumerate(_rules(wl)):
        if rule[0] == "cycle8":
            out[b] = BLOCK_K
        else:
            out[b] = geometric_capped(child_rng(wl.seed, _P_ACCEPT, b), rule[1])
    return out


def pending_tokens(wl: Workload) -> np.ndarray:
    """Uniform pending tokens, used when the KV cache is synthetic."""
    return child_rng(wl.seed, _P_PENDING).integers(0, wl.model.vocab, size=wl.batch).astype(np.int32)


def plant_block(cont: np.ndarray, L: int, vocab: int, g: np.random.Generator) -> np.ndarray:
    """Assemble a 16-token block from a greedy continuation.

    cont[0] is the pending token and cont[j] the greedy token that follows
    cont[0..j-1] (16 entries).  The block copies cont for j < L; block[L]
    (if L < 16) is uniform but redrawn until it differs from cont[L], so the
    first mismatch sits exactly at L; later entries are uniform."""
    cont = np.asarray(cont)
    assert cont.shape[0] >= min(L + 1, BLOCK_K) and 1 <= L <= BLOCK_K
    t = g.integers(0, vocab, size=BLOCK_K).astype(np.int32)
    t[:L] = cont[:L]
    if L < BLOCK_K:
        while t[L] == cont[L]:
            t[L] = g.integers(0, vocab)
    return t


def draft_rng(wl: Workload, b: int, round_: int = 0) -> np.random.Generator:
    return child_rng(wl.seed, _P_DRAFT, b, round_)


def synthetic_kv_layer(m: ModelShape, seed: int, layer: int, lens, max_ctx: int, max_batch=None):
    """BF16 K and V for one layer, [max_batch, Hkv, max_ctx, D] uint16 bits;
    positions < lens[b] hold N(0, (0.02*sqrt(H))^2) draws, the rest zero."""
    B = len(lens) if max_batch is None else max_batch
    sigma = 0.02 * np.sqrt(m.hidden)
    K = np.zeros((B, m.n_kv_heads, max_ctx, m.head_dim), dtype=np.uint16)
    V = np.zeros_like(K)

    def fill(args):
        which, b = args
        n = int(lens[b])
        w = _draw(seed, (_P_KV, layer, which, b), (m.n_kv_heads, n, m.head_dim), std=sigma)
        (K if which == 0 else V)[b, :, :n, :] = to_bf16_bits(w)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, [(w, b) for w in (0, 1) for b in range(len(lens))]))
    return K, V
