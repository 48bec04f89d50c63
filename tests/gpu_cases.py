"""Builds one parity case on both sides from the seeded inputs, and compares.

Both sides receive bit-identical arrays from ``workload``: FP8/MXFP4 weight
codes and scales, BF16 embedding, BF16 KV caches (the oracle's own prefill
rounded to BF16 once, or synthetic draws), pending tokens and planted blocks.
Drafts are planted from the ORACLE's greedy continuation; nothing the HIP
path computes is ever fed to the oracle.

Parity rule for floating point (hidden states and logits): per row
||gpu - oracle|| / ||oracle|| <= 2e-2 (BF16 activations against a float64
reference).  Integer outputs: the argmax of a row must equal the oracle's
wherever the oracle's top-2 margin exceeds 1e-2; tau and bonus must equal the
oracle's for every sequence whose deciding rows (0 .. tau*-1) all clear that
margin; every sequence's tau must equal the first mismatch of the GPU's own
argmax (self-consistency).
"""
from __future__ import annotations

import json
import os
import sys
import time
from dataclasses import dataclass

import numpy as np
import torch

import oracle
import workload as W
from block_draft_verification_amd import DeviceModel, Verifier

MARGIN = 1e-2
REL_TOL = 2e-2
# When set, every comparison appends its statistics (rows and sequences
# exempt under the margin rule, largest relative errors) as one JSON line.
PARITY_LOG = os.environ.get("SPEC_PARITY_LOG")


def log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


@dataclass
class Case:
    wl: W.Workload
    weights: dict
    lens: np.ndarray
    kv_layers: list          # [(K, V)] uint16 [B, Hkv, max_ctx, D] per layer
    pending: np.ndarray
    blocks: np.ndarray       # [B, 16] int32
    om: oracle.OracleModel
    okv: oracle.OracleKV


def _bf16_cache_from_oracle(okv, m, B, max_ctx):
    layers = []
    for l in range(m.n_layers):
        K = np.zeros((B, m.n_kv_heads, max_ctx, m.head_dim), np.uint16)
        V = np.zeros_like(K)
        for b in range(B):
            n = int(okv.n[b])
            K[b, :, :n] = W.to_bf16_bits(okv.K[l][b][:, :n].astype(np.float32))
            V[b, :, :n] = W.to_bf16_bits(okv.V[l][b][:, :n].astype(np.float32))
        layers.append((K, V))
    return layers


def build_case(name: str, seqs_planted=None, batch=None, gains="ones", extra=16, oracle_seqs=None) -> Case:
    """oracle_seqs: the sequences the oracle will be asked about (default all);
    the others enter the oracle's cache with length 0, which keeps the
    float64 copy of a large cache small."""
    wl = W.WORKLOADS[name]
    m = wl.model
    B = batch or wl.batch
    log(f"case {name}: weights")
    wts = W.model_weights(m, wl.seed, gains=gains)
    lens = W.context_lengths(wl)[:B]
    om = oracle.OracleModel(m, wts, cache=m.hidden < 4096)  # the 8B shape decodes per use
    if wl.kv_fill == "prefill":
        log(f"case {name}: oracle prefill of {lens.tolist()} tokens")
        pr = W.prompts(wl, lens)[:B]
        okv0 = oracle.OracleKV(m, B, lens + 16)
        pend = oracle.prefill(om, okv0, pr)
        kv_layers = _bf16_cache_from_oracle(okv0, m, B, wl.max_ctx)
    else:
        log(f"case {name}: synthetic KV")
        kv_layers = [W.synthetic_kv_layer(m, wl.seed, l, lens, wl.max_ctx) for l in range(m.n_layers)]
        pend = W.pending_tokens(wl)[:B]
    olens = lens.copy()
    if oracle_seqs is not None:
        olens[[b for b in range(B) if b not in set(oracle_seqs)]] = 0
    okv = oracle.OracleKV.from_bf16(m, [k for k, _ in kv_layers], [v for _, v in kv_layers], olens, extra=extra)
    L = W.accept_lengths(wl)[:B]
    planted = range(B) if seqs_planted is None else seqs_planted
    blocks = np.empty((B, 16), np.int32)
    for b in range(B):
        g = W.draft_rng(wl, b)
        blocks[b] = g.integers(0, m.vocab, size=16)
        blocks[b, 0] = pend[b]
    if len(planted):
        log(f"case {name}: oracle greedy continuation for {len(planted)} sequences")
        sub = oracle.OracleKV.__new__(oracle.OracleKV)
        sub.m, sub.caps, sub.n = okv.m, okv.caps[list(planted)], okv.n[list(planted)].copy()
        sub.K = [[okv.K[l][b] for b in planted] for l in range(m.n_layers)]
        sub.V = [[okv.V[l][b] for b in planted] for l in range(m.n_layers)]
        cont = oracle.greedy_continuation(om, sub, pend[list(planted)])
        for i, b in enumerate(planted):
            blocks[b] = W.plant_block(cont[i], int(L[b]), m.vocab, W.draft_rng(wl, b))
    return Case(wl, wts, lens, kv_layers, pend, blocks, om, okv)


def oracle_verify(case: Case, seqs=None):
    log("oracle verify pass")
    seqs = list(range(len(case.lens))) if seqs is None else list(seqs)
    okv = case.okv
    if len(seqs) != len(case.lens):
        sub = oracle.OracleKV.__new__(oracle.OracleKV)
        sub.m, sub.caps, sub.n = okv.m, okv.caps[seqs], okv.n[seqs].copy()
        sub.K = [[okv.K[l][b] for b in seqs] for l in range(okv.m.n_layers)]
        sub.V = [[okv.V[l][b] for b in seqs] for l in range(okv.m.n_layers)]
        okv = sub
    return oracle.verify_block(case.om, okv, case.blocks[seqs]), okv


def gpu_setup(case: Case, max_batch=None):
    m = case.wl.model
    B = len(case.lens)
    log("upload to the device")
    dev = DeviceModel(m, case.weights, max_batch=max_batch or B, max_ctx=case.wl.max_ctx,
                      kv_layers=case.kv_layers, kv_len=case.lens)
    return dev, Verifier(dev)


def gpu_verify(ver: Verifier, case: Case, dump_logits=True):
    m = case.wl.model
    B = len(case.lens)
    hid = torch.full((B * 16, m.hidden), float("nan"), device="cuda")
    lg = torch.full((B * 16, m.vocab), float("nan"), device="cuda") if dump_logits else None
    ver.set_dump(hidden=hid, logits=lg)
    out = ver.verify(torch.from_numpy(case.blocks).cuda())
    torch.cuda.synchronize()
    ver.set_dump(None, None)
    res = {k: v.cpu().numpy() for k, v in out.items()}
    res["hidden"] = hid.cpu().numpy().reshape(B, 16, -1)
    if lg is not None:
        res["logits"] = lg.cpu().numpy().reshape(B, 16, -1)
    return res


def row_rel(a, ref):
    return np.linalg.norm(a - ref, axis=-1) / np.maximum(np.linalg.norm(ref, axis=-1), 1e-30)


def compare(ref, got, blocks, seqs=None, check_logits=True):
    """Apply the parity rule; returns a stats dict, raises AssertionError."""
    seqs = list(range(ref.g.shape[0])) if seqs is None else list(seqs)
    g = got["argmax"].reshape(-1, 16)[seqs]
    tau, bonus = got["accept_len"][seqs], got["bonus"][seqs]
    blocks = blocks[seqs]
    stats = {}
    rel_h = row_rel(got["hidden"][seqs].astype(np.float64), ref.hidden)
    stats["max_rel_hidden"] = float(rel_h.max())
    assert np.all(np.isfinite(got["hidden"][seqs])), "non-finite hidden state"
    assert rel_h.max() <= REL_TOL, f"hidden rel {rel_h.max():.3g}"
    if check_logits and "logits" in got:
        rel_l = row_rel(got["logits"][seqs].astype(np.float64), ref.logits)
        stats["max_rel_logits"] = float(rel_l.max())
        assert rel_l.max() <= REL_TOL, f"logits rel {rel_l.max():.3g}"
    sure = ref.margin > MARGIN
    stats["rows_exempt"] = float(1 - sure.mean())
    bad = (g != ref.g) & sure
    assert not bad.any(), f"argmax differs on {bad.sum()} decided rows"
    # self-consistency of the GPU's tau and bonus with its own argmax
    for i in range(len(seqs)):
        t = 16
        for j in range(1, 16):
            if blocks[i, j] != g[i, j - 1]:
                t = j
                break
        assert tau[i] == t and bonus[i] == g[i, t - 1], f"seq {seqs[i]}: tau/bonus not self-consistent"
    decided = np.array([np.all(ref.margin[i, :ref.tau[i]] > MARGIN) for i in range(len(seqs))])
    stats["seqs_exempt"] = float(1 - decided.mean())
    assert np.array_equal(tau[decided], ref.tau[decided]), "tau differs from the oracle"
    assert np.array_equal(bonus[decided], ref.bonus[decided]), "bonus differs from the oracle"
    stats["seqs_compared"] = len(seqs)
    stats["seqs_decided"] = int(decided.sum())
    stats["tau_gpu"] = tau.tolist()
    stats["tau_oracle"] = ref.tau.tolist()
    record(stats)
    return stats


def record(stats):
    """Print the parity statistics and, with SPEC_PARITY_LOG set, append them
    (tagged with the running test) to that file."""
    test = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
    log(f"parity {test}: {json.dumps(stats)}")
    if PARITY_LOG:
        with open(PARITY_LOG, "a") as f:
            f.write(json.dumps({"test": test, **stats}) + "\n")
