"""End-to-end greedy decoding on the GPU: the block-speculative loop must
emit exactly the autoregressive greedy stream (the lossless property of
greedy speculative decoding), and the GPU's autoregressive stream must follow
the float64 oracle's wherever the oracle's top-2 margin decides it."""
import numpy as np
import pytest
import torch

import oracle
import workload as W
from block_draft_verification_amd import DeviceModel, Verifier
from block_draft_verification_amd.decode import ar_decode, planted_drafts, spec_decode
from gpu_cases import MARGIN, log

pytestmark = pytest.mark.gpu


def _lossless(m, ver, dev, pending, n_rounds, seed, p=0.1):
    """GPU AR stream, then GPU speculative decoding with drafts planted from it."""
    B = pending.shape[0]
    kv0 = dev.kv_len.clone()
    n_ref = n_rounds * 16 + 16
    ar = ar_decode(ver, pending, n_ref)
    dev.kv_len.copy_(kv0)
    stream = torch.cat([pending[:, None], ar], dim=1)
    L = np.minimum(W.child_rng(seed, 950).geometric(p, size=(B, n_rounds)), 16)
    draft = planted_drafts(stream, torch.from_numpy(L).cuda(), m.vocab)
    toks, counts, taus = spec_decode(ver, pending, n_rounds, draft, capacity=n_ref)
    torch.cuda.synchronize()
    counts = counts.cpu().numpy()
    toks, ar_np, taus = toks.cpu().numpy(), ar.cpu().numpy(), taus.cpu().numpy()
    assert np.array_equal(taus, L), "the target did not accept exactly the planted prefixes"
    for b in range(B):
        assert counts[b] == L[b].sum()
        assert np.array_equal(toks[b, :counts[b]], ar_np[b, :counts[b]]), f"seq {b}: speculative != AR stream"
    assert np.array_equal(dev.kv_len.cpu().numpy()[:B], kv0.cpu().numpy()[:B] + counts)
    return ar_np, counts


def test_decode_tiny_against_oracle_and_lossless():
    m = W.TINY
    wts = W.model_weights(m, seed=4, gains="random")
    rng = W.child_rng(4, 930)
    prompts = [rng.integers(0, m.vocab, size=n) for n in (40, 23)]
    B, T = 2, 40
    P = np.zeros((B, T), np.int32)
    for b, pr in enumerate(prompts):
        P[b, :len(pr)] = pr
    lens = np.array([40, 23], np.int32)
    cap = 448
    dev = DeviceModel(m, wts, max_batch=B, max_ctx=cap)
    ver = Verifier(dev)
    pending = ver.prefill(torch.from_numpy(P).cuda(), torch.from_numpy(lens).cuda())
    n_rounds = 12
    ar, counts = _lossless(m, ver, dev, pending, n_rounds, seed=4)
    # the GPU's AR stream against the oracle's, up to the first step the oracle's margin leaves open
    om = oracle.OracleModel(m, wts)
    okv = oracle.OracleKV(m, B, cap)
    opend, _, pmarg = oracle.prefill(om, okv, prompts, return_hidden=True)
    otoks, omarg = oracle.ar_decode(om, okv, opend, 64, return_margin=True)
    for b in range(B):
        if pmarg[b] <= MARGIN:  # the pending token itself is not decided: nothing to compare
            continue
        assert opend[b] == pending[b].item()
        open_steps = np.nonzero(omarg[b] <= MARGIN)[0]
        k = int(open_steps[0]) if len(open_steps) else 64
        assert np.array_equal(ar[b, :k], otoks[b, :k]), f"seq {b}: GPU AR differs from the oracle before step {k}"
        log(f"seq {b}: GPU AR == oracle for {k} decided steps; speculative == AR for {counts[b]} tokens")
    assert ver.device_error() == 0
    ver.close()


def test_decode_05b_lossless_batch4():
    m = W.M05B
    wl = W.WORKLOADS["0.5b-fp8-b32-ctx512to4096"]
    wts = W.model_weights(m, seed=0)
    B, cap = 4, 1024
    lens = np.array([600, 512, 700, 531], np.int32)
    kvs = [W.synthetic_kv_layer(m, 0, l, lens, cap) for l in range(m.n_layers)]
    dev = DeviceModel(m, wts, max_batch=B, max_ctx=cap, kv_layers=kvs, kv_len=lens)
    ver = Verifier(dev)
    pending = torch.from_numpy(W.pending_tokens(wl)[:B].astype(np.int32)).cuda()
    _, counts = _lossless(m, ver, dev, pending, n_rounds=16, seed=5)
    log(f"0.5b: speculative == AR for {counts.tolist()} tokens")
    assert ver.device_error() == 0
    ver.close()
