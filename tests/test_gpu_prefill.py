"""Chunked prefill through the verify pass and the export of the target's
hidden state, on the GPU, against the float64 oracle.  Each side prefills its
own cache (the GPU through spec_prefill, the oracle through its own chunked
forward); then one verify pass on top of each cache is compared with the
usual parity rule."""
import numpy as np
import pytest
import torch

import oracle
import workload as W
from block_draft_verification_amd import DeviceModel, Verifier
from gpu_cases import MARGIN, REL_TOL, compare, log, row_rel

pytestmark = pytest.mark.gpu


def _f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def _prefill_both(m, wts, prompts, cap):
    B, T = len(prompts), max(len(p) for p in prompts)
    lens = np.array([len(p) for p in prompts], np.int32)
    P = np.zeros((B, T), np.int32)
    for b, p in enumerate(prompts):
        P[b, :len(p)] = p
    dev = DeviceModel(m, wts, max_batch=B, max_ctx=cap)
    ver = Verifier(dev)
    anchor = torch.empty(B, m.hidden, dtype=torch.bfloat16, device="cuda")
    pend = ver.prefill(torch.from_numpy(P).cuda(), torch.from_numpy(lens).cuda(), anchor)
    torch.cuda.synchronize()
    log("oracle prefill")
    om = oracle.OracleModel(m, wts, cache=m.hidden < 4096)
    okv = oracle.OracleKV(m, B, np.full(B, cap))
    opend, ohid, omargin = oracle.prefill(om, okv, prompts, return_hidden=True)
    return dev, ver, om, okv, lens, pend.cpu().numpy(), _f64(anchor), opend, ohid, omargin


def _check_prefill(m, dev, ver, okv, lens, pend, anchor, opend, ohid, omargin):
    assert ver.device_error() == 0
    assert np.array_equal(dev.kv_len.cpu().numpy()[:len(lens)], lens), "kv_len after prefill"
    sure = omargin > MARGIN
    assert np.array_equal(pend[sure], opend[sure]), f"pending {pend} vs oracle {opend}"
    rel = row_rel(anchor, ohid)
    assert rel.max() <= REL_TOL, f"anchor hidden rel {rel.max():.3g}"
    worst = 0.0
    for l in range(m.n_layers):
        for b, n in enumerate(lens):
            for cache, ref in ((dev.k_cache, okv.K[l][b]), (dev.v_cache, okv.V[l][b])):
                got = oracle.decode_bf16(cache[l, b, :, :n].cpu().numpy().view(np.uint16))
                worst = max(worst, row_rel(got, ref[:, :n]).max())
    assert worst <= REL_TOL, f"committed K/V rel {worst:.3g}"
    return {"anchor_rel": float(rel.max()), "kv_rel": float(worst), "pending_exempt": int((~sure).sum())}


def _verify_on_top(m, ver, om, okv, opend, seed):
    """One verify pass on each side's own prefilled cache, planted from the
    oracle's greedy continuation; then the exported hidden state."""
    B = len(opend)
    cont = oracle.greedy_continuation(om, okv, opend)
    g = W.child_rng(seed, 900)
    L = np.minimum(g.geometric(0.3, size=B), 16)
    blocks = np.stack([W.plant_block(cont[b], int(L[b]), m.vocab, W.child_rng(seed, 901, b))
                       for b in range(B)]).astype(np.int32)
    ref = oracle.verify_block(om, okv, blocks)
    hid = torch.full((B * 16, m.hidden), float("nan"), device="cuda")
    ver.set_dump(hidden=hid)
    out = ver.verify(torch.from_numpy(blocks).cuda())
    feat = ver.export_hidden(B)
    torch.cuda.synchronize()
    ver.set_dump(None, None)
    got = {k: v.cpu().numpy() for k, v in out.items()}
    got["hidden"] = hid.cpu().numpy().reshape(B, 16, -1)
    stats = compare(ref, got, blocks, check_logits=False)
    tau = got["accept_len"]
    feat_ref = np.stack([ref.hidden[b, tau[b] - 1] for b in range(B)])
    # the export is the BF16 rounding of the pass's final hidden state at row tau-1
    rows = np.stack([got["hidden"][b, tau[b] - 1] for b in range(B)]).astype(np.float32)
    assert np.array_equal(feat.view(torch.int16).cpu().numpy().view(np.uint16), W.to_bf16_bits(rows)), \
        "exported hidden is not row tau-1 of the pass"
    rel = row_rel(_f64(feat), feat_ref)
    assert rel.max() <= REL_TOL, f"exported hidden rel {rel.max():.3g}"
    stats["export_rel"] = float(rel.max())
    return stats


def test_prefill_tiny_ragged():
    m = W.TINY
    wts = W.model_weights(m, seed=3, gains="random")
    rng = W.child_rng(3, 800)
    prompts = [rng.integers(0, m.vocab, size=n) for n in (37, 128, 5, 16)]
    dev, ver, om, okv, lens, pend, anchor, opend, ohid, omargin = _prefill_both(m, wts, prompts, cap=192)
    log(f"tiny prefill: {_check_prefill(m, dev, ver, okv, lens, pend, anchor, opend, ohid, omargin)}")
    log(f"tiny verify after prefill: {_verify_on_top(m, ver, om, okv, opend, seed=3)}")
    assert ver.device_error() == 0
    ver.close()


def test_prefill_05b_two_prompts():
    m = W.M05B
    wts = W.model_weights(m, seed=0)
    rng = W.child_rng(0, 810)
    prompts = [rng.integers(0, m.vocab, size=n) for n in (70, 33)]
    dev, ver, om, okv, lens, pend, anchor, opend, ohid, omargin = _prefill_both(m, wts, prompts, cap=128)
    log(f"0.5b prefill: {_check_prefill(m, dev, ver, okv, lens, pend, anchor, opend, ohid, omargin)}")
    log(f"0.5b verify after prefill: {_verify_on_top(m, ver, om, okv, opend, seed=0)}")
    assert ver.device_error() == 0
    ver.close()


def test_prefill_rejects_bad_length():
    """A length outside [1, T] sets the device error bit and leaves that
    sequence's kv_len alone; the other sequences are prefilled."""
    m = W.TINY
    wts = W.model_weights(m, seed=0)
    dev = DeviceModel(m, wts, max_batch=2, max_ctx=128)
    ver = Verifier(dev)
    P = torch.from_numpy(W.child_rng(0, 820).integers(0, m.vocab, size=(2, 20)).astype(np.int32)).cuda()
    ver.prefill(P, torch.tensor([0, 20], dtype=torch.int32, device="cuda"))
    assert ver.device_error() & 8, "SPEC_DERR_LENGTH not reported"
    assert dev.kv_len.cpu().tolist() == [0, 20]
    ver.close()
