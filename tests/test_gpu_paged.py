"""Paged KV cache ("The Inference Stack Behind OCRia", KV-cache section:
block table and slot mapping): the same verify pass over a page pool reached
through a page table.  The paged pass is held to the float64 oracle on its
own, and, since paging only moves where rows live, every result must also be
bit-identical to the contiguous layout."""
import numpy as np
import pytest
import torch

import oracle
import workload as W
from block_draft_verification_amd import DeviceModel, Verifier
from block_draft_verification_amd.decode import ar_decode, planted_drafts, spec_decode
from gpu_cases import compare, log

pytestmark = pytest.mark.gpu


def _shuffled_table(B, pages_per_seq, num_pages, seed):
    perm = W.child_rng(seed, 970).permutation(num_pages)[:B * pages_per_seq]
    return perm.reshape(B, pages_per_seq).astype(np.int32)


def _verify_dump(dev, ver, blocks):
    m = dev.shape
    B = blocks.shape[0]
    hid = torch.full((B * 16, m.hidden), float("nan"), device="cuda")
    ver.set_dump(hidden=hid)
    out = ver.verify(torch.from_numpy(blocks).cuda())
    torch.cuda.synchronize()
    ver.set_dump(None, None)
    return {k: v.cpu().numpy() for k, v in out.items()}, hid.cpu().numpy()


def test_paged_vs_oracle_05b():
    """The 0.5B model over a shuffled pool of 64-row pages (4 ragged
    sequences, blocks planted from the oracle's greedy continuation with L =
    16, 5, 9, 1): hidden states, logits, argmax, tau and bonus against the
    oracle under the whole-pass parity rule; every block K/V row written
    through the page table within 2e-2 of the oracle's, committed rows
    untouched bit for bit."""
    m = W.M05B
    wts = W.model_weights(m, seed=0)
    B, cap, ps = 4, 1024, 64
    lens = np.array([600, 512, 700, 531], np.int32)
    kvs = [W.synthetic_kv_layer(m, 0, l, lens, cap) for l in range(m.n_layers)]
    num_pages = B * (cap // ps) + 7
    table = _shuffled_table(B, cap // ps, num_pages, seed=3)
    om = oracle.OracleModel(m, wts)
    okv = oracle.OracleKV.from_bf16(m, [k for k, _ in kvs], [v for _, v in kvs], lens)
    pend = W.child_rng(0, 975).integers(0, m.vocab, size=B)
    log("oracle greedy continuation of 4 sequences")
    cont = oracle.greedy_continuation(om, okv, pend)
    L = [16, 5, 9, 1]
    blocks = np.stack([W.plant_block(cont[b], L[b], m.vocab, W.child_rng(0, 976, b)) for b in range(B)])
    ref = oracle.verify_block(om, okv, blocks)
    assert ref.tau.tolist() == L
    dp = DeviceModel(m, wts, max_batch=B, max_ctx=cap, kv_layers=kvs, kv_len=lens,
                     page_table=table, page_size=ps, num_pages=num_pages)
    vp = Verifier(dp)
    hid = torch.full((B * 16, m.hidden), float("nan"), device="cuda")
    lg = torch.full((B * 16, m.vocab), float("nan"), device="cuda")
    vp.set_dump(hidden=hid, logits=lg)
    out = vp.verify(torch.from_numpy(blocks.astype(np.int32)).cuda())
    torch.cuda.synchronize()
    vp.set_dump(None, None)
    got = {k: v.cpu().numpy() for k, v in out.items()}
    got["hidden"] = hid.cpu().numpy().reshape(B, 16, -1)
    got["logits"] = lg.cpu().numpy().reshape(B, 16, -1)
    stats = compare(ref, got, blocks)
    log(f"paged vs oracle: {stats}")
    for l in (0, m.n_layers - 1):
        for b in range(B):
            n = int(lens[b])
            for which, cache0, ocache in (("k", kvs[l][0], okv.K[l][b]), ("v", kvs[l][1], okv.V[l][b])):
                rows = dp.cache_rows(l, b, n + 16, which).cpu().numpy().view(np.uint16)
                assert np.array_equal(rows[:, :n], cache0[b, :, :n]), f"layer {l} seq {b} {which}: prefix changed"
                blk = oracle.decode_bf16(rows[:, n:])
                ref_rows = ocache[:, n:n + 16]
                rel = np.linalg.norm(blk - ref_rows, axis=-1) / np.linalg.norm(ref_rows, axis=-1)
                assert rel.max() < 2e-2, f"layer {l} seq {b} {which}: block rows {rel.max():.3g}"
    assert vp.device_error() == 0
    vp.close()


def test_paged_equals_contiguous_05b():
    m = W.M05B
    wl = W.WORKLOADS["0.5b-fp8-b32-ctx512to4096"]
    wts = W.model_weights(m, seed=0)
    B, cap, ps = 4, 1024, 64
    lens = np.array([600, 512, 700, 531], np.int32)
    kvs = [W.synthetic_kv_layer(m, 0, l, lens, cap) for l in range(m.n_layers)]
    table = _shuffled_table(B, cap // ps, B * (cap // ps) + 7, seed=1)
    dc = DeviceModel(m, wts, max_batch=B, max_ctx=cap, kv_layers=kvs, kv_len=lens)
    dp = DeviceModel(m, wts, max_batch=B, max_ctx=cap, kv_layers=kvs, kv_len=lens,
                     page_table=table, page_size=ps, num_pages=B * (cap // ps) + 7)
    vc, vp = Verifier(dc), Verifier(dp)
    blocks = np.stack([W.draft_rng(wl, b).integers(0, m.vocab, size=16) for b in range(B)]).astype(np.int32)
    blocks[:, 0] = W.pending_tokens(wl)[:B]
    for rnd in range(3):  # verify, commit, repeat with the argmax as the next blocks' tokens
        oc, hc = _verify_dump(dc, vc, blocks)
        op, hp = _verify_dump(dp, vp, blocks)
        for k in oc:
            assert np.array_equal(oc[k], op[k]), f"round {rnd}: {k} differs between layouts"
        assert np.array_equal(hc, hp), f"round {rnd}: hidden states differ between layouts"
        vc.commit(B)
        vp.commit(B)
        blocks = np.concatenate([oc["bonus"][:, None], oc["argmax"][:, :15]], axis=1).astype(np.int32)
    torch.cuda.synchronize()
    n = dc.kv_len.cpu().numpy()
    assert np.array_equal(n, dp.kv_len.cpu().numpy())
    for l in (0, m.n_layers // 2, m.n_layers - 1):
        for b in range(B):
            for which in ("k", "v"):
                assert torch.equal(dc.cache_rows(l, b, int(n[b]) + 16, which),
                                   dp.cache_rows(l, b, int(n[b]) + 16, which)), f"layer {l} seq {b} {which}"
    assert vc.device_error() == 0 and vp.device_error() == 0
    log(f"paged == contiguous over 3 rounds, kv_len {n.tolist()}")
    vc.close()
    vp.close()


def test_paged_prefill_and_decode_tiny():
    """Prefill and lossless speculative decoding on a paged cache (128-row pages)."""
    m = W.TINY
    wts = W.model_weights(m, seed=6, gains="random")
    B, cap, ps = 3, 384, 128
    num_pages = B * (cap // ps) + 2
    table = _shuffled_table(B, cap // ps, num_pages, seed=2)
    rng = W.child_rng(6, 980)
    lens = np.array([50, 17, 64], np.int32)
    P = np.zeros((B, 64), np.int32)
    for b in range(B):
        P[b, :lens[b]] = rng.integers(0, m.vocab, size=lens[b])
    dc = DeviceModel(m, wts, max_batch=B, max_ctx=cap)
    dp = DeviceModel(m, wts, max_batch=B, max_ctx=cap, page_table=table, page_size=ps, num_pages=num_pages)
    vc, vp = Verifier(dc), Verifier(dp)
    pc = vc.prefill(torch.from_numpy(P).cuda(), torch.from_numpy(lens).cuda())
    pp = vp.prefill(torch.from_numpy(P).cuda(), torch.from_numpy(lens).cuda())
    assert torch.equal(pc, pp)
    kv0 = dp.kv_len.clone()
    ar = ar_decode(vp, pp, 10 * 16 + 16)
    dp.kv_len.copy_(kv0)
    L = np.minimum(W.child_rng(6, 981).geometric(0.15, size=(B, 10)), 16)
    draft = planted_drafts(torch.cat([pp[:, None], ar], dim=1), torch.from_numpy(L).cuda(), m.vocab)
    toks, counts, _ = spec_decode(vp, pp, 10, draft, capacity=176)
    ar_c = ar_decode(vc, pc, 10 * 16 + 16)
    torch.cuda.synchronize()
    assert torch.equal(ar, ar_c), "paged AR stream differs from the contiguous one"
    for b in range(B):
        n = int(counts[b])
        assert n == L[b].sum() and torch.equal(toks[b, :n], ar[b, :n]), f"seq {b}: speculative != AR"
    assert vc.device_error() == 0 and vp.device_error() == 0
    vc.close()
    vp.close()


def test_paged_bad_page_index_is_reported():
    m = W.TINY
    wts = W.model_weights(m, seed=0)
    B, cap, ps = 2, 256, 64
    table = np.arange(B * (cap // ps), dtype=np.int32).reshape(B, -1)
    table[1, 0] = 99  # outside the pool of 8 pages
    dev = DeviceModel(m, wts, max_batch=B, max_ctx=cap, page_table=table, page_size=ps, num_pages=B * (cap // ps))
    ver = Verifier(dev)
    ver.verify(torch.zeros(B, 16, dtype=torch.int32, device="cuda"))
    assert ver.device_error() & 16, "SPEC_DERR_PAGE not reported"
    ver.close()
