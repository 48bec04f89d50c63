"""Paged KV cache: the same verify pass over a page pool reached through a
page table.  Paging only moves where rows live, so every result must be
bit-identical to the contiguous layout (and the contiguous layout is the one
held to the oracle elsewhere)."""
import numpy as np
import pytest
import torch

import workload as W
from block_draft_verification_amd import DeviceModel, Verifier
from block_draft_verification_amd.decode import ar_decode, planted_drafts, spec_decode
from gpu_cases import log

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
