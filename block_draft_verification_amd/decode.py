"""Greedy decoding loops on top of the verify pass: plain autoregressive (one
committed row per pass) and block-speculative (HunyuanOCR-1.5 / DFlash
write-up, inference loop, steps 2-5: draft a block, verify it in one target
pass, keep the longest agreeing prefix plus the target's own next token).

Both loops only orchestrate the library's entry points (spec_verify_block,
spec_commit_kv) on the current stream; the bookkeeping between passes stays
on the device.  One step (AR) or one round (speculative) is captured once in
a graph and replayed, so the host neither synchronises nor launches the
pass's kernels one by one inside a loop.  Drafting is the caller's:
`draft_fn(pending, pos, round)` returns the [B, 16] int32 block whose row 0 is
the pending token, using only device tensor operations.  A trained block
drafter is out of scope here; tests and the benchmark plant drafts from a
reference greedy stream.
"""
from __future__ import annotations

import torch

from ._binding import BLOCK, Verifier


def _replay(step, n: int, timing: dict | None = None):
    """Capture step() once (after one eager warm-up) and replay it n-1 times.
    With `timing`, the replays alone are bracketed by events on the stream and
    timing["ms"], timing["steps"] are filled in (after a synchronisation)."""
    if n <= 0:
        return
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # eager first step (also warms up the allocator)
    torch.cuda.current_stream().wait_stream(side)
    if n == 1:
        return
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n - 1):
        g.replay()
    e1.record()
    if timing is not None:
        e1.synchronize()
        timing["ms"], timing["steps"] = e0.elapsed_time(e1), n - 1


def ar_decode(ver: Verifier, pending: torch.Tensor, n_tokens: int, timing: dict | None = None) -> torch.Tensor:
    """n_tokens greedy tokens per sequence, one per pass: the block's row 0 is
    the current token, one row is committed and the argmax of row 0 is the
    next token.  Returns int32 [B, n_tokens] on the device."""
    B = pending.shape[0]
    dev = pending.device
    block = torch.zeros(B, BLOCK, dtype=torch.int32, device=dev)
    ones = torch.ones(B, dtype=torch.int32, device=dev)
    out = torch.zeros(B, n_tokens, dtype=torch.int32, device=dev)
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    bon = torch.empty(B, dtype=torch.int32, device=dev)
    amx = torch.empty(B, BLOCK, dtype=torch.int32, device=dev)
    i = torch.zeros(1, dtype=torch.int64, device=dev)
    block[:, 0] = pending

    def step():
        ver.verify(block, acc, bon, amx)
        ver.commit(B, ones)
        out.index_copy_(1, i, amx[:, :1])
        block[:, 0].copy_(amx[:, 0])
        i.add_(1)

    _replay(step, n_tokens, timing)
    return out


def spec_decode(ver: Verifier, pending: torch.Tensor, n_rounds: int, draft_fn, capacity: int,
                timing: dict | None = None):
    """n_rounds verify passes with drafted blocks.  Each round emits
    t[1 .. tau-1] and the bonus token, commits tau rows and makes the bonus the
    next pending token.  Returns (tokens int32 [B, capacity], counts int32 [B],
    accepted int64 [B, n_rounds]) on the device: the first counts[b] entries of
    row b are the emitted tokens (recording stops at `capacity`), accepted
    holds each round's tau."""
    B = pending.shape[0]
    dev = pending.device
    out = torch.zeros(B, capacity + BLOCK, dtype=torch.int32, device=dev)
    taus = torch.zeros(B, n_rounds + 1, dtype=torch.int64, device=dev)
    pos = torch.zeros(B, dtype=torch.int64, device=dev)
    rnd = torch.zeros(1, dtype=torch.int64, device=dev)
    cur = pending.clone()
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    bon = torch.empty(B, dtype=torch.int32, device=dev)
    j = torch.arange(BLOCK, device=dev)
    rows = torch.arange(B, device=dev)[:, None]

    def step():
        block = draft_fn(cur, pos, rnd)
        ver.verify(block, acc, bon, None)
        ver.commit(B)  # tau rows of each sequence
        tau = acc.long()
        # emitted this iteration, at pos .. pos+tau-1: block[1 .. tau-1], then the bonus
        nxt = torch.cat([block[:, 1:], bon[:, None]], dim=1)
        emit = torch.where(j[None, :] < tau[:, None] - 1, nxt, bon[:, None])
        idx = torch.clamp(pos[:, None] + j[None, :], max=capacity + BLOCK - 1)
        keep = (j[None, :] < tau[:, None]) & (pos[:, None] + j[None, :] < capacity)
        out[rows, idx] = torch.where(keep, emit, out[rows, idx])
        taus.index_copy_(1, torch.clamp(rnd, max=n_rounds), tau[:, None])
        pos.copy_(torch.clamp(pos + tau, max=capacity))
        cur.copy_(bon)
        rnd.add_(1)

    _replay(step, n_rounds, timing)
    return out[:, :capacity], pos.to(torch.int32), taus[:, :n_rounds]


def planted_drafts(stream: torch.Tensor, accept_len: torch.Tensor, vocab: int):
    """A draft_fn that plants blocks from a reference greedy stream.

    stream int32 [B, N]: stream[:, 0] is the first pending token and
    stream[:, k] the k-th greedy token after it.  accept_len int64 [B, R]: the
    planted acceptance length L of each round, in [1, 16].  At emitted
    position p the block is stream[p .. p+L-1] followed by tokens that differ
    from the stream (so the target accepts exactly L rows when its greedy
    stream equals the reference)."""
    B, N = stream.shape
    R = accept_len.shape[1]
    j = torch.arange(BLOCK, device=stream.device)

    def draft(cur, pos, rnd):
        L = torch.gather(accept_len, 1, torch.clamp(rnd, max=R - 1).expand(B)[:, None])
        idx = torch.clamp(pos[:, None] + j[None, :], max=N - 1)
        ref = torch.gather(stream, 1, idx)
        block = torch.where(j[None, :] < L, ref, (ref + 1) % vocab)
        block = torch.cat([cur[:, None], block[:, 1:]], dim=1)
        return block.to(torch.int32).contiguous()

    return draft
