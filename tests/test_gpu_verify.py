"""Whole verify pass on the GPU against the float64 oracle, through the C ABI
(spec_verify_init / spec_verify_block / spec_commit_kv), on the synthetic
workloads; plus the data-movement, error-path, determinism and graph-replay
properties of the boundary.  The parity rule is documented in gpu_cases."""
import dataclasses
import types

import numpy as np
import pytest
import torch

import oracle
import workload as W
from block_draft_verification_amd import DERR_CAPACITY, DERR_COMMIT, DERR_TOKEN, DeviceModel, Verifier

from gpu_cases import build_case, compare, gpu_setup, gpu_verify, log, oracle_verify, row_rel

pytestmark = pytest.mark.gpu


def _kv_rows(dev, l, b, lo, hi):
    K = dev.k_cache[l, b, :, lo:hi].cpu().numpy().view(np.uint16)
    V = dev.v_cache[l, b, :, lo:hi].cpu().numpy().view(np.uint16)
    return K, V


def _check_block_kv(case, dev, okv, seqs, layers):
    """Block rows land in slots n..n+15 (within tolerance of the oracle's);
    committed rows below n are untouched, bit for bit."""
    for l in layers:
        for i, b in enumerate(seqs):
            n = int(case.lens[b])
            K, V = _kv_rows(dev, l, b, 0, n + 16)
            K0, V0 = case.kv_layers[l]
            assert np.array_equal(K[:, :n], K0[b, :, :n]) and np.array_equal(V[:, :n], V0[b, :, :n])
            kr = okv.K[l][i][:, n:n + 16]
            vr = okv.V[l][i][:, n:n + 16]
            assert row_rel(oracle.decode_bf16(K[:, n:]), kr).max() < 2e-2
            assert row_rel(oracle.decode_bf16(V[:, n:]), vr).max() < 2e-2


def _full_case(name, check_layers=(0, -1), min_decided=0.0):
    """min_decided: the share of sequences whose tau and bonus the margin rule
    must leave decided (compared bit for bit), so that a batched workload
    cannot pass on exempt sequences alone."""
    case = build_case(name)
    ref, okv = oracle_verify(case)
    dev, ver = gpu_setup(case)
    got = gpu_verify(ver, case)
    stats = compare(ref, got, case.blocks)
    assert stats["seqs_decided"] >= min_decided * stats["seqs_compared"], stats
    m = case.wl.model
    _check_block_kv(case, dev, okv, range(len(case.lens)), [l % m.n_layers for l in check_layers])
    # commit the accepted rows: a length bump by tau
    ver.commit(len(case.lens))
    torch.cuda.synchronize()
    assert np.array_equal(dev.kv_len.cpu().numpy()[:len(case.lens)], case.lens + got["accept_len"])
    assert ver.device_error() == 0
    ver.close()
    return stats


def test_verify_tiny():
    _full_case("tiny-b1-ctx128")


def test_verify_05b_b1_ctx2048():
    _full_case("0.5b-fp8-b1-ctx2048")


def test_verify_05b_b32_ragged():
    _full_case("0.5b-fp8-b32-ctx512to4096", min_decided=0.4)


def test_verify_05b_mxfp4_b16():
    _full_case("0.5b-mxfp4mlp-b16-ctx3072", min_decided=0.4)


def _golden_blocks(name):
    """Planted blocks stored by a committed script (tests/golden/make_*.py)
    that calls only the oracle and the input generators: {seq: (L, block)}."""
    import os
    rows = {}
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", name)) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            v = [int(x) for x in line.split()]
            rows[v[0]] = (v[1], np.array(v[2:18], np.int32))
    return rows


def test_verify_8b_planted():
    """8B shape at full size (32 layers, 8 sequences at context 4096).  Two
    sequences carry blocks planted from the oracle's greedy continuation
    (planted L = 16 and 12, stored in tests/golden/planted_8b_blocks.txt), so
    tau > 1 and the bonus after a long accepted prefix are compared with the
    oracle at head_dim 128 / G = 4; every sequence is checked for
    self-consistency and untouched committed rows."""
    gold = _golden_blocks("planted_8b_blocks.txt")
    seqs = sorted(gold)
    case = build_case("8b-fp8-b8-ctx4096", seqs_planted=[], oracle_seqs=seqs)
    for b in seqs:
        case.blocks[b] = gold[b][1]
    ref, okv = oracle_verify(case, seqs=seqs)
    assert ref.tau.tolist() == [gold[b][0] for b in seqs], "the oracle's tau must equal the planted L"
    dev, ver = gpu_setup(case)
    got = gpu_verify(ver, case)
    stats = compare(ref, got, case.blocks, seqs=seqs)
    log(f"8b: {stats}")
    _check_block_kv(case, dev, okv, seqs, [0, 31])
    g = got["argmax"].reshape(-1, 16)
    for b in range(8):
        t = next((j for j in range(1, 16) if case.blocks[b, j] != g[b, j - 1]), 16)
        assert got["accept_len"][b] == t
    ver.close()


def test_multi_round_tiny_with_explicit_commits():
    """Four rounds of verify + commit on the tiny model; each round is planted
    from the oracle's continuation of the committed history, both sides commit
    the oracle's tau (explicit counts on the GPU side)."""
    case = build_case("tiny-b1-ctx128", batch=1, extra=16 * 6)
    m = case.wl.model
    dev, ver = gpu_setup(case)
    okv = case.okv
    pend = case.pending.copy()
    for rnd in range(4):
        cont = oracle.greedy_continuation(case.om, okv, pend)
        L = int(W.geometric_capped(W.child_rng(5, 200 + rnd), 0.3))
        case.blocks = W.plant_block(cont[0], L, m.vocab, W.child_rng(5, 300 + rnd))[None].astype(np.int32)
        ref = oracle.verify_block(case.om, okv, case.blocks)
        got = gpu_verify(ver, case)
        compare(ref, got, case.blocks)
        n_commit = torch.tensor(ref.tau.astype(np.int32), device="cuda")
        ver.commit(1, n_commit)
        oracle.commit(okv, ref.tau)
        pend = ref.bonus
        torch.cuda.synchronize()
        assert dev.kv_len[0].item() == okv.n[0]
    assert ver.device_error() == 0
    ver.close()


def test_split_down_matches_oracle_and_repeats():
    """At batch 1 the down projection (K = 4864 over 28 workgroups) splits K
    four ways inside its launch: each split's partial goes out with
    device-coherent stores, and the last split of a tile to arrive adds the
    partials in split order, resets the tile's arrival counter and runs the
    epilogue.  Two layers of the 0.5B shape: the pass matches the oracle,
    two eager passes give identical bits, and graph replays (the counters
    reused launch after launch) give the eager results."""
    m = dataclasses.replace(W.M05B, name="0.5b-L2", n_layers=2)
    seed, cap = 13, 1024
    wts = W.model_weights(m, seed)
    lens = np.array([700], np.int32)
    kvs = [W.synthetic_kv_layer(m, seed, l, lens, cap) for l in range(m.n_layers)]
    blocks = W.child_rng(seed, 996).integers(0, m.vocab, size=(1, 16)).astype(np.int32)
    om = oracle.OracleModel(m, wts)
    okv = oracle.OracleKV.from_bf16(m, [k for k, _ in kvs], [v for _, v in kvs], lens)
    ref = oracle.verify_block(om, okv, blocks)
    dev = DeviceModel(m, wts, max_batch=1, max_ctx=cap, kv_layers=kvs, kv_len=lens)
    ver = Verifier(dev)
    case = types.SimpleNamespace(wl=types.SimpleNamespace(model=m), lens=lens, blocks=blocks)
    a = gpu_verify(ver, case)
    log(f"split down: {compare(ref, a, blocks)}")
    b = gpu_verify(ver, case)
    for k in ("hidden", "logits", "argmax", "accept_len", "bonus"):
        assert np.array_equal(a[k], b[k], equal_nan=True), k
    tokens = torch.from_numpy(blocks).cuda()
    tau = torch.empty(1, dtype=torch.int32, device="cuda")
    bonus = torch.empty(1, dtype=torch.int32, device="cuda")
    amax = torch.empty(1, 16, dtype=torch.int32, device="cuda")
    kv0 = dev.kv_len.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ver.verify(tokens, tau, bonus, amax)
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ver.verify(tokens, tau, bonus, amax)
    for rep in range(3):
        dev.kv_len.copy_(kv0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert tau.item() == a["accept_len"][0] and bonus.item() == a["bonus"][0], rep
        assert np.array_equal(amax.cpu().numpy().reshape(-1), a["argmax"].reshape(-1)), rep
    assert ver.device_error() == 0
    ver.close()


def test_determinism_and_graph_replay():
    """Two eager verifies give identical bits; a captured graph of verify +
    commit replays to the same outputs, with kv_len restored between replays."""
    case = build_case("tiny-b1-ctx128", seqs_planted=[])
    m = case.wl.model
    dev, ver = gpu_setup(case)
    a = gpu_verify(ver, case)
    b = gpu_verify(ver, case)
    for k in ("hidden", "logits", "argmax", "accept_len", "bonus"):
        assert np.array_equal(a[k], b[k], equal_nan=True), k
    tokens = torch.from_numpy(case.blocks).cuda()
    outs = {k: torch.empty(1, dtype=torch.int32, device="cuda") for k in ("tau", "bonus")}
    amax = torch.empty(1, 16, dtype=torch.int32, device="cuda")
    kv0 = dev.kv_len.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm up on the capture stream
        ver.verify(tokens, outs["tau"], outs["bonus"], amax)
        ver.commit(1)
    torch.cuda.current_stream().wait_stream(s)
    dev.kv_len.copy_(kv0)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ver.verify(tokens, outs["tau"], outs["bonus"], amax)
        ver.commit(1)
    for rep in range(3):
        dev.kv_len.copy_(kv0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert outs["tau"].item() == a["accept_len"][0] and outs["bonus"].item() == a["bonus"][0]
        assert np.array_equal(amax.cpu().numpy(), a["argmax"])
        assert dev.kv_len[0].item() == case.lens[0] + a["accept_len"][0]
    ver.close()


def test_error_paths_are_reported_without_stray_writes():
    case = build_case("tiny-b1-ctx128", seqs_planted=[])
    m = case.wl.model
    cap = case.wl.max_ctx
    dev, ver = gpu_setup(case)
    # token id out of range -> DERR_TOKEN, pass still completes
    bad = case.blocks.copy()
    bad[0, 3] = m.vocab + 5
    ver.verify(torch.from_numpy(bad).cuda())
    assert ver.device_error() & DERR_TOKEN
    assert ver.device_error() == 0                      # reading clears the word
    # a commit count past 16 -> DERR_COMMIT, kv_len unchanged
    before = dev.kv_len[0].item()
    ver.commit(1, torch.tensor([17], dtype=torch.int32, device="cuda"))
    assert ver.device_error() & DERR_COMMIT and dev.kv_len[0].item() == before
    # a cache that cannot take the block -> DERR_CAPACITY and no block K/V writes
    dev.kv_len[0] = cap - 8
    snap = [(_kv_rows(dev, l, 0, cap - 8, cap)) for l in range(m.n_layers)]
    ver.verify(torch.from_numpy(case.blocks).cuda())
    assert ver.device_error() & DERR_CAPACITY
    for l in range(m.n_layers):
        K, V = _kv_rows(dev, l, 0, cap - 8, cap)
        assert np.array_equal(K, snap[l][0]) and np.array_equal(V, snap[l][1])
    ver.close()


def test_batch_bounds_rejected():
    case = build_case("tiny-b1-ctx128", seqs_planted=[])
    dev, ver = gpu_setup(case)
    with pytest.raises(Exception):
        ver.verify(torch.zeros(2, 16, dtype=torch.int32, device="cuda"))   # batch > max_batch
    ver.close()


def test_lanes_parity_and_graph_replay():
    """spec_verify_set_lanes: a batch of 7 ragged sequences cut into 2 and 3
    concurrent ranges meets the same oracle parity rule as one lane; a captured
    graph of verify + commit with 3 lanes replays to the eager outputs."""
    case = build_case("0.5b-fp8-b32-ctx512to4096", batch=7)
    ref, _ = oracle_verify(case)
    dev, ver = gpu_setup(case)
    B = len(case.lens)
    for lanes in (2, 3):
        ver.set_lanes(lanes)
        got = gpu_verify(ver, case)
        log(f"lanes {lanes}: {compare(ref, got, case.blocks)}")
    tokens = torch.from_numpy(case.blocks).cuda()
    eager = ver.verify(tokens)
    torch.cuda.synchronize()
    outs = {k: torch.empty(B, dtype=torch.int32, device="cuda") for k in ("tau", "bonus")}
    amax = torch.empty(B, 16, dtype=torch.int32, device="cuda")
    kv0 = dev.kv_len.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ver.verify(tokens, outs["tau"], outs["bonus"], amax)
        ver.commit(B)
    torch.cuda.current_stream().wait_stream(s)
    dev.kv_len.copy_(kv0)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ver.verify(tokens, outs["tau"], outs["bonus"], amax)
        ver.commit(B)
    for rep in range(3):
        dev.kv_len.copy_(kv0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(outs["tau"], eager["accept_len"]) and torch.equal(outs["bonus"], eager["bonus"])
        assert torch.equal(amax, eager["argmax"])
        assert torch.equal(dev.kv_len[:B], kv0[:B] + eager["accept_len"])
    assert ver.device_error() == 0
    ver.close()
