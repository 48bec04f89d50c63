"""Throughput of the block verify pass on one MI355X.

A step is one verify pass plus its commit (every step of the hot path) over
one batch: the 0.5B-class FP8 target (24 layers, hidden 896, 14/2 heads,
head_dim 64, SwiGLU 4864, vocab 151936, tied BF16 lm_head), 32 sequences with
contexts uniform in [512, 4096], 16-token blocks (512 rows per GEMM).  All
inputs are seeded synthetic data resident in HBM before timing: FP8 weights
drawn N(0, 0.02^2), BF16 KV caches drawn N(0, (0.02*sqrt(H))^2), drafts
planted from the pass's own greedy continuation with acceptance lengths
min(Geometric(0.1), 16).  The timed region replays a captured graph of
{restore kv_len, verify, commit} K times between two events.

Also measured, as keys of the same JSON line: per-step percentiles with the
caches warm and after a 512 MB eviction write (outside the timed events),
every kernel class's duration inside a pass (the kernel's own dispatch
events), the roofline of the dominant kernel and of the whole pass, the other
single-GPU workloads (the batch-1 and MXFP4 shapes, and the 8B shape unless
--no-8b), batch-1 decoding loops, the FP8-activation mode, and the CPU
oracle on a bounded sample.

Prints one JSON line.  --gpus N > 1 is refused: the path runs on one GPU.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # bytes/s, MI355X HBM3E
MFMA_BF16_PEAK = 2.5e15    # flop/s, dense BF16 / FP16 MFMA
MFMA_FP8_PEAK = 5.0e15     # flop/s, dense FP8 MFMA
RIDGE = MFMA_BF16_PEAK / HBM_PEAK
METRIC = "verify passes/s & accepted tok/s, 0.5B FP8 target, K=16 block; % of HBM peak"
WORKLOAD = "0.5b-fp8-b32-ctx512to4096"
OTHER_WORKLOADS = ["0.5b-fp8-b1-ctx2048", "0.5b-mxfp4mlp-b16-ctx3072"]
WORKLOAD_8B = "8b-fp8-b8-ctx4096"
EVICT_BYTES = 512 << 20

# Hardware-counter figures per kernel class, from rocprofv3 --pmc runs of
# `bench.py --no-cpu --no-extras --no-kernel-times` (profiles/ holds the summary):
#   traffic = FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0 per launch (the factors that
#             make a plain 1 GiB device copy read back as 1 GiB), bytes
#   mfma_util = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x 2.4 GHz x the launch's
#             measured duration): the busy cycles are the MFMA instructions'
#             own cycles (32 per 32x32x16 MFMA), so this is the share of the
#             chip's MFMA time the launch keeps busy
# valid for the kernel sources whose digest is recorded; any other source
# reports null.
SIMD_CLOCK = 2.4e9
N_SIMD = 1024
COUNTERS_PROFILE = "profiles/verify_pass_0.5b-fp8-b32-ctx512to4096_counters.md"
SOURCES = ("gemm.hip", "attention.hip", "attn_plan.h", "misc.hip", "common.h", "kernels.h")
COUNTERS = {  # per launch at the batch-32 grid: FETCH_SIZE / WRITE_SIZE (KiB, medians over dispatches), traffic (bytes), MFMA busy (SIMD cycles)
    "embed": {"fetch_kib": 509.4, "write_kib": 2752.5, "traffic": 3861920, "mfma_busy_cycles": 0},
    "qkv": {"fetch_kib": 5002.9, "write_kib": 1152.0, "traffic": 11425664, "mfma_busy_cycles": 1032192},
    "attention": {"fetch_kib": 19696.6, "write_kib": 3778.2, "traffic": 44207488, "mfma_busy_cycles": 4616192},
    "attn_merge": {"fetch_kib": 1924.6, "write_kib": 896.0, "traffic": 4859136, "mfma_busy_cycles": 0},
    "o_proj": {"fetch_kib": 5112.5, "write_kib": 2840.0, "traffic": 13378560, "mfma_busy_cycles": 802816},
    "gate_up": {"fetch_kib": 9735.0, "write_kib": 4864.0, "traffic": 24918016, "mfma_busy_cycles": 8716288},
    "down": {"fetch_kib": 23642.5, "write_kib": 2840.0, "traffic": 51328000, "mfma_busy_cycles": 4358144},
    "lm_head": {"fetch_kib": 137936.0, "write_kib": 8684.6, "traffic": 291386048, "mfma_busy_cycles": 136134656},
    "accept": {"fetch_kib": 2399.3, "write_kib": 5.0, "traffic": 4918912, "mfma_busy_cycles": 0},
    "commit": {"fetch_kib": 1.5, "write_kib": 0.1, "traffic": 3200, "mfma_busy_cycles": 0},
}
COUNTERS_DIGEST = "d91ef063ce46a412"


def _sources_digest():
    d = os.path.join(ROOT, "block_draft_verification_amd", "csrc")
    h = hashlib.sha256()
    for f in SOURCES:
        h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()[:16]


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def weight_bytes_per_layer(m):
    H, I, D = m.hidden, m.intermediate, m.head_dim
    qkv = m.qkv_rows * H + m.qkv_rows * 4
    o = H * m.n_q_heads * D + H * 4
    if m.mlp_format == "fp8":
        gu, dn = 2 * I * H + 2 * I * 4, H * I + H * 4
    else:
        gu, dn = 2 * I * H // 2 + 2 * I * H // 32, H * I // 2 + H * I // 32
    return {"qkv": qkv, "o_proj": o, "gate_up": gu, "down": dn, "norms": 2 * H * 4}


def kernel_work(kind, m, lens):
    """Algorithmic (bytes, flops) of ONE launch of a kernel class: the bytes it
    must read and write (weights, its activation inputs and outputs, KV rows)
    and the multiply-add flops of its products."""
    B = len(lens)
    M, H, D, I, V = B * 16, m.hidden, m.head_dim, m.intermediate, m.vocab
    wb = weight_bytes_per_layer(m)
    HqD = m.n_q_heads * D
    kvd = m.n_kv_heads * D
    if kind == "attention":
        kv = int(np.sum(lens + 16)) * kvd * 2 * 2
        flops = sum(int(np.sum(n + 1 + np.arange(16))) for n in lens) * m.n_q_heads * D * 4
        return kv + 2 * M * HqD * 2, flops
    if kind == "attn_merge":
        return 2 * M * HqD * 2, 0
    if kind == "qkv":  # h*g in, per-row partial sums in, q out, block K/V rows out
        return wb["qkv"] + M * H * 2 + M * (HqD + 2 * kvd) * 2, 2 * M * m.qkv_rows * H
    if kind == "o_proj":  # attention out and h in; h, h*g and partial sums out
        return wb["o_proj"] + M * HqD * 2 + M * H * (4 + 4 + 2), 2 * M * H * HqD
    if kind == "gate_up":
        return wb["gate_up"] + M * H * 2 + M * I * 2, 2 * M * 2 * I * H
    if kind == "down":
        return wb["down"] + M * I * 2 + M * H * (4 + 4 + 2), 2 * M * H * I
    if kind == "lm_head":
        return V * H * 2 + M * H * 2 + (V // 128) * M * 8, 2 * M * V * H
    if kind == "embed":
        return M * H * (2 + 4 + 2), 0
    if kind == "rmsnorm":
        return M * H * 4 * 3 + M * H * 2, 4 * M * H
    return 0, 0


def pass_bytes(m, lens):
    """Algorithmic HBM bytes of one verify pass + commit: every weight byte once,
    the KV read (committed rows plus the block rows), the block's KV write,
    the embedding gather."""
    B = len(lens)
    wb = weight_bytes_per_layer(m)
    w = m.n_layers * sum(wb.values()) + m.vocab * m.hidden * 2 + m.hidden * 4
    per_tok = m.n_layers * m.n_kv_heads * m.head_dim * 2 * 2
    kv_read = int(np.sum(lens + 16)) * per_tok
    kv_write = B * 16 * per_tok
    return w + kv_read + kv_write + B * 16 * m.hidden * 2


def roofline_time(kind, m, lens):
    """The roofline time of one launch: max(bytes / HBM peak, flops / MFMA peak)."""
    by, fl = kernel_work(kind, m, lens)
    return max(by / HBM_PEAK, fl / MFMA_BF16_PEAK)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, weights, kv_layers, lens, n_seq, min_seconds=10.0):
    """The oracle (float64 numpy) timed on this host for a bounded sample: the
    verify pass of the first n_seq sequences (random drafts; the oracle's
    work does not depend on draft values), repeated until min_seconds have
    passed.  Scaled to passes/s of the whole batch by n_seq / B."""
    import oracle
    import workload as W
    from threadpoolctl import threadpool_info
    m = wl.model
    om = oracle.OracleModel(m, weights)
    sl = lens[:n_seq]
    okv = oracle.OracleKV.from_bf16(m, [k[:n_seq] for k, _ in kv_layers], [v[:n_seq] for _, v in kv_layers], sl)
    blocks = np.stack([W.draft_rng(wl, b, 1).integers(0, m.vocab, size=16) for b in range(n_seq)])
    oracle.verify_block(om, okv, blocks[:1, :1], seqs=[0])  # decode weights once (untimed)
    t0 = time.time()
    reps = 0
    while reps == 0 or time.time() - t0 < min_seconds:
        oracle.verify_block(om, okv, blocks)
        reps += 1
    dt = (time.time() - t0) / reps
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": (n_seq / len(lens)) / dt, "unit": "verify passes/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"float64 numpy oracle, {reps} verify passes of {n_seq} of {len(lens)} sequences "
                      f"({dt:.2f} s each), scaled by {n_seq}/{len(lens)}; weight decoding untimed",
            "cpu_model": cpu_model()}


def e2e_batch1(ver, dev, m, lens, seed, n_rounds=32):
    """End-to-end greedy decoding of one sequence (the 0.5B model at the
    batch-1 shape, ~2k context): plain autoregressive (one pass per token)
    against block-speculative with drafts planted from that AR stream
    (acceptance lengths min(Geometric(0.1), 16)).  The sequence whose context
    is closest to 2048 is moved into slot 0 for the run and restored after."""
    import torch
    from block_draft_verification_amd.decode import ar_decode, planted_drafts, spec_decode
    import workload as W
    b = int(np.argmin(np.abs(lens - 2048)))
    save_k, save_v = dev.k_cache[:, 0].clone(), dev.v_cache[:, 0].clone()
    kv0 = dev.kv_len.clone()
    dev.k_cache[:, 0].copy_(dev.k_cache[:, b])
    dev.v_cache[:, 0].copy_(dev.v_cache[:, b])
    dev.kv_len[0] = int(lens[b])
    start = dev.kv_len[:1].clone()
    pending = torch.tensor([int(W.child_rng(seed, 960).integers(0, m.vocab))], dtype=torch.int32, device="cuda")
    n_ref = n_rounds * 16 + 16
    t_ar, t_sp = {}, {}
    ar = ar_decode(ver, pending, n_ref, t_ar)
    dev.kv_len[:1].copy_(start)
    L = np.minimum(W.child_rng(seed, 961).geometric(0.1, size=(1, n_rounds)), 16)
    draft = planted_drafts(torch.cat([pending[:, None], ar], dim=1), torch.from_numpy(L).cuda(), m.vocab)
    toks, counts, taus = spec_decode(ver, pending, n_rounds, draft, capacity=n_ref, timing=t_sp)
    torch.cuda.synchronize()
    n = int(counts[0].item())
    lossless = bool(torch.equal(toks[0, :n], ar[0, :n])) and bool(torch.equal(taus.cpu(), torch.from_numpy(L)))
    dev.k_cache[:, 0].copy_(save_k)
    dev.v_cache[:, 0].copy_(save_v)
    dev.kv_len.copy_(kv0)
    torch.cuda.synchronize()
    # rates from the graph replays alone (the first, eager step and the capture excluded)
    ms_pass_ar = t_ar["ms"] / t_ar["steps"]
    ms_round = t_sp["ms"] / t_sp["steps"]
    ar_tps = 1000.0 / ms_pass_ar
    spec_tps = (n / n_rounds) * 1000.0 / ms_round
    return {"batch": 1, "context": int(lens[b]), "ar_tokens": n_ref, "ar_ms_per_token": ms_pass_ar,
            "ar_tok_per_s": ar_tps, "spec_rounds": n_rounds, "spec_tokens": n, "spec_ms_per_round": ms_round,
            "spec_tok_per_s": spec_tps, "speedup": spec_tps / ar_tps, "mean_tau": n / n_rounds,
            "lossless": lossless, "drafts": "planted from the AR stream, acceptance min(Geometric(0.1), 16)",
            "ar_rows_per_pass": 16,
            "ar_note": "the autoregressive arm runs the library's 16-row pass with one committed row per token; "
                       "at batch 1 both arms stream the same weight bytes per pass, so this is an upper bound "
                       "on a one-row pass's time by the attention and MFMA work of 15 extra rows"}


def make_graph(ver, dev, tok, kv0):
    """Capture one step (restore kv_len, verify, commit) in a graph."""
    import torch
    B = tok.shape[0]
    acc = torch.empty(B, dtype=torch.int32, device="cuda")
    bon = torch.empty(B, dtype=torch.int32, device="cuda")
    amx = torch.empty(B, 16, dtype=torch.int32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            dev.kv_len.copy_(kv0)
            ver.verify(tok, acc, bon, amx)
            ver.commit(B)
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dev.kv_len.copy_(kv0)
        ver.verify(tok, acc, bon, amx)
        ver.commit(B)
    return graph, acc


def time_graph(graph, steps, warmup):
    """`warmup` replays, then `steps` replays timed between two events on the
    stream, bracketed by synchronisations.  Returns ms per step."""
    import torch
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def step_percentiles(graph, n, evict=None):
    """Each of n replays timed on its own (an event pair around it); with
    `evict` (a device buffer), a full write of that buffer before each replay,
    outside the events, so the replay starts with the caches holding none of
    the pass's data.  Returns (p10, p50, p90) in ms."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for e0, e1 in evs:
        if evict is not None:
            evict.fill_(1)
        e0.record()
        graph.replay()
        e1.record()
    torch.cuda.synchronize()
    t = np.array([e0.elapsed_time(e1) for e0, e1 in evs])
    return [float(np.percentile(t, q)) for q in (10, 50, 90)]


def kernel_times(ver, dev, tok, kv0, kinds, reps):
    """Per kernel class: the duration of each of its launches inside eager
    passes, recorded by events bound to that launch's dispatch (its own
    start and end); the mean over `reps` passes."""
    import torch
    B = tok.shape[0]
    acc = torch.empty(B, dtype=torch.int32, device="cuda")
    bon = torch.empty(B, dtype=torch.int32, device="cuda")
    per_kind = {}
    ver.set_repeat(1)
    for k in kinds:
        ver.time_kernel(k)
        for _ in range(reps):
            dev.kv_len.copy_(kv0)
            ver.verify(tok, acc, bon, None)
            ver.commit(B)
        ver.time_kernel(None)
        tot, n = ver.kernel_time()
        if n:
            per_kind[k] = {"ms_per_pass": tot / reps, "us_per_launch": 1000 * tot / n, "launches_per_pass": n // reps}
    dev.kv_len.copy_(kv0)
    return per_kind


def plant(ver, wl, m, tok_np):
    """Drafts from the pass's own greedy continuation: row j-1's argmax depends
    only on tokens 0..j-1, so 15 uncommitted passes fill the block."""
    import torch
    import workload as W
    B = wl.batch
    L = W.accept_lengths(wl)
    blocks = tok_np
    tok = torch.from_numpy(blocks).cuda()
    for j in range(1, 16):
        g = ver.verify(tok)["argmax"].cpu().numpy()
        for b in range(B):
            if j < L[b]:
                blocks[b, j] = g[b, j - 1]
            elif j == L[b]:
                redraw = W.draft_rng(wl, b, 2)
                while blocks[b, j] == g[b, j - 1]:
                    blocks[b, j] = redraw.integers(0, m.vocab)
        tok.copy_(torch.from_numpy(blocks))
    tau = ver.verify(tok)["accept_len"].cpu().numpy()
    return tok, tau, L


def setup(wl, weights=None):
    import workload as W
    from block_draft_verification_amd import DeviceModel, Verifier
    m = wl.model
    if weights is None:
        log(f"workload {wl.name}: generating weights")
        weights = W.model_weights(m, wl.seed)
    lens = W.context_lengths(wl)
    log(f"{wl.name}: synthetic KV")
    kv_layers = [W.synthetic_kv_layer(m, wl.seed, l, lens, wl.max_ctx) for l in range(m.n_layers)]
    log(f"{wl.name}: upload")
    dev = DeviceModel(m, weights, max_batch=wl.batch, max_ctx=wl.max_ctx, kv_layers=kv_layers, kv_len=lens)
    return weights, lens, kv_layers, dev


def device_setup(wl):
    """The workload's model and KV cache drawn on the GPU, for throughput only:
    the shapes, distributions and encodings of workload/'s host generator
    (N(0, 0.02^2) weights encoded FP8-e4m3 with one fp32 scale per output row,
    BF16 embedding and lm_head, unit norm gains, KV rows N(0, (0.02 sqrt(H))^2)
    on each sequence's first n_b positions), drawn by torch's generator on the
    device in seconds instead of minutes of host work.  The parity tests use
    the host generator; the throughput does not depend on the values."""
    import torch
    import workload as W
    from block_draft_verification_amd import DeviceModel
    m = wl.model
    assert m.mlp_format == "fp8"
    g = torch.Generator(device="cuda")
    g.manual_seed(wl.seed * 1_000_003 + 7919)
    log(f"workload {wl.name}: drawing weights on the device")

    def fp8_rows(rows, cols):
        w = torch.randn(rows, cols, generator=g, device="cuda") * 0.02
        s = w.abs().amax(dim=1) / 448.0
        s = torch.where(s > 0, s, torch.ones_like(s))
        return (w / s[:, None]).to(torch.float8_e4m3fn).view(torch.uint8), s.float().contiguous()

    def bf16(rows, cols, std=0.02):
        return (torch.randn(rows, cols, generator=g, device="cuda") * std).to(torch.bfloat16).view(torch.int16)

    H, D, I = m.hidden, m.head_dim, m.intermediate
    ones = torch.ones(H, device="cuda")
    layers = []
    for _ in range(m.n_layers):
        lw = {"attn_norm": ones, "mlp_norm": ones}
        lw["w_qkv"], lw["s_qkv"] = fp8_rows(m.qkv_rows, H)
        lw["w_o"], lw["s_o"] = fp8_rows(H, m.n_q_heads * D)
        lw["w_gate_up"], lw["s_gate_up"] = fp8_rows(2 * I, H)
        lw["w_down"], lw["s_down"] = fp8_rows(H, I)
        layers.append(lw)
    weights = {"layers": layers, "embed": bf16(m.vocab, H),
               "lm_head": None if m.tied_lm_head else bf16(m.vocab, H), "final_norm": ones}
    lens = W.context_lengths(wl)
    dev = DeviceModel(m, weights, max_batch=wl.batch, max_ctx=wl.max_ctx, kv_layers=None, kv_len=lens)
    sigma = 0.02 * float(np.sqrt(H))
    for l in range(m.n_layers):
        for cache in (dev.k_cache, dev.v_cache):
            for b, n in enumerate(lens):
                cache[l, b, :, :int(n)] = (torch.randn(m.n_kv_heads, int(n), D, generator=g, device="cuda")
                                           * sigma).to(torch.bfloat16).view(torch.int16)
    torch.cuda.synchronize()
    return weights, lens, None, dev


def config_line(wl, weights, steps, warmup, on_device=False):
    """Throughput of one more workload, timed like the headline one."""
    import torch
    import workload as W
    from block_draft_verification_amd import Verifier
    m = wl.model
    weights, lens, kv_layers, dev = device_setup(wl) if on_device else setup(wl, weights)
    ver = Verifier(dev)
    blocks = np.stack([W.draft_rng(wl, b).integers(0, m.vocab, size=16) for b in range(wl.batch)]).astype(np.int32)
    blocks[:, 0] = W.pending_tokens(wl)
    log(f"{wl.name}: planting drafts")
    tok, tau, L = plant(ver, wl, m, blocks)
    kv0 = dev.kv_len.clone()
    graph, acc = make_graph(ver, dev, tok, kv0)
    ms = time_graph(graph, steps, warmup)
    assert np.array_equal(acc.cpu().numpy(), tau)
    assert ver.device_error() == 0
    nb = pass_bytes(m, lens)
    # the split merge is no algorithmic step of the pass: its bound leaves it out
    kinds = ["embed", "qkv", "attention", "o_proj", "gate_up", "down", "lm_head", "accept", "commit"]
    roof = sum(roofline_time(k, m, lens) * (1 if k in ("embed", "lm_head", "accept", "commit") else m.n_layers)
               for k in kinds)
    ver.close()
    del graph
    out = {"value": 1000.0 / ms, "unit": "verify passes/s", "ms_per_step": ms, "batch": wl.batch,
           "rows": wl.batch * 16, "sum_tau": int(tau.sum()), "planted_L_equals_tau": bool(np.array_equal(tau, L)),
           "emitted_tok_per_s": 1000.0 / ms * float(tau.sum()),
           "accepted_draft_tok_per_s": 1000.0 / ms * float((tau - 1).sum()),
           "hbm_frac_of_peak": nb / (ms * 1e-3) / HBM_PEAK, "algorithmic_bytes_per_pass": nb,
           "pass_roofline_frac": roof / (ms * 1e-3),
           "kv_fill": "synthetic BF16 draws (the KV values do not change the work)"}
    del dev
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=WORKLOAD)
    ap.add_argument("--cpu-seqs", type=int, default=8)
    ap.add_argument("--lanes", type=int, default=1, help="concurrent sequence ranges per pass (spec_verify_set_lanes)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="only the headline workload (no other workloads, decoding loops, FP8 mode; for counter runs)")
    ap.add_argument("--no-kernel-times", action="store_true", help="skip the per-kernel-class timing passes")
    ap.add_argument("--no-8b", action="store_true", help="skip the 8B workload (its model is drawn on the device)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB three times (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the path runs on a single device)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": 3}), flush=True)
        return
    import workload as W
    from block_draft_verification_amd import Verifier

    wl = W.WORKLOADS[args.workload]
    m = wl.model
    B = wl.batch
    on_device = args.workload == WORKLOAD_8B
    if on_device and not (args.no_cpu and args.no_extras):
        sys.exit("the 8B workload as the main line needs --no-cpu --no-extras (its model is drawn on the device)")
    weights, lens, kv_layers, dev = device_setup(wl) if on_device else setup(wl)
    ver = Verifier(dev, lanes=args.lanes)
    torch.cuda.synchronize()
    blocks = np.stack([W.draft_rng(wl, b).integers(0, m.vocab, size=16) for b in range(B)]).astype(np.int32)
    blocks[:, 0] = W.pending_tokens(wl)
    log("planting drafts (15 passes)")
    tok, tau, L = plant(ver, wl, m, blocks)
    log(f"planted L == tau: {np.array_equal(tau, L)}; sum tau = {tau.sum()}")

    kv0 = dev.kv_len.clone()
    graph, acc = make_graph(ver, dev, tok, kv0)
    log(f"timing {args.steps} steps")
    ms = time_graph(graph, args.steps, args.warmup)
    assert np.array_equal(acc.cpu().numpy(), tau)
    assert ver.device_error() == 0
    n_pct = max(20, min(100, args.steps))
    warm = step_percentiles(graph, n_pct)
    evict = torch.empty(EVICT_BYTES, dtype=torch.uint8, device="cuda")
    cold = step_percentiles(graph, n_pct, evict)
    del evict

    passes = 1000.0 / ms
    nbytes = pass_bytes(m, lens)
    kinds = ["embed", "qkv", "attention", "attn_merge", "o_proj", "rmsnorm", "gate_up", "down", "lm_head", "accept",
             "commit"]
    counts = {k: (1 if k in ("embed", "lm_head", "accept", "commit") else m.n_layers) for k in kinds}
    roof_pass = sum(roofline_time(k, m, lens) * counts[k] for k in kinds if k not in ("rmsnorm", "attn_merge"))
    res = {
        "metric": METRIC, "value": passes, "unit": "verify passes/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp16", "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "block": 16, "rows": B * 16,
                   "context": "uniform [512, 4096]", "weights": "fp8-e4m3 per-row, bf16 tied lm_head",
                   "activations": "fp16 MFMA inputs, fp32 accumulate and residual; bf16 KV cache and lm_head"},
        "emitted_tok_per_s": passes * float(tau.sum()),
        "accepted_draft_tok_per_s": passes * float((tau - 1).sum()),
        "sum_tau": int(tau.sum()),
        "hbm_frac_of_peak": nbytes / (ms * 1e-3) / HBM_PEAK,
        "algorithmic_bytes_per_pass": nbytes,
        "pass_roofline_frac": roof_pass / (ms * 1e-3),
        "pass_roofline_us": roof_pass * 1e6,
        "step_ms_warm_p10_p50_p90": warm,
        "step_ms_cold_p10_p50_p90": cold,
    }
    if not args.no_kernel_times:
        reps = max(3, min(10, args.steps // 10))
        per_kind = kernel_times(ver, dev, tok, kv0, kinds, reps)
        dom = max(per_kind, key=lambda k: per_kind[k]["ms_per_pass"])
        by, fl = kernel_work(dom, m, lens)
        t_launch = per_kind[dom]["us_per_launch"] * 1e-6
        if fl / max(by, 1) > RIDGE:
            roof = {"bound": "mfma", "achieved": fl / t_launch / 1e12, "peak": MFMA_BF16_PEAK / 1e12, "unit": "TFLOP/s"}
        else:
            roof = {"bound": "hbm", "achieved": by / t_launch / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s"}
        roof["frac"] = roof["achieved"] / roof["peak"]
        counters_ok = COUNTERS_DIGEST == _sources_digest()
        cnt = COUNTERS.get(dom) if counters_ok else None
        roof["traffic"] = cnt["traffic"] if cnt else None
        roof["mfma_util"] = cnt["mfma_busy_cycles"] / (N_SIMD * SIMD_CLOCK * t_launch) if cnt else None
        roof["kernel"] = dom
        roof["us_per_launch"] = per_kind[dom]["us_per_launch"]
        roof["algorithmic_bytes_per_launch"] = by
        roof["algorithmic_flops_per_launch"] = fl
        roof["timing"] = "the kernel's own dispatch events inside eager passes (every layer's weights from HBM)"
        for k, v in per_kind.items():
            v["roofline_us"] = roofline_time(k, m, lens) * 1e6
            v["roofline_frac"] = v["roofline_us"] / v["us_per_launch"] if v["us_per_launch"] else None
            c = COUNTERS.get(k) if counters_ok else None
            v["algorithmic_bytes"] = kernel_work(k, m, lens)[0]
            v["traffic"] = c["traffic"] if c else None
            if c and c["mfma_busy_cycles"] and v["us_per_launch"]:
                v["mfma_util"] = c["mfma_busy_cycles"] / (N_SIMD * SIMD_CLOCK * v["us_per_launch"] * 1e-6)
        res["roofline"] = roof
        res["kernels"] = per_kind
        res["kernel_sum_ms_per_pass"] = sum(v["ms_per_pass"] for v in per_kind.values())
    if args.no_extras:
        ver.close()
        print(json.dumps(res), flush=True)
        return
    log("end-to-end decoding at batch 1")
    res["e2e"] = e2e_batch1(ver, dev, m, lens, wl.seed)
    ver.close()
    # the FP8-activation mode on the same cache and blocks (drafts planted from
    # the FP16 mode's greedy continuation, so tau also shows the mode's drift)
    log("FP8-activation mode")
    dev.kv_len.copy_(kv0)
    ver8 = Verifier(dev, act_fmt="mxfp8")
    g8, acc8 = make_graph(ver8, dev, tok, kv0)
    ms8 = time_graph(g8, args.steps, args.warmup)
    assert ver8.device_error() == 0
    ver8.close()
    acc8 = acc8.cpu().numpy()
    res["fp8_activations"] = {
        "value": 1000.0 / ms8, "unit": "verify passes/s", "ms_per_step": ms8,
        "activations": "MXFP8 (e4m3 + e8m0 per 32) into QKV, gate/up and down on the scaled FP8 MFMA; "
                       "FP16 into O-proj and attention",
        "sum_tau": int(acc8.sum()), "tau_rows_equal_fp16_mode": int((acc8 == tau).sum()),
        "mean_tau_fp16_mode": float(tau.mean()), "mean_tau": float(acc8.mean())}
    del g8, graph
    cpu = None
    if not args.no_cpu:
        log(f"cpu baseline: oracle on {args.cpu_seqs} sequences")
        cpu = cpu_baseline(wl, weights, kv_layers, lens, args.cpu_seqs)
    del dev, kv_layers
    torch.cuda.empty_cache()
    res["configs"] = {}
    for name in OTHER_WORKLOADS + ([] if args.no_8b else [WORKLOAD_8B]):
        w2 = W.WORKLOADS[name]
        res["configs"][name] = config_line(w2, weights if w2.model == m else None, args.steps, args.warmup,
                                           on_device=name == WORKLOAD_8B)
        if name == WORKLOAD_8B:
            res["configs"][name]["weights_and_kv"] = ("drawn on the device (bench.py device_setup): the host "
                                                      "generator's shapes, distributions and encodings")
        torch.cuda.empty_cache()
    if cpu is not None:
        res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
