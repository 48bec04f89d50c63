"""Writes planted_8b_blocks.txt: verify blocks for two sequences of the 8B
workload (32 layers, hidden 4096, 32/8 heads, head_dim 128, vocab 128256;
8 sequences at context 4096, synthetic BF16 KV), planted from the ORACLE's
own greedy continuation with the workload's acceptance lengths.

The HunyuanOCR-1.5 / DFlash write-up (inference loop, steps 3-4) fixes what a
block verify must return: the longest prefix of drafts equal to the target's
greedy choices, plus the target's next token.  A block planted from the
target's greedy continuation with first mismatch at L therefore has accepted
length L and bonus = continuation[L]; these blocks let a GPU test check that
at the 8B shape for L > 1 without running 15 oracle steps at test time.

Only ``oracle`` and ``workload`` are called.  Run from the repository root:

    python tests/golden/make_planted_8b.py

It takes several minutes (the float64 oracle decodes every layer's weights
once per step: 15 steps of 32 layers).
"""
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workload as W  # noqa: E402

WORKLOAD = "8b-fp8-b8-ctx4096"
SEQS = (0, 2)  # planted L = 16 and 12
OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "planted_8b_blocks.txt")


def main():
    wl = W.WORKLOADS[WORKLOAD]
    m = wl.model
    t0 = time.time()
    wts = W.model_weights(m, wl.seed)
    lens = W.context_lengths(wl)
    print(f"weights {time.time() - t0:.0f} s", flush=True)
    olens = np.zeros_like(lens)
    olens[list(SEQS)] = lens[list(SEQS)]
    Ks, Vs = [], []
    for l in range(m.n_layers):
        K, V = W.synthetic_kv_layer(m, wl.seed, l, lens, wl.max_ctx)
        Ks.append(K[list(SEQS)])
        Vs.append(V[list(SEQS)])
    print(f"kv {time.time() - t0:.0f} s", flush=True)
    om = oracle.OracleModel(m, wts, cache=False)
    okv = oracle.OracleKV.from_bf16(m, Ks, Vs, lens[list(SEQS)])
    pend = W.pending_tokens(wl)[list(SEQS)]
    cont = oracle.greedy_continuation(om, okv, pend)
    print(f"continuation {time.time() - t0:.0f} s", flush=True)
    L = W.accept_lengths(wl)
    lines = [f"# {WORKLOAD}: oracle-planted verify blocks (written by tests/golden/make_planted_8b.py)",
             "# columns: sequence, planted L, then the 16 block tokens (t[0] = pending token)"]
    for i, b in enumerate(SEQS):
        blk = W.plant_block(cont[i], int(L[b]), m.vocab, W.draft_rng(wl, b))
        lines.append(" ".join(str(int(v)) for v in [b, L[b], *blk]))
    lines.append("# oracle greedy continuation of each sequence (pending token first)")
    for i, b in enumerate(SEQS):
        lines.append("# " + " ".join(str(int(v)) for v in [b, *cont[i]]))
    with open(OUT, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {OUT} ({time.time() - t0:.0f} s)")


if __name__ == "__main__":
    main()
