"""Why the decoder GEMM inputs are FP16 rather than BF16 (CPU, slow).

The pass holds its hidden states and logits to a 2e-2 relative bar per row
against the float64 oracle.  FP16 and BF16 run the same dense MFMA rate on
gfx950, so the choice between them is a numerics one.  This test measures
it on the 0.5B shape with its 24 random-weight layers: the oracle is run with
its activation hook (the normed rows that enter the QKV and gate/up
projections, and the SwiGLU output that enters the down projection) rounded
to BF16, then to FP16, and each is compared with the exact oracle on the same
blocks.  BF16 rounding at those two points alone moves the pass by several
times more than FP16 rounding does, and by a sizeable part of the bar.  The
test needs no GPU and shares nothing with the HIP path; it reads only
`oracle/` and the seeded input generators."""
import numpy as np
import pytest

import oracle
import workload as W

N_SEQ = 3  # sequences of the 32-sequence 0.5B workload (its first three)


def round_bf16(x):
    """Round to the nearest BF16 (ties to even), via the float32 bit pattern."""
    f = np.asarray(x, dtype=np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


def round_fp16(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def test_rounding_helpers():
    # BF16 keeps 8 significant bits: 1 + 2^-8 is a tie that rounds to even (1),
    # 1 + 3 * 2^-8 rounds up to 1 + 2^-6; FP16 keeps 11 bits
    assert round_bf16(1 + 2.0 ** -8) == 1.0
    assert round_bf16(1 + 3 * 2.0 ** -8) == 1 + 2.0 ** -6
    assert round_bf16(-3.0) == -3.0
    assert round_fp16(1 + 2.0 ** -11) == 1.0
    assert round_fp16(1 + 3 * 2.0 ** -11) == 1 + 2.0 ** -9


def _row_rel(a, ref):
    return np.linalg.norm(a - ref, axis=-1) / np.linalg.norm(ref, axis=-1)


@pytest.mark.slow
def test_bf16_activations_move_the_pass_more_than_fp16():
    wl = W.WORKLOADS["0.5b-fp8-b32-ctx512to4096"]
    m = wl.model
    weights = W.model_weights(m, wl.seed)
    lens = W.context_lengths(wl)[:N_SEQ]
    kv_layers = [W.synthetic_kv_layer(m, wl.seed, l, lens, int(lens.max())) for l in range(m.n_layers)]
    kv0 = oracle.OracleKV.from_bf16(m, [k for k, _ in kv_layers], [v for _, v in kv_layers], lens)
    blocks = np.stack([W.draft_rng(wl, b).integers(0, m.vocab, size=16) for b in range(N_SEQ)])

    om = oracle.OracleModel(m, weights)
    out = {}
    for name, act in (("exact", None), ("bf16", round_bf16), ("fp16", round_fp16)):
        om.act = act if act is not None else (lambda x: x)
        x = oracle.forward(om, kv0.copy(), blocks).reshape(-1, m.hidden)
        out[name] = (x, om.logits(x))
    ref_x, ref_l = out["exact"]
    err = {k: (_row_rel(out[k][0], ref_x).max(), _row_rel(out[k][1], ref_l).max()) for k in ("bf16", "fp16")}
    print("max row rel err (hidden, logits):", {k: tuple(float(f"{e:.4g}") for e in v) for k, v in err.items()})
    # FP16 leaves a wide margin under the bar; BF16 takes a large share of it
    # from these two rounding points alone, and several times FP16's error
    assert err["fp16"][0] < 5e-3 and err["fp16"][1] < 5e-3
    assert err["bf16"][0] > 4 * err["fp16"][0] and err["bf16"][1] > 4 * err["fp16"][1]
    assert err["bf16"][0] > 1e-2
