"""CPU oracle for the block-draft verify pass.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls it, and it shares no code
with that path: the only thing both consume is the seeded input module
``workload``.

What it computes (plain, slow, float64 throughout):

* the target decoder forward over a block of rows per sequence, each row at
  position n_b + j, attending to the committed KV cache plus the block rows
  up to itself (block-causal);
* greedy argmax of the lm_head at every row, lowest id on ties;
* the accepted length: the first index j >= 1 where the draft differs from
  the argmax of row j-1, or 16 when none does; the bonus token is the argmax
  of the last accepted row;
* commit: the committed length grows by the accepted count.

Sources: "The Inference Stack Behind OCRia" (speculative decoding section:
the target verifies all drafted tokens in one forward pass, losslessly), and
the HunyuanOCR-1.5 / DFlash write-up (inference loop, steps 3-5: verify the
16-token block in one forward, keep the longest valid prefix cut at the
first left-to-right mismatch, append and repeat).  Architecture details the
pages leave open (pre-norm RMSNorm, rotate-half RoPE, SwiGLU, no biases,
contiguous GQA grouping) take the plainest reading; each is listed as a
reading in the design notes.

Parity pins: every function here is checked in ``tests/test_oracle_*.py``
against something other than itself (library routines in float64, closed
forms, brute force, the speculative == autoregressive invariant).
"""
from .codecs import decode_bf16, decode_e2m1, decode_e4m3, decode_e8m0, mxfp8_roundtrip  # noqa: F401
from .model import (  # noqa: F401
    OracleKV, OracleModel, VerifyResult, accept, ar_decode, attention, commit, forward,
    greedy, greedy_continuation, prefill, rms_norm, rope, silu, spec_decode, verify_block)
