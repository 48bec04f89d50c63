"""spec_debug_attention_noalloc, the allocation-free variant of
spec_debug_attention for callers that cannot allocate device memory: on the
same inputs its output must equal the allocating entry point's bit for bit
(the two run the same kernels with the same split plan, so any difference is
a fault of the static buffer's use).  Two calls in a row, the second smaller
than the first, so stale contents of the shared buffer would show; a launch
whose partials exceed the buffer is refused on the host."""
import ctypes

import numpy as np
import pytest
import torch

import workload as W
from block_draft_verification_amd import SpecError, debug_attention, load_library

pytestmark = pytest.mark.gpu


def _case(B, Hq, Hkv, D, lens, max_ctx, seed):
    rng = np.random.default_rng(seed)
    q = torch.from_numpy(rng.standard_normal((B * 16, Hq * D)).astype(np.float16).view(np.int16)).cuda()
    K = W.to_bf16_bits(rng.standard_normal((B, Hkv, max_ctx, D)).astype(np.float32))
    V = W.to_bf16_bits(rng.standard_normal((B, Hkv, max_ctx, D)).astype(np.float32))
    kc = torch.from_numpy(K.view(np.int16)).cuda()
    vc = torch.from_numpy(V.view(np.int16)).cuda()
    kl = torch.tensor(np.asarray(lens, np.int32)).cuda()
    return q, kc, vc, kl


@pytest.mark.parametrize("split_len", [0, 128])
def test_noalloc_attention_equals_allocating(split_len):
    shapes = [  # the second call is smaller than the first
        dict(B=4, Hq=14, Hkv=2, D=64, lens=[600, 100, 0, 1072], max_ctx=1088, seed=1),
        dict(B=2, Hq=32, Hkv=8, D=128, lens=[300, 17], max_ctx=576, seed=2),
    ]
    for sh in shapes:
        q, kc, vc, kl = _case(sh["B"], sh["Hq"], sh["Hkv"], sh["D"], sh["lens"], sh["max_ctx"], sh["seed"])
        args = (q, kc, vc, kl, sh["B"], sh["Hq"], sh["Hkv"], sh["D"], split_len)
        ref = debug_attention(*args)
        out = torch.full_like(q, 0x7e00)  # NaN bits: every element must be written
        got = debug_attention(*args, noalloc=True, out=out)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"noalloc attention differs from the allocating one for {sh}"


def test_noalloc_attention_rejects_oversize():
    """1024 (sequence, KV head) units of head_dim 128 with 8 query heads each
    need more partial storage than the static buffer holds: refused before any
    launch, with the reason in spec_last_error()."""
    t = torch.zeros(16, dtype=torch.int16, device="cuda")
    kl = torch.zeros(128, dtype=torch.int32, device="cuda")
    lib = load_library()
    rc = lib.spec_debug_attention_noalloc(128, 64, 8, 128, 128, 128, t.data_ptr(), t.data_ptr(), t.data_ptr(),
                                          kl.data_ptr(), t.data_ptr(), 0,
                                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == -1 and b"SPEC_ATTN_SCRATCH_BYTES" in lib.spec_last_error()
    with pytest.raises(SpecError):
        debug_attention(torch.zeros(128 * 16, 64 * 128, dtype=torch.int16, device="cuda"),
                        torch.zeros(128, 8, 128, 128, dtype=torch.int16, device="cuda"),
                        torch.zeros(128, 8, 128, 128, dtype=torch.int16, device="cuda"), kl, 128, 64, 8, 128,
                        noalloc=True)
