"""The C-ABI library without a GPU: it loads, exports every function the
header declares (with the binding's prototypes), and rejects bad arguments on
the host before touching the device."""
import ctypes
import os
import re
import subprocess

import pytest

import block_draft_verification_amd as bdv
from block_draft_verification_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec_verify.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(spec_\w+)\s*\(", src, flags=re.M))


def test_header_declares_the_boundary():
    names = _declared()
    for n in ["spec_verify_init", "spec_verify_block", "spec_commit_kv", "spec_verify_destroy",
              "spec_get_device_error", "spec_status_str"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = bdv.load_library()
    out = subprocess.run(["nm", "-D", "--defined-only", bdv.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (spec_\w+)", out))
    assert _declared() <= exported
    assert set(B.EXPORTS) == _declared()
    for n in _declared():
        assert getattr(lib, n) is not None


def test_status_strings():
    lib = bdv.load_library()
    assert lib.spec_status_str(0) == b"ok"
    assert b"argument" in lib.spec_status_str(-1)
    assert lib.spec_status_str(-99) == b"unknown status"


def test_host_side_argument_checks():
    lib = bdv.load_library()
    # no context / bad batch: rejected before any device work
    assert lib.spec_verify_block(None, 1, None, None, None, None, None) == -1
    assert lib.spec_commit_kv(None, 1, None, None) == -1
    assert lib.spec_verify_destroy(None) == 0
    v = ctypes.c_int32()
    assert lib.spec_get_device_error(None, ctypes.byref(v), None) == -1
    assert lib.spec_debug_set_dump(None, None, None) == -1
    assert lib.spec_prefill(None, 1, 16, 16, 16, 16, None, None) == -1
    assert lib.spec_export_hidden(None, 1, 16, None) == -1
    assert lib.spec_verify_set_lanes(None, 2) == -1
    m0 = B.SpecModelDesc(2, 4096 + 64, 4, 2, 64, 704, 1024, 1e-6, 1e4, 1, 1, 1)  # hidden > 4096
    w0 = B.SpecWeights((B.SpecLayerWeights * 2)(), 16, None, 16)
    kv0 = B.SpecKV(16, 16, 16, 1, 128)
    h0 = ctypes.c_void_p()
    assert lib.spec_verify_init(ctypes.byref(m0), ctypes.byref(w0), ctypes.byref(kv0), None, ctypes.byref(h0)) == -2
    # shapes the kernels do not support are refused at init
    m = B.SpecModelDesc(2, 256, 4, 2, 96, 704, 1024, 1e-6, 1e4, 1, 1, 1)       # head_dim 96
    arr = (B.SpecLayerWeights * 2)()
    w = B.SpecWeights(arr, 16, None, 16)
    kv = B.SpecKV(16, 16, 16, 1, 128)
    h = ctypes.c_void_p()
    assert lib.spec_verify_init(ctypes.byref(m), ctypes.byref(w), ctypes.byref(kv), None, ctypes.byref(h)) == -2
    m.head_dim = 64
    m.mlp_wfmt = 3                                                            # BF16 MLP not supported
    assert lib.spec_verify_init(ctypes.byref(m), ctypes.byref(w), ctypes.byref(kv), None, ctypes.byref(h)) == -3
    m.mlp_wfmt = 1
    m.act_fmt = 2                                                             # no such activation format
    assert lib.spec_verify_init(ctypes.byref(m), ctypes.byref(w), ctypes.byref(kv), None, ctypes.byref(h)) == -3
    m.act_fmt = 1
    m.n_q_heads = 3                                                           # Hq % Hkv != 0
    assert lib.spec_verify_init(ctypes.byref(m), ctypes.byref(w), ctypes.byref(kv), None, ctypes.byref(h)) == -2
    m.n_q_heads = 4
    # NULL per-layer weight pointers
    assert lib.spec_verify_init(ctypes.byref(m), ctypes.byref(w), ctypes.byref(kv), None, ctypes.byref(h)) == -1
    assert h.value is None
    # debug entry points validate before launching
    assert lib.spec_debug_linear(16, 100, 64, 16, 16, 16, 1, 16, None) == -1  # N % 64
    assert lib.spec_debug_quant_mx8(4, 48, 16, 16, 16, None) == -1              # K % 32
    assert lib.spec_debug_linear(16, 64, 64, 16, 16, None, 1, 16, None) == -1   # FP8 without scales
    assert b"scales" in lib.spec_last_error()                                   # the failure is described
    assert lib.spec_debug_residual(16, 96, 64, 16, 16, 16, 1, 16, 16, 0, 32, 16, 16, None) == -1  # N % 64
    assert lib.spec_debug_residual(16, 64, 64, 16, 16, 16, 3, 16, 16, 0, 32, 16, 16, None) == -3  # BF16 weights
    assert lib.spec_debug_residual(16, 64, 64, 16, 16, 16, 1, 16, 16, 0, 16, 16, 16, None) == -1  # h_in == h_out
    assert lib.spec_debug_quant_mx8(4, 64, 16, 24, 16, None) == -1              # codes not 16-byte aligned
    assert lib.spec_debug_linear_mx8(16, 64, 96, 16, 16, 16, 16, 1, 16, None) == -1   # K % 64
    assert lib.spec_debug_linear_mx8(16, 64, 64, 16, 16, 16, None, 2, 16, None) == -1  # MXFP4 without scales
    assert lib.spec_debug_linear_mx8(16, 64, 64, 16, 16, 16, 16, 3, 16, None) == -3    # BF16 weights
    assert lib.spec_debug_rmsnorm(4, 4096 + 32, 16, 16, 1e-6, 0, 16, None, None) == -1  # H > 4096
    assert lib.spec_debug_rmsnorm(4, 64, 16, 16, 1e-6, 1, 16, None, None) == -1         # MXFP8 without scales
    assert lib.spec_debug_rmsnorm(4, 64, 16, 16, 1e-6, 5, 16, 16, None) == -3           # unknown format
    assert lib.spec_debug_swiglu(4, 64, 96, 16, None, 16, 16, 1, 0, 16, None, None) == -1  # I % 64
    assert lib.spec_debug_swiglu(4, 64, 64, 16, None, 16, 16, 1, 1, 16, None, None) == -1  # MXFP8 out, no scales
    assert lib.spec_debug_attention(1, 4, 2, 80, 1, 128, 16, 16, 16, 16, 16, 0, None) == -2


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", "/nonexistent/libspecverify.so")
    with pytest.raises(RuntimeError, match="missing"):
        B.load_library()
