"""ctypes binding of libspecverify.so: argument marshalling only.

Every step of the verify pass runs in the HIP library; this module only
places caller-owned buffers in device memory (torch tensors, weights in the
row-major layout a checkpoint holds), fills the descriptor structs of
include/spec_verify.h and forwards pointers and the current HIP stream.  It
fails loudly when the library is missing.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspecverify.so")

SPEC_OK = 0
WFMT_FP8_E4M3_ROW, WFMT_MXFP4, WFMT_BF16 = 1, 2, 3
ACT_FMTS = {"fp16": 0, "mxfp8": 1}
DERR_TOKEN, DERR_CAPACITY, DERR_COMMIT, DERR_LENGTH, DERR_PAGE, DERR_RANGE = 1, 2, 4, 8, 16, 32
BLOCK = 16

_P = ctypes.c_void_p
_I = ctypes.c_int32


class SpecModelDesc(ctypes.Structure):
    _fields_ = [("n_layers", _I), ("hidden", _I), ("n_q_heads", _I), ("n_kv_heads", _I), ("head_dim", _I),
                ("intermediate", _I), ("vocab", _I), ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
                ("attn_wfmt", _I), ("mlp_wfmt", _I), ("tied_lm_head", _I), ("act_fmt", _I)]


class SpecLayerWeights(ctypes.Structure):
    _fields_ = [(n, _P) for n in ("w_qkv", "s_qkv", "w_o", "s_o", "w_gate_up", "s_gate_up", "w_down", "s_down",
                                  "attn_norm", "mlp_norm")]


class SpecWeights(ctypes.Structure):
    _fields_ = [("layers", ctypes.POINTER(SpecLayerWeights)), ("embed", _P), ("lm_head", _P), ("final_norm", _P)]


class SpecKV(ctypes.Structure):
    _fields_ = [("k_cache", _P), ("v_cache", _P), ("kv_len", _P), ("max_batch", _I), ("max_ctx", _I),
                ("page_table", _P), ("page_size", _I), ("num_pages", _I)]


EXPORTS = {
    "spec_verify_init": (_I, [ctypes.POINTER(SpecModelDesc), ctypes.POINTER(SpecWeights), ctypes.POINTER(SpecKV),
                              _P, ctypes.POINTER(_P)]),
    "spec_verify_block": (_I, [_P, _I, _P, _P, _P, _P, _P]),
    "spec_verify_set_lanes": (_I, [_P, _I]),
    "spec_commit_kv": (_I, [_P, _I, _P, _P]),
    "spec_prefill": (_I, [_P, _I, _P, _I, _P, _P, _P, _P]),
    "spec_export_hidden": (_I, [_P, _I, _P, _P]),
    "spec_verify_destroy": (_I, [_P]),
    "spec_get_device_error": (_I, [_P, ctypes.POINTER(_I), _P]),
    "spec_status_str": (ctypes.c_char_p, [_I]),
    "spec_last_error": (ctypes.c_char_p, []),
    "spec_debug_set_dump": (_I, [_P, _P, _P]),
    "spec_debug_linear": (_I, [_I, _I, _I, _P, _P, _P, _I, _P, _P]),
    "spec_debug_residual": (_I, [_I, _I, _I, _P, _P, _P, _I, _P, _P, _I, _P, _P, _P, _P]),
    "spec_debug_quant_mx8": (_I, [_I, _I, _P, _P, _P, _P]),
    "spec_debug_linear_mx8": (_I, [_I, _I, _I, _P, _P, _P, _P, _I, _P, _P]),
    "spec_debug_rmsnorm": (_I, [_I, _I, _P, _P, ctypes.c_float, _I, _P, _P, _P]),
    "spec_debug_swiglu": (_I, [_I, _I, _I, _P, _P, _P, _P, _I, _I, _P, _P, _P]),
    "spec_debug_attention": (_I, [_I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _I, _P]),
    "spec_debug_attention_noalloc": (_I, [_I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _I, _P]),
    "spec_debug_time_kernel": (_I, [_P, _I]),
    "spec_debug_set_repeat": (_I, [_P, _I]),
    "spec_debug_kernel_time": (_I, [_P, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(_I)]),
}

KERNEL_KINDS = {"embed": 1, "rmsnorm": 2, "qkv": 3, "attention": 4, "o_proj": 5, "gate_up": 6, "down": 7,
                "lm_head": 8, "accept": 9, "commit": 10, "attn_merge": 11}

_lib = None


def load_library():
    """Load libspecverify.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build the HIP library first "
                               "(python -c 'import __graft_entry__ as g; g.build()')")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(lib, name)
            fn.restype, fn.argtypes = res, args
        _lib = lib
    return _lib


class SpecError(RuntimeError):
    pass


def _check(rc: int, what: str):
    if rc != SPEC_OK:
        lib = load_library()
        raise SpecError(f"{what}: {lib.spec_status_str(rc).decode()} ({rc}): {lib.spec_last_error().decode()}")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(a, device):
    if isinstance(a, torch.Tensor):  # already a tensor (drawn on the device): used as it is
        return a.contiguous().to(device)
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def _wfmt(name: str) -> int:
    return {"fp8": WFMT_FP8_E4M3_ROW, "mxfp4": WFMT_MXFP4}[name]


class DeviceModel:
    """Caller-owned device buffers: row-major weights (the library repacks its
    own copy at init), the BF16 KV cache for K and V, and kv_len.  Contiguous cache: [L][max_batch][Hkv]
    [max_ctx][D].  Paged cache (page_table given, int [max_batch][max_ctx /
    page_size]): a pool [L][num_pages][Hkv][page_size][D]; kv_layers are then
    given in the contiguous shape and scattered into the pages."""

    def __init__(self, shape, weights: dict, max_batch: int, max_ctx: int, kv_layers=None, kv_len=None,
                 device="cuda", page_table=None, page_size: int = 0, num_pages: int = 0):
        self.shape, self.max_batch, self.max_ctx, self.device = shape, max_batch, max_ctx, device
        self.page_size, self.num_pages = page_size, num_pages
        self.page_table = None if page_table is None else torch.as_tensor(
            np.asarray(page_table, np.int32), device=device).contiguous()
        m = shape
        self.layers = [{k: _dev(v, device) for k, v in lw.items()} for lw in weights["layers"]]
        self.embed = _dev(weights["embed"], device)
        self.lm_head = None if weights.get("lm_head") is None else _dev(weights["lm_head"], device)
        self.final_norm = _dev(weights["final_norm"], device)
        if self.page_table is None:
            cache_shape = (m.n_layers, max_batch, m.n_kv_heads, max_ctx, m.head_dim)
        else:
            cache_shape = (m.n_layers, num_pages, m.n_kv_heads, page_size, m.head_dim)
        self.k_cache = torch.zeros(cache_shape, dtype=torch.int16, device=device)
        self.v_cache = torch.zeros(cache_shape, dtype=torch.int16, device=device)
        self.kv_len = torch.zeros(max_batch, dtype=torch.int32, device=device)
        if kv_layers is not None:
            for l, (K, V) in enumerate(kv_layers):
                self.load_kv_layer(l, K, V)
        if kv_len is not None:
            self.kv_len[:len(kv_len)] = torch.as_tensor(np.asarray(kv_len, np.int32), device=device)

    def load_kv_layer(self, l, K, V):
        """K, V: uint16 [b, Hkv, max_ctx, D] for sequences 0 .. b-1."""
        b = K.shape[0]
        if self.page_table is None:
            self.k_cache[l, :b].copy_(_dev(K, "cpu"))
            self.v_cache[l, :b].copy_(_dev(V, "cpu"))
            return
        ps, pt = self.page_size, self.page_table.cpu().numpy()
        for s in range(b):
            for j in range(self.max_ctx // ps):
                pg = int(pt[s, j])
                self.k_cache[l, pg].copy_(_dev(np.ascontiguousarray(K[s, :, j * ps:(j + 1) * ps]), "cpu"))
                self.v_cache[l, pg].copy_(_dev(np.ascontiguousarray(V[s, :, j * ps:(j + 1) * ps]), "cpu"))

    def cache_rows(self, l: int, b: int, n: int, which: str = "k") -> torch.Tensor:
        """Positions 0 .. n-1 of sequence b in layer l, [Hkv, n, D] int16, in either layout."""
        cache = self.k_cache if which == "k" else self.v_cache
        if self.page_table is None:
            return cache[l, b, :, :n]
        ps = self.page_size
        pages = self.page_table[b, :(n + ps - 1) // ps].long()
        return cache[l, pages].permute(1, 0, 2, 3).reshape(self.shape.n_kv_heads, -1, self.shape.head_dim)[:, :n]

    def structs(self):
        m = self.shape
        desc = SpecModelDesc(m.n_layers, m.hidden, m.n_q_heads, m.n_kv_heads, m.head_dim, m.intermediate, m.vocab,
                             m.rms_eps, m.rope_theta, WFMT_FP8_E4M3_ROW, _wfmt(m.mlp_format),
                             1 if m.tied_lm_head else 0)
        arr = (SpecLayerWeights * m.n_layers)()
        for i, lw in enumerate(self.layers):
            for name in SpecLayerWeights._fields_:
                setattr(arr[i], name[0], lw[name[0]].data_ptr())
        w = SpecWeights(arr, self.embed.data_ptr(), None if self.lm_head is None else self.lm_head.data_ptr(),
                        self.final_norm.data_ptr())
        pt = None if self.page_table is None else self.page_table.data_ptr()
        kv = SpecKV(self.k_cache.data_ptr(), self.v_cache.data_ptr(), self.kv_len.data_ptr(), self.max_batch,
                    self.max_ctx, pt, self.page_size, self.num_pages)
        return desc, arr, w, kv


class Verifier:
    """One spec_ctx bound to a DeviceModel.  act_fmt: "fp16" or "mxfp8" (the
    activation format of the QKV, gate/up and down projections)."""

    def __init__(self, dev: DeviceModel, act_fmt: str = "fp16", lanes: int = 1):
        lib = load_library()
        self.dev = dev
        self._desc, self._arr, self._w, self._kv = dev.structs()
        self._desc.act_fmt = ACT_FMTS[act_fmt]
        h = ctypes.c_void_p()
        _check(lib.spec_verify_init(ctypes.byref(self._desc), ctypes.byref(self._w), ctypes.byref(self._kv),
                                    _stream(), ctypes.byref(h)), "spec_verify_init")
        self._h = h
        self._dump = (None, None)
        if lanes != 1:
            self.set_lanes(lanes)

    def set_lanes(self, lanes: int):
        """Run the batch as `lanes` concurrent sequence ranges (spec_verify_set_lanes)."""
        _check(load_library().spec_verify_set_lanes(self._h, lanes), "spec_verify_set_lanes")

    def verify(self, tokens: torch.Tensor, accept_len=None, bonus=None, argmax="alloc"):
        """tokens int32 [B, 16] on the device.  Returns the output tensors."""
        B = tokens.shape[0]
        assert tokens.dtype == torch.int32 and tokens.is_contiguous() and tokens.shape[1] == BLOCK
        d = tokens.device
        accept_len = torch.empty(B, dtype=torch.int32, device=d) if accept_len is None else accept_len
        bonus = torch.empty(B, dtype=torch.int32, device=d) if bonus is None else bonus
        if isinstance(argmax, str):
            argmax = torch.empty(B, BLOCK, dtype=torch.int32, device=d)
        _check(load_library().spec_verify_block(self._h, B, _ptr(tokens), _ptr(accept_len), _ptr(bonus),
                                                _ptr(argmax), _stream()), "spec_verify_block")
        return {"accept_len": accept_len, "bonus": bonus, "argmax": argmax}

    def commit(self, batch: int, n_commit: torch.Tensor | None = None):
        _check(load_library().spec_commit_kv(self._h, batch, _ptr(n_commit), _stream()), "spec_commit_kv")

    def prefill(self, prompt: torch.Tensor, lengths: torch.Tensor, anchor_hidden: torch.Tensor | None = None,
                pending: torch.Tensor | None = None):
        """prompt int32 [B, T], lengths int32 [B] on the device; appends each
        prompt to its cache.  Returns the pending tokens (int32 [B])."""
        B, T = prompt.shape
        assert prompt.dtype == torch.int32 and prompt.is_contiguous() and lengths.dtype == torch.int32
        pending = torch.empty(B, dtype=torch.int32, device=prompt.device) if pending is None else pending
        _check(load_library().spec_prefill(self._h, B, _ptr(prompt), T, _ptr(lengths), _ptr(pending),
                                           _ptr(anchor_hidden), _stream()), "spec_prefill")
        return pending

    def export_hidden(self, batch: int, out: torch.Tensor | None = None) -> torch.Tensor:
        """BF16 [batch, hidden] final normed hidden state of row tau-1 of the last pass."""
        if out is None:
            out = torch.empty(batch, self.dev.shape.hidden, dtype=torch.bfloat16, device="cuda")
        _check(load_library().spec_export_hidden(self._h, batch, _ptr(out), _stream()), "spec_export_hidden")
        return out

    def device_error(self) -> int:
        v = ctypes.c_int32()
        _check(load_library().spec_get_device_error(self._h, ctypes.byref(v), _stream()), "spec_get_device_error")
        return v.value

    def set_dump(self, hidden=None, logits=None):
        self._dump = (hidden, logits)
        _check(load_library().spec_debug_set_dump(self._h, _ptr(hidden), _ptr(logits)), "spec_debug_set_dump")

    def time_kernel(self, kind: str | None):
        """Start (or stop, with None) event timing of one kernel class."""
        _check(load_library().spec_debug_time_kernel(self._h, 0 if kind is None else KERNEL_KINDS[kind]),
               "spec_debug_time_kernel")

    def set_repeat(self, repeat: int):
        """While a kernel class is timed, issue each of its launches `repeat` times."""
        _check(load_library().spec_debug_set_repeat(self._h, repeat), "spec_debug_set_repeat")

    def kernel_time(self):
        """(total ms, launches) recorded since the last call."""
        ms, n = ctypes.c_float(), ctypes.c_int32()
        _check(load_library().spec_debug_kernel_time(self._h, ctypes.byref(ms), ctypes.byref(n)),
               "spec_debug_kernel_time")
        return ms.value, n.value

    def close(self):
        if self._h is not None:
            _check(load_library().spec_verify_destroy(self._h), "spec_verify_destroy")
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def debug_linear(x_bf16: torch.Tensor, w: torch.Tensor, scales, wfmt: int, N: int) -> torch.Tensor:
    """y = x W^T (fp32) through the library's linear kernel."""
    M, K = x_bf16.shape
    y = torch.empty(M, N, dtype=torch.float32, device=x_bf16.device)
    _check(load_library().spec_debug_linear(M, N, K, _ptr(x_bf16), _ptr(w), _ptr(scales), wfmt, _ptr(y),
                                            _stream()), "spec_debug_linear")
    return y


def debug_residual(x_f16: torch.Tensor, w: torch.Tensor, scales, wfmt: int, h_in: torch.Tensor,
                   gain: torch.Tensor, xg_bf16: bool = False):
    """One residual projection with the next RMSNorm folded in (spec_debug_residual):
    returns (h_out fp32 [M, N], xg 16-bit bits int16 [M, N], ssp fp32 [M, ld])."""
    M, K = x_f16.shape
    N = h_in.shape[1]
    ld = ((N // 32 + 3) // 4) * 4
    h_out = torch.empty_like(h_in)
    xg = torch.empty(M, N, dtype=torch.int16, device=h_in.device)
    ssp = torch.full((M, ld), float("nan"), dtype=torch.float32, device=h_in.device)
    _check(load_library().spec_debug_residual(M, N, K, _ptr(x_f16), _ptr(w), _ptr(scales), wfmt, _ptr(h_in),
                                              _ptr(gain), 1 if xg_bf16 else 0, _ptr(h_out), _ptr(xg), _ptr(ssp),
                                              _stream()), "spec_debug_residual")
    return h_out, xg, ssp


def debug_quant_mx8(x: torch.Tensor):
    """MXFP8 encoding of fp32 rows x [M, K]: (e4m3 codes uint8 [M, K], e8m0 uint8 [M, K/32])."""
    M, K = x.shape
    codes = torch.empty(M, K, dtype=torch.uint8, device=x.device)
    scales = torch.empty(M, K // 32, dtype=torch.uint8, device=x.device)
    _check(load_library().spec_debug_quant_mx8(M, K, _ptr(x), _ptr(codes), _ptr(scales), _stream()),
           "spec_debug_quant_mx8")
    return codes, scales


def debug_linear_mx8(codes: torch.Tensor, scales: torch.Tensor, w: torch.Tensor, wscales, wfmt: int,
                     N: int) -> torch.Tensor:
    """y = x W^T (fp32) with MXFP8 activations (codes [M, K], e8m0 [M, K/32])."""
    M, K = codes.shape
    y = torch.empty(M, N, dtype=torch.float32, device=codes.device)
    _check(load_library().spec_debug_linear_mx8(M, N, K, _ptr(codes), _ptr(scales), _ptr(w), _ptr(wscales), wfmt,
                                                _ptr(y), _stream()), "spec_debug_linear_mx8")
    return y


def debug_rmsnorm(h: torch.Tensor, gain: torch.Tensor, eps: float, act_fmt: str = "fp16"):
    """The pass's RMSNorm on fp32 rows h [M, H]: FP16 bits (int16 [M, H]) or
    MXFP8 (codes uint8 [M, H], e8m0 uint8 [M, H/32])."""
    M, H = h.shape
    if act_fmt == "fp16":
        x, xs = torch.empty(M, H, dtype=torch.int16, device=h.device), None
    else:
        x = torch.empty(M, H, dtype=torch.uint8, device=h.device)
        xs = torch.empty(M, H // 32, dtype=torch.uint8, device=h.device)
    _check(load_library().spec_debug_rmsnorm(M, H, _ptr(h), _ptr(gain), eps, ACT_FMTS[act_fmt], _ptr(x), _ptr(xs),
                                             _stream()), "spec_debug_rmsnorm")
    return x if xs is None else (x, xs)


def debug_swiglu(x: torch.Tensor, x_scales, w: torch.Tensor, wscales, wfmt: int, I: int, out_fmt: str = "fp16"):
    """SiLU(x Wg^T) * (x Wu^T) through the gate/up kernel.  x: FP16 bits
    [M, H] (x_scales None) or MXFP8 codes [M, H] with e8m0 x_scales."""
    M, H = x.shape
    if out_fmt == "fp16":
        a, as_ = torch.empty(M, I, dtype=torch.int16, device=x.device), None
    else:
        a = torch.empty(M, I, dtype=torch.uint8, device=x.device)
        as_ = torch.empty(M, I // 32, dtype=torch.uint8, device=x.device)
    _check(load_library().spec_debug_swiglu(M, H, I, _ptr(x), _ptr(x_scales), _ptr(w), _ptr(wscales), wfmt,
                                            ACT_FMTS[out_fmt], _ptr(a), _ptr(as_), _stream()), "spec_debug_swiglu")
    return a if as_ is None else (a, as_)


def debug_attention(q, k_cache, v_cache, kv_len, batch, n_q_heads, n_kv_heads, head_dim, split_len=0,
                    noalloc=False, out=None):
    """One layer's block-causal attention through the library's kernel;
    noalloc=True goes through spec_debug_attention_noalloc (no device
    allocation, asynchronous) with `out` as the caller's output buffer."""
    max_batch, _, max_ctx, _ = k_cache.shape
    o = torch.empty_like(q) if out is None else out
    fn = "spec_debug_attention_noalloc" if noalloc else "spec_debug_attention"
    _check(getattr(load_library(), fn)(batch, n_q_heads, n_kv_heads, head_dim, max_batch, max_ctx, _ptr(q),
                                       _ptr(k_cache), _ptr(v_cache), _ptr(kv_len), _ptr(o), split_len, _stream()), fn)
    return o
