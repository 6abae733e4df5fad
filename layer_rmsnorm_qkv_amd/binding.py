"""Thin ctypes binding of liblrq (include/lrq.h): argument marshalling only.

Every function has the name of the C entry point it calls.  Array arguments may be
torch tensors (their ``data_ptr()`` is passed) or plain integers (raw device
addresses; 0 = NULL).  A non-OK status raises :class:`LrqError` carrying the
library's message.  There is no fallback: if ``liblrq.so`` is missing, loading it
raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblrq.so")

LRQ_OK, LRQ_ERR_INVALID_ARG, LRQ_ERR_UNSUPPORTED, LRQ_ERR_HIP = 0, 1, 2, 3
LRQ_F32, LRQ_BF16 = 0, 1
LRQ_TARGET_Q, LRQ_TARGET_K, LRQ_TARGET_V = 1, 2, 4
LRQ_VARIANT_AUTO, LRQ_VARIANT_GENERIC, LRQ_VARIANT_TILED, LRQ_VARIANT_DECODE = 0, 1, 2, 3
VARIANT_NAMES = {LRQ_VARIANT_GENERIC: "generic", LRQ_VARIANT_TILED: "tiled", LRQ_VARIANT_DECODE: "decode"}
LRQ_WEIGHT_DENSE, LRQ_WEIGHT_NF4 = 0, 1

# every symbol include/lrq.h declares
EXPORTED = ("lrq_forward", "lrq_forward_kv", "lrq_backward", "lrq_workspace_size", "lrq_select_variant",
            "lrq_status_string", "lrq_last_error", "lrq_abi_version", "lrq_kernel_timing",
            "lrq_kernel_time_ms", "lrq_prepared_size", "lrq_prepare_weights", "lrq_forward_prepared",
            "lrq_backward_prepared", "lrq_workspace_size_prepared", "lrq_forward_noalloc",
            "lrq_mlp_workspace_size", "lrq_mlp_forward", "lrq_nf4_weight_size", "lrq_quantize_nf4",
            "lrq_attention")
LRQ_MLP_GATE, LRQ_MLP_UP, LRQ_MLP_DOWN = 1, 2, 4


class LrqDesc(ctypes.Structure):
    _fields_ = [("n_tokens", ctypes.c_int64), ("d_model", ctypes.c_int64),
                ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
                ("lora_rank", ctypes.c_int32), ("lora_alpha", ctypes.c_float),
                ("lora_targets", ctypes.c_uint32), ("has_bias", ctypes.c_int32),
                ("variant", ctypes.c_int32), ("lora_dropout", ctypes.c_float),
                ("dropout_offset", ctypes.c_uint32), ("dropout_seed", ctypes.c_uint64),
                ("weight_format", ctypes.c_int32)]


class LrqMlpDesc(ctypes.Structure):
    _fields_ = [("n_tokens", ctypes.c_int64), ("d_model", ctypes.c_int64), ("d_ff", ctypes.c_int64),
                ("dtype", ctypes.c_int32), ("lora_rank", ctypes.c_int32), ("lora_alpha", ctypes.c_float),
                ("lora_targets", ctypes.c_uint32)]


class LrqAttnDesc(ctypes.Structure):
    _fields_ = [("n_seqs", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32), ("max_q_len", ctypes.c_int32),
                ("ld_q", ctypes.c_int64), ("num_slots", ctypes.c_int64), ("scale", ctypes.c_float),
                ("causal", ctypes.c_int32)]


class LrqKvCache(ctypes.Structure):
    _fields_ = [("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p), ("slots", ctypes.c_void_p),
                ("num_slots", ctypes.c_int64)]


class LrqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


_STATUS = {0: "LRQ_OK", 1: "LRQ_ERR_INVALID_ARG", 2: "LRQ_ERR_UNSUPPORTED", 3: "LRQ_ERR_HIP"}
_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load liblrq.so once (raises OSError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise OSError(f"{path} not found: build it with `python -m layer_rmsnorm_qkv_amd.build`")
        # The library must bind to the HIP runtime that owns the caller's device memory and
        # streams.  PyTorch-ROCm ships its own libamdhip64.so.7; loading torch first makes the
        # dynamic linker resolve liblrq's libamdhip64.so.7 to that same copy.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        lib = ctypes.CDLL(path)
        P, S = ctypes.c_void_p, ctypes.c_size_t
        PP = ctypes.POINTER(ctypes.c_void_p)
        lib.lrq_forward.argtypes = [ctypes.POINTER(LrqDesc), P, P, P, P, PP, PP, P, P, P, S, P]
        lib.lrq_forward.restype = ctypes.c_int
        lib.lrq_forward_kv.argtypes = [ctypes.POINTER(LrqDesc), P, P, P, P, PP, PP, P, P,
                                       ctypes.POINTER(LrqKvCache), P, S, P]
        lib.lrq_forward_kv.restype = ctypes.c_int
        lib.lrq_backward.argtypes = [ctypes.POINTER(LrqDesc), P, P, P, P, PP, PP, P, P, P, P, PP, PP, P, S, P]
        lib.lrq_backward.restype = ctypes.c_int
        lib.lrq_workspace_size.argtypes = [ctypes.POINTER(LrqDesc), ctypes.c_int]
        lib.lrq_workspace_size.restype = ctypes.c_size_t
        lib.lrq_workspace_size_prepared.argtypes = [ctypes.POINTER(LrqDesc), ctypes.c_int]
        lib.lrq_workspace_size_prepared.restype = ctypes.c_size_t
        lib.lrq_attention.argtypes = [ctypes.POINTER(LrqAttnDesc), P, P, P, P, P, P, P, P]
        lib.lrq_attention.restype = ctypes.c_int
        lib.lrq_nf4_weight_size.argtypes = [ctypes.POINTER(LrqDesc)]
        lib.lrq_nf4_weight_size.restype = ctypes.c_size_t
        lib.lrq_quantize_nf4.argtypes = [ctypes.POINTER(LrqDesc), P, P, S, P]
        lib.lrq_quantize_nf4.restype = ctypes.c_int
        lib.lrq_prepared_size.argtypes = [ctypes.POINTER(LrqDesc), ctypes.c_int]
        lib.lrq_prepared_size.restype = ctypes.c_size_t
        lib.lrq_prepare_weights.argtypes = [ctypes.POINTER(LrqDesc), ctypes.c_int, P, P, P, S, P]
        lib.lrq_prepare_weights.restype = ctypes.c_int
        lib.lrq_forward_prepared.argtypes = [ctypes.POINTER(LrqDesc), P, P, P, P, S, P, PP, PP, P, P,
                                             ctypes.POINTER(LrqKvCache), P, S, P]
        lib.lrq_forward_prepared.restype = ctypes.c_int
        lib.lrq_backward_prepared.argtypes = [ctypes.POINTER(LrqDesc), P, P, P, P, S, P, PP, PP, P, P, P, P, PP,
                                              PP, P, S, P]
        lib.lrq_backward_prepared.restype = ctypes.c_int
        lib.lrq_forward_noalloc.argtypes = [ctypes.POINTER(LrqDesc), P, P, P, P, S, P, PP, PP, P, P,
                                            ctypes.POINTER(LrqKvCache), P]
        lib.lrq_forward_noalloc.restype = ctypes.c_int
        lib.lrq_mlp_workspace_size.argtypes = [ctypes.POINTER(LrqMlpDesc)]
        lib.lrq_mlp_workspace_size.restype = ctypes.c_size_t
        lib.lrq_mlp_forward.argtypes = [ctypes.POINTER(LrqMlpDesc), P, P, P, P, PP, PP, P, P, S, P]
        lib.lrq_mlp_forward.restype = ctypes.c_int
        lib.lrq_select_variant.argtypes = [ctypes.POINTER(LrqDesc), ctypes.c_int]
        lib.lrq_select_variant.restype = ctypes.c_int
        lib.lrq_status_string.argtypes = [ctypes.c_int]
        lib.lrq_status_string.restype = ctypes.c_char_p
        lib.lrq_last_error.argtypes = []
        lib.lrq_last_error.restype = ctypes.c_char_p
        lib.lrq_abi_version.argtypes = []
        lib.lrq_abi_version.restype = ctypes.c_int
        lib.lrq_kernel_timing.argtypes = [ctypes.c_int]
        lib.lrq_kernel_timing.restype = ctypes.c_int
        lib.lrq_kernel_time_ms.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                                           ctypes.POINTER(ctypes.c_int)]
        lib.lrq_kernel_time_ms.restype = ctypes.c_int
        _lib = lib
    return _lib


def make_desc(n_tokens, d_model, n_q_heads, n_kv_heads, head_dim, dtype, eps=1e-6, rope_theta=10000.0,
              lora_rank=0, lora_alpha=0.0, lora_targets=0, has_bias=0, variant=LRQ_VARIANT_AUTO,
              lora_dropout=0.0, dropout_offset=0, dropout_seed=0, weight_format=LRQ_WEIGHT_DENSE) -> LrqDesc:
    return LrqDesc(int(n_tokens), int(d_model), int(n_q_heads), int(n_kv_heads), int(head_dim), int(dtype),
                   float(eps), float(rope_theta), int(lora_rank), float(lora_alpha), int(lora_targets),
                   int(has_bias), int(variant), float(lora_dropout), int(dropout_offset) & 0xFFFFFFFF,
                   int(dropout_seed) & 0xFFFFFFFFFFFFFFFF, int(weight_format))


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t or None
    return t.data_ptr()


def _ptr3(ts: Optional[Sequence]):
    if ts is None:
        return None
    vals = [_ptr(t) for t in ts] + [None] * (3 - len(ts))
    return (ctypes.c_void_p * 3)(*vals[:3])


def _stream(stream, tensors) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    for t in tensors:
        if t is not None and not isinstance(t, int) and getattr(t, "is_cuda", False):
            import torch
            return torch.cuda.current_stream(t.device).cuda_stream
    return None


def _ws_bytes(workspace, workspace_bytes) -> int:
    if workspace_bytes is not None:
        return int(workspace_bytes)
    if workspace is None or isinstance(workspace, int):
        return 0
    return workspace.numel() * workspace.element_size()


def _check(st: int):
    if st != LRQ_OK:
        raise LrqError(st, load().lrq_last_error().decode())


def lrq_forward(desc: LrqDesc, x, gamma, w_qkv, bias, lora_a, lora_b, positions, out,
                workspace=None, workspace_bytes: Optional[int] = None, stream=None) -> None:
    lib = load()
    workspace_bytes = _ws_bytes(workspace, workspace_bytes)
    st = lib.lrq_forward(ctypes.byref(desc), _ptr(x), _ptr(gamma), _ptr(w_qkv), _ptr(bias),
                         _ptr3(lora_a), _ptr3(lora_b), _ptr(positions), _ptr(out), _ptr(workspace),
                         int(workspace_bytes), _stream(stream, (x, out)))
    _check(st)


def lrq_forward_kv(desc: LrqDesc, x, gamma, w_qkv, bias, lora_a, lora_b, positions, out,
                   k_cache, v_cache, slots, num_slots: int, workspace=None,
                   workspace_bytes: Optional[int] = None, stream=None) -> None:
    """lrq_forward plus the k and v rows written to k_cache / v_cache at rows ``slots``."""
    lib = load()
    workspace_bytes = _ws_bytes(workspace, workspace_bytes)
    kv = LrqKvCache(_ptr(k_cache), _ptr(v_cache), _ptr(slots), int(num_slots))
    st = lib.lrq_forward_kv(ctypes.byref(desc), _ptr(x), _ptr(gamma), _ptr(w_qkv), _ptr(bias),
                            _ptr3(lora_a), _ptr3(lora_b), _ptr(positions), _ptr(out), ctypes.byref(kv),
                            _ptr(workspace), int(workspace_bytes), _stream(stream, (x, out)))
    _check(st)


def lrq_backward(desc: LrqDesc, x, gamma, w_qkv, bias, lora_a, lora_b, positions, y, dy, dx,
                 d_lora_a, d_lora_b, workspace=None, workspace_bytes: Optional[int] = None, stream=None) -> None:
    lib = load()
    workspace_bytes = _ws_bytes(workspace, workspace_bytes)
    st = lib.lrq_backward(ctypes.byref(desc), _ptr(x), _ptr(gamma), _ptr(w_qkv), _ptr(bias),
                          _ptr3(lora_a), _ptr3(lora_b), _ptr(positions), _ptr(y), _ptr(dy), _ptr(dx),
                          _ptr3(d_lora_a), _ptr3(d_lora_b), _ptr(workspace), int(workspace_bytes),
                          _stream(stream, (x, dx)))
    _check(st)


def lrq_prepared_size(desc: LrqDesc, for_backward: bool = False) -> int:
    return int(load().lrq_prepared_size(ctypes.byref(desc), int(bool(for_backward))))


def lrq_workspace_size_prepared(desc: LrqDesc, for_backward: bool = False) -> int:
    return int(load().lrq_workspace_size_prepared(ctypes.byref(desc), int(bool(for_backward))))


def make_attn_desc(n_seqs, n_q_heads, n_kv_heads, head_dim, max_q_len, ld_q, num_slots, dtype=LRQ_BF16,
                   scale=0.0, causal=1) -> LrqAttnDesc:
    return LrqAttnDesc(int(n_seqs), int(n_q_heads), int(n_kv_heads), int(head_dim), int(dtype), int(max_q_len),
                       int(ld_q), int(num_slots), float(scale), int(causal))


def lrq_attention(desc: LrqAttnDesc, q, k_cache, v_cache, q_indptr, kv_indptr, kv_slots, out,
                  stream=None) -> None:
    lib = load()
    _check(lib.lrq_attention(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(q_indptr),
                             _ptr(kv_indptr), _ptr(kv_slots), _ptr(out), _stream(stream, (q, out))))


def lrq_nf4_weight_size(desc: LrqDesc) -> int:
    return int(load().lrq_nf4_weight_size(ctypes.byref(desc)))


def lrq_quantize_nf4(desc: LrqDesc, w_qkv, w_nf4, nf4_bytes: Optional[int] = None, stream=None) -> None:
    lib = load()
    nbytes = _ws_bytes(w_nf4, nf4_bytes)
    _check(lib.lrq_quantize_nf4(ctypes.byref(desc), _ptr(w_qkv), _ptr(w_nf4), int(nbytes),
                                _stream(stream, (w_qkv,))))


def lrq_prepare_weights(desc: LrqDesc, for_backward: bool, gamma, w_qkv, prepared,
                        prepared_bytes: Optional[int] = None, stream=None) -> None:
    lib = load()
    nbytes = _ws_bytes(prepared, prepared_bytes)
    _check(lib.lrq_prepare_weights(ctypes.byref(desc), int(bool(for_backward)), _ptr(gamma), _ptr(w_qkv),
                                   _ptr(prepared), int(nbytes), _stream(stream, (w_qkv,))))


def lrq_forward_prepared(desc: LrqDesc, x, gamma, w_qkv, prepared, bias, lora_a, lora_b, positions, out,
                         kv: Optional[tuple] = None, workspace=None, workspace_bytes: Optional[int] = None,
                         prepared_bytes: Optional[int] = None, stream=None) -> None:
    """kv: None or (k_cache, v_cache, slots, num_slots)."""
    lib = load()
    kvs = None if kv is None else LrqKvCache(_ptr(kv[0]), _ptr(kv[1]), _ptr(kv[2]), int(kv[3]))
    st = lib.lrq_forward_prepared(ctypes.byref(desc), _ptr(x), _ptr(gamma), _ptr(w_qkv), _ptr(prepared),
                                  int(_ws_bytes(prepared, prepared_bytes)), _ptr(bias), _ptr3(lora_a),
                                  _ptr3(lora_b), _ptr(positions), _ptr(out),
                                  ctypes.byref(kvs) if kvs is not None else None, _ptr(workspace),
                                  int(_ws_bytes(workspace, workspace_bytes)), _stream(stream, (x, out)))
    _check(st)


NOALLOC_SCRATCH_BYTES = 16 << 20  # LRQ_NOALLOC_SCRATCH_BYTES


def lrq_forward_noalloc(desc: LrqDesc, x, gamma, w_qkv, prepared, bias, lora_a, lora_b, positions, out,
                        kv: Optional[tuple] = None, prepared_bytes: Optional[int] = None, stream=None) -> None:
    """lrq_forward_prepared with the library's own scratch (no workspace argument)."""
    lib = load()
    kvs = None if kv is None else LrqKvCache(_ptr(kv[0]), _ptr(kv[1]), _ptr(kv[2]), int(kv[3]))
    st = lib.lrq_forward_noalloc(ctypes.byref(desc), _ptr(x), _ptr(gamma), _ptr(w_qkv), _ptr(prepared),
                                 int(_ws_bytes(prepared, prepared_bytes)), _ptr(bias), _ptr3(lora_a),
                                 _ptr3(lora_b), _ptr(positions), _ptr(out),
                                 ctypes.byref(kvs) if kvs is not None else None, _stream(stream, (x, out)))
    _check(st)


def lrq_backward_prepared(desc: LrqDesc, x, gamma, w_qkv, prepared, bias, lora_a, lora_b, positions, y, dy, dx,
                          d_lora_a, d_lora_b, workspace=None, workspace_bytes: Optional[int] = None,
                          prepared_bytes: Optional[int] = None, stream=None) -> None:
    lib = load()
    st = lib.lrq_backward_prepared(ctypes.byref(desc), _ptr(x), _ptr(gamma), _ptr(w_qkv), _ptr(prepared),
                                   int(_ws_bytes(prepared, prepared_bytes)), _ptr(bias), _ptr3(lora_a),
                                   _ptr3(lora_b), _ptr(positions), _ptr(y), _ptr(dy), _ptr(dx), _ptr3(d_lora_a),
                                   _ptr3(d_lora_b), _ptr(workspace), int(_ws_bytes(workspace, workspace_bytes)),
                                   _stream(stream, (x, dx)))
    _check(st)


def lrq_workspace_size(desc: LrqDesc, for_backward: bool = False) -> int:
    return int(load().lrq_workspace_size(ctypes.byref(desc), int(bool(for_backward))))


def lrq_select_variant(desc: LrqDesc, for_backward: bool = False) -> int:
    return int(load().lrq_select_variant(ctypes.byref(desc), int(bool(for_backward))))


def lrq_status_string(status: int) -> str:
    return load().lrq_status_string(int(status)).decode()


def lrq_last_error() -> str:
    return load().lrq_last_error().decode()


def lrq_abi_version() -> int:
    return int(load().lrq_abi_version())


def lrq_kernel_timing(enable: bool) -> None:
    _check(load().lrq_kernel_timing(1 if enable else 0))


def lrq_kernel_time_ms(for_backward: bool = False):
    """(mean milliseconds, number of calls) of the dominant kernel since timing was enabled."""
    ms, n = ctypes.c_double(0.0), ctypes.c_int(0)
    _check(load().lrq_kernel_time_ms(1 if for_backward else 0, ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def make_mlp_desc(n_tokens, d_model, d_ff, dtype=LRQ_BF16, lora_rank=0, lora_alpha=0.0, lora_targets=0) -> LrqMlpDesc:
    return LrqMlpDesc(int(n_tokens), int(d_model), int(d_ff), int(dtype), int(lora_rank), float(lora_alpha),
                      int(lora_targets))


def lrq_mlp_workspace_size(desc: LrqMlpDesc) -> int:
    return int(load().lrq_mlp_workspace_size(ctypes.byref(desc)))


def lrq_mlp_forward(desc: LrqMlpDesc, h, w_gate, w_up, w_down, lora_a, lora_b, out, workspace=None,
                    workspace_bytes: Optional[int] = None, stream=None) -> None:
    lib = load()
    st = lib.lrq_mlp_forward(ctypes.byref(desc), _ptr(h), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr3(lora_a),
                             _ptr3(lora_b), _ptr(out), _ptr(workspace), int(_ws_bytes(workspace, workspace_bytes)),
                             _stream(stream, (h, out)))
    _check(st)
