"""Python binding of libmoe_decode.so (argument marshalling only).

Every function here forwards to the C entry point of the same name declared
in include/moe.h; all arithmetic runs in the library's HIP kernels.  Tensors
are torch CUDA tensors (used for device memory and streams only); bf16
values travel as int16/uint16 bit patterns.  A missing or unbuilt library
raises immediately: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_decode.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "moe.h")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
MOE_MAX_LAYER_KERNELS = 8
MOE_STREAM_SINK_WORDS = 4096
MOE_NOALLOC_SCRATCH_BYTES = 16 << 20


class MoeError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed: {msg} ({status})")
        self.status = status


class MoeShape(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("ffn", ctypes.c_int32),
                ("n_shared", ctypes.c_int32), ("shared_ffn", ctypes.c_int32)]


class MoeMxMat(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class MoeLayerWeights(ctypes.Structure):
    _fields_ = [("router_w", ctypes.c_void_p), ("gate", MoeMxMat), ("up", MoeMxMat),
                ("down", MoeMxMat), ("s_gate", MoeMxMat), ("s_up", MoeMxMat),
                ("s_down", MoeMxMat)]


_lib = None
_P = ctypes.c_void_p
_SIG = {
    "moe_workspace_size": ([ctypes.POINTER(MoeShape), ctypes.c_int32,
                            ctypes.POINTER(ctypes.c_size_t)]),
    "moe_workspace_init": ([_P, ctypes.c_size_t, _P]),
    "moe_router_topk": ([ctypes.POINTER(MoeShape), _P, _P, ctypes.c_int32, _P, _P, _P, _P,
                         ctypes.c_size_t, _P]),
    "moe_expert_gateup": ([ctypes.POINTER(MoeShape), ctypes.POINTER(MoeLayerWeights), _P, _P,
                           ctypes.c_int32, _P, _P, ctypes.c_size_t, _P]),
    "moe_decode_layer": ([ctypes.POINTER(MoeShape), ctypes.POINTER(MoeLayerWeights), _P, _P,
                          _P, ctypes.c_int32, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_decode_stack": ([ctypes.POINTER(MoeShape), ctypes.POINTER(MoeLayerWeights),
                          ctypes.POINTER(ctypes.c_void_p), ctypes.c_float, ctypes.c_int32, _P,
                          ctypes.c_int32, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_group_by_expert": ([_P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P, _P,
                             ctypes.c_size_t, _P]),
    "moe_decode_layer_timed": ([ctypes.POINTER(MoeShape), ctypes.POINTER(MoeLayerWeights), _P,
                                _P, _P, ctypes.c_int32, _P, _P, _P, ctypes.c_size_t, _P,
                                ctypes.POINTER(ctypes.c_void_p), ctypes.c_int32,
                                ctypes.POINTER(ctypes.c_int32)]),
    "moe_stream_read": ([_P, ctypes.c_size_t, _P, _P]),
    "moe_decode_layer_noalloc": ([ctypes.POINTER(MoeShape), ctypes.POINTER(MoeLayerWeights), _P,
                                  _P, _P, ctypes.c_int32, _P, _P, _P]),
}


def lib():
    """The loaded library (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIG.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def header_functions():
    """Names of the functions declared in include/moe.h."""
    with open(HEADER) as f:
        text = f.read()
    return re.findall(r"^\s*(?:int|const char\*)\s+(moe_\w+)\s*\(", text, re.M)


def _check(fn, rc):
    if rc != MOE_OK:
        raise MoeError(fn, rc, lib().moe_status_string(rc).decode())


def _ptr(t):
    if t is None:
        return None
    return t if isinstance(t, int) else t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def make_shape(H, E, k, F, S=0, Fs=0) -> MoeShape:
    return MoeShape(H, E, k, F, S, Fs if S else 0)


def make_weights(router, gate, up, down, s_gate=None, s_up=None, s_down=None) -> MoeLayerWeights:
    """Each matrix is a (codes, scales) pair of tensors (or raw pointers)."""
    def mat(m):
        return MoeMxMat(_ptr(m[0]), _ptr(m[1])) if m is not None else MoeMxMat(None, None)
    return MoeLayerWeights(_ptr(router), mat(gate), mat(up), mat(down), mat(s_gate),
                           mat(s_up), mat(s_down))


# ------------------------------------------------------------ entry points

def workspace_size(shape: MoeShape, max_tokens: int) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_workspace_size", lib().moe_workspace_size(ctypes.byref(shape), max_tokens,
                                                           ctypes.byref(n)))
    return n.value


def workspace_init(ws, stream=None):
    _check("moe_workspace_init", lib().moe_workspace_init(_ptr(ws), ws.numel() * ws.element_size(),
                                                           _stream(stream)))


def router_topk(shape, x, router_w, n_tokens, topk_idx, topk_w, logits, ws, stream=None):
    _check("moe_router_topk", lib().moe_router_topk(
        ctypes.byref(shape), _ptr(x), _ptr(router_w), n_tokens, _ptr(topk_idx), _ptr(topk_w),
        _ptr(logits), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def expert_gateup(shape, weights, x, topk_idx, n_tokens, act, ws, stream=None):
    _check("moe_expert_gateup", lib().moe_expert_gateup(
        ctypes.byref(shape), ctypes.byref(weights), _ptr(x), _ptr(topk_idx), n_tokens, _ptr(act),
        _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def decode_layer(shape, weights, x, residual, out, n_tokens, topk_idx_out, topk_w_out, ws,
                 stream=None):
    _check("moe_decode_layer", lib().moe_decode_layer(
        ctypes.byref(shape), ctypes.byref(weights), _ptr(x), _ptr(residual), _ptr(out), n_tokens,
        _ptr(topk_idx_out), _ptr(topk_w_out), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream)))


def decode_stack(shape, layers, gammas, eps, hidden, n_tokens, topk_idx_out, hidden_trace, ws,
                 stream=None):
    n = len(layers)
    arr = (MoeLayerWeights * n)(*layers)
    garr = (ctypes.c_void_p * n)(*[_ptr(g) for g in gammas])
    _check("moe_decode_stack", lib().moe_decode_stack(
        ctypes.byref(shape), arr, garr, eps, n, _ptr(hidden), n_tokens, _ptr(topk_idx_out),
        _ptr(hidden_trace), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def group_by_expert(topk_idx, n_tokens, top_k, n_experts, offsets, pairs, ws, stream=None):
    _check("moe_group_by_expert", lib().moe_group_by_expert(
        _ptr(topk_idx), n_tokens, top_k, n_experts, _ptr(offsets), _ptr(pairs), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream)))


def decode_layer_timed(shape, weights, x, residual, out, n_tokens, topk_idx_out, topk_w_out, ws,
                       events, stream=None) -> int:
    """``events``: list of (start, stop) torch.cuda.Event pairs (timing
    enabled, already created); returns the number of kernels launched."""
    n = len(events)
    handles = (ctypes.c_void_p * (2 * n))(*[h for a, b in events for h in (a.cuda_event,
                                                                          b.cuda_event)])
    nk = ctypes.c_int32(0)
    _check("moe_decode_layer_timed", lib().moe_decode_layer_timed(
        ctypes.byref(shape), ctypes.byref(weights), _ptr(x), _ptr(residual), _ptr(out), n_tokens,
        _ptr(topk_idx_out), _ptr(topk_w_out), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream), handles, n, ctypes.byref(nk)))
    return nk.value


def decode_layer_noalloc(shape, weights, x, residual, out, n_tokens, topk_idx_out, topk_w_out,
                         stream=None):
    _check("moe_decode_layer_noalloc", lib().moe_decode_layer_noalloc(
        ctypes.byref(shape), ctypes.byref(weights), _ptr(x), _ptr(residual), _ptr(out), n_tokens,
        _ptr(topk_idx_out), _ptr(topk_w_out), _stream(stream)))


def stream_read(buf, sink, stream=None):
    _check("moe_stream_read", lib().moe_stream_read(
        _ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream(stream)))
