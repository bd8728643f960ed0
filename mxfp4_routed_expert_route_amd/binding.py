"""ctypes binding of libmoe_mxfp4.so (argument marshalling only).

Each function has the name of the C entry point it calls and takes torch
tensors that live on the GPU; it checks dtypes, shapes and contiguity, passes
raw device pointers and the current HIP stream, and raises MoeError on a
non-OK status.  No step of the layer runs here: every one runs in the HIP
library.  If the library is missing, load() raises instead of falling back to
anything else.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_mxfp4.so")

STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARGUMENT", 2: "MOE_ERR_UNSUPPORTED",
          3: "MOE_ERR_MISALIGNED", 4: "MOE_ERR_WORKSPACE_TOO_SMALL", 5: "MOE_ERR_HIP"}

EXPORTS = ("moe_route", "moe_build_bitmatrix", "moe_expert_offsets", "moe_route_and_group",
           "moe_grouped_ffn_mxfp4", "moe_combine", "moe_workspace_bytes", "moe_status_string")


# bf16 buffers may be given as bfloat16 tensors or as int16 tensors of bit patterns
BF16 = (torch.bfloat16, torch.int16)


class MoeError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} returned {STATUS.get(code, code)}")
        self.code = code


_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SIG = {
    "moe_route": [_P, _I64, _I32, _I32, _P, _P, _P],
    "moe_build_bitmatrix": [_P, _I64, _I32, _I32, _P, _P],
    "moe_expert_offsets": [_P, _P, _I64, _I32, _I32, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "moe_route_and_group": [_P, _I64, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t,
                            _P],
    "moe_grouped_ffn_mxfp4": [_P, _I64, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P,
                              ctypes.c_float, _P, _P, ctypes.c_size_t, _P],
    "moe_combine": [_P, _P, _P, _I64, _I32, _I32, _P, _P],
    "moe_forward_mxfp4": [_P, _P, _I64, _I32, _I32, _I32, _I32, _P, _P, _P, _P, ctypes.c_float,
                          _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "moe_forward_mxfp4_noalloc": [_P, _P, _I64, _I32, _I32, _I32, _I32, _P, _P, _P, _P,
                                  ctypes.c_float, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "moe_forward_mxfp4_timed": [_P, _P, _I64, _I32, _I32, _I32, _I32, _P, _P, _P, _P,
                                ctypes.c_float, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                ctypes.c_size_t, _P, _P],
    "moe_read_probe": [_P, ctypes.c_size_t, _P, _P],
    "moe_workspace_bytes": [_I64, _I32, _I32, _I32, _I32],
    "moe_status_string": [ctypes.c_int],
}


def load(path: str = LIB_PATH):
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not found: build it with `python -m "
                           "mxfp4_routed_expert_route_amd.build` (no CPU fallback exists)")
    lib = ctypes.CDLL(path)
    for name, args in _SIG.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.moe_workspace_bytes.restype = ctypes.c_size_t
    lib.moe_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _ptr(t: torch.Tensor | None, dtype=None, name="tensor") -> int | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None:
        ok = t.dtype in dtype if isinstance(dtype, tuple) else t.dtype == dtype
        if not ok:
            raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(fn: str, code: int):
    if code != 0:
        raise MoeError(fn, code)


def moe_workspace_bytes(T: int, E: int, k: int, H: int, I: int) -> int:
    return int(load().moe_workspace_bytes(T, E, k, H, I))


def moe_status_string(code: int) -> str:
    return load().moe_status_string(code).decode()


def moe_route(logits, k: int, topk_ids, topk_weights, stream=None):
    T, E = logits.shape
    _check("moe_route", load().moe_route(
        _ptr(logits, torch.float32, "logits"), T, E, k, _ptr(topk_ids, torch.int32, "topk_ids"),
        _ptr(topk_weights, torch.float32, "topk_weights"), _stream(stream)))


def moe_build_bitmatrix(topk_ids, E: int, bitmatrix, stream=None):
    T, k = topk_ids.shape
    _check("moe_build_bitmatrix", load().moe_build_bitmatrix(
        _ptr(topk_ids, torch.int32, "topk_ids"), T, E, k,
        _ptr(bitmatrix, torch.int32, "bitmatrix"), _stream(stream)))


def moe_expert_offsets(bitmatrix, topk_ids, E: int, counts, offsets, gather, scatter, ws,
                       stream=None):
    T, k = topk_ids.shape
    _check("moe_expert_offsets", load().moe_expert_offsets(
        _ptr(bitmatrix, torch.int32, "bitmatrix"), _ptr(topk_ids, torch.int32, "topk_ids"), T, E, k,
        _ptr(counts, torch.int32, "counts"), _ptr(offsets, torch.int32, "offsets"),
        _ptr(gather, torch.int32, "gather"), _ptr(scatter, torch.int32, "scatter"),
        _ptr(ws, torch.uint8, "ws"), ws.numel() if ws is not None else 0, _stream(stream)))


def moe_route_and_group(logits, k: int, topk_ids, topk_weights, bitmatrix, counts, offsets,
                        gather, scatter, ws, stream=None):
    T, E = logits.shape
    _check("moe_route_and_group", load().moe_route_and_group(
        _ptr(logits, torch.float32, "logits"), T, E, k, _ptr(topk_ids, torch.int32, "topk_ids"),
        _ptr(topk_weights, torch.float32, "topk_weights"), _ptr(bitmatrix, torch.int32, "bitmatrix"),
        _ptr(counts, torch.int32, "counts"), _ptr(offsets, torch.int32, "offsets"),
        _ptr(gather, torch.int32, "gather"), _ptr(scatter, torch.int32, "scatter"),
        _ptr(ws, torch.uint8, "ws"), ws.numel() if ws is not None else 0, _stream(stream)))


def moe_grouped_ffn_mxfp4(x, k: int, w1, w1_scale, w2, w2_scale, counts, offsets, gather,
                          swiglu_limit: float, y_sorted, ws, stream=None):
    T, H = x.shape
    E, two_i, _ = w1.shape
    _check("moe_grouped_ffn_mxfp4", load().moe_grouped_ffn_mxfp4(
        _ptr(x, BF16, "x"), T, H, two_i // 2, E, k, _ptr(w1, torch.uint8, "w1"),
        _ptr(w1_scale, torch.uint8, "w1_scale"), _ptr(w2, torch.uint8, "w2"),
        _ptr(w2_scale, torch.uint8, "w2_scale"), _ptr(counts, torch.int32, "counts"),
        _ptr(offsets, torch.int32, "offsets"), _ptr(gather, torch.int32, "gather"),
        float(swiglu_limit), _ptr(y_sorted, BF16, "y_sorted"), _ptr(ws, torch.uint8, "ws"),
        ws.numel() if ws is not None else 0, _stream(stream)))


def moe_combine(y_sorted, topk_weights, scatter, y, stream=None):
    T, k = topk_weights.shape
    H = y.shape[1]
    _check("moe_combine", load().moe_combine(
        _ptr(y_sorted, BF16, "y_sorted"), _ptr(topk_weights, torch.float32, "topk_weights"),
        _ptr(scatter, torch.int32, "scatter"), T, H, k, _ptr(y, BF16, "y"), _stream(stream)))


def moe_forward_mxfp4(logits, x, k: int, w1, w1_scale, w2, w2_scale, swiglu_limit: float,
                      topk_ids, topk_weights, bitmatrix, counts, offsets, gather, scatter,
                      y_sorted, y, ws, stream=None):
    T, E = logits.shape
    H = x.shape[1]
    two_i = w1.shape[1]
    _check("moe_forward_mxfp4", load().moe_forward_mxfp4(
        _ptr(logits, torch.float32, "logits"), _ptr(x, BF16, "x"), T, H, two_i // 2, E, k,
        _ptr(w1, torch.uint8, "w1"), _ptr(w1_scale, torch.uint8, "w1_scale"),
        _ptr(w2, torch.uint8, "w2"), _ptr(w2_scale, torch.uint8, "w2_scale"),
        float(swiglu_limit), _ptr(topk_ids, torch.int32, "topk_ids"),
        _ptr(topk_weights, torch.float32, "topk_weights"),
        _ptr(bitmatrix, torch.int32, "bitmatrix"), _ptr(counts, torch.int32, "counts"),
        _ptr(offsets, torch.int32, "offsets"), _ptr(gather, torch.int32, "gather"),
        _ptr(scatter, torch.int32, "scatter"), _ptr(y_sorted, BF16, "y_sorted"),
        _ptr(y, BF16, "y"), _ptr(ws, torch.uint8, "ws"), ws.numel() if ws is not None else 0,
        _stream(stream)))


def moe_forward_mxfp4_timed(logits, x, k: int, w1, w1_scale, w2, w2_scale, swiglu_limit: float,
                            topk_ids, topk_weights, bitmatrix, counts, offsets, gather, scatter,
                            y_sorted, y, ws, events, stream=None):
    """moe_forward_mxfp4 plus three HIP events recorded around its W1 and W2
    kernels; `events` holds three hipEvent_t handles (ints) created by the caller."""
    T, E = logits.shape
    H = x.shape[1]
    two_i = w1.shape[1]
    ev = None
    if events is not None:
        if len(events) != 3:
            raise ValueError("events must hold three hipEvent_t handles")
        ev = (ctypes.c_void_p * 3)(*events)
    _check("moe_forward_mxfp4_timed", load().moe_forward_mxfp4_timed(
        _ptr(logits, torch.float32, "logits"), _ptr(x, BF16, "x"), T, H, two_i // 2, E, k,
        _ptr(w1, torch.uint8, "w1"), _ptr(w1_scale, torch.uint8, "w1_scale"),
        _ptr(w2, torch.uint8, "w2"), _ptr(w2_scale, torch.uint8, "w2_scale"),
        float(swiglu_limit), _ptr(topk_ids, torch.int32, "topk_ids"),
        _ptr(topk_weights, torch.float32, "topk_weights"),
        _ptr(bitmatrix, torch.int32, "bitmatrix"), _ptr(counts, torch.int32, "counts"),
        _ptr(offsets, torch.int32, "offsets"), _ptr(gather, torch.int32, "gather"),
        _ptr(scatter, torch.int32, "scatter"), _ptr(y_sorted, BF16, "y_sorted"),
        _ptr(y, BF16, "y"), _ptr(ws, torch.uint8, "ws"), ws.numel() if ws is not None else 0,
        ev, _stream(stream)))


# moe_forward_mxfp4_noalloc's static device scratch (MOE_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 128 << 20


def moe_forward_mxfp4_noalloc(logits, x, k: int, w1, w1_scale, w2, w2_scale,
                              swiglu_limit: float, topk_ids, topk_weights, bitmatrix, counts,
                              offsets, gather, scatter, y_sorted, y, stream=None):
    T, E = logits.shape
    H = x.shape[1]
    two_i = w1.shape[1]
    _check("moe_forward_mxfp4_noalloc", load().moe_forward_mxfp4_noalloc(
        _ptr(logits, torch.float32, "logits"), _ptr(x, BF16, "x"), T, H, two_i // 2, E, k,
        _ptr(w1, torch.uint8, "w1"), _ptr(w1_scale, torch.uint8, "w1_scale"),
        _ptr(w2, torch.uint8, "w2"), _ptr(w2_scale, torch.uint8, "w2_scale"),
        float(swiglu_limit), _ptr(topk_ids, torch.int32, "topk_ids"),
        _ptr(topk_weights, torch.float32, "topk_weights"),
        _ptr(bitmatrix, torch.int32, "bitmatrix"), _ptr(counts, torch.int32, "counts"),
        _ptr(offsets, torch.int32, "offsets"), _ptr(gather, torch.int32, "gather"),
        _ptr(scatter, torch.int32, "scatter"), _ptr(y_sorted, BF16, "y_sorted"),
        _ptr(y, BF16, "y"), _stream(stream)))


READ_PROBE_SINK_WORDS = 8192


def moe_read_probe(buf, sink, stream=None):
    """Streaming read of every byte of `buf` (a contiguous device tensor, 16-byte
    aligned, size a multiple of 16); `sink` is an int32 device tensor of
    READ_PROBE_SINK_WORDS entries that receives the per-workgroup XORs."""
    if not buf.is_contiguous():
        raise ValueError("buf must be contiguous")
    if sink.dtype != torch.int32 or sink.numel() < READ_PROBE_SINK_WORDS:
        raise ValueError(f"sink must be int32 with >= {READ_PROBE_SINK_WORDS} entries")
    _check("moe_read_probe", load().moe_read_probe(
        _ptr(buf, None, "buf"), buf.numel() * buf.element_size(), _ptr(sink, torch.int32, "sink"),
        _stream(stream)))
