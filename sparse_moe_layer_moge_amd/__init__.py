"""Python binding of libmoge.so, the MI355X MoGE expert-layer library.

Argument marshalling only: every function passes device pointers of torch tensors
and the current HIP stream to the C entry point of the same name and raises
MogeError on a non-zero status.  Every step of the layer runs in the library's
HIP kernels; there is no fallback.  Importing this package fails loudly if the
library has not been built (python sparse_moe_layer_moge_amd/build.py).
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoge.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "moge.h")

MOGE_F32, MOGE_BF16 = 0, 1
STATUS = {0: "MOGE_OK", 1: "MOGE_ERR_INVALID_ARG", 2: "MOGE_ERR_UNSUPPORTED",
          3: "MOGE_ERR_WORKSPACE", 4: "MOGE_ERR_HIP"}


class MogeError(RuntimeError):
    def __init__(self, status: int, fn: str, msg: str):
        super().__init__(f"{fn}: {STATUS.get(status, status)}: {msg}")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("N", ctypes.c_int32),
                ("M", ctypes.c_int32), ("k_per_group", ctypes.c_int32),
                ("inter", ctypes.c_int32), ("shared_inter", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]

    @property
    def K(self) -> int:
        return self.M * self.k_per_group

    @property
    def R(self) -> int:
        return self.T * self.K

    def __repr__(self) -> str:
        return ("Dims(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")")


def make_dims(T: int, d: int, N: int, M: int, k_per_group: int, inter: int,
              shared_inter: int, dtype: int) -> Dims:
    return Dims(T, d, N, M, k_per_group, inter, shared_inter, dtype)


_P = ctypes.c_void_p
_SIGS = {
    "moge_abi_version": (ctypes.c_int32, []),
    "moge_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(Dims)]),
    "moge_last_error": (ctypes.c_char_p, []),
    "moge_route": (ctypes.c_int, [ctypes.POINTER(Dims), _P, _P, _P, _P, _P]),
    "moge_permute": (ctypes.c_int, [ctypes.POINTER(Dims), _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                    ctypes.c_size_t, _P]),
    "moge_expert_ffn": (ctypes.c_int, [ctypes.POINTER(Dims), _P, _P, _P, _P, _P, _P, _P,
                                       ctypes.c_size_t, _P]),
    "moge_combine": (ctypes.c_int, [ctypes.POINTER(Dims), _P, _P, _P, _P, _P, _P]),
    "moge_layer_forward": (ctypes.c_int, [ctypes.POINTER(Dims), _P, _P, _P, _P, _P, _P, _P, _P,
                                          _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moge_set_stage_events": (ctypes.c_int, [ctypes.POINTER(_P), ctypes.c_int32]),
    "moge_packed_weights_size": (ctypes.c_size_t, [ctypes.POINTER(Dims)]),
    "moge_pack_weights": (ctypes.c_int, [ctypes.POINTER(Dims), _P, _P, _P, _P, _P, _P, _P,
                                         ctypes.c_size_t, _P]),
    "moge_layer_forward_packed": (ctypes.c_int, [ctypes.POINTER(Dims), _P, _P, _P, _P, _P, _P,
                                                 _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moge_layer_forward_packed_noalloc": (ctypes.c_int, [ctypes.POINTER(Dims), _P, _P, _P, _P,
                                                         _P, _P, _P, _P, _P, _P, _P]),
    "moge_w8_weights_size": (ctypes.c_size_t, [ctypes.POINTER(Dims)]),
    "moge_pack_weights_w8": (ctypes.c_int, [ctypes.POINTER(Dims)] + [_P] * 13
                             + [ctypes.c_size_t, _P]),
    "moge_quantize_weights_w8": (ctypes.c_int, [ctypes.POINTER(Dims), _P, _P, _P, _P, _P, _P, _P,
                                                ctypes.c_size_t, _P]),
    "moge_layer_forward_w8": (ctypes.c_int, [ctypes.POINTER(Dims), _P, _P, _P, _P, _P, _P, _P,
                                             _P, _P, _P, _P, ctypes.c_size_t, _P]),
}
STAGE_EVENTS = 7
STAGE_NAMES = ("router_scores", "route", "permute", "gate_up", "down", "combine")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    # PyTorch-ROCm carries its own HIP runtime under the same soname; loading torch
    # first makes the library bind to that one runtime, so torch's device memory
    # and streams are valid handles for it.
    import torch  # noqa: F401
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python sparse_moe_layer_moge_amd/build.py` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def header_functions(path: str = HEADER):
    """Names of the functions include/moge.h declares."""
    with open(path) as f:
        text = f.read()
    decls = [ln for ln in text.splitlines() if not ln.lstrip().startswith(("*", "/*", "//"))]
    return sorted(set(m for ln in decls for m in re.findall(r"\b(moge_[a-z0-9_]+)\(", ln)))


lib = load_library()


def last_error() -> str:
    return lib.moge_last_error().decode()


def _check(status: int, fn: str) -> None:
    if status != 0:
        raise MogeError(status, fn, last_error())


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors passed to the MoGE library must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to the MoGE library must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def workspace_size(dims: Dims) -> int:
    return int(lib.moge_workspace_size(ctypes.byref(dims)))


def route(dims: Dims, logits, topk_idx, topk_gate, probs=None, stream=None) -> None:
    _check(lib.moge_route(ctypes.byref(dims), _ptr(logits), _ptr(probs), _ptr(topk_idx),
                          _ptr(topk_gate), _stream(stream)), "moge_route")


def permute(dims: Dims, topk_idx, x, counts, offsets, group_counts, sorted_pair, pair_row,
            x_perm, ws, stream=None) -> None:
    _check(lib.moge_permute(ctypes.byref(dims), _ptr(topk_idx), _ptr(x), _ptr(counts),
                            _ptr(offsets), _ptr(group_counts), _ptr(sorted_pair),
                            _ptr(pair_row), _ptr(x_perm), _ptr(ws),
                            ws.numel() * ws.element_size(), _stream(stream)), "moge_permute")


def expert_ffn(dims: Dims, x_perm, offsets, w_gate, w_up, w_down, y_perm, ws,
               stream=None) -> None:
    _check(lib.moge_expert_ffn(ctypes.byref(dims), _ptr(x_perm), _ptr(offsets), _ptr(w_gate),
                               _ptr(w_up), _ptr(w_down), _ptr(y_perm), _ptr(ws),
                               ws.numel() * ws.element_size(), _stream(stream)),
           "moge_expert_ffn")


def combine(dims: Dims, y_perm, pair_row, topk_gate, shared_out, y, stream=None) -> None:
    _check(lib.moge_combine(ctypes.byref(dims), _ptr(y_perm), _ptr(pair_row), _ptr(topk_gate),
                            _ptr(shared_out), _ptr(y), _stream(stream)), "moge_combine")


def layer_forward(dims: Dims, x, w_router, router_bias, w_gate, w_up, w_down, ws_gate, ws_up,
                  ws_down, y, ws, logits_in=None, logits_out=None, topk_idx_out=None,
                  topk_gate_out=None, group_counts_out=None, stream=None) -> None:
    _check(lib.moge_layer_forward(ctypes.byref(dims), _ptr(x), _ptr(w_router), _ptr(router_bias),
                                  _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(ws_gate),
                                  _ptr(ws_up), _ptr(ws_down), _ptr(logits_in), _ptr(y),
                                  _ptr(logits_out), _ptr(topk_idx_out), _ptr(topk_gate_out),
                                  _ptr(group_counts_out), _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream(stream)),
           "moge_layer_forward")


def set_stage_events(events) -> None:
    """events: a sequence of STAGE_EVENTS raw hipEvent_t handles (ints; None skips
    that point), or None to stop recording."""
    if events is None:
        _check(lib.moge_set_stage_events(None, 0), "moge_set_stage_events")
        return
    arr = (_P * len(events))(*events)
    _check(lib.moge_set_stage_events(arr, len(events)), "moge_set_stage_events")


def packed_weights_size(dims: Dims) -> int:
    return int(lib.moge_packed_weights_size(ctypes.byref(dims)))


def pack_weights(dims: Dims, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, packed,
                 stream=None) -> None:
    _check(lib.moge_pack_weights(ctypes.byref(dims), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
                                 _ptr(ws_gate), _ptr(ws_up), _ptr(ws_down), _ptr(packed),
                                 packed.numel() * packed.element_size(), _stream(stream)),
           "moge_pack_weights")


def layer_forward_packed(dims: Dims, x, w_router, router_bias, packed, y, ws, logits_in=None,
                         logits_out=None, topk_idx_out=None, topk_gate_out=None,
                         group_counts_out=None, stream=None) -> None:
    _check(lib.moge_layer_forward_packed(ctypes.byref(dims), _ptr(x), _ptr(w_router),
                                         _ptr(router_bias), _ptr(packed), _ptr(logits_in), _ptr(y),
                                         _ptr(logits_out), _ptr(topk_idx_out),
                                         _ptr(topk_gate_out), _ptr(group_counts_out), _ptr(ws),
                                         ws.numel() * ws.element_size(), _stream(stream)),
           "moge_layer_forward_packed")


NOALLOC_SCRATCH_BYTES = 128 << 20


def layer_forward_packed_noalloc(dims: Dims, x, w_router, router_bias, packed, y,
                                 logits_in=None, logits_out=None, topk_idx_out=None,
                                 topk_gate_out=None, group_counts_out=None, stream=None) -> None:
    _check(lib.moge_layer_forward_packed_noalloc(ctypes.byref(dims), _ptr(x), _ptr(w_router),
                                                 _ptr(router_bias), _ptr(packed),
                                                 _ptr(logits_in), _ptr(y), _ptr(logits_out),
                                                 _ptr(topk_idx_out), _ptr(topk_gate_out),
                                                 _ptr(group_counts_out), _stream(stream)),
           "moge_layer_forward_packed_noalloc")


def w8_weights_size(dims: Dims) -> int:
    return int(lib.moge_w8_weights_size(ctypes.byref(dims)))


def pack_weights_w8(dims: Dims, q_gate, q_up, q_down, s_gate, s_up, s_down, qs_gate, qs_up,
                    qs_down, ss_gate, ss_up, ss_down, w8, stream=None) -> None:
    _check(lib.moge_pack_weights_w8(ctypes.byref(dims), _ptr(q_gate), _ptr(q_up), _ptr(q_down),
                                    _ptr(s_gate), _ptr(s_up), _ptr(s_down), _ptr(qs_gate),
                                    _ptr(qs_up), _ptr(qs_down), _ptr(ss_gate), _ptr(ss_up),
                                    _ptr(ss_down), _ptr(w8), w8.numel() * w8.element_size(),
                                    _stream(stream)),
           "moge_pack_weights_w8")


def quantize_weights_w8(dims: Dims, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, w8,
                        stream=None) -> None:
    _check(lib.moge_quantize_weights_w8(ctypes.byref(dims), _ptr(w_gate), _ptr(w_up),
                                        _ptr(w_down), _ptr(ws_gate), _ptr(ws_up), _ptr(ws_down),
                                        _ptr(w8), w8.numel() * w8.element_size(),
                                        _stream(stream)),
           "moge_quantize_weights_w8")


def layer_forward_w8(dims: Dims, x, w_router, router_bias, w8, y, ws, logits_in=None,
                     logits_out=None, topk_idx_out=None, topk_gate_out=None,
                     group_counts_out=None, stream=None) -> None:
    _check(lib.moge_layer_forward_w8(ctypes.byref(dims), _ptr(x), _ptr(w_router),
                                     _ptr(router_bias), _ptr(w8), _ptr(logits_in), _ptr(y),
                                     _ptr(logits_out), _ptr(topk_idx_out), _ptr(topk_gate_out),
                                     _ptr(group_counts_out), _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(stream)),
           "moge_layer_forward_w8")
