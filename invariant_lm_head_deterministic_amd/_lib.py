"""ctypes binding of ``librlk_logprob.so``: the C entry points under the same names.

Argument marshalling only — every step of the computation runs in the library's HIP kernels.
Pointers are plain integers (device addresses) and streams are hipStream_t integers.
"""

from __future__ import annotations

import ctypes
import os
import re

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "librlk_logprob.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "rlk_logprob.h")

RLK_OK = 0
RLK_ERR_INVALID_ARGUMENT = 1
RLK_ERR_NO_DEVICE = 2
RLK_ERR_UNSUPPORTED_ARCH = 3
RLK_ERR_UNSUPPORTED_SHAPE = 4
RLK_ERR_ALIGNMENT = 5
RLK_ERR_WORKSPACE = 6
RLK_ERR_CONTRACT = 7
RLK_ERR_HIP = 8

RLK_FLAG_RMSNORM = 1
RLK_FLAG_ENTROPY = 2
RLK_FLAG_PORTABLE_EXP = 4
RLK_BWD_ACCUMULATE = 1
RLK_DEVICE_STATUS_BAD_TARGET = 1


class rlk_logprob_config_t(ctypes.Structure):
    _fields_ = [
        ("hidden_size", ctypes.c_int32),
        ("vocab_segments", ctypes.c_int32),
        ("vocab_size", ctypes.c_int64),
        ("inv_temperature", ctypes.c_float),
        ("rms_eps", ctypes.c_float),
        ("flags", ctypes.c_uint32),
        ("reserved", ctypes.c_uint32),
    ]


class rlk_layout_desc_t(ctypes.Structure):
    _fields_ = [
        ("num_rows", ctypes.c_int64),
        ("num_batches", ctypes.c_int32),
        ("vocab_shards", ctypes.c_int32),
        ("batch_offsets", ctypes.POINTER(ctypes.c_int64)),
        ("row_chunk", ctypes.c_int64),
        ("token_tile", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class rlk_segment_record_t(ctypes.Structure):
    _fields_ = [("m", ctypes.c_float), ("s", ctypes.c_float), ("u", ctypes.c_float),
                ("tgt", ctypes.c_float)]


_H = ctypes.c_void_p  # rlk_logprob_t
_P = ctypes.c_void_p  # device pointer
_S = ctypes.c_void_p  # stream
_ST = ctypes.c_int    # rlk_status_t

_SIGS = {
    "rlk_logprob_create": (_ST, [ctypes.POINTER(rlk_logprob_config_t), ctypes.c_int,
                                 ctypes.POINTER(_H)]),
    "rlk_logprob_destroy": (_ST, [_H]),
    "rlk_logprob_workspace_size": (_ST, [ctypes.POINTER(rlk_logprob_config_t),
                                         ctypes.POINTER(rlk_layout_desc_t),
                                         ctypes.POINTER(ctypes.c_size_t)]),
    "rlk_layout_check": (_ST, [ctypes.POINTER(rlk_logprob_config_t),
                               ctypes.POINTER(rlk_layout_desc_t), ctypes.POINTER(ctypes.c_int64)]),
    "rlk_logprob_forward": (_ST, [_H, _P, _P, _P, ctypes.POINTER(rlk_layout_desc_t), _P, _P, _P,
                                  _P, _P, ctypes.c_size_t, _S]),
    "rlk_logprob_forward_timed": (_ST, [_H, _P, _P, _P, ctypes.POINTER(rlk_layout_desc_t), _P, _P,
                                        _P, _P, _P, ctypes.c_size_t, _S,
                                        ctypes.POINTER(ctypes.c_void_p), ctypes.c_int32]),
    "rlk_logprob_forward_noalloc": (_ST, [_H, _P, _P, _P, ctypes.POINTER(rlk_layout_desc_t), _P,
                                          _P, _P, _P, _S]),
    "rlk_logprob_partials_workspace_size": (_ST, [ctypes.POINTER(rlk_logprob_config_t),
                                                  ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                                  ctypes.POINTER(ctypes.c_size_t)]),
    "rlk_logprob_partials": (_ST, [_H, _P, _P, ctypes.c_int64, ctypes.c_int64, _P, ctypes.c_int64,
                                   _P, _P, _P, ctypes.c_size_t, _S]),
    "rlk_logprob_merge": (_ST, [_H, _P, _P, ctypes.c_int64, _P, _P, _P, _P, _S]),
    "rlk_logprob_device_status": (_ST, [_H, _P, _S, ctypes.POINTER(ctypes.c_uint32)]),
    "rlk_logprob_backward_workspace_size": (_ST, [ctypes.POINTER(rlk_logprob_config_t),
                                                  ctypes.c_int64, ctypes.c_int64,
                                                  ctypes.POINTER(ctypes.c_size_t)]),
    "rlk_logprob_backward": (_ST, [_H, _P, _P, _P, ctypes.c_int64, _P, _P, _P, _P, _P, _P, _P, _P,
                                   ctypes.c_uint32, ctypes.c_int64, _P, ctypes.c_size_t, _S]),
    "rlk_logprob_backward_partials_workspace_size": (_ST, [ctypes.POINTER(rlk_logprob_config_t),
                                                           ctypes.c_int64, ctypes.c_int64,
                                                           ctypes.c_int64, ctypes.c_int64,
                                                           ctypes.POINTER(ctypes.c_size_t)]),
    "rlk_logprob_backward_partials": (_ST, [_H, _P, _P, ctypes.c_int64, ctypes.c_int64, _P,
                                            ctypes.c_int64, _P, _P, _P, _P, _P, _P, _P,
                                            ctypes.c_uint32, ctypes.c_int64, _P, ctypes.c_size_t,
                                            _S]),
    "rlk_logprob_backward_merge_workspace_size": (_ST, [ctypes.POINTER(rlk_logprob_config_t),
                                                        ctypes.c_int64,
                                                        ctypes.POINTER(ctypes.c_size_t)]),
    "rlk_logprob_backward_merge": (_ST, [_H, _P, _P, _P, ctypes.c_int64, _P, _P, ctypes.c_uint32,
                                         _P, ctypes.c_size_t, _S]),
    "rlk_logprob_contract_id": (ctypes.c_char_p, [_H]),
    "rlk_build_fingerprint": (ctypes.c_char_p, []),
    "rlk_status_string": (ctypes.c_char_p, [_ST]),
    "rlk_last_error": (ctypes.c_char_p, []),
}

_lib = None


class RlkError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        lib = load()
        msg = lib.rlk_status_string(status).decode()
        detail = lib.rlk_last_error().decode()
        super().__init__(f"{where}: {msg} ({status}): {detail}")


def load():
    """Load the built library; raises if it was not built (there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                           "(run `python -c 'import __graft_entry__ as g; g.build()'`)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def header_functions() -> list[str]:
    """Names of the entry points the public header declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const char\*|rlk_status_t)\s+(rlk_\w+)\s*\(", text, re.M)))


def check(status: int, where: str) -> None:
    if status != RLK_OK:
        raise RlkError(status, where)


# ---- same-name thin wrappers (plain integers for pointers and streams) ----

def rlk_logprob_create(config: rlk_logprob_config_t, device: int) -> int:
    h = _H()
    check(load().rlk_logprob_create(ctypes.byref(config), device, ctypes.byref(h)),
          "rlk_logprob_create")
    return h.value


def rlk_logprob_destroy(handle: int) -> None:
    check(load().rlk_logprob_destroy(handle), "rlk_logprob_destroy")


def rlk_logprob_workspace_size(config: rlk_logprob_config_t, layout: rlk_layout_desc_t) -> int:
    n = ctypes.c_size_t()
    check(load().rlk_logprob_workspace_size(ctypes.byref(config), ctypes.byref(layout),
                                            ctypes.byref(n)), "rlk_logprob_workspace_size")
    return n.value


def rlk_layout_check(config: rlk_logprob_config_t, layout: rlk_layout_desc_t) -> int:
    n = ctypes.c_int64()
    check(load().rlk_layout_check(ctypes.byref(config), ctypes.byref(layout), ctypes.byref(n)),
          "rlk_layout_check")
    return n.value


def rlk_logprob_forward(handle, hidden, W_lm, targets, layout, rms_gamma, logp, lse, entropy,
                        workspace, workspace_bytes, stream) -> None:
    check(load().rlk_logprob_forward(handle, hidden, W_lm, targets, ctypes.byref(layout),
                                     rms_gamma, logp, lse, entropy, workspace, workspace_bytes,
                                     stream), "rlk_logprob_forward")


def rlk_logprob_forward_timed(handle, hidden, W_lm, targets, layout, rms_gamma, logp, lse,
                              entropy, workspace, workspace_bytes, stream, events) -> None:
    """events: a sequence of hipEvent_t integers (2 per LM-head launch to bracket)."""
    arr = (ctypes.c_void_p * max(1, len(events)))(*events)
    check(load().rlk_logprob_forward_timed(handle, hidden, W_lm, targets, ctypes.byref(layout),
                                           rms_gamma, logp, lse, entropy, workspace,
                                           workspace_bytes, stream, arr, len(events)),
          "rlk_logprob_forward_timed")


def rlk_logprob_forward_noalloc(handle, hidden, W_lm, targets, layout, rms_gamma, logp, lse,
                                entropy, stream) -> None:
    check(load().rlk_logprob_forward_noalloc(handle, hidden, W_lm, targets, ctypes.byref(layout),
                                             rms_gamma, logp, lse, entropy, stream),
          "rlk_logprob_forward_noalloc")


def rlk_logprob_partials_workspace_size(config, num_rows, vocab_begin, vocab_end) -> int:
    n = ctypes.c_size_t()
    check(load().rlk_logprob_partials_workspace_size(ctypes.byref(config), num_rows, vocab_begin,
                                                     vocab_end, ctypes.byref(n)),
          "rlk_logprob_partials_workspace_size")
    return n.value


def rlk_logprob_partials(handle, hidden, W_shard, vocab_begin, vocab_end, targets, num_rows,
                         rms_gamma, records, workspace, workspace_bytes, stream) -> None:
    check(load().rlk_logprob_partials(handle, hidden, W_shard, vocab_begin, vocab_end, targets,
                                      num_rows, rms_gamma, records, workspace, workspace_bytes,
                                      stream), "rlk_logprob_partials")


def rlk_logprob_merge(handle, records, targets, num_rows, logp, lse, entropy, status,
                      stream) -> None:
    check(load().rlk_logprob_merge(handle, records, targets, num_rows, logp, lse, entropy, status,
                                   stream), "rlk_logprob_merge")


def rlk_logprob_device_status(handle, workspace, stream) -> int:
    v = ctypes.c_uint32()
    check(load().rlk_logprob_device_status(handle, workspace, stream, ctypes.byref(v)),
          "rlk_logprob_device_status")
    return v.value


def rlk_logprob_backward_workspace_size(config: rlk_logprob_config_t, num_rows: int,
                                        row_chunk: int) -> int:
    n = ctypes.c_size_t()
    check(load().rlk_logprob_backward_workspace_size(ctypes.byref(config), num_rows, row_chunk,
                                                     ctypes.byref(n)),
          "rlk_logprob_backward_workspace_size")
    return n.value


def rlk_logprob_backward(handle, hidden, W_lm, targets, num_rows, rms_gamma, lse, entropy,
                         grad_logp, grad_entropy, grad_hidden, grad_W, grad_gamma, flags,
                         row_chunk, workspace, workspace_bytes, stream) -> None:
    check(load().rlk_logprob_backward(handle, hidden, W_lm, targets, num_rows, rms_gamma, lse,
                                      entropy, grad_logp, grad_entropy, grad_hidden, grad_W,
                                      grad_gamma, flags, row_chunk, workspace, workspace_bytes,
                                      stream), "rlk_logprob_backward")


def rlk_logprob_backward_partials_workspace_size(config: rlk_logprob_config_t, num_rows: int,
                                                 vocab_begin: int, vocab_end: int,
                                                 row_chunk: int) -> int:
    n = ctypes.c_size_t()
    check(load().rlk_logprob_backward_partials_workspace_size(ctypes.byref(config), num_rows,
                                                              vocab_begin, vocab_end, row_chunk,
                                                              ctypes.byref(n)),
          "rlk_logprob_backward_partials_workspace_size")
    return n.value


def rlk_logprob_backward_partials(handle, hidden, W_shard, vocab_begin, vocab_end, targets,
                                  num_rows, rms_gamma, lse, entropy, grad_logp, grad_entropy,
                                  dh_parts, grad_W_shard, flags, row_chunk, workspace,
                                  workspace_bytes, stream) -> None:
    check(load().rlk_logprob_backward_partials(handle, hidden, W_shard, vocab_begin, vocab_end,
                                               targets, num_rows, rms_gamma, lse, entropy,
                                               grad_logp, grad_entropy, dh_parts, grad_W_shard,
                                               flags, row_chunk, workspace, workspace_bytes,
                                               stream), "rlk_logprob_backward_partials")


def rlk_logprob_backward_merge_workspace_size(config: rlk_logprob_config_t, num_rows: int) -> int:
    n = ctypes.c_size_t()
    check(load().rlk_logprob_backward_merge_workspace_size(ctypes.byref(config), num_rows,
                                                           ctypes.byref(n)),
          "rlk_logprob_backward_merge_workspace_size")
    return n.value


def rlk_logprob_backward_merge(handle, dh_parts, hidden, rms_gamma, num_rows, grad_hidden,
                               grad_gamma, flags, workspace, workspace_bytes, stream) -> None:
    check(load().rlk_logprob_backward_merge(handle, dh_parts, hidden, rms_gamma, num_rows,
                                            grad_hidden, grad_gamma, flags, workspace,
                                            workspace_bytes, stream),
          "rlk_logprob_backward_merge")


def rlk_logprob_contract_id(handle) -> str:
    return load().rlk_logprob_contract_id(handle).decode()


def rlk_build_fingerprint() -> str:
    return load().rlk_build_fingerprint().decode()


def rlk_status_string(status: int) -> str:
    return load().rlk_status_string(status).decode()


def rlk_last_error() -> str:
    return load().rlk_last_error().decode()
