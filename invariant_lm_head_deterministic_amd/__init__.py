"""Strict-path selected-token logprob on MI355X (gfx950): LM head -> log-softmax -> gather.

``Logprob`` marshals torch tensors (device memory, the current stream) into the C ABI of
``librlk_logprob.so``; all arithmetic runs in the library's HIP kernels. If the library is not
built, every call raises: there is no CPU or eager fallback.
"""

from __future__ import annotations

import ctypes
from typing import Sequence

import numpy as np

from . import _lib
from ._lib import (  # noqa: F401
    RLK_BWD_ACCUMULATE,
    RLK_DEVICE_STATUS_BAD_TARGET,
    RLK_FLAG_ENTROPY,
    RLK_FLAG_PORTABLE_EXP,
    RLK_FLAG_RMSNORM,
    RlkError,
    rlk_build_fingerprint,
    rlk_layout_check,
    rlk_logprob_config_t,
    rlk_logprob_contract_id,
    rlk_logprob_backward,
    rlk_logprob_backward_merge,
    rlk_logprob_backward_merge_workspace_size,
    rlk_logprob_backward_partials,
    rlk_logprob_backward_partials_workspace_size,
    rlk_logprob_backward_workspace_size,
    rlk_logprob_create,
    rlk_logprob_destroy,
    rlk_logprob_device_status,
    rlk_logprob_forward,
    rlk_logprob_forward_noalloc,
    rlk_logprob_forward_timed,
    rlk_logprob_merge,
    rlk_logprob_partials,
    rlk_logprob_partials_workspace_size,
    rlk_logprob_workspace_size,
    rlk_layout_desc_t,
    rlk_segment_record_t,
    rlk_status_string,
)

__all__ = ["Logprob", "make_config", "make_layout", "require_library", "RlkError"]


def require_library():
    """Load the HIP library or raise."""
    return _lib.load()


def inv_temperature(tau: float) -> float:
    """fl32(1/tau): the reciprocal is formed in float64 on the host and rounded once."""
    return float(np.float32(1.0 / float(tau)))


def make_config(hidden_size: int, vocab_size: int, vocab_segments: int = 4,
                temperature: float = 1.0, rmsnorm: bool = False, rms_eps: float = 1e-6,
                entropy: bool = False, portable: bool = False) -> rlk_logprob_config_t:
    c = rlk_logprob_config_t()
    c.hidden_size = hidden_size
    c.vocab_segments = vocab_segments
    c.vocab_size = vocab_size
    c.inv_temperature = inv_temperature(temperature)
    c.rms_eps = rms_eps if rmsnorm else 0.0
    c.flags = ((RLK_FLAG_RMSNORM if rmsnorm else 0) | (RLK_FLAG_ENTROPY if entropy else 0)
               | (RLK_FLAG_PORTABLE_EXP if portable else 0))
    c.reserved = 0
    return c


def make_layout(num_rows: int, batch_sizes: Sequence[int] | None = None, row_chunk: int = 0,
                vocab_shards: int = 1, token_tile: int = 0):
    """A layout descriptor plus the host array its pointer refers to (keep both alive)."""
    l = rlk_layout_desc_t()
    l.num_rows = num_rows
    l.vocab_shards = vocab_shards
    l.row_chunk = row_chunk
    l.token_tile = token_tile
    l.reserved = 0
    keep = None
    if batch_sizes is not None and len(batch_sizes) > 1:
        offs = [0]
        for s in batch_sizes:
            offs.append(offs[-1] + int(s))
        keep = (ctypes.c_int64 * len(offs))(*offs)
        l.num_batches = len(batch_sizes)
        l.batch_offsets = ctypes.cast(keep, ctypes.POINTER(ctypes.c_int64))
    else:
        l.num_batches = 1
        l.batch_offsets = None
    return l, keep


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _on_stream(s, dev, *tensors) -> None:
    """Tensors the binding allocated from torch's caching allocator on the current stream but
    handed to work enqueued on another stream `s`: record that use, so that the allocator does not
    hand their memory out again before the work on `s` is done."""
    import torch

    if s == torch.cuda.current_stream(dev):
        return
    for t in tensors:
        if t is not None:
            t.record_stream(s)


class Logprob:
    """A handle of the C library bound to one device and one numeric configuration."""

    def __init__(self, hidden_size: int, vocab_size: int, vocab_segments: int = 4,
                 temperature: float = 1.0, rmsnorm: bool = False, rms_eps: float = 1e-6,
                 entropy: bool = False, device: int = 0, portable: bool = False):
        self.config = make_config(hidden_size, vocab_size, vocab_segments, temperature, rmsnorm,
                                  rms_eps, entropy, portable)
        self.device = device
        self.entropy = entropy
        self.rmsnorm = rmsnorm
        self.handle = rlk_logprob_create(self.config, device)

    def __del__(self):
        h = getattr(self, "handle", None)
        if h:
            try:
                rlk_logprob_destroy(h)
            except Exception:
                pass
            self.handle = None

    @property
    def contract_id(self) -> str:
        return rlk_logprob_contract_id(self.handle)

    def workspace_size(self, num_rows: int, **layout_kw) -> int:
        layout, _keep = make_layout(num_rows, **layout_kw)
        return rlk_logprob_workspace_size(self.config, layout)

    def _check(self, t, dtype, name: str, shape=None):
        """Device, layout, dtype and shape of a tensor handed to the library: the C ABI takes
        bare pointers, so a wrong shape here would become an out-of-bounds access there."""
        import torch

        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.device.type != "cuda" or t.device.index != self.device:
            raise ValueError(f"{name} must be on cuda:{self.device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dtype not in dtype:
            raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtype}")
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        return torch

    def _targets(self, targets):
        import torch

        self._check(targets, (torch.int32,), "targets")
        if targets.dim() != 1:
            raise ValueError("targets must be 1-D [T]")
        return targets.shape[0]

    def _gamma(self, gamma):
        import torch

        if gamma is not None:
            self._check(gamma, (torch.bfloat16, torch.int16, torch.uint16), "gamma",
                        (self.config.hidden_size,))

    def forward(self, hidden, W, targets, *, batch_sizes=None, row_chunk: int = 0,
                vocab_shards: int = 1, token_tile: int = 0, gamma=None, workspace=None,
                out=None, stream=None) -> dict:
        """Selected-token logprob of every row. hidden [T,H] and W [V,H] bf16 (or int16 bit
        views), targets int32 [T] (negative = padded). Returns {"logp", "lse"[, "entropy"]}
        fp32 [T] on the device, enqueued on ``stream`` (default: torch's current stream)."""
        import torch

        bf = (torch.bfloat16, torch.int16, torch.uint16)
        H = self.config.hidden_size
        T = self._targets(targets)
        self._check(hidden, bf, "hidden", (T, H))
        self._check(W, bf, "W", (self.config.vocab_size, H))
        self._gamma(gamma)
        layout, keep = make_layout(T, batch_sizes, row_chunk, vocab_shards, token_tile)
        need = rlk_logprob_workspace_size(self.config, layout)
        dev = torch.device("cuda", self.device)
        if workspace is not None:
            self._check(workspace, (torch.uint8, torch.int8), "workspace")
        if workspace is None or workspace.numel() < need:
            workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        if out is None:
            out = {"logp": torch.empty(T, dtype=torch.float32, device=dev),
                   "lse": torch.empty(T, dtype=torch.float32, device=dev)}
            if self.entropy:
                out["entropy"] = torch.empty(T, dtype=torch.float32, device=dev)
        else:
            for k in ("logp", "lse") + (("entropy",) if self.entropy else ()):
                self._check(out[k], (torch.float32,), f"out[{k!r}]", (T,))
        s = stream if stream is not None else torch.cuda.current_stream(dev)
        rlk_logprob_forward(self.handle, hidden.data_ptr(), W.data_ptr(), targets.data_ptr(),
                            layout, _ptr(gamma), out["logp"].data_ptr(), out["lse"].data_ptr(),
                            _ptr(out.get("entropy")), workspace.data_ptr(),
                            workspace.numel() * workspace.element_size(), s.cuda_stream)
        _on_stream(s, dev, workspace, *out.values())
        del keep
        res = dict(out)  # the caller's dict is left as it was given
        res["_workspace"] = workspace
        return res

    def device_status(self, workspace, stream=None) -> int:
        import torch

        self._check(workspace, (torch.uint8, torch.int8), "workspace")
        s = stream if stream is not None else torch.cuda.current_stream(
            torch.device("cuda", self.device))
        return rlk_logprob_device_status(self.handle, workspace.data_ptr(), s.cuda_stream)

    def partials(self, hidden, W_shard, vocab_begin: int, vocab_end: int, targets, *, gamma=None,
                 records=None, stream=None):
        """One vocab shard's per-segment records, shape [n_local_segments, T, 4] fp32."""
        import torch

        bf = (torch.bfloat16, torch.int16, torch.uint16)
        H = self.config.hidden_size
        T = self._targets(targets)
        dev = torch.device("cuda", self.device)
        # validates the range (segment boundaries) before any shape is derived from it
        need = rlk_logprob_partials_workspace_size(self.config, T, vocab_begin, vocab_end)
        self._check(hidden, bf, "hidden", (T, H))
        self._check(W_shard, bf, "W_shard", (vocab_end - vocab_begin, H))
        self._gamma(gamma)
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        seg_len = self.config.vocab_size // self.config.vocab_segments
        nloc = (vocab_end - vocab_begin) // seg_len
        if records is None:
            records = torch.empty((nloc, T, 4), dtype=torch.float32, device=dev)
        else:
            self._check(records, (torch.float32,), "records", (nloc, T, 4))
        s = stream if stream is not None else torch.cuda.current_stream(dev)
        rlk_logprob_partials(self.handle, hidden.data_ptr(), W_shard.data_ptr(), vocab_begin,
                             vocab_end, targets.data_ptr(), T, _ptr(gamma), records.data_ptr(),
                             ws.data_ptr(), ws.numel(), s.cuda_stream)
        _on_stream(s, dev, ws, records)
        return records

    def backward(self, hidden, W, targets, lse, grad_logp, *, entropy=None, grad_entropy=None,
                 gamma=None, want_hidden: bool = True, want_W: bool = True,
                 want_gamma: bool | None = None, grad_W=None, grad_gamma=None,
                 accumulate: bool = False, row_chunk: int = 0, workspace=None,
                 stream=None) -> dict:
        """Gradients of sum_t grad_logp[t] logp[t] (+ grad_entropy[t] entropy[t]) with respect
        to the hidden rows ("grad_hidden", fp32 [T, H]; through the RMSNorm when the handle has
        one), W ("grad_W", fp32 [V, H]) and the RMSNorm's gamma ("grad_gamma", fp32 [H]).
        lse (and entropy) are the forward's outputs for these rows. grad_W / grad_gamma may be
        given to write into; with accumulate=True their chains continue from their contents."""
        import torch

        bf = (torch.bfloat16, torch.int16, torch.uint16)
        H = self.config.hidden_size
        V = self.config.vocab_size
        T = self._targets(targets)
        self._check(hidden, bf, "hidden", (T, H))
        self._check(W, bf, "W", (V, H))
        self._check(lse, (torch.float32,), "lse", (T,))
        self._check(grad_logp, (torch.float32,), "grad_logp", (T,))
        if grad_entropy is not None:
            self._check(grad_entropy, (torch.float32,), "grad_entropy", (T,))
            if entropy is None:
                raise ValueError("grad_entropy needs the forward's entropy")
        if entropy is not None:
            self._check(entropy, (torch.float32,), "entropy", (T,))
        self._gamma(gamma)
        if want_gamma is None:
            want_gamma = self.rmsnorm
        dev = torch.device("cuda", self.device)
        need = rlk_logprob_backward_workspace_size(self.config, T, row_chunk)
        if workspace is not None:
            self._check(workspace, (torch.uint8, torch.int8), "workspace")
        if workspace is None or workspace.numel() < need:
            workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        out = {}
        if want_hidden:
            out["grad_hidden"] = torch.empty((T, H), dtype=torch.float32, device=dev)
        if want_W:
            if grad_W is None:
                if accumulate:
                    raise ValueError("accumulate=True needs grad_W")
                grad_W = torch.empty((V, H), dtype=torch.float32, device=dev)
            else:
                self._check(grad_W, (torch.float32,), "grad_W", (V, H))
            out["grad_W"] = grad_W
        if want_gamma:
            if grad_gamma is None:
                if accumulate:
                    raise ValueError("accumulate=True needs grad_gamma")
                grad_gamma = torch.empty((H,), dtype=torch.float32, device=dev)
            else:
                self._check(grad_gamma, (torch.float32,), "grad_gamma", (H,))
            out["grad_gamma"] = grad_gamma
        s = stream if stream is not None else torch.cuda.current_stream(dev)
        rlk_logprob_backward(self.handle, hidden.data_ptr(), W.data_ptr(), targets.data_ptr(), T,
                             _ptr(gamma), lse.data_ptr(), _ptr(entropy), grad_logp.data_ptr(),
                             _ptr(grad_entropy), _ptr(out.get("grad_hidden")),
                             _ptr(out.get("grad_W")), _ptr(out.get("grad_gamma")),
                             RLK_BWD_ACCUMULATE if accumulate else 0, row_chunk,
                             workspace.data_ptr(), workspace.numel(), s.cuda_stream)
        _on_stream(s, dev, workspace, *out.values())
        out["_workspace"] = workspace
        return out

    def backward_partials(self, hidden, W_shard, vocab_begin: int, vocab_end: int, targets, lse,
                          grad_logp, *, entropy=None, grad_entropy=None, gamma=None,
                          want_W: bool = True, grad_W_shard=None, accumulate: bool = False,
                          row_chunk: int = 0, stream=None) -> dict:
        """One vocab shard's backward: "dh_parts" fp32 [segments of the shard, T, H] and
        "grad_W_shard" fp32 [vocab_end - vocab_begin, H]."""
        import torch

        bf = (torch.bfloat16, torch.int16, torch.uint16)
        H = self.config.hidden_size
        T = self._targets(targets)
        # validates the range (segment boundaries) before any shape is derived from it
        need = rlk_logprob_backward_partials_workspace_size(self.config, T, vocab_begin,
                                                            vocab_end, row_chunk)
        self._check(hidden, bf, "hidden", (T, H))
        self._check(W_shard, bf, "W_shard", (vocab_end - vocab_begin, H))
        self._check(lse, (torch.float32,), "lse", (T,))
        self._check(grad_logp, (torch.float32,), "grad_logp", (T,))
        if grad_entropy is not None:
            self._check(grad_entropy, (torch.float32,), "grad_entropy", (T,))
            if entropy is None:
                raise ValueError("grad_entropy needs the forward's entropy")
        if entropy is not None:
            self._check(entropy, (torch.float32,), "entropy", (T,))
        self._gamma(gamma)
        dev = torch.device("cuda", self.device)
        seg_len = self.config.vocab_size // self.config.vocab_segments
        nloc = (vocab_end - vocab_begin) // seg_len
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        out = {"dh_parts": torch.empty((nloc, T, H), dtype=torch.float32, device=dev)}
        if want_W:
            if grad_W_shard is None:
                if accumulate:
                    raise ValueError("accumulate=True needs grad_W_shard")
                grad_W_shard = torch.empty((vocab_end - vocab_begin, H), dtype=torch.float32,
                                           device=dev)
            else:
                self._check(grad_W_shard, (torch.float32,), "grad_W_shard",
                            (vocab_end - vocab_begin, H))
            out["grad_W_shard"] = grad_W_shard
        s = stream if stream is not None else torch.cuda.current_stream(dev)
        rlk_logprob_backward_partials(self.handle, hidden.data_ptr(), W_shard.data_ptr(),
                                      vocab_begin, vocab_end, targets.data_ptr(), T, _ptr(gamma),
                                      lse.data_ptr(), _ptr(entropy), grad_logp.data_ptr(),
                                      _ptr(grad_entropy), out["dh_parts"].data_ptr(),
                                      _ptr(out.get("grad_W_shard")),
                                      RLK_BWD_ACCUMULATE if accumulate else 0, row_chunk,
                                      ws.data_ptr(), ws.numel(), s.cuda_stream)
        _on_stream(s, dev, ws, *out.values())
        out["_workspace"] = ws
        return out

    def backward_merge(self, dh_parts, *, hidden=None, gamma=None, want_gamma: bool | None = None,
                       grad_gamma=None, accumulate: bool = False, stream=None) -> dict:
        """Merge of every shard's dh partials ([S_c, T, H] fp32) into "grad_hidden" (and
        "grad_gamma" with the RMSNorm, which needs the hidden rows and gamma)."""
        import torch

        H = self.config.hidden_size
        S = self.config.vocab_segments
        self._check(dh_parts, (torch.float32,), "dh_parts")
        if dh_parts.dim() != 3 or dh_parts.shape[0] != S or dh_parts.shape[2] != H:
            raise ValueError(f"dh_parts must be [{S}, T, {H}]")
        T = dh_parts.shape[1]
        if hidden is not None:
            self._check(hidden, (torch.bfloat16, torch.int16, torch.uint16), "hidden", (T, H))
        self._gamma(gamma)
        if want_gamma is None:
            want_gamma = self.rmsnorm
        dev = torch.device("cuda", self.device)
        need = rlk_logprob_backward_merge_workspace_size(self.config, T)
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        out = {"grad_hidden": torch.empty((T, H), dtype=torch.float32, device=dev)}
        if want_gamma:
            if grad_gamma is None:
                if accumulate:
                    raise ValueError("accumulate=True needs grad_gamma")
                grad_gamma = torch.empty((H,), dtype=torch.float32, device=dev)
            else:
                self._check(grad_gamma, (torch.float32,), "grad_gamma", (H,))
            out["grad_gamma"] = grad_gamma
        s = stream if stream is not None else torch.cuda.current_stream(dev)
        rlk_logprob_backward_merge(self.handle, dh_parts.data_ptr(), _ptr(hidden), _ptr(gamma), T,
                                   out["grad_hidden"].data_ptr(), _ptr(out.get("grad_gamma")),
                                   RLK_BWD_ACCUMULATE if accumulate else 0, ws.data_ptr(),
                                   ws.numel(), s.cuda_stream)
        _on_stream(s, dev, ws, *out.values())
        out["_workspace"] = ws
        return out

    def merge(self, records, targets, *, status=None, stream=None) -> dict:
        """Merge the records of all segments ([S_c, T, 4] fp32) into logp, lse[, entropy]."""
        import torch

        T = self._targets(targets)
        self._check(records, (torch.float32,), "records", (self.config.vocab_segments, T, 4))
        if status is not None:
            self._check(status, (torch.int32, torch.uint32), "status", (1,))
        dev = torch.device("cuda", self.device)
        out = {"logp": torch.empty(T, dtype=torch.float32, device=dev),
               "lse": torch.empty(T, dtype=torch.float32, device=dev)}
        if self.entropy:
            out["entropy"] = torch.empty(T, dtype=torch.float32, device=dev)
        s = stream if stream is not None else torch.cuda.current_stream(dev)
        rlk_logprob_merge(self.handle, records.data_ptr(), targets.data_ptr(), T,
                          out["logp"].data_ptr(), out["lse"].data_ptr(), _ptr(out.get("entropy")),
                          _ptr(status), s.cuda_stream)
        _on_stream(s, dev, *out.values())
        return out
