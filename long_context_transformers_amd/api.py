"""Thin Python binding of libringattn with the C ABI's names.

Argument marshalling only: tensors become device pointers, streams become
hipStream_t handles, structs are filled; every step of the computation runs
in the library's HIP kernels.  PyTorch is used for device memory and streams.
"""
from __future__ import annotations

import ctypes
import dataclasses
from typing import List, Optional

from . import _lib as L

c_vp_t = ctypes.c_void_p
from ._lib import (RA_BF16, RA_F32, RA_MASK_NONE, RA_MASK_CAUSAL, RA_LAYOUT_CONTIGUOUS,
                   RA_LAYOUT_STRIPED, RA_LAYOUT_ZIGZAG, RA_BLK_SKIP, RA_BLK_FULL, RA_BLK_TRI_INCL,
                   RA_BLK_TRI_STRICT, RA_BLK_BAND, RA_BLK_QUADRANTS, RA_FLAG_ELIDE_SKIPPED_COPIES,
                   RA_FLAG_SERIALIZE, RA_COPY_NONE, RA_COPY_DMA_ENGINES, RA_COPY_FALLBACK,
                   RingAttnError)


@dataclasses.dataclass
class Dims:
    batch: int
    heads_q: int
    heads_kv: int
    head_dim: int
    block_len: int
    dtype: int = RA_BF16
    scale: float = 0.0

    def c(self) -> L.RaDims:
        return L.RaDims(self.batch, self.heads_q, self.heads_kv, self.head_dim,
                        self.block_len, self.dtype, self.scale)


@dataclasses.dataclass
class RingCfg:
    dims: Dims
    n_hosts: int
    host_begin: int
    host_end: int
    layout: int = RA_LAYOUT_CONTIGUOUS
    mask: int = RA_MASK_NONE
    flags: int = 0
    debug_copy_delay_us: int = 0
    step_events: Optional[list] = None   # 2 * n_hosts torch.cuda.Event (created with timing)

    def c(self) -> L.RaRingCfg:
        ev = None
        if self.step_events is not None:
            if len(self.step_events) != 2 * self.n_hosts:
                raise ValueError("step_events needs 2 * n_hosts events")
            for e in self.step_events:
                if getattr(e, "cuda_event", 0) == 0:
                    e.record()   # torch creates the HIP event lazily
            arr = (c_vp_t * len(self.step_events))(*[e.cuda_event for e in self.step_events])
            self._keep = arr
            ev = ctypes.cast(arr, ctypes.POINTER(c_vp_t))
        return L.RaRingCfg(self.dims.c(), self.n_hosts, self.host_begin, self.host_end,
                           self.layout, self.mask, self.flags, self.debug_copy_delay_us, ev)


def _ptr(t) -> Optional[int]:
    """Device address of a tensor (None stays NULL)."""
    if t is None:
        return None
    if hasattr(t, "data_ptr"):
        if not t.is_contiguous():
            raise ValueError("tensors passed to libringattn must be contiguous")
        return t.data_ptr()
    return int(t)


def _stream(s) -> Optional[int]:
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if hasattr(s, "cuda_stream"):
        return s.cuda_stream
    return int(s)


def version() -> int:
    return int(L.load().ra_version())


def token_index(layout: int, n_hosts: int, block_len: int, host: int, r: int) -> int:
    return int(L.load().ra_token_index(layout, n_hosts, block_len, host, r))


def block_class_of(mask: int, q_offset: int, kv_offset: int, stride: int, block_len: int) -> int:
    return int(L.load().ra_block_class_of(mask, q_offset, kv_offset, stride, block_len))


def schedule(n_hosts: int, host: int, block_len: int, layout: int, mask: int) -> List[dict]:
    out = (L.RaStep * n_hosts)()
    L.check(L.load().ra_schedule(n_hosts, host, block_len, layout, mask, out), "ra_schedule")
    return [dict(step=o.step, src=o.src, cls=o.cls, q_offset=o.q_offset,
                 kv_offset=o.kv_offset, stride=o.stride) for o in out]


def state_init(dims: Dims, m, l, O, stream=None):
    d = dims.c()
    L.check(L.load().ra_state_init(ctypes.byref(d), _ptr(m), _ptr(l), _ptr(O), _stream(stream)),
            "ra_state_init")


def block_fwd(dims: Dims, q, k, v, mask: int, q_offset: int, kv_offset: int, stride: int,
              m, l, O, stream=None):
    d = dims.c()
    L.check(L.load().ra_block_fwd(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), mask, q_offset,
                                  kv_offset, stride, _ptr(m), _ptr(l), _ptr(O), _stream(stream)),
            "ra_block_fwd")


def merge_lse(dims: Dims, O_a, lse_a, O_b, lse_b, O_out, lse_out, stream=None):
    d = dims.c()
    L.check(L.load().ra_merge_lse(ctypes.byref(d), _ptr(O_a), _ptr(lse_a), _ptr(O_b), _ptr(lse_b),
                                  _ptr(O_out), _ptr(lse_out), _stream(stream)), "ra_merge_lse")


def finalize(dims: Dims, m, l, O, O_out, lse, stream=None):
    d = dims.c()
    L.check(L.load().ra_finalize(ctypes.byref(d), _ptr(m), _ptr(l), _ptr(O), _ptr(O_out), _ptr(lse),
                                 _stream(stream)), "ra_finalize")


def bwd_preprocess(dims: Dims, O, dO, D, stream=None):
    d = dims.c()
    L.check(L.load().ra_bwd_preprocess(ctypes.byref(d), _ptr(O), _ptr(dO), _ptr(D), _stream(stream)),
            "ra_bwd_preprocess")


def block_bwd(dims: Dims, q, k, v, dO, lse, D, mask: int, q_offset: int, kv_offset: int,
              stride: int, dQ, dK, dV, stream=None):
    d = dims.c()
    L.check(L.load().ra_block_bwd(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(dO), _ptr(lse),
                                  _ptr(D), mask, q_offset, kv_offset, stride, _ptr(dQ), _ptr(dK),
                                  _ptr(dV), _stream(stream)), "ra_block_bwd")


def layout_permute(dims: Dims, heads: int, n_hosts: int, layout: int, to_host_major: bool, src, dst,
                   stream=None):
    d = dims.c()
    L.check(L.load().ra_layout_permute(ctypes.byref(d), heads, n_hosts, layout, int(bool(to_host_major)),
                                       _ptr(src), _ptr(dst), _stream(stream)), "ra_layout_permute")


def mask_tile(q_offset: int, kv_offset: int, stride: int, rows: int, cols: int, out, stream=None):
    L.check(L.load().ra_mask_tile(q_offset, kv_offset, stride, rows, cols, _ptr(out), _stream(stream)),
            "ra_mask_tile")


def ring_workspace_size(cfg: RingCfg, is_bwd: bool = False) -> int:
    c = cfg.c()
    n = ctypes.c_size_t(0)
    L.check(L.load().ra_ring_workspace_size(ctypes.byref(c), int(bool(is_bwd)), ctypes.byref(n)),
            "ra_ring_workspace_size")
    return int(n.value)


def _stats(s: L.RaRingStats) -> dict:
    return {f: getattr(s, f) for f, _ in L.RaRingStats._fields_}


def ring_fwd(cfg: RingCfg, q, k, v, O, lse, workspace, compute_stream=None, comm_stream=None) -> dict:
    c = cfg.c()
    st = L.RaRingStats()
    nbytes = workspace.numel() * workspace.element_size()
    cs = _stream(compute_stream)
    ms = _stream(comm_stream) if comm_stream is not None else cs
    L.check(L.load().ra_ring_fwd(ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v), _ptr(O), _ptr(lse),
                                 _ptr(workspace), nbytes, cs, ms, ctypes.byref(st)), "ra_ring_fwd")
    return _stats(st)


def ring_bwd(cfg: RingCfg, q, k, v, O, lse, dO, dQ, dK, dV, workspace, compute_stream=None,
             comm_stream=None) -> dict:
    c = cfg.c()
    st = L.RaRingStats()
    nbytes = workspace.numel() * workspace.element_size()
    cs = _stream(compute_stream)
    ms = _stream(comm_stream) if comm_stream is not None else cs
    L.check(L.load().ra_ring_bwd(ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v), _ptr(O), _ptr(lse),
                                 _ptr(dO), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(workspace), nbytes,
                                 cs, ms, ctypes.byref(st)), "ra_ring_bwd")
    return _stats(st)


def decode_workspace_size(dims: Dims, n_hosts: int) -> int:
    d = dims.c()
    n = ctypes.c_size_t(0)
    L.check(L.load().ra_decode_workspace_size(ctypes.byref(d), n_hosts, ctypes.byref(n)),
            "ra_decode_workspace_size")
    return int(n.value)


def ring_decode(dims: Dims, n_hosts: int, q, k, v, kv_len, O, lse, workspace, o_dtype=None,
                stream=None):
    """One decode step over n_hosts KV-cache shards (ra_ring_decode); o_dtype
    defaults to the dtype of O (bf16 or float32)."""
    d = dims.c()
    if o_dtype is None:
        o_dtype = RA_BF16 if str(O.dtype) == "torch.bfloat16" else RA_F32
    nbytes = workspace.numel() * workspace.element_size()
    L.check(L.load().ra_ring_decode(ctypes.byref(d), n_hosts, _ptr(q), _ptr(k), _ptr(v), _ptr(kv_len),
                                    _ptr(O), o_dtype, _ptr(lse), _ptr(workspace), nbytes,
                                    _stream(stream)), "ra_ring_decode")


def ring_decode_noalloc(dims: Dims, n_hosts: int, q, k, v, kv_len, O, lse, o_dtype=None, stream=None):
    """ra_ring_decode without a workspace (ra_ring_decode_noalloc): the
    partials live in the library's fixed device array; calls that overlap on
    one GPU race."""
    d = dims.c()
    if o_dtype is None:
        o_dtype = RA_BF16 if str(O.dtype) == "torch.bfloat16" else RA_F32
    L.check(L.load().ra_ring_decode_noalloc(ctypes.byref(d), n_hosts, _ptr(q), _ptr(k), _ptr(v), _ptr(kv_len),
                                            _ptr(O), o_dtype, _ptr(lse), _stream(stream)),
            "ra_ring_decode_noalloc")


def ffn_workspace_size(block_rows: int, h: int, f: int) -> int:
    n = ctypes.c_size_t(0)
    L.check(L.load().ra_ffn_workspace_size(block_rows, h, f, ctypes.byref(n)), "ra_ffn_workspace_size")
    return int(n.value)


def block_ffn(X, W1, W2, Y, block_rows: int, workspace, stream=None):
    """Blockwise feedforward Y = GELU(X W1^T) W2^T of [rows][h] bf16 X
    (ra_block_ffn); W1 [f][h], W2 [h][f]."""
    rows, h = X.shape[-2], X.shape[-1]
    f = W1.shape[0]
    nbytes = workspace.numel() * workspace.element_size()
    L.check(L.load().ra_block_ffn(_ptr(X), _ptr(W1), _ptr(W2), _ptr(Y), X.numel() // h, h, f, block_rows,
                                  _ptr(workspace), nbytes, _stream(stream)), "ra_block_ffn")


def raw_call(name: str, *args) -> int:
    """Call an exported symbol directly (tests of argument checking)."""
    return int(getattr(L.load(), name)(*args))


def last_error() -> str:
    return L.load().ra_last_error().decode(errors="replace")
