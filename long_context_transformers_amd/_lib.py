"""ctypes declarations of libringattn's C ABI (include/ringattn.h).

Argument marshalling only.  The library is the in-tree ``libringattn.so``
built by ``long_context_transformers_amd.build``; if it is missing this
module raises -- there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libringattn.so")

RA_OK, RA_ERR_INVALID_ARG, RA_ERR_UNSUPPORTED, RA_ERR_HIP, RA_ERR_WORKSPACE = range(5)
RA_BF16, RA_F32 = 0, 1
RA_MASK_NONE, RA_MASK_CAUSAL = 0, 1
RA_LAYOUT_CONTIGUOUS, RA_LAYOUT_STRIPED, RA_LAYOUT_ZIGZAG = 0, 1, 2
RA_BLK_SKIP, RA_BLK_FULL, RA_BLK_TRI_INCL, RA_BLK_TRI_STRICT, RA_BLK_BAND, RA_BLK_QUADRANTS = range(6)
RA_FLAG_ELIDE_SKIPPED_COPIES = 1
RA_FLAG_SERIALIZE = 2
RA_COPY_NONE, RA_COPY_DMA_ENGINES, RA_COPY_FALLBACK = 0, 1, 2

c_i32, c_i64, c_u32, c_f32, c_vp = (ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32,
                                    ctypes.c_float, ctypes.c_void_p)


class RaDims(ctypes.Structure):
    _fields_ = [("batch", c_i32), ("heads_q", c_i32), ("heads_kv", c_i32),
                ("head_dim", c_i32), ("block_len", c_i32), ("dtype", c_i32),
                ("scale", c_f32)]


class RaStep(ctypes.Structure):
    _fields_ = [("step", c_i32), ("src", c_i32), ("cls", c_i32), ("pad_", c_i32),
                ("q_offset", c_i64), ("kv_offset", c_i64), ("stride", c_i64)]


class RaRingCfg(ctypes.Structure):
    _fields_ = [("dims", RaDims), ("n_hosts", c_i32), ("host_begin", c_i32),
                ("host_end", c_i32), ("layout", c_i32), ("mask", c_i32),
                ("flags", c_u32), ("debug_copy_delay_us", c_u32),
                ("step_events", ctypes.POINTER(c_vp))]


class RaRingStats(ctypes.Structure):
    _fields_ = [("compute_steps", c_i32), ("transfers", c_i32),
                ("skipped_blocks", c_i32), ("kernel_launches", c_i32),
                ("copy_bytes", c_i64), ("resident_bytes_per_host", c_i64),
                ("copy_kind", c_i32), ("pad_", c_i32)]


P = ctypes.POINTER
# (name, restype, argtypes) for every exported symbol of include/ringattn.h
SIGNATURES = [
    ("ra_token_index", c_i64, [c_i32, c_i32, c_i64, c_i32, c_i64]),
    ("ra_schedule", c_i32, [c_i32, c_i32, c_i32, c_i32, c_i32, P(RaStep)]),
    ("ra_block_class_of", c_i32, [c_i32, c_i64, c_i64, c_i64, c_i32]),
    ("ra_state_init", c_i32, [P(RaDims), c_vp, c_vp, c_vp, c_vp]),
    ("ra_block_fwd", c_i32, [P(RaDims), c_vp, c_vp, c_vp, c_i32, c_i64, c_i64, c_i64,
                             c_vp, c_vp, c_vp, c_vp]),
    ("ra_merge_lse", c_i32, [P(RaDims), c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    ("ra_finalize", c_i32, [P(RaDims), c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    ("ra_bwd_preprocess", c_i32, [P(RaDims), c_vp, c_vp, c_vp, c_vp]),
    ("ra_block_bwd", c_i32, [P(RaDims), c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i64,
                             c_i64, c_i64, c_vp, c_vp, c_vp, c_vp]),
    ("ra_layout_permute", c_i32, [P(RaDims), c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp]),
    ("ra_mask_tile", c_i32, [c_i64, c_i64, c_i64, c_i32, c_i32, c_vp, c_vp]),
    ("ra_ring_workspace_size", c_i32, [P(RaRingCfg), c_i32, P(ctypes.c_size_t)]),
    ("ra_ring_fwd", c_i32, [P(RaRingCfg), c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, ctypes.c_size_t,
                            c_vp, c_vp, P(RaRingStats)]),
    ("ra_ring_bwd", c_i32, [P(RaRingCfg), c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                            c_vp, ctypes.c_size_t, c_vp, c_vp, P(RaRingStats)]),
    ("ra_decode_workspace_size", c_i32, [P(RaDims), c_i32, P(ctypes.c_size_t)]),
    ("ra_ring_decode", c_i32, [P(RaDims), c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp,
                               ctypes.c_size_t, c_vp]),
    ("ra_ring_decode_noalloc", c_i32, [P(RaDims), c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp]),
    ("ra_ffn_workspace_size", c_i32, [c_i64, c_i32, c_i32, P(ctypes.c_size_t)]),
    ("ra_block_ffn", c_i32, [c_vp, c_vp, c_vp, c_vp, c_i64, c_i32, c_i32, c_i64, c_vp, ctypes.c_size_t,
                             c_vp]),
    ("ra_status_str", ctypes.c_char_p, [c_i32]),
    ("ra_last_error", ctypes.c_char_p, []),
    ("ra_version", c_i32, []),
]

_LIB = None


class RingAttnError(RuntimeError):
    def __init__(self, status: int, fn: str, detail: str):
        self.status = status
        super().__init__(f"{fn}: status {status}: {detail}")


def load():
    """Load libringattn.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        # The library must run on the HIP runtime that torch loaded: device
        # pointers and streams come from torch.  Loaded first, it would pull
        # in the system runtime, and torch would then load its bundled copy
        # beside it (it names the runtime without the version suffix), leaving
        # two runtimes in the process.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} not found: build it with "
                "`python -m long_context_transformers_amd.build` (no fallback exists)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, res, args in SIGNATURES:
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


def check(status: int, fn: str):
    if status != RA_OK:
        detail = load().ra_last_error().decode(errors="replace")
        raise RingAttnError(status, fn, detail)
