"""ctypes binding of the C fp64 oracle (``ra_oracle.c``).  TEST INFRASTRUCTURE.

Every function here evaluates the plain definition of attention (see the
header of ``ra_oracle.c`` for the page passages it follows).  Pins: see
``tests/test_oracle_pins.py`` (brute force, closed forms, order invariance,
merge identity, finite differences).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(dtype=np.int64, flags="C_CONTIGUOUS")
_u8p = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")


def lib():
    global _LIB
    if _LIB is None:
        path = os.path.join(_HERE, "liboracle.so")
        if not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        L.oracle_token_index.restype = ctypes.c_longlong
        L.oracle_token_index.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_longlong,
                                         ctypes.c_int, ctypes.c_longlong]
        L.oracle_visible.restype = ctypes.c_int
        L.oracle_visible.argtypes = [ctypes.c_int, ctypes.c_longlong, ctypes.c_longlong]
        L.oracle_block_mask.restype = None
        L.oracle_block_mask.argtypes = [ctypes.c_int] * 6 + [_u8p]
        ci = ctypes.c_int
        L.oracle_attn_rows.restype = ci
        L.oracle_attn_rows.argtypes = [_f32p, _f32p, _f32p] + [ci] * 8 + [
            ctypes.c_double, ci, ci, ctypes.c_longlong, _i64p, _f64p, _f64p, _f64p, _f64p]
        L.oracle_attn_bwd_q_rows.restype = ci
        L.oracle_attn_bwd_q_rows.argtypes = [_f32p] * 4 + [ci] * 8 + [
            ctypes.c_double, ci, ci, ctypes.c_longlong, _i64p, _f64p, _f64p, _f64p]
        L.oracle_attn_rows_plain.restype = ci
        L.oracle_attn_rows_plain.argtypes = L.oracle_attn_rows.argtypes
        L.oracle_attn_bwd_q_rows_plain.restype = ci
        L.oracle_attn_bwd_q_rows_plain.argtypes = L.oracle_attn_bwd_q_rows.argtypes
        L.oracle_attn_bwd_kv_rows.restype = ci
        L.oracle_attn_bwd_kv_rows.argtypes = [_f32p] * 4 + [_f64p, _f64p] + [ci] * 8 + [
            ctypes.c_double, ctypes.c_longlong, _i64p, _f64p, _f64p]
        L.oracle_num_threads.restype = ci
        L.oracle_num_threads.argtypes = []
        _LIB = L
    return _LIB


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def token_index(layout: int, n_hosts: int, block_len: int, host: int, r: int) -> int:
    return int(lib().oracle_token_index(layout, n_hosts, block_len, host, r))


def block_mask(layout: int, causal: int, n_hosts: int, block_len: int, qhost: int,
               khost: int) -> np.ndarray:
    out = np.zeros((block_len, block_len), dtype=np.uint8)
    lib().oracle_block_mask(layout, causal, n_hosts, block_len, qhost, khost, out)
    return out


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def attn_rows(q, k, v, *, n_hosts, layout, causal, rows, scale: Optional[float] = None,
              q_host_base: int = 0, plain: bool = False):
    """Forward rows.  q: [nq_hosts][B][Hq][c][d] float32 (host ``h`` at index
    ``h - q_host_base``); k, v: [N][B][Hkv][c][d]; rows: int64 [n, 4] of
    (host, batch, q_head, local row).  Returns (O [n,d], lse, max, l) fp64.
    ``plain``: evaluate one row at a time (the per-row form the row sets must
    match bit for bit; slow on long sequences)."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    nq, B, Hq, c, d = q.shape
    Hkv = k.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 4)
    n = rows.shape[0]
    O = np.zeros((n, d)); lse = np.zeros(n); mx = np.zeros(n); l = np.zeros(n)
    fn = lib().oracle_attn_rows_plain if plain else lib().oracle_attn_rows
    rc = fn(q, k, v, n_hosts, B, Hq, Hkv, c, d, layout, causal, float(scale), q_host_base,
            nq, n, rows, O, lse, mx, l)
    if rc != 0:
        raise ValueError("oracle_attn_rows: bad argument")
    return O, lse, mx, l


def attn_bwd_q_rows(q, k, v, do, *, n_hosts, layout, causal, rows, scale=None,
                    q_host_base: int = 0, plain: bool = False):
    """dQ for query rows; also returns the oracle's LSE and D for those rows.
    ``plain``: one row at a time, as in ``attn_rows``."""
    q, k, v, do = _f32(q), _f32(k), _f32(v), _f32(do)
    nq, B, Hq, c, d = q.shape
    Hkv = k.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 4)
    n = rows.shape[0]
    dQ = np.zeros((n, d)); lse = np.zeros(n); D = np.zeros(n)
    fn = lib().oracle_attn_bwd_q_rows_plain if plain else lib().oracle_attn_bwd_q_rows
    rc = fn(q, k, v, do, n_hosts, B, Hq, Hkv, c, d, layout, causal, float(scale),
            q_host_base, nq, n, rows, dQ, lse, D)
    if rc != 0:
        raise ValueError("oracle_attn_bwd_q_rows: bad argument")
    return dQ, lse, D


def attn_bwd_kv_rows(q, k, v, do, lse_all, D_all, *, n_hosts, layout, causal, rows,
                     scale=None):
    """dK, dV for key rows (host, batch, kv_head, local row).  q, do hold all
    N hosts; lse_all, D_all: [N][B][Hq][c] from the oracle's own forward."""
    q, k, v, do = _f32(q), _f32(k), _f32(v), _f32(do)
    N, B, Hq, c, d = q.shape
    Hkv = k.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    lse_all = np.ascontiguousarray(lse_all, dtype=np.float64)
    D_all = np.ascontiguousarray(D_all, dtype=np.float64)
    assert lse_all.shape == (N, B, Hq, c) and D_all.shape == (N, B, Hq, c)
    rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 4)
    n = rows.shape[0]
    dK = np.zeros((n, d)); dV = np.zeros((n, d))
    rc = lib().oracle_attn_bwd_kv_rows(q, k, v, do, lse_all, D_all, n_hosts, B, Hq, Hkv,
                                       c, d, layout, causal, float(scale), n, rows, dK, dV)
    if rc != 0:
        raise ValueError("oracle_attn_bwd_kv_rows: bad argument")
    return dK, dV


def row_desc(hosts, batches, heads, rows) -> np.ndarray:
    """Cartesian product of (host, batch, head, row) as an int64 [n,4] array."""
    H, B, Hh, R = np.meshgrid(np.asarray(hosts), np.asarray(batches), np.asarray(heads),
                              np.asarray(rows), indexing="ij")
    return np.stack([H.ravel(), B.ravel(), Hh.ravel(), R.ravel()], axis=1).astype(np.int64)
