"""Seeded synthetic inputs for the ring-attention workloads.

This module is shared by the fp64 oracle (``oracle/``) and the HIP path
(``long_context_transformers_amd``).  It holds no attention arithmetic: it
only draws iid N(0, 1) samples from NumPy's PCG64, rounds them to bfloat16
(round to nearest, ties to even), widens bfloat16 bit patterns back to
float32 (exact), picks seeded row samples, and names the five workload
shapes.

Arrays are drawn directly in the host-major layout ``[N][B][H][c][d]``: block
``h`` holds host ``h``'s share.  Which global token a local row ``r`` of host
``h`` stands for is fixed by the token layout (contiguous or striped), which
both sides compute on their own.  Because the samples are iid, drawing them in
host-major order gives the same distribution as drawing a full sequence and
permuting it.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

LAYOUT_CONTIGUOUS = 0
LAYOUT_STRIPED = 1
LAYOUT_ZIGZAG = 2
MASK_NONE = 0
MASK_CAUSAL = 1
DT_BF16 = 0
DT_F32 = 1


@dataclasses.dataclass(frozen=True)
class Workload:
    """One workload shape.  ``hosts`` lists the simulated hosts that run."""

    name: str
    cfg: int                 # workload number, used to derive seeds
    batch: int
    heads_q: int
    heads_kv: int
    head_dim: int
    n_hosts: int
    block_len: int
    dtype: int               # DT_BF16 or DT_F32
    mask: int                # MASK_NONE or MASK_CAUSAL
    layout: int              # LAYOUT_CONTIGUOUS, LAYOUT_STRIPED or LAYOUT_ZIGZAG
    host_begin: int
    host_end: int
    q_scale: float = 1.0     # multiplies Q before rounding (large-logit variant)
    seed_offset: int = 0     # second seed set

    @property
    def seq_len(self) -> int:
        return self.n_hosts * self.block_len

    @property
    def n_active(self) -> int:
        return self.host_end - self.host_begin

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def workloads() -> dict:
    """The five workload shapes (b=1 everywhere)."""
    w = {}
    w["tiny"] = Workload("tiny_f32_noncausal_N4_c64", 1, 1, 2, 2, 64, 4, 64,
                         DT_F32, MASK_NONE, LAYOUT_CONTIGUOUS, 0, 4)
    w["tiny_bigq"] = w["tiny"].replace(name="tiny_f32_noncausal_N4_c64_qx8",
                                       q_scale=8.0, seed_offset=100)
    w["noncausal_32k"] = Workload("noncausal_32k_H8_d128_N8_c4096", 2, 1, 8, 8, 128,
                                  8, 4096, DT_BF16, MASK_NONE,
                                  LAYOUT_CONTIGUOUS, 0, 8)
    w["causal_256k_contig"] = Workload("causal_256k_contiguous_H32_N8_c32768_host7",
                                       3, 1, 32, 32, 128, 8, 32768, DT_BF16,
                                       MASK_CAUSAL, LAYOUT_CONTIGUOUS, 7, 8)
    w["causal_256k_striped"] = w["causal_256k_contig"].replace(
        name="causal_256k_striped_H32_N8_c32768_host7", layout=LAYOUT_STRIPED)
    w["causal_256k_zigzag"] = w["causal_256k_contig"].replace(
        name="causal_256k_zigzag_H32_N8_c32768_host7", layout=LAYOUT_ZIGZAG)
    w["striped_786k_gqa"] = Workload("striped_786k_gqa_Hq32_Hkv8_N16_c49152_host15",
                                     4, 1, 32, 8, 128, 16, 49152, DT_BF16,
                                     MASK_CAUSAL, LAYOUT_STRIPED, 15, 16)
    w["bwd_64k"] = Workload("bwd_64k_causal_contiguous_H32_N8_c8192", 5, 1, 32, 32,
                            128, 8, 8192, DT_BF16, MASK_CAUSAL,
                            LAYOUT_CONTIGUOUS, 0, 8)
    return w


# ----------------------------------------------------------------------------
# bfloat16 helpers (input quantisation only)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16, nearest-even; returns uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = (u >> 16) & np.uint32(1)          # 32-bit arithmetic: a carry past bit 31 only
    r += u                                # wraps where the 64-bit form would drop it
    r += np.uint32(0x7FFF)                # under the & 0xFFFF of the top half
    r >>= 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------
# seeded draws
# ----------------------------------------------------------------------------

def normal_f32(seed, shape, scale: float = 1.0) -> np.ndarray:
    """iid N(0,1) float32 from PCG64(seed) (seed: int or tuple of ints),
    optionally multiplied by ``scale``."""
    rng = np.random.default_rng(list(seed) if isinstance(seed, tuple) else seed)
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x = x * np.float32(scale)
    return x


def q_shape(w: Workload, hosts: Optional[int] = None):
    n = w.n_hosts if hosts is None else hosts
    return (n, w.batch, w.heads_q, w.block_len, w.head_dim)


def kv_shape(w: Workload, hosts: Optional[int] = None):
    n = w.n_hosts if hosts is None else hosts
    return (n, w.batch, w.heads_kv, w.block_len, w.head_dim)


@dataclasses.dataclass
class Inputs:
    """Host-major inputs.  ``*_f32`` hold the exact values the device reads
    (bf16 values widened to float32 for bf16 workloads); ``*_dev`` hold the
    device representation (uint16 bf16 bit patterns, or float32).
    ``q_*`` / ``do_*`` cover hosts [q_host_base, q_host_base + len)."""

    q_f32: np.ndarray
    k_f32: np.ndarray
    v_f32: np.ndarray
    q_dev: np.ndarray
    k_dev: np.ndarray
    v_dev: np.ndarray
    q_host_base: int = 0
    do_f32: Optional[np.ndarray] = None
    do_dev: Optional[np.ndarray] = None


def _draw_blocks(w: Workload, base_seed: int, hosts, shape_one, scale: float = 1.0):
    """Blocks of the given hosts; block h is drawn from seed (base_seed, h).
    Returns (exact float32 values, device representation)."""
    n = len(hosts)
    f = np.empty((n,) + shape_one, dtype=np.float32)
    dev = np.empty((n,) + shape_one, dtype=np.uint16 if w.dtype == DT_BF16 else np.float32)
    for i, h in enumerate(hosts):
        x = normal_f32((base_seed, h), shape_one, scale)
        if w.dtype == DT_BF16:
            bits = f32_to_bf16_bits(x)
            dev[i] = bits
            f[i] = bf16_bits_to_f32(bits)
        else:
            dev[i] = x
            f[i] = x
    return f, dev


def make_inputs(w: Workload, with_do: bool = False, q_hosts_only: bool = False) -> Inputs:
    """Draw Q, K, V (and dO) for workload ``w``.

    Block h of each tensor comes from PCG64 seeded with (base + cfg +
    seed_offset, h), base = 1000 (Q), 2000 (K), 3000 (V), 4000 (dO).  K and V
    cover all N hosts; Q and dO cover the active hosts only when
    ``q_hosts_only`` (else all N)."""
    so = w.seed_offset
    qh = list(range(w.host_begin, w.host_end)) if q_hosts_only else list(range(w.n_hosts))
    one_q = q_shape(w, 1)[1:]
    one_kv = kv_shape(w, 1)[1:]
    qf, qd = _draw_blocks(w, 1000 + w.cfg + so, qh, one_q, w.q_scale)
    kf, kd = _draw_blocks(w, 2000 + w.cfg + so, range(w.n_hosts), one_kv)
    vf, vd = _draw_blocks(w, 3000 + w.cfg + so, range(w.n_hosts), one_kv)
    inp = Inputs(qf, kf, vf, qd, kd, vd, q_host_base=qh[0])
    if with_do:
        inp.do_f32, inp.do_dev = _draw_blocks(w, 4000 + w.cfg + so, qh, one_q)
    return inp


def row_sample(w: Workload, n_rows: int = 1024, seed: Optional[int] = None) -> np.ndarray:
    """Seeded sample of ``n_rows`` distinct local rows in [0, c), always
    including rows 0, 1 and c-1; sorted."""
    c = w.block_len
    if n_rows >= c:
        return np.arange(c, dtype=np.int64)
    rng = np.random.default_rng(9000 + w.cfg if seed is None else seed)
    fixed = {0, 1, c - 1}
    pool = rng.choice(c, size=min(c, n_rows + 8), replace=False)
    rows = list(fixed)
    for p in pool:
        if len(rows) >= n_rows:
            break
        if int(p) not in fixed:
            rows.append(int(p))
    return np.array(sorted(rows), dtype=np.int64)


# ----------------------------------------------------------------------------
# decoding against a ring-sharded KV cache
# ----------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    """One decode step: `batch` sequences, each with one new query token,
    against a KV cache sharded over `n_hosts` shards of `block_len` rows."""
    name: str
    cfg: int
    batch: int
    heads_q: int
    heads_kv: int
    head_dim: int
    n_hosts: int
    block_len: int

    @property
    def capacity(self) -> int:
        return self.n_hosts * self.block_len


def decode_workloads() -> dict:
    """The decode shapes.  decode_8m follows the pages' inference example
    (a 7B model with 32 heads of d = 128 served from 32 hosts): 32 shards of
    256K rows, an 8M-token cache; decode_512k_gqa is a grouped-head case small
    enough for the oracle to read every key."""
    return {
        "decode_8m": DecodeWorkload("decode_8m_H32_d128_N32_c262144", 20, 1, 32, 32, 128, 32, 262144),
        "decode_512k_gqa": DecodeWorkload("decode_512k_Hq32_Hkv8_N8_c65536_B2", 21, 2, 32, 8, 128, 8, 65536),
    }


def decode_lens(n_hosts: int, batch: int, block_len: int, seed: int, full: bool = True) -> np.ndarray:
    """Valid rows per shard, int32 [n_hosts][batch], for contiguous sharding
    of each sequence's tokens: sequence b of length T_b puts tokens
    [h c, (h+1) c) on shard h.  full=True draws T_b in ((N-1) c, N c] (every
    shard but the last one full, as in a long-context server); full=False
    draws T_b in [0, N c] (ragged, empty shards and sequences included)."""
    rng = np.random.default_rng(seed)
    cap = n_hosts * block_len
    lo = (n_hosts - 1) * block_len + 1 if full else 0
    T = rng.integers(lo, cap + 1, size=batch)
    h = np.arange(n_hosts)[:, None]
    return np.clip(T[None, :] - h * block_len, 0, block_len).astype(np.int32)


# ----------------------------------------------------------------------------
# the blockwise feedforward of the local block
# ----------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class FfnWorkload:
    """Feedforward of one host's block: `rows` tokens of width h, hidden f,
    evaluated in row blocks of `block_rows`."""
    name: str
    cfg: int
    rows: int
    h: int
    f: int
    block_rows: int


def ffn_workloads() -> dict:
    """ffn_7b_c4096: a 7B-like layer (h = 4096, f = 4h) on one host's block of
    4096 tokens (the block size of the non-causal 32K ring), evaluated as one
    row block (the host's block is the unit of the blockwise schedule)."""
    return {"ffn_7b_c4096": FfnWorkload("ffn_7b_h4096_f16384_c4096", 30, 4096, 4096, 16384, 4096)}
