"""Overlap arithmetic of the ring: when does a block's compute hide its transfer?

[P2] "Ring Attention with Blockwise Transformers for Near Infinite Context"
(reading notes), section 5.4: one block pair costs 4 d c^2 FLOPs and moving a
K/V block costs 4 c d bytes (bf16 K and V), so the transfer hides behind the
compute when 4 d c^2 / F >= 4 c d / B, i.e. c >= F / B; the minimal local
sequence is 6 c (the paper's Table 2, repeated in the notes' 结果 2).
[P3] aiqz.cc explainer, 隐藏通信: total time ~ m * max(t_calc, t_comm).
"""
from __future__ import annotations


def min_block_size(flops: float, bandwidth: float) -> float:
    """Smallest block length c (tokens) whose compute hides its transfer: F / B."""
    return flops / bandwidth


def min_local_sequence(flops: float, bandwidth: float) -> float:
    return 6.0 * min_block_size(flops, bandwidth)


def block_flops(head_dim: int, block_len: int, heads: int = 1) -> float:
    """4 d c^2 per head for one unmasked block pair."""
    return 4.0 * head_dim * block_len * block_len * heads


def kv_transfer_bytes(head_dim: int, block_len: int, heads_kv: int = 1, elem_bytes: int = 2) -> float:
    """K and V of one block: 2 * c * d * elem_bytes per kv head (4 c d at bf16)."""
    return 2.0 * block_len * head_dim * heads_kv * elem_bytes


def t_comm(head_dim: int, block_len: int, heads_kv: int, bandwidth: float, elem_bytes: int = 2) -> float:
    return kv_transfer_bytes(head_dim, block_len, heads_kv, elem_bytes) / bandwidth


def ring_time(n_steps: int, t_calc: float, t_comm_: float) -> float:
    """Overlapped ring time: n * max(t_calc, t_comm)."""
    return n_steps * max(t_calc, t_comm_)


def crossing_block_len(t_calc_by_c: dict, heads_kv: int, head_dim: int, bandwidth: float,
                       elem_bytes: int = 2):
    """Smallest measured c with t_calc(c) >= t_comm(c); None if none qualifies."""
    for c in sorted(t_calc_by_c):
        if t_calc_by_c[c] >= t_comm(head_dim, c, heads_kv, bandwidth, elem_bytes):
            return c
    return None
