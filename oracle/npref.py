"""NumPy fp64 forms of the ring-attention computation.  TEST INFRASTRUCTURE.

Pages (short names):
  [P1] "Ring Attention如何让大模型突破百万token上下文：从环形通信到计算重叠的技术突围"
  [P2] "Ring Attention with Blockwise Transformers for Near Infinite Context"
       (reading notes on arXiv 2310.01889)
  [P3] aiqz.cc Ring Attention explainer

Functions and what they follow:
  token_index          -- [P1] 因果掩码的负载均衡挑战 (contiguous split; striped
                          lists "device 0: tokens 0, 4, 8, 12 ...").
  explicit_mask        -- [P3] 工程实现 (a token sees tokens with index <= its own).
  dense_attention      -- [P2] 5.1 softmax(QK^T/sqrt(d))V, written out densely.
  ring_host_blocked    -- [P3] 分块注意力 per-block update (normalised form) and
                          [P1] Flash Attention paragraph / [P2] 5.2 (max,
                          numerator, denominator form); ring order from [P1]
                          Ring Attention的核心洞察 (device i receives from i-1)
                          and [P3] 环状拓扑.
  lse_merge            -- [P1] Online Softmax, the LogSumExp form.
  brute_force_row      -- pure-Python loops over the definition (tiny inputs).
  dense_attention_grad -- closed-form gradient of dense_attention (the pages do not
                          print it; [P2] 5.2 only says dQ, dK, dV accumulate along
                          the ring).
  blockwise_ffn        -- [P2] 2 and 5.2-5.3 (the Blockwise Parallel Transformer's
                          feedforward acts on the local block only, so its
                          activation stays within 2bch): Y = GELU(X W1^T) W2^T per
                          token, evaluated block by block.
  decode_attention     -- [P2] 5.6 (Appendix C: autoregressive decoding with the KV
                          cache spread over the ring) and [P3] 超长序列推理与KV Cache
                          分发: one new query token per sequence attends to every
                          valid cached key of every host's shard.

Every function is pinned in tests/test_oracle_pins.py.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence

import numpy as np

LAYOUT_CONTIGUOUS = 0
LAYOUT_STRIPED = 1
LAYOUT_ZIGZAG = 2


def token_index(layout: int, n_hosts: int, block_len: int, host, r):
    """Global token of local row r on host ``host``.  Zigzag (named, not
    defined, in P1 "工程实践指南" as the causal load-balancing variant beside
    Striped; reading used here): 2N chunks of c/2 tokens, host h holds chunk h
    in rows 0..c/2-1 and chunk 2N-1-h in rows c/2..c-1."""
    host = np.asarray(host, dtype=np.int64)
    r = np.asarray(r, dtype=np.int64)
    if layout == LAYOUT_STRIPED:
        return r * n_hosts + host
    if layout == LAYOUT_ZIGZAG:
        half = block_len // 2
        return np.where(r < half, host * half + r, (2 * n_hosts - 1 - host) * half + (r - half))
    return host * block_len + r


def explicit_mask(causal: bool, tq, tk) -> np.ndarray:
    """mask[a, b] = key token tk[b] visible to query token tq[a]."""
    tq = np.asarray(tq, dtype=np.int64)[:, None]
    tk = np.asarray(tk, dtype=np.int64)[None, :]
    if not causal:
        return np.ones((tq.shape[0], tk.shape[1]), dtype=bool)
    return tk <= tq


def gather_full(x_hm: np.ndarray, layout: int) -> np.ndarray:
    """Host-major [N][B][H][c][d] -> full sequence [B][H][S][d] (fp64)."""
    N, B, H, c, d = x_hm.shape
    out = np.empty((B, H, N * c, d), dtype=np.float64)
    r = np.arange(c)
    for h in range(N):
        t = token_index(layout, N, c, h, r)
        out[:, :, t, :] = x_hm[h].astype(np.float64)
    return out


def dense_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray,
                    scale: float):
    """q [Sq,d], k, v [Sk,d], mask [Sq,Sk] bool.  Returns O, lse, max, l.
    A row with no visible key gets O = 0, lse = max = -inf, l = 0."""
    s = (q.astype(np.float64) @ k.astype(np.float64).T) * scale
    s = np.where(mask, s, -np.inf)
    mx = s.max(axis=1)
    safe = np.where(np.isfinite(mx), mx, 0.0)
    p = np.exp(s - safe[:, None])
    l = p.sum(axis=1)
    num = p @ v.astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        O = np.where(l[:, None] > 0, num / np.where(l > 0, l, 1.0)[:, None], 0.0)
        lse = np.where(l > 0, safe + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return O, lse, mx, l


def dense_attention_grad(q, k, v, do, mask, scale):
    """Closed-form gradient of dense_attention's O with cotangent ``do``.
    Returns dQ, dK, dV (fp64)."""
    q = q.astype(np.float64); k = k.astype(np.float64); v = v.astype(np.float64)
    do = do.astype(np.float64)
    O, lse, _, _ = dense_attention(q, k, v, mask, scale)
    s = (q @ k.T) * scale
    safe = np.where(np.isfinite(lse), lse, 0.0)
    p = np.where(mask, np.exp(s - safe[:, None]), 0.0)
    D = (do * O).sum(axis=1)
    dv = p.T @ do
    dp = do @ v.T
    ds = p * (dp - D[:, None])
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


# ----------------------------------------------------------------------------
# the blocked ring procedure
# ----------------------------------------------------------------------------

def _update_normalised(m, ell, O, s_b, v_b):
    """One block of the [P3] 分块注意力 update, normalised-output form:
        m   <- max(m, rowmax S_b)
        ell <- ell * e^(m_old - m) + rowsum(e^(S_b - m))
        O   <- (ell_old e^(m_old - m) / ell) O + (e^(S_b - m) / ell) V_b
    Rows whose running max is still -inf keep the initial state (no visible
    key yet): e^(-inf - (-inf)) is taken as contributing nothing."""
    m_new = np.maximum(m, s_b.max(axis=1))
    live = np.isfinite(m_new)
    base = np.where(live, m_new, 0.0)
    alpha = np.where(live, np.exp(np.where(np.isfinite(m), m, -np.inf) - base), 1.0)
    p = np.exp(s_b - base[:, None])          # masked scores are -inf -> 0
    ell_new = ell * alpha + p.sum(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        w_old = np.where(ell_new > 0, ell * alpha / np.where(ell_new > 0, ell_new, 1.0), 0.0)
        w_new = np.where(ell_new > 0, 1.0 / np.where(ell_new > 0, ell_new, 1.0), 0.0)
    O_new = w_old[:, None] * O + w_new[:, None] * (p @ v_b)
    return m_new, ell_new, O_new


def _update_numerator(m, num, den, s_b, v_b):
    """One block in the (max, numerator, denominator) form of [P1] (Flash
    Attention paragraph) and [P2] 5.2: both accumulators are rescaled by
    e^(m_old - m) when the max grows; the output is num / den at the end."""
    m_new = np.maximum(m, s_b.max(axis=1))
    live = np.isfinite(m_new)
    base = np.where(live, m_new, 0.0)
    alpha = np.where(live, np.exp(np.where(np.isfinite(m), m, -np.inf) - base), 1.0)
    p = np.exp(s_b - base[:, None])
    return m_new, den * alpha + p.sum(axis=1), num * alpha[:, None] + p @ v_b


def ring_order(n_hosts: int, host: int) -> list:
    """Source host of the K/V block that host ``host`` holds at each step: the
    host's own block first, then the block its predecessor passed on."""
    return [(host - s) % n_hosts for s in range(n_hosts)]


def ring_host_blocked(q_hm, k_hm, v_hm, host: int, *, layout: int, causal: bool,
                      scale: float, batch: int = 0, head: int = 0, kv_head: int = 0,
                      order: Optional[Sequence[int]] = None, form: str = "normalised"):
    """Attention output of ``host``'s query block computed block by block in
    ring order (or in any given order of source blocks).
    Returns O [c,d], lse [c], m [c], ell [c] (fp64)."""
    N, c, d = k_hm.shape[0], k_hm.shape[3], k_hm.shape[4]
    order = ring_order(N, host) if order is None else list(order)
    q = q_hm[host, batch, head].astype(np.float64)
    tq = token_index(layout, N, c, host, np.arange(c))
    m = np.full(c, -np.inf)
    ell = np.zeros(c)
    O = np.zeros((c, d))
    for j in order:
        kb = k_hm[j, batch, kv_head].astype(np.float64)
        vb = v_hm[j, batch, kv_head].astype(np.float64)
        tk = token_index(layout, N, c, j, np.arange(c))
        s_b = np.where(explicit_mask(causal, tq, tk), (q @ kb.T) * scale, -np.inf)
        if form == "normalised":
            m, ell, O = _update_normalised(m, ell, O, s_b, vb)
        elif form == "numerator":
            m, ell, O = _update_numerator(m, O, ell, s_b, vb)  # O holds the numerator
        else:
            raise ValueError(form)
    if form == "numerator":
        with np.errstate(divide="ignore", invalid="ignore"):
            O = np.where(ell[:, None] > 0, O / np.where(ell > 0, ell, 1.0)[:, None], 0.0)
    with np.errstate(divide="ignore"):
        lse = np.where(ell > 0, m + np.log(np.where(ell > 0, ell, 1.0)), -np.inf)
    return O, lse, m, ell


def lse_merge(O_a, lse_a, O_b, lse_b):
    """Combine two partial results over disjoint key sets ([P1] Online
    Softmax, LogSumExp form): with M = max(lse_a, lse_b),
    lse = M + ln(e^(lse_a - M) + e^(lse_b - M)) and
    O = e^(lse_a - lse) O_a + e^(lse_b - lse) O_b.  An empty part has
    lse = -inf and weight 0; two empty parts give O = 0, lse = -inf."""
    lse_a = np.asarray(lse_a, dtype=np.float64)
    lse_b = np.asarray(lse_b, dtype=np.float64)
    M = np.maximum(lse_a, lse_b)
    live = np.isfinite(M)
    base = np.where(live, M, 0.0)
    ea = np.exp(lse_a - base)
    eb = np.exp(lse_b - base)
    with np.errstate(divide="ignore"):
        lse = np.where(live, base + np.log(ea + eb), -np.inf)
    wa = np.where(live, np.exp(lse_a - np.where(live, lse, 0.0)), 0.0)
    wb = np.where(live, np.exp(lse_b - np.where(live, lse, 0.0)), 0.0)
    return wa[..., None] * O_a + wb[..., None] * O_b, lse


def brute_force_row(q: Sequence[float], keys: Iterable[Sequence[float]],
                    values: Iterable[Sequence[float]], visible: Iterable[bool],
                    scale: float):
    """Pure-Python loops: softmax over visible keys of scale * q.k, times V.
    Returns (O list, lse)."""
    keys = list(keys); values = list(values); visible = list(visible)
    scores = []
    for kk, vis in zip(keys, visible):
        if vis:
            acc = 0.0
            for a, b in zip(q, kk):
                acc += float(a) * float(b)
            scores.append(scale * acc)
        else:
            scores.append(None)
    live = [s for s in scores if s is not None]
    d = len(values[0])
    if not live:
        return [0.0] * d, -math.inf
    mx = max(live)
    total = 0.0
    out = [0.0] * d
    for s, vv in zip(scores, values):
        if s is None:
            continue
        w = math.exp(s - mx)
        total += w
        for e in range(d):
            out[e] += w * float(vv[e])
    return [o / total for o in out], mx + math.log(total)


# ----------------------------------------------------------------------------
# decoding against a ring-sharded KV cache
# ----------------------------------------------------------------------------

def decode_keys(x_hm: np.ndarray, lens: np.ndarray, b: int, kvh: int) -> np.ndarray:
    """The valid cached rows of sequence b, KV head kvh, over all shards in
    host order: x_hm [N][B][Hkv][c][d], lens [N][B] valid rows per shard."""
    N = x_hm.shape[0]
    return np.concatenate([x_hm[h, b, kvh, :int(lens[h][b])].astype(np.float64) for h in range(N)], axis=0)


def decode_attention(q: np.ndarray, k_hm: np.ndarray, v_hm: np.ndarray, lens: np.ndarray,
                     scale: float):
    """One decode step ([P2] 5.6; [P3] KV-cache distribution over the ring):
    q [B][Hq][d] holds each sequence's newest query token; the KV cache is
    sharded over N hosts, host h holding lens[h][b] valid rows of sequence b.
    The new token sees every cached key (all earlier tokens and its own, so
    the causal mask removes nothing), so each (sequence, query head) is the
    plain softmax(q K^T * scale) V over the valid keys of its KV head
    (query head g uses KV head g // (Hq / Hkv)).  Returns O [B][Hq][d],
    lse [B][Hq]; a sequence with no valid key gets O = 0, lse = -inf."""
    B, Hq, d = q.shape
    Hkv = k_hm.shape[2]
    group = Hq // Hkv
    O = np.zeros((B, Hq, d))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        for kvh in range(Hkv):
            k = decode_keys(k_hm, lens, b, kvh)
            v = decode_keys(v_hm, lens, b, kvh)
            heads = slice(kvh * group, (kvh + 1) * group)
            if k.shape[0] == 0:
                continue
            qq = q[b, heads].astype(np.float64)
            o, l_, _, _ = dense_attention(qq, k, v, np.ones((group, k.shape[0]), dtype=bool), scale)
            O[b, heads] = o
            lse[b, heads] = l_
    return O, lse


# ----------------------------------------------------------------------------
# the blockwise feedforward of the local block
# ----------------------------------------------------------------------------

def gelu(x: np.ndarray) -> np.ndarray:
    """GELU with the exact Gaussian CDF: x * Phi(x) = x (1 + erf(x / sqrt 2)) / 2."""
    from scipy.special import erf
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def blockwise_ffn(x: np.ndarray, w1: np.ndarray, w2: np.ndarray, block_rows: Optional[int] = None):
    """Feedforward of a block of tokens ([P2] 2 and 5.2-5.3: it acts on each
    token of the local block alone, so the layer's activation stays within
    2bch when it is evaluated block by block).  The pages do not fix the
    network; the reading is the standard two-layer feedforward with GELU:
    Y = GELU(X W1^T) W2^T, x [rows][h], w1 [f][h], w2 [h][f] (the weights of
    two linear layers, out-features major).  ``block_rows`` evaluates the
    rows in blocks of that size, as a blockwise schedule would; the result
    does not depend on it."""
    x = np.asarray(x, dtype=np.float64)
    w1 = np.asarray(w1, dtype=np.float64)
    w2 = np.asarray(w2, dtype=np.float64)
    n = x.shape[0]
    step = n if not block_rows else block_rows
    out = np.empty((n, w2.shape[0]))
    for r0 in range(0, n, max(step, 1)):
        hblk = gelu(x[r0:r0 + step] @ w1.T)
        out[r0:r0 + step] = hblk @ w2.T
    return out
