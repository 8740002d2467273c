"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test ties the oracle to something other than itself: values printed on
the pages (tests/golden), closed forms, brute force on tiny inputs, a library
softmax for the special case N = 1, order invariance, the merge identity and
finite differences for the gradient.  A dropped term, a wrong sign or index,
or a transposed operand in the oracle fails at least one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import cref, npref
import ra_synth as rs

C, S, Z = rs.LAYOUT_CONTIGUOUS, rs.LAYOUT_STRIPED, rs.LAYOUT_ZIGZAG


def _rand(seed, shape, scale=1.0):
    return rs.normal_f32(seed, shape, scale)


def _all_rows(nq_hosts, B, H, c, base=0):
    return cref.row_desc(range(base, base + nq_hosts), range(B), range(H), range(c))


# ---------------------------------------------------------------------------
# token layout, ring order, block counts: printed examples
# ---------------------------------------------------------------------------

def test_striped_token_lists(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "striped_tokens_N4.json")))
    N = g["n_hosts"]
    for dev, toks in g["tokens_per_device_prefix"].items():
        dev = int(dev)
        got_c = [cref.token_index(S, N, 1000, dev, r) for r in range(len(toks))]
        got_n = list(npref.token_index(S, N, 1000, dev, np.arange(len(toks))))
        assert got_c == toks and got_n == toks


def test_contiguous_split(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "contiguous_split_4dev_100tok.json")))
    N, c = g["n_hosts"], g["block_len"]
    for dev, (lo, hi) in g["device_token_range"].items():
        dev = int(dev)
        assert cref.token_index(C, N, c, dev, 0) == lo
        assert cref.token_index(C, N, c, dev, c - 1) == hi
        assert int(npref.token_index(C, N, c, dev, c - 1)) == hi


def test_ring_holdings(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "ring_holdings_N4.json")))
    N = g["n_hosts"]
    for step, held in g["held"].items():
        for host, blk in enumerate(held):
            assert npref.ring_order(N, host)[int(step)] == blk
    # every host sees every block exactly once in N steps (N - 1 transfers)
    for host in range(N):
        assert sorted(npref.ring_order(N, host)) == list(range(N))


def test_contiguous_causal_imbalance(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "contiguous_split_4dev_100tok.json")))
    N, c = g["n_hosts"], g["block_len"]
    work = []
    for i in range(N):
        blocks = 0
        pairs = 0
        for j in range(N):
            m = cref.block_mask(C, 1, N, c, i, j)
            blocks += int(m.any())
            pairs += int(m.sum())
        # block granularity: host i attends to i + 1 blocks of c keys
        rows, cols = g["attention_shape"][str(i)]
        assert blocks * c == cols and rows == c
        assert pairs == c * c * i + c * (c + 1) // 2
        work.append(blocks)
    assert work[-1] / work[0] == g["work_ratio_last_to_first"]


def test_striped_masks_are_triangles():
    # striped causal: block j <= i keeps r' <= r, block j > i keeps r' < r
    N, c = 4, 6
    tri_incl = np.tril(np.ones((c, c), dtype=np.uint8))
    tri_strict = np.tril(np.ones((c, c), dtype=np.uint8), -1)
    for i in range(N):
        for j in range(N):
            m = cref.block_mask(S, 1, N, c, i, j)
            assert np.array_equal(m, tri_incl if j <= i else tri_strict)


@pytest.mark.parametrize("N,c", [(1, 2), (2, 4), (3, 6), (4, 128), (8, 10)])
def test_zigzag_token_map_is_a_bijection(N, c):
    """Zigzag places every token of the sequence on exactly one (host, row)."""
    tc = sorted(cref.token_index(Z, N, c, h, r) for h in range(N) for r in range(c))
    tn = np.sort(np.concatenate([npref.token_index(Z, N, c, h, np.arange(c)) for h in range(N)]))
    assert tc == list(range(N * c))
    assert np.array_equal(tn, np.arange(N * c))


@pytest.mark.parametrize("N,c", [(2, 4), (3, 6), (4, 8), (8, 16)])
def test_zigzag_balances_causal_work(N, c):
    """The pages name Zigzag beside Striped as the causal layout that avoids
    load imbalance (P1, 工程实践指南, 因果掩码).  Closed form: every host sees
    exactly S(S+1)/(2N) visible (query, key) pairs, S = N c (half h = c/2:
    h^2 (2N-1) + h (h+1) per host), while contiguous hosts differ."""
    S_ = N * c
    h = c // 2
    want = S_ * (S_ + 1) // (2 * N)
    assert want == h * h * (2 * N - 1) + h * (h + 1)
    contig = []
    for i in range(N):
        got = sum(int(cref.block_mask(Z, 1, N, c, i, j).sum()) for j in range(N))
        assert got == want, (i, got, want)
        contig.append(sum(int(cref.block_mask(C, 1, N, c, i, j).sum()) for j in range(N)))
    assert len(set(contig)) == N                       # contiguous: every host differs


def test_mask_c_vs_numpy():
    for layout in (C, S, Z):
        for causal in (0, 1):
            for N, c in ((3, 5), (4, 4), (5, 2)):
                if layout == Z and c % 2:
                    continue
                for i in range(N):
                    for j in range(N):
                        mc = cref.block_mask(layout, causal, N, c, i, j)
                        tq = npref.token_index(layout, N, c, i, np.arange(c))
                        tk = npref.token_index(layout, N, c, j, np.arange(c))
                        mn = npref.explicit_mask(bool(causal), tq, tk)
                        assert np.array_equal(mc.astype(bool), mn)


# ---------------------------------------------------------------------------
# forward definition
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("layout,causal", [(C, 0), (C, 1), (S, 1), (Z, 1)])
@pytest.mark.parametrize("hq,hkv", [(2, 2), (4, 2)])
def test_forward_vs_brute_force(layout, causal, hq, hkv):
    N, B, c, d = 3, 2, 4, 5
    q = _rand(11, (N, B, hq, c, d))
    k = _rand(12, (N, B, hkv, c, d))
    v = _rand(13, (N, B, hkv, c, d))
    scale = 1.0 / math.sqrt(d)
    rows = _all_rows(N, B, hq, c)
    O, lse, mx, l = cref.attn_rows(q, k, v, n_hosts=N, layout=layout, causal=causal,
                                   rows=rows)
    group = hq // hkv
    for n, (h, b, hd, r) in enumerate(rows):
        tq = npref.token_index(layout, N, c, h, r)
        keys, vals, vis = [], [], []
        for j in range(N):
            for rk in range(c):
                keys.append(k[j, b, hd // group, rk]); vals.append(v[j, b, hd // group, rk])
                tk = npref.token_index(layout, N, c, j, rk)
                vis.append((not causal) or tk <= tq)
        o_bf, lse_bf = npref.brute_force_row(q[h, b, hd, r], keys, vals, vis, scale)
        assert np.allclose(O[n], o_bf, rtol=0, atol=1e-13)
        assert abs(lse[n] - lse_bf) <= 1e-13
        assert abs(mx[n] + math.log(l[n]) - lse[n]) <= 1e-13


@pytest.mark.parametrize("layout,causal,hq,hkv,c,d", [
    (C, 0, 2, 2, 37, 64), (C, 1, 4, 2, 33, 128), (S, 1, 2, 1, 40, 5), (Z, 1, 2, 2, 34, 128)])
def test_row_sets_equal_per_row_form(layout, causal, hq, hkv, c, d):
    """The row-set sweeps (up to 16 rows of one head per pass over the keys)
    reorder only the loop over independent rows: forward outputs, dQ, LSE and
    D are bitwise equal to the one-row-at-a-time form, for whole sets, ragged
    tail sets and rows in shuffled order (sets of one)."""
    N, B = 3, 1
    q = _rand(71, (N, B, hq, c, d)); k = _rand(72, (N, B, hkv, c, d))
    v = _rand(73, (N, B, hkv, c, d)); do = _rand(74, (N, B, hq, c, d))
    rows = _all_rows(N, B, hq, c)
    shuffled = rows[np.random.default_rng(75).permutation(len(rows))[:40]]
    for rr in (rows, shuffled):
        kw = dict(n_hosts=N, layout=layout, causal=causal, rows=rr)
        for a, b in zip(cref.attn_rows(q, k, v, **kw), cref.attn_rows(q, k, v, plain=True, **kw)):
            assert np.array_equal(a, b)
        for a, b in zip(cref.attn_bwd_q_rows(q, k, v, do, **kw),
                        cref.attn_bwd_q_rows(q, k, v, do, plain=True, **kw)):
            assert np.array_equal(a, b)


def test_single_host_noncausal_is_library_softmax():
    """N = 1, non-causal: plain softmax attention.  Checked against
    scipy.special.softmax and torch's fp64 CPU scaled_dot_product_attention."""
    from scipy.special import softmax, logsumexp
    import torch
    c, d, H = 17, 8, 3
    q = _rand(21, (1, 1, H, c, d)); k = _rand(22, (1, 1, H, c, d)); v = _rand(23, (1, 1, H, c, d))
    O, lse, _, _ = cref.attn_rows(q, k, v, n_hosts=1, layout=C, causal=0,
                                  rows=_all_rows(1, 1, H, c))
    O = O.reshape(H, c, d); lse = lse.reshape(H, c)
    for h in range(H):
        s = q[0, 0, h].astype(np.float64) @ k[0, 0, h].astype(np.float64).T / math.sqrt(d)
        ref = softmax(s, axis=1) @ v[0, 0, h].astype(np.float64)
        assert np.allclose(O[h], ref, atol=1e-13, rtol=0)
        assert np.allclose(lse[h], logsumexp(s, axis=1), atol=1e-13, rtol=0)
        t = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[0, 0, h].astype(np.float64))[None],
            torch.from_numpy(k[0, 0, h].astype(np.float64))[None],
            torch.from_numpy(v[0, 0, h].astype(np.float64))[None])
        assert np.allclose(O[h], t[0].numpy(), atol=1e-12, rtol=0)


def test_causal_library_sdpa_full_sequence():
    """Contiguous causal over the whole sequence equals torch's fp64 causal
    SDPA on the gathered sequence (a library routine with its own mask)."""
    import torch
    N, c, d, H = 4, 5, 8, 2
    q = _rand(31, (N, 1, H, c, d)); k = _rand(32, (N, 1, H, c, d)); v = _rand(33, (N, 1, H, c, d))
    for layout in (C, S):
        O, _, _, _ = cref.attn_rows(q, k, v, n_hosts=N, layout=layout, causal=1,
                                    rows=_all_rows(N, 1, H, c))
        O = O.reshape(N, H, c, d)
        qf, kf, vf = (torch.from_numpy(npref.gather_full(x, layout)[0]) for x in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(qf, kf, vf, is_causal=True)
        for h in range(N):
            t = npref.token_index(layout, N, c, h, np.arange(c))
            assert np.allclose(O[h], ref[:, t].numpy(), atol=1e-12, rtol=0)


@pytest.mark.parametrize("layout,causal", [(C, 0), (C, 1), (S, 1), (Z, 1)])
def test_numpy_dense_matches_c(layout, causal):
    N, B, H, c, d = 4, 1, 2, 8, 16
    q = _rand(41, (N, B, H, c, d)); k = _rand(42, (N, B, H, c, d)); v = _rand(43, (N, B, H, c, d))
    O, lse, mx, l = cref.attn_rows(q, k, v, n_hosts=N, layout=layout, causal=causal,
                                   rows=_all_rows(N, B, H, c))
    O = O.reshape(N, B, H, c, d); lse = lse.reshape(N, B, H, c)
    qf, kf, vf = (npref.gather_full(x, layout) for x in (q, k, v))
    S_ = N * c
    tok = np.arange(S_)
    mask = npref.explicit_mask(bool(causal), tok, tok)
    for h in range(H):
        Od, lsed, _, _ = npref.dense_attention(qf[0, h], kf[0, h], vf[0, h], mask, 1 / math.sqrt(d))
        for host in range(N):
            t = npref.token_index(layout, N, c, host, np.arange(c))
            assert np.allclose(O[host, 0, h], Od[t], atol=1e-12, rtol=0)
            assert np.allclose(lse[host, 0, h], lsed[t], atol=1e-12, rtol=0)


# ---------------------------------------------------------------------------
# blocked ring procedure: equals the definition, in any block order
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("layout,causal", [(C, 0), (C, 1), (S, 1), (Z, 1)])
def test_blocked_ring_all_orders(layout, causal):
    N, c, d = 4, 6, 8
    q = _rand(51, (N, 1, 1, c, d), 3.0)
    k = _rand(52, (N, 1, 1, c, d)); v = _rand(53, (N, 1, 1, c, d))
    scale = 1 / math.sqrt(d)
    for host in range(N):
        O, lse, _, _ = cref.attn_rows(q, k, v, n_hosts=N, layout=layout, causal=causal,
                                      rows=cref.row_desc([host], [0], [0], range(c)))
        for order in itertools.permutations(range(N)):
            for form in ("normalised", "numerator"):
                Ob, lseb, _, _ = npref.ring_host_blocked(q, k, v, host, layout=layout,
                                                         causal=bool(causal), scale=scale,
                                                         order=order, form=form)
                assert np.allclose(Ob, O, atol=1e-12, rtol=0)
                assert np.allclose(lseb, lse, atol=1e-12, rtol=0)


def test_blocked_ring_large_logits():
    """Q scaled x8 forces frequent max updates; the two accumulator forms and
    the definition still agree."""
    w = rs.workloads()["tiny_bigq"].replace(block_len=16)
    inp = rs.make_inputs(w)
    scale = 1 / math.sqrt(w.head_dim)
    for host in range(w.n_hosts):
        O, lse, _, _ = cref.attn_rows(inp.q_f32, inp.k_f32, inp.v_f32, n_hosts=w.n_hosts,
                                      layout=C, causal=0,
                                      rows=cref.row_desc([host], [0], [1], range(16)))
        for form in ("normalised", "numerator"):
            Ob, lseb, _, _ = npref.ring_host_blocked(inp.q_f32, inp.k_f32, inp.v_f32, host,
                                                     layout=C, causal=False, scale=scale,
                                                     head=1, kv_head=1, form=form)
            assert np.allclose(Ob, O, atol=1e-11, rtol=0)
            assert np.allclose(lseb, lse, atol=1e-11, rtol=0)


def test_strict_row_without_keys_stays_empty():
    """Striped strict block alone: row 0 sees no key.  The update keeps the
    initial state (m = -inf, l = 0, O = 0) instead of producing NaN."""
    N, c, d = 4, 5, 4
    q = _rand(61, (N, 1, 1, c, d)); k = _rand(62, (N, 1, 1, c, d)); v = _rand(63, (N, 1, 1, c, d))
    O, lse, m, ell = npref.ring_host_blocked(q, k, v, 0, layout=S, causal=True,
                                             scale=0.5, order=[1])
    assert m[0] == -np.inf and ell[0] == 0 and np.all(O[0] == 0) and lse[0] == -np.inf
    assert np.all(np.isfinite(O))


# ---------------------------------------------------------------------------
# merge identity
# ---------------------------------------------------------------------------

def test_merge_identity_random_partitions():
    rng = np.random.default_rng(71)
    c, Sk, d = 6, 40, 8
    q = rng.standard_normal((c, d)) * 2; k = rng.standard_normal((Sk, d)); v = rng.standard_normal((Sk, d))
    full = np.ones((c, Sk), dtype=bool)
    O, lse, m, l = npref.dense_attention(q, k, v, full, 0.4)
    for trial in range(20):
        a = rng.random(Sk) < rng.random()
        ma = np.broadcast_to(a, (c, Sk)); mb = ~ma
        Oa, lsea, m_a, la = npref.dense_attention(q, k, v, ma, 0.4)
        Ob, lseb, m_b, lb = npref.dense_attention(q, k, v, mb, 0.4)
        # l = l1 e^(m1 - m) + l2 e^(m2 - m)   ([P1] Online Softmax)
        with np.errstate(invalid="ignore"):
            ea = np.where(np.isfinite(m_a), np.exp(m_a - m), 0.0)
            eb = np.where(np.isfinite(m_b), np.exp(m_b - m), 0.0)
        assert np.allclose(la * ea + lb * eb, l, rtol=1e-12, atol=0)
        assert np.allclose(np.maximum(m_a, m_b), m)
        # log-space form
        assert np.allclose(np.logaddexp(lsea, lseb), lse, rtol=0, atol=1e-12)
        Om, lsem = npref.lse_merge(Oa, lsea, Ob, lseb)
        assert np.allclose(Om, O, atol=1e-12, rtol=0) and np.allclose(lsem, lse, atol=1e-12)


def test_merge_with_empty_parts():
    O = np.arange(6.0).reshape(2, 3)
    lse = np.array([0.3, -1.0])
    empty = np.full(2, -np.inf)
    Om, lsem = npref.lse_merge(O, lse, np.zeros_like(O), empty)
    assert np.array_equal(Om, O) and np.array_equal(lsem, lse)
    Om, lsem = npref.lse_merge(np.zeros_like(O), empty, np.zeros_like(O), empty)
    assert np.all(Om == 0) and np.all(lsem == -np.inf)


# ---------------------------------------------------------------------------
# closed forms (these also run at full scale against the GPU)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("layout", [C, S, Z])
def test_closed_form_q_zero(layout):
    """Q = 0: every visible score is 0, so l = number of visible keys,
    LSE = ln(count), O = mean of V over visible keys (count = t_q + 1 causal)."""
    N, c, d = 4, (8 if layout == Z else 7), 5             # zigzag halves need even c
    q = np.zeros((N, 1, 1, c, d), np.float32)
    k = _rand(81, (N, 1, 1, c, d)); v = _rand(82, (N, 1, 1, c, d))
    O, lse, mx, l = cref.attn_rows(q, k, v, n_hosts=N, layout=layout, causal=1,
                                   rows=_all_rows(N, 1, 1, c))
    vf = npref.gather_full(v, layout)[0, 0]
    csum = np.cumsum(vf, axis=0)
    for n, (h, _, _, r) in enumerate(_all_rows(N, 1, 1, c)):
        t = int(npref.token_index(layout, N, c, h, r))
        assert l[n] == t + 1 and mx[n] == 0.0
        assert abs(lse[n] - math.log(t + 1)) < 1e-14
        assert np.allclose(O[n], csum[t] / (t + 1), atol=1e-14, rtol=0)


def test_closed_form_index_digits():
    """Q = 0 and V = base-16 digits of the key's token index: the visible set
    of query token t is exactly {0..t} iff count = t+1 and sum = t(t+1)/2."""
    N, c, d = 4, 9, 8
    q = np.zeros((N, 1, 1, c, d), np.float32)
    k = _rand(91, (N, 1, 1, c, d))
    for layout in (C, S):
        v = np.zeros((N, 1, 1, c, d), np.float32)
        for h in range(N):
            t = npref.token_index(layout, N, c, h, np.arange(c))
            for ch in range(5):
                v[h, 0, 0, :, ch] = (t >> (4 * ch)) & 15
        O, _, _, l = cref.attn_rows(q, k, v, n_hosts=N, layout=layout, causal=1,
                                    rows=_all_rows(N, 1, 1, c))
        for n, (h, _, _, r) in enumerate(_all_rows(N, 1, 1, c)):
            t = int(npref.token_index(layout, N, c, h, r))
            num = O[n] * l[n]
            s = sum(num[ch] * 16 ** ch for ch in range(5))
            assert l[n] == t + 1 and round(s) == t * (t + 1) // 2


def test_closed_form_k_zero_prefix_mean():
    N, c, d = 3, 6, 4
    q = _rand(95, (N, 1, 1, c, d)); k = np.zeros((N, 1, 1, c, d), np.float32)
    v = _rand(96, (N, 1, 1, c, d))
    O, _, _, _ = cref.attn_rows(q, k, v, n_hosts=N, layout=C, causal=1,
                                rows=_all_rows(N, 1, 1, c))
    vf = npref.gather_full(v, C)[0, 0]
    ref = np.cumsum(vf, axis=0) / np.arange(1, N * c + 1)[:, None]
    assert np.allclose(O, ref, atol=1e-14, rtol=0)


# ---------------------------------------------------------------------------
# backward: finite differences and special cases
# ---------------------------------------------------------------------------

def _loss_and_grads(q, k, v, do, layout, causal, N):
    B, Hq, c, d = q.shape[1:]
    Hkv = k.shape[2]
    rows = _all_rows(N, B, Hq, c)
    O, lse, _, _ = cref.attn_rows(q, k, v, n_hosts=N, layout=layout, causal=causal, rows=rows)
    O = O.reshape(q.shape)
    loss = float((O * do.astype(np.float64)).sum())
    dQ, lse_q, D = cref.attn_bwd_q_rows(q, k, v, do, n_hosts=N, layout=layout,
                                        causal=causal, rows=rows)
    krows = cref.row_desc(range(N), range(B), range(Hkv), range(c))
    dK, dV = cref.attn_bwd_kv_rows(q, k, v, do, lse_q.reshape(N, B, Hq, c),
                                   D.reshape(N, B, Hq, c), n_hosts=N, layout=layout,
                                   causal=causal, rows=krows)
    return loss, dQ.reshape(q.shape), dK.reshape(k.shape), dV.reshape(v.shape)


@pytest.mark.parametrize("layout,causal,hq,hkv", [(C, 0, 2, 2), (C, 1, 2, 1), (S, 1, 2, 2)])
def test_backward_finite_differences(layout, causal, hq, hkv):
    """Central differences of L = sum(dO * O) in fp64 (h = 1e-6).  The inputs
    are float32 arrays, so perturbations are applied in a float64 copy through
    a wrapper that evaluates the dense numpy definition."""
    N, B, c, d = 2, 1, 3, 4
    q = _rand(101, (N, B, hq, c, d)); k = _rand(102, (N, B, hkv, c, d))
    v = _rand(103, (N, B, hkv, c, d)); do = _rand(104, (N, B, hq, c, d))
    _, dQ, dK, dV = _loss_and_grads(q, k, v, do, layout, causal, N)
    scale = 1 / math.sqrt(d)
    group = hq // hkv
    tok = np.arange(N * c)
    mask = npref.explicit_mask(bool(causal), tok, tok)

    def loss64(q64, k64, v64):
        qf, kf, vf = (npref.gather_full(x, layout) for x in (q64, k64, v64))
        dof = npref.gather_full(do, layout)
        tot = 0.0
        for b in range(B):
            for h in range(hq):
                O, _, _, _ = npref.dense_attention(qf[b, h], kf[b, h // group],
                                                   vf[b, h // group], mask, scale)
                tot += float((O * dof[b, h]).sum())
        return tot

    eps = 1e-6
    base = [x.astype(np.float64) for x in (q, k, v)]
    for which, grad in ((0, dQ), (1, dK), (2, dV)):
        x = base[which]
        for idx in np.ndindex(x.shape):
            xp = [b.copy() for b in base]; xm = [b.copy() for b in base]
            xp[which][idx] += eps; xm[which][idx] -= eps
            fd = (loss64(*xp) - loss64(*xm)) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-7 * max(1.0, abs(fd)), (which, idx, fd, grad[idx])


def test_backward_numpy_closed_form_matches_c():
    N, c, d = 3, 4, 6
    q = _rand(111, (N, 1, 1, c, d)); k = _rand(112, (N, 1, 1, c, d))
    v = _rand(113, (N, 1, 1, c, d)); do = _rand(114, (N, 1, 1, c, d))
    for layout, causal in ((C, 1), (S, 1), (C, 0)):
        _, dQ, dK, dV = _loss_and_grads(q, k, v, do, layout, causal, N)
        tok = np.arange(N * c)
        mask = npref.explicit_mask(bool(causal), tok, tok)
        qf, kf, vf, dof = (npref.gather_full(x, layout)[0, 0] for x in (q, k, v, do))
        dq, dk, dv = npref.dense_attention_grad(qf, kf, vf, dof, mask, 1 / math.sqrt(d))
        for h in range(N):
            t = npref.token_index(layout, N, c, h, np.arange(c))
            assert np.allclose(dQ[h, 0, 0], dq[t], atol=1e-12)
            assert np.allclose(dK[h, 0, 0], dk[t], atol=1e-12)
            assert np.allclose(dV[h, 0, 0], dv[t], atol=1e-12)


def test_backward_zero_keys_closed_form():
    """K = 0 under the causal contiguous mask: token t_q gives probability
    1/(t_q + 1) to each of tokens 0..t_q, so dQ = 0, dV_k is the reverse
    cumulative sum of dO_q/(q + 1), and dK_k = scale * sum over q >= k of
    (dO_q . v_k - D_q) Q_q/(q + 1) with D_q = dO_q . (prefix mean of V)_q."""
    N, c, d = 3, 5, 4
    S = N * c
    q = _rand(131, (N, 1, 1, c, d)); k = np.zeros((N, 1, 1, c, d), np.float32)
    v = _rand(132, (N, 1, 1, c, d)); do = _rand(133, (N, 1, 1, c, d))
    _, dQ, dK, dV = _loss_and_grads(q, k, v, do, C, 1, N)
    qf, vf, dof = (npref.gather_full(x, C)[0, 0].astype(np.float64) for x in (q, v, do))
    inv = 1.0 / np.arange(1, S + 1)
    dv_ref = np.cumsum((dof * inv[:, None])[::-1], axis=0)[::-1]
    D = (dof * np.cumsum(vf, axis=0) * inv[:, None]).sum(axis=1)
    dk_ref = np.array([sum((dof[t] @ vf[j] - D[t]) * inv[t] * qf[t] for t in range(j, S))
                       for j in range(S)]) / math.sqrt(d)
    assert np.abs(dQ).max() == 0.0
    assert np.allclose(dV.reshape(S, d), dv_ref, atol=1e-13, rtol=0)
    assert np.allclose(dK.reshape(S, d), dk_ref, atol=1e-13, rtol=0)


def test_backward_equal_value_rows_give_zero_dq_dk():
    """All V rows equal => O is that row for every query, dP - D = 0 on every
    visible pair, so dQ = dK = 0 exactly (up to rounding)."""
    N, c, d = 3, 4, 5
    q = _rand(121, (N, 1, 2, c, d)); k = _rand(122, (N, 1, 2, c, d))
    v = np.broadcast_to(_rand(123, (1, 1, 2, 1, d)), (N, 1, 2, c, d)).copy()
    do = _rand(124, (N, 1, 2, c, d))
    _, dQ, dK, dV = _loss_and_grads(q, k, v, do, C, 1, N)
    assert np.abs(dQ).max() < 1e-12 and np.abs(dK).max() < 1e-12
    assert np.abs(dV).max() > 0.1


def test_oracle_rejects_bad_rows():
    q = np.zeros((1, 1, 1, 4, 4), np.float32)
    k = np.zeros((2, 1, 1, 4, 4), np.float32)
    with pytest.raises(ValueError):
        cref.attn_rows(q, k, k, n_hosts=2, layout=C, causal=0,
                       rows=np.array([[1, 0, 0, 0]]))   # host 1's Q block not passed
    with pytest.raises(ValueError):
        cref.attn_rows(q, k, k, n_hosts=2, layout=C, causal=0,
                       rows=np.array([[0, 0, 0, 4]]))


def test_bf16_rounding_helper():
    x = np.array([1.0, 1.00390625, 1.005859375, -3.14159, 0.0, 65504.0], np.float32)
    b = rs.f32_to_bf16_bits(x)
    back = rs.bf16_bits_to_f32(b)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: nearest-even gives 1
    assert back[1] == 1.0
    assert back[2] == np.float32(1.0078125)
    assert back[0] == 1.0 and back[4] == 0.0
    assert abs(back[3] - x[3]) <= abs(x[3]) * 2 ** -8


# ---------------------------------------------------------------------------
# decoding against a ring-sharded KV cache ([P2] 5.6, [P3] KV-cache distribution)
# ---------------------------------------------------------------------------

def _decode_case(seed, N=3, B=2, Hq=4, Hkv=2, c=6, d=8):
    q = _rand(seed, (B, Hq, d))
    k = _rand(seed + 1, (N, B, Hkv, c, d))
    v = _rand(seed + 2, (N, B, Hkv, c, d))
    lens = np.random.default_rng(seed + 3).integers(0, c + 1, size=(N, B))
    lens[0, 0] = 0
    lens[N - 1, B - 1] = c
    return q, k, v, lens


def test_decode_vs_library_sdpa():
    """Each (sequence, head) equals torch's fp64 SDPA with query length 1 over
    the concatenated valid keys (a library routine, no mask)."""
    import torch
    q, k, v, lens = _decode_case(61)
    scale = 8 ** -0.5
    O, lse = npref.decode_attention(q, k, v, lens, scale)
    B, Hq, d = q.shape
    group = Hq // k.shape[2]
    for b in range(B):
        for hd in range(Hq):
            kk = npref.decode_keys(k, lens, b, hd // group)
            vv = npref.decode_keys(v, lens, b, hd // group)
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q[b, hd].astype(np.float64))[None, None], torch.from_numpy(kk)[None],
                torch.from_numpy(vv)[None])
            assert np.allclose(O[b, hd], ref[0, 0].numpy(), atol=1e-12, rtol=0)
            s = (kk @ q[b, hd].astype(np.float64)) * scale
            assert abs(lse[b, hd] - (s.max() + np.log(np.exp(s - s.max()).sum()))) < 1e-12


def test_decode_vs_brute_force_and_causal_last_row():
    """Pure-Python loops on a tiny case; and the decode of token S-1 equals the
    last row of causal attention over the whole contiguous sequence."""
    q, k, v, _ = _decode_case(71, N=2, B=1, Hq=2, Hkv=2, c=3, d=4)
    N, c = k.shape[0], k.shape[3]
    lens = np.full((N, 1), c)
    scale = 0.5
    O, lse = npref.decode_attention(q, k, v, lens, scale)
    for hd in range(2):
        keys = npref.decode_keys(k, lens, 0, hd)
        vals = npref.decode_keys(v, lens, 0, hd)
        ob, lb = npref.brute_force_row(q[0, hd], keys, vals, [True] * len(keys), scale)
        assert np.allclose(O[0, hd], ob, atol=1e-13) and abs(lse[0, hd] - lb) < 1e-13
    # whole-sequence view: replace the last token's query by q, causal row S-1
    qs = _rand(72, (N, 1, 2, c, 4))
    qs[N - 1, 0, :, c - 1] = q[0]
    full = cref.attn_rows(qs, k, v, n_hosts=N, layout=C, causal=1,
                          rows=cref.row_desc([N - 1], [0], [0, 1], [c - 1]), scale=scale)
    assert np.allclose(full[0], O[0], atol=1e-12) and np.allclose(full[1], lse[0], atol=1e-12)


def test_decode_closed_form_q_zero():
    """Q = 0: every score is 0, so O is the mean of the valid V rows and
    LSE = ln(number of valid keys)."""
    q, k, v, lens = _decode_case(81)
    O, lse = npref.decode_attention(np.zeros_like(q), k, v, lens, 0.3)
    B, Hq = q.shape[:2]
    group = Hq // k.shape[2]
    for b in range(B):
        n = int(lens[:, b].sum())
        for hd in range(Hq):
            vv = np.concatenate([v[h, b, hd // group, :lens[h, b]] for h in range(k.shape[0])])
            assert np.allclose(O[b, hd], vv.mean(axis=0), atol=1e-13)
            assert abs(lse[b, hd] - np.log(n)) < 1e-13


def test_decode_shards_merge_in_any_order():
    """The ring form: per-shard partials merged with the LSE merge, in any
    host order, give the decode over all shards; an empty shard is neutral."""
    q, k, v, lens = _decode_case(91, N=4)
    scale = 8 ** -0.5
    O, lse = npref.decode_attention(q, k, v, lens, scale)
    N = k.shape[0]
    parts = []
    for h in range(N):
        one = np.zeros_like(lens)
        one[h] = lens[h]
        parts.append(npref.decode_attention(q, k, v, one, scale))
    for order in itertools.permutations(range(N)):
        Om, lm = parts[order[0]]
        for h in order[1:]:
            Om, lm = npref.lse_merge(Om, lm, *parts[h])
        assert np.allclose(Om, O, atol=1e-12) and np.allclose(lm, lse, atol=1e-12)
    # a sequence with no valid key at all: O = 0, lse = -inf
    Oz, lz = npref.decode_attention(q, k, v, np.zeros_like(lens), scale)
    assert np.all(Oz == 0) and np.all(lz == -np.inf)


# ---------------------------------------------------------------------------
# blockwise feedforward ([P2] 2, 5.2-5.3)
# ---------------------------------------------------------------------------

def test_gelu_vs_math_erf_and_torch():
    import torch
    x = np.concatenate([np.linspace(-9, 9, 181), _rand(101, (50,)).astype(np.float64) * 3])
    g = npref.gelu(x)
    loops = np.array([0.5 * v * (1 + math.erf(v / math.sqrt(2))) for v in x])
    assert np.allclose(g, loops, atol=1e-15, rtol=1e-14)
    t = torch.nn.functional.gelu(torch.from_numpy(x), approximate="none").numpy()
    assert np.allclose(g, t, atol=1e-15, rtol=1e-14)
    assert npref.gelu(np.array([0.0]))[0] == 0.0


def test_ffn_brute_force_and_identity():
    """Pure-Python loops on a tiny case; identity weights reduce the
    feedforward to the elementwise GELU."""
    x = _rand(111, (3, 4)).astype(np.float64)
    w1 = _rand(112, (5, 4)).astype(np.float64)
    w2 = _rand(113, (4, 5)).astype(np.float64)
    y = npref.blockwise_ffn(x, w1, w2)
    for r in range(3):
        hid = []
        for j in range(5):
            acc = sum(float(x[r, k]) * float(w1[j, k]) for k in range(4))
            hid.append(0.5 * acc * (1 + math.erf(acc / math.sqrt(2))))
        for i in range(4):
            assert abs(y[r, i] - sum(hid[j] * float(w2[i, j]) for j in range(5))) < 1e-13
    eye = np.eye(4)
    assert np.allclose(npref.blockwise_ffn(x, eye, eye), npref.gelu(x), atol=1e-15)


def test_ffn_is_per_token():
    """Blocks of any size give the same result, and permuting the tokens
    permutes the output: the feedforward never mixes tokens."""
    x = _rand(121, (37, 16)).astype(np.float64)
    w1 = _rand(122, (24, 16)).astype(np.float64) * 0.25
    w2 = _rand(123, (16, 24)).astype(np.float64) * 0.25
    y = npref.blockwise_ffn(x, w1, w2)
    for b in (1, 5, 16, 37, 64):
        assert np.allclose(npref.blockwise_ffn(x, w1, w2, block_rows=b), y, atol=1e-13)
    perm = np.random.default_rng(124).permutation(37)
    assert np.allclose(npref.blockwise_ffn(x[perm], w1, w2), y[perm], atol=1e-13)
