"""GPU parity of the ring backward at the sizes that are timed, and of the
fp32 backward, against the fp64 oracle (calls through the C ABI).

- fp32 inputs (the tiny exact-check workload with both seed sets, plus small
  causal, striped and grouped-head shapes): every row, max-abs 1e-4 times
  max(1, largest reference magnitude).
- The non-causal 32K ring (8 hosts x 4096, 8 heads, d = 128) and a striped
  causal ring at c = 4096 with grouped heads: dQ on 1024 seeded rows of every
  (host, head), dK and dV on 1024 seeded key rows of seeded KV heads.
- The striped causal 256K ring over all 8 hosts (32 heads, c = 32768), the
  workload whose forward + backward the benchmark times: forward and dQ on
  seeded rows of every (host, head); with K = 0 every score is 0 and the
  gradient has closed forms in token order (dQ = 0 exactly, dV a reverse
  cumulative sum over every row, dK on seeded rows).
Tolerances: max-abs 2e-2 on dQ, dK, dV and O, 1e-3 on LSE for bf16; 1e-4
(scaled as above) for fp32.  The forward that produces (O, LSE) is the library's own."""
import numpy as np
import pytest

import ra_synth as rs
from oracle import cref
from tests import gpu_helpers as H
from tests.test_gpu_backward import _compare, _gather, _oracle_grads

pytestmark = pytest.mark.gpu
C, S = rs.LAYOUT_CONTIGUOUS, rs.LAYOUT_STRIPED
TOL_BWD = 2e-2
TOL_F32 = 1e-4


@pytest.fixture(scope="module")
def torch():
    import torch
    assert torch.cuda.is_available()
    import long_context_transformers_amd as ra
    ra.version()
    return torch


def _ring_fwd_bwd(torch, w, q, k, v, do):
    import long_context_transformers_amd as ra
    O, lse, fst = H.run_ring_fwd(w, None, tensors=(q, k, v))
    cfg = H.cfg_of(w)
    dQ = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    dK = torch.empty(k.shape, dtype=torch.float32, device="cuda")
    dV = torch.empty(v.shape, dtype=torch.float32, device="cuda")
    ws = torch.empty(ra.ring_workspace_size(cfg, True), dtype=torch.uint8, device="cuda")
    st = ra.ring_bwd(cfg, q, k, v, O, lse, do, dQ, dK, dV, ws, torch.cuda.current_stream(),
                     torch.cuda.Stream())
    torch.cuda.synchronize()
    del ws
    return O, lse, dQ, dK, dV, fst, st


F32 = [
    # (workload or (hq, hkv, d, layout, mask, N, c))
    "tiny",
    "tiny_bigq",
    (4, 2, 64, S, 1, 3, 100),
    (2, 2, 128, C, 1, 2, 70),
    (4, 1, 128, C, 0, 2, 65),
]


@pytest.mark.parametrize("spec", F32, ids=[s if isinstance(s, str) else "x".join(map(str, s)) for s in F32])
def test_ring_bwd_f32_all_rows(torch, spec):
    if isinstance(spec, str):
        w = rs.workloads()[spec]
    else:
        hq, hkv, d, layout, mask, N, c = spec
        w = rs.Workload("bwd_f32", 94, 1, hq, hkv, d, N, c, rs.DT_F32, mask, layout, 0, N)
    inp = rs.make_inputs(w, with_do=True)
    q, k, v, do = (H.dev_tensor(x, w.dtype) for x in (inp.q_dev, inp.k_dev, inp.v_dev, inp.do_dev))
    O, lse, dQ, dK, dV, _, st = _ring_fwd_bwd(torch, w, q, k, v, do)
    assert st["compute_steps"] == w.n_hosts
    rows = np.arange(w.block_len)
    dQr, dKr, dVr = _oracle_grads(w, inp, rows, rows, range(w.heads_kv))
    # fp32 gradients: 1e-4 relative to the gradient's scale.  The LSE the
    # forward hands over is fp32, so every recomputed P carries a relative
    # error up to |LSE| 2^-24 (4e-6 at |LSE| = 60, reached with Q x 8), which
    # the gradient inherits at its own magnitude (|dK| up to 26 there).
    for nm, got, ref in (("dQ", dQ, dQr), ("dK", dK, dKr), ("dV", dV, dVr)):
        tol = TOL_F32 * max(1.0, float(np.abs(ref).max()))
        _compare(f"ring_bwd f32 {w.name} {spec} {nm}", _gather(got, rows), ref, tol)


def _sampled_bwd(torch, w, kv_heads, n_rows=1024):
    inp = H.inputs(w, with_do=True)
    q, k, v, do = (H.dev_tensor(x, w.dtype) for x in (inp.q_dev, inp.k_dev, inp.v_dev, inp.do_dev))
    O, lse, dQ, dK, dV, fst, st = _ring_fwd_bwd(torch, w, q, k, v, do)
    assert st["compute_steps"] == w.n_hosts and st["transfers"] == w.n_hosts - 1
    assert st["copy_kind"] == 1, "ring transfers must run on the DMA engines on MI355X"
    rows = rs.row_sample(w, n_rows)
    krows = rs.row_sample(w, n_rows, seed=9500 + w.cfg)
    dQr, dKr, dVr = _oracle_grads(w, inp, rows, krows, kv_heads)
    _compare(f"ring_bwd {w.name} dQ", _gather(dQ, rows), dQr)
    _compare(f"ring_bwd {w.name} dK", _gather(dK, krows, kv_heads), dKr)
    _compare(f"ring_bwd {w.name} dV", _gather(dV, krows, kv_heads), dVr)


@pytest.mark.timeout(900)
def test_ring_bwd_noncausal_32k_sampled(torch):
    """The non-causal 32K ring (8 hosts x 4096, 8 heads, d = 128): dQ on 1024
    seeded rows of every (host, head); dK, dV on 1024 seeded key rows of 2
    seeded KV heads."""
    w = rs.workloads()["noncausal_32k"]
    heads = sorted(np.random.default_rng(9600 + w.cfg).choice(w.heads_kv, 2, replace=False).tolist())
    _sampled_bwd(torch, w, heads)


@pytest.mark.timeout(900)
def test_ring_bwd_striped_causal_4096_gqa_sampled(torch):
    """Striped causal ring, 8 hosts x 4096, 8 query heads on 2 KV heads,
    d = 128 (32 key tiles per block, every host's blocks TRI_INCL or
    TRI_STRICT): dQ on 1024 seeded rows of every (host, head); dK, dV on 1024
    seeded key rows of KV head 1."""
    w = rs.Workload("bwd_striped_gqa_N8_c4096", 92, 1, 8, 2, 128, 8, 4096, rs.DT_BF16,
                    rs.MASK_CAUSAL, S, 0, 8)
    _sampled_bwd(torch, w, [1])


def _token_order(layout, N, c):
    """t[h, r] = token index of local row r on host h (contiguous, striped or
    zigzag), pinned against the oracle's token map on a few rows."""
    r = np.arange(c, dtype=np.int64)[None, :]
    h = np.arange(N, dtype=np.int64)[:, None]
    if layout == rs.LAYOUT_ZIGZAG:
        half = c // 2
        t = np.where(r < half, h * half + r, (2 * N - 1 - h) * half + (r - half))
    else:
        t = r * N + h if layout == S else h * c + r
    for hh, rr in ((0, 0), (N - 1, c - 1), (1, c // 2), (N // 2, 7), (0, c // 2 - 1), (N - 1, c // 2)):
        assert t[hh, rr] == cref.token_index(layout, N, c, hh, rr)
    return t


@pytest.mark.timeout(1200)
def test_ring_fwd_bwd_striped_256k_all_hosts(torch):
    """The timed workload: striped causal 256K over all 8 hosts (32 heads,
    d = 128, c = 32768), forward + backward in the configuration the
    benchmark launches.  (1) Random inputs: O and LSE on 16 seeded rows of
    every (host, head), and dQ on the same rows.  (2) K = 0: every visible
    score is 0, so the forward gives LSE = ln(t + 1) and O = the prefix mean
    of V; the backward gives dQ = 0 exactly, dV_k = sum over t_q >= t_k of
    dO_q / (t_q + 1) on every row of every head, and
    dK_k = scale sum over t_q >= t_k of (dO_q . v_k - D_q) Q_q / (t_q + 1)
    on 64 seeded rows of 2 seeded heads."""
    base = rs.workloads()["causal_256k_striped"]
    w = base.replace(name="causal_256k_striped_H32_N8_c32768_all_hosts", host_begin=0,
                     host_end=base.n_hosts)
    N, Hq, c, d = w.n_hosts, w.heads_q, w.block_len, w.head_dim
    n = N * c
    # inputs drawn on the device (seeded); the oracle reads the same bf16
    # values, widened to float32 on the host
    print(f"[inputs] drawing {w.name} on the device", flush=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(9100 + w.cfg)
    q, k, v, do = (torch.randn(rs.q_shape(w), generator=g, device="cuda").to(torch.bfloat16)
                   for _ in range(4))
    inp = rs.Inputs(*(t.float().cpu().numpy() for t in (q, k, v)), None, None, None, q_host_base=0,
                    do_f32=do.float().cpu().numpy())
    O, lse, dQ, dK, dV, fst, st = _ring_fwd_bwd(torch, w, q, k, v, do)
    assert fst["skipped_blocks"] == 0 and st["skipped_blocks"] == 0
    rows = rs.row_sample(w, 16)
    Os, Ls = H.sampled(O, lse, w, rows)
    O_ref, lse_ref = H.oracle_rows(w, inp, rows)
    eo, el = float(np.abs(Os - O_ref).max()), float(np.abs(Ls - lse_ref).max())
    H.report(f"ring_fwd {w.name}", tol={"max_abs_O": 2e-2, "max_abs_lse": 1e-3}, max_abs_O=eo, max_abs_lse=el)
    assert eo <= 2e-2 and el <= 1e-3
    desc = cref.row_desc(range(N), range(w.batch), range(Hq), rows)
    dQr, _, _ = cref.attn_bwd_q_rows(inp.q_f32, inp.k_f32, inp.v_f32, inp.do_f32, n_hosts=N,
                                     layout=w.layout, causal=w.mask, rows=desc)
    _compare(f"ring_bwd {w.name} dQ", _gather(dQ, rows), dQr)
    del O, lse, dQ, dK, dV, inp

    # (2) zero keys: closed forms in token order
    k.zero_()
    O, lse, dQ, dK, dV, _, _ = _ring_fwd_bwd(torch, w, q, k, v, do)
    assert int(torch.count_nonzero(dQ)) == 0, "dQ must be exactly zero when K = 0"
    del dQ
    t = torch.as_tensor(_token_order(w.layout, N, c), device="cuda")
    want = torch.log((t + 1).double()).float()[:, None, None, :].expand_as(lse)
    ulp = torch.abs(torch.nextafter(want, torch.full_like(want, np.inf)) - want)
    err_l = float(((lse - want).abs() / ulp).max())
    H.report(f"{w.name} K=0 lse (all rows)", max_err_ulps=err_l)
    assert err_l <= 2.0
    tq = t.cpu().numpy()
    order = np.argsort(tq.reshape(-1))            # token position -> flat (host, row)

    def tok(x, h):   # host-major [N][1][H][c][d] device tensor -> token-ordered [n, d] fp64 (host)
        return x[:, 0, h].double().cpu().numpy().reshape(n, d)[order]

    inv = 1.0 / np.arange(1, n + 1, dtype=np.float64)
    err_v = 0.0
    for h in range(Hq):
        want_v = np.cumsum((tok(do, h) * inv[:, None])[::-1], axis=0)[::-1]
        got = tok(dV, h)
        assert np.all(np.isfinite(got))
        err_v = max(err_v, float(np.abs(got - want_v).max()))
    H.report(f"{w.name} K=0 dV (all rows)", tol=TOL_BWD, max_abs=err_v)
    assert err_v <= TOL_BWD
    rng = np.random.default_rng(9700 + w.cfg)
    heads = sorted(rng.choice(Hq, 2, replace=False).tolist())
    scale = 1.0 / np.sqrt(d)
    err_k = 0.0
    for h in heads:
        Qh, Vh, dOh = tok(q, h), tok(v, h), tok(do, h)
        Oh = np.cumsum(Vh, axis=0) * inv[:, None]
        Dq = (dOh * Oh).sum(axis=1)
        ks = np.sort(np.unique(np.concatenate([[0, 1, n - 1], rng.choice(n, 61, replace=False)])))[::-1]
        M = np.zeros((d, d))
        u = np.zeros(d)
        hi = n
        want_k = np.empty((len(ks), d))
        for i, kr in enumerate(ks):
            wq = Qh[kr:hi] * inv[kr:hi, None]
            M += wq.T @ dOh[kr:hi]
            u += (wq * Dq[kr:hi, None]).sum(axis=0)
            hi = kr
            want_k[i] = scale * (M @ Vh[kr] - u)
        got = tok(dK, h)[ks]
        err_k = max(err_k, float(np.abs(got - want_k).max()))
    H.report(f"{w.name} K=0 dK (sampled rows)", tol=TOL_BWD, max_abs=err_k, heads=heads)
    assert err_k <= TOL_BWD


# ---------------------------------------------------------------------------
# one host's share of the backward (a subset of the hosts)
# ---------------------------------------------------------------------------

def _bwd_hosts(torch, w, q, k, v, O, lse, do, hb, he, flags=0):
    """ra_ring_bwd for hosts [hb, he): q, O, lse, do hold those hosts' blocks."""
    import long_context_transformers_amd as ra
    wh = w.replace(host_begin=hb, host_end=he)
    cfg = H.cfg_of(wh, flags)
    dQ = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    dK = torch.empty(k.shape, dtype=torch.float32, device="cuda")
    dV = torch.empty(v.shape, dtype=torch.float32, device="cuda")
    ws = torch.empty(ra.ring_workspace_size(cfg, True), dtype=torch.uint8, device="cuda")
    st = ra.ring_bwd(cfg, q, k, v, O, lse, do, dQ, dK, dV, ws, torch.cuda.current_stream(), torch.cuda.Stream())
    torch.cuda.synchronize()
    return dQ, dK, dV, st


SUBSETS = [
    # (hq, hkv, d, layout, mask, N, c, dtype)
    (2, 2, 128, C, 1, 4, 130, rs.DT_BF16),
    (4, 2, 128, S, 1, 3, 192, rs.DT_BF16),
    (2, 2, 128, rs.LAYOUT_ZIGZAG, 1, 3, 256, rs.DT_BF16),
    (4, 1, 64, C, 0, 3, 100, rs.DT_BF16),
    (2, 2, 64, S, 1, 4, 64, rs.DT_F32),
]


@pytest.mark.parametrize("hq,hkv,d,layout,mask,N,c,dtype", SUBSETS)
def test_ring_bwd_one_host_shares_sum_to_full_ring(torch, hq, hkv, d, layout, mask, N, c, dtype):
    """Every host's one-host backward: its dQ equals the full ring's dQ of that
    host bit for bit (same kernels, same step order), and the dK, dV
    contributions of all hosts sum to the full ring's gradient and to the
    oracle's.  A two-host range equals the sum of its two one-host runs."""
    w = rs.Workload("bwd_hosts", 91, 1, hq, hkv, d, N, c, dtype, mask, layout, 0, N)
    inp = rs.make_inputs(w, with_do=True)
    q, k, v, do = (H.dev_tensor(x, w.dtype) for x in (inp.q_dev, inp.k_dev, inp.v_dev, inp.do_dev))
    O, lse, dQf, dKf, dVf, _, _ = _ring_fwd_bwd(torch, w, q, k, v, do)
    sK = torch.zeros(k.shape, dtype=torch.float64, device="cuda")
    sV = torch.zeros_like(sK)
    for h in range(N):
        dQh, dKh, dVh, st = _bwd_hosts(torch, w, q[h:h + 1], k, v, O[h:h + 1], lse[h:h + 1], do[h:h + 1], h, h + 1)
        assert torch.equal(dQh[0], dQf[h]), h
        assert st["transfers"] == N - 1
        sK += dKh.double()
        sV += dVh.double()
    scale = max(1.0, float(dKf.abs().max()), float(dVf.abs().max()))
    assert float((sK - dKf.double()).abs().max()) <= 1e-5 * scale
    assert float((sV - dVf.double()).abs().max()) <= 1e-5 * scale
    tol = TOL_F32 * scale if dtype == rs.DT_F32 else TOL_BWD
    rows = np.arange(c)
    _, dKr, dVr = _oracle_grads(w, inp, rows, rows, range(hkv))
    _compare(f"one-host shares summed {w.name} {layout}/{mask} dK", _gather(sK, rows), dKr, tol)
    _compare(f"one-host shares summed {w.name} {layout}/{mask} dV", _gather(sV, rows), dVr, tol)
    if N >= 3:
        dQ2, dK2, dV2, _ = _bwd_hosts(torch, w, q[1:3], k, v, O[1:3], lse[1:3], do[1:3], 1, 3)
        assert torch.equal(dQ2, dQf[1:3])
        d1 = _bwd_hosts(torch, w, q[1:2], k, v, O[1:2], lse[1:2], do[1:2], 1, 2)
        d2 = _bwd_hosts(torch, w, q[2:3], k, v, O[2:3], lse[2:3], do[2:3], 2, 3)
        assert float((dK2.double() - d1[1].double() - d2[1].double()).abs().max()) <= 1e-5 * scale
        assert float((dV2.double() - d1[2].double() - d2[2].double()).abs().max()) <= 1e-5 * scale


def _one_host_inputs(torch, w, seed):
    """Device-drawn bf16 inputs of a one-host workload (Q, dO of the host, the
    K/V pool), and their float32 copies for the oracle."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    q = torch.randn(rs.q_shape(w, 1), generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn(rs.kv_shape(w), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn(rs.kv_shape(w), generator=g, device="cuda").to(torch.bfloat16)
    do = torch.randn(rs.q_shape(w, 1), generator=g, device="cuda").to(torch.bfloat16)
    inp = rs.Inputs(q.float().cpu().numpy(), k.float().cpu().numpy(), v.float().cpu().numpy(), None, None, None,
                    q_host_base=w.host_begin, do_f32=do.float().cpu().numpy())
    return q, k, v, do, inp


def _one_host_fwd_bwd(torch, w, q, k, v, do):
    O, lse, _ = H.run_ring_fwd(w, None, tensors=(q, k, v))
    dQ, dK, dV, st = _bwd_hosts(torch, w, q, k, v, O, lse, do, w.host_begin, w.host_end)
    return O, lse, dQ, dK, dV, st


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("name", ["causal_256k_contig", "causal_256k_striped", "causal_256k_zigzag",
                                  "striped_786k_gqa"])
def test_ring_bwd_one_host_share_full_size(torch, name):
    """One host's share of the backward at full size: the last host of the
    causal 256K workload (contiguous, striped and zigzag, 32 heads,
    c = 32768) and of
    the 786K striped workload with 32 query heads on 8 KV heads (c = 49152).
    dQ on 128 seeded rows of every head against the oracle.  For the 256K
    workloads also K = 0, where every visible score is 0: dQ = 0 exactly, and
    the host's contribution to dV_k is the sum over its own queries q with
    t_q >= t_k of dO_q / (t_q + 1), checked on every key row of every head;
    its contribution to dK_k, scale times the sum over the same queries of
    (dO_q . v_k - D_q) Q_q / (t_q + 1), on 48 seeded key tokens of 2 heads."""
    w = rs.workloads()[name]
    N, c, d, Hq, Hkv = w.n_hosts, w.block_len, w.head_dim, w.heads_q, w.heads_kv
    print(f"[inputs] drawing {w.name} on the device", flush=True)
    q, k, v, do, inp = _one_host_inputs(torch, w, 9200 + w.cfg)
    O, lse, dQ, dK, dV, st = _one_host_fwd_bwd(torch, w, q, k, v, do)
    assert st["compute_steps"] == N - st["skipped_blocks"] and st["transfers"] == N - 1
    rows = rs.row_sample(w, 128)
    desc = cref.row_desc([w.host_begin], range(w.batch), range(Hq), rows)
    dQr, _, _ = cref.attn_bwd_q_rows(inp.q_f32, inp.k_f32, inp.v_f32, inp.do_f32, n_hosts=N, layout=w.layout,
                                     causal=w.mask, rows=desc, q_host_base=w.host_begin)
    _compare(f"one-host ring_bwd {w.name} dQ", _gather(dQ, rows), dQr)
    if Hq != Hkv:
        return
    del O, lse, dQ, dK, dV, inp
    k.zero_()
    O, lse, dQ, dK, dV, _ = _one_host_fwd_bwd(torch, w, q, k, v, do)
    assert int(torch.count_nonzero(dQ)) == 0, "dQ must be exactly zero when K = 0"
    n = N * c
    t_all = _token_order(w.layout, N, c)                        # [N, c] token of (host, row)
    order = np.argsort(t_all.reshape(-1))                       # token -> flat (host, row)
    tq = t_all[w.host_begin]                                    # tokens of the host's query rows
    inv = 1.0 / (tq + 1.0)
    err_v = 0.0
    for h in range(Hq):
        wq = do[0, 0, h].double().cpu().numpy() * inv[:, None]  # dO_q / (t_q + 1) at token t_q
        acc = np.zeros((n, d))
        acc[tq] = wq
        want = np.cumsum(acc[::-1], axis=0)[::-1]               # sum over q with t_q >= t_k, token order
        got = dV[:, 0, h].double().cpu().numpy().reshape(n, d)[order]
        assert np.all(np.isfinite(got))
        err_v = max(err_v, float(np.abs(got - want).max()))
    H.report(f"one-host {w.name} K=0 dV (all rows)", tol=TOL_BWD, max_abs=err_v)
    assert err_v <= TOL_BWD
    rng = np.random.default_rng(9800 + w.cfg)
    scale = 1.0 / np.sqrt(d)
    err_k = 0.0
    qsort = np.argsort(tq)[::-1]                                 # the host's rows by descending token
    for h in sorted(rng.choice(Hq, 2, replace=False).tolist()):
        Vt = v[:, 0, h].double().cpu().numpy().reshape(n, d)[order]
        pref = np.cumsum(Vt, axis=0)
        Qh = q[0, 0, h].double().cpu().numpy()
        dOh = do[0, 0, h].double().cpu().numpy()
        Oq = pref[tq] / (tq + 1.0)[:, None]                      # prefix mean of V up to t_q
        Dq = (dOh * Oq).sum(axis=1)
        ks = np.sort(np.unique(np.concatenate([[0, n - 1], rng.choice(n, 46, replace=False)])))[::-1]
        M = np.zeros((d, d))
        u = np.zeros(d)
        pos = 0
        want = np.empty((len(ks), d))
        for i, kt in enumerate(ks):
            while pos < len(qsort) and tq[qsort[pos]] >= kt:
                r = qsort[pos]
                wr = Qh[r] * inv[r]
                M += np.outer(wr, dOh[r])
                u += Dq[r] * wr
                pos += 1
            want[i] = scale * (M @ Vt[kt] - u)
        got = dK[:, 0, h].double().cpu().numpy().reshape(n, d)[order][ks]
        err_k = max(err_k, float(np.abs(got - want).max()))
    H.report(f"one-host {w.name} K=0 dK (sampled rows)", tol=TOL_BWD, max_abs=err_k)
    assert err_k <= TOL_BWD
