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
    """t[h, r] = token index of local row r on host h (contiguous or striped),
    pinned against the oracle's token map on a few rows."""
    r = np.arange(c, dtype=np.int64)[None, :]
    h = np.arange(N, dtype=np.int64)[:, None]
    t = r * N + h if layout == S else h * c + r
    for hh, rr in ((0, 0), (N - 1, c - 1), (1, c // 2), (N // 2, 7)):
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
