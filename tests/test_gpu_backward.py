"""GPU parity of the backward path against the fp64 oracle's closed-form
gradient (calls through the C ABI).  Tolerance: max-abs 2e-2 on dQ, dK, dV
(fp32 outputs from bf16 inputs); the relative L2 error is reported too.
The forward that produces (O, LSE) for the backward is the library's own."""
import numpy as np
import pytest

import ra_synth as rs
from oracle import cref
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu
C, S, Z = rs.LAYOUT_CONTIGUOUS, rs.LAYOUT_STRIPED, rs.LAYOUT_ZIGZAG
TOL_BWD = 2e-2


@pytest.fixture(scope="module")
def torch():
    import torch
    assert torch.cuda.is_available()
    import long_context_transformers_amd as ra
    ra.version()
    return torch


def _fwd(torch, w, q, k, v):
    import long_context_transformers_amd as ra
    O, lse, _ = H.run_ring_fwd(w, None, tensors=(q, k, v))
    return O, lse


def _oracle_grads(w, inp, q_rows, k_rows, heads_for_kv):
    """dQ on (host, b, head, row) samples; dK, dV on (host, b, kv_head, row)
    samples whose kv_head is in heads_for_kv (LSE and D of every query row
    of those groups come from the oracle's own forward)."""
    N, B, Hq, Hkv, c, d = w.n_hosts, w.batch, w.heads_q, w.heads_kv, w.block_len, w.head_dim
    dq_desc = cref.row_desc(range(N), range(B), range(Hq), q_rows)
    dQ, _, _ = cref.attn_bwd_q_rows(inp.q_f32, inp.k_f32, inp.v_f32, inp.do_f32, n_hosts=N,
                                    layout=w.layout, causal=w.mask, rows=dq_desc)
    group = Hq // Hkv
    qheads = [g * group + u for g in heads_for_kv for u in range(group)]
    all_desc = cref.row_desc(range(N), range(B), qheads, range(c))
    O, lse, _, _ = cref.attn_rows(inp.q_f32, inp.k_f32, inp.v_f32, n_hosts=N, layout=w.layout,
                                  causal=w.mask, rows=all_desc)
    dO = inp.do_f32[:, :, qheads].reshape(-1, d).astype(np.float64)
    Dv = (dO * O).sum(axis=1)
    lse_all = np.full((N, B, Hq, c), np.nan)
    D_all = np.full((N, B, Hq, c), np.nan)
    lse_all[:, :, qheads] = lse.reshape(N, B, len(qheads), c)
    D_all[:, :, qheads] = Dv.reshape(N, B, len(qheads), c)
    kv_desc = cref.row_desc(range(N), range(B), heads_for_kv, k_rows)
    dK, dV = cref.attn_bwd_kv_rows(inp.q_f32, inp.k_f32, inp.v_f32, inp.do_f32, lse_all, D_all,
                                   n_hosts=N, layout=w.layout, causal=w.mask, rows=kv_desc)
    return dQ, dK, dV


def _compare(name, got, want, tol=TOL_BWD):
    err = float(np.abs(got - want).max())
    rel = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30))
    H.report(name, tol=tol, max_abs=err, rel_l2=rel)
    assert np.all(np.isfinite(got))
    assert err <= tol, (name, err)
    return err


def _gather(t, rows, heads=None):
    import torch
    idx = torch.as_tensor(rows, device=t.device)
    x = t if heads is None else t[:, :, heads]
    return x.index_select(3, idx).float().cpu().numpy().reshape(-1, t.shape[-1]).astype(np.float64)


SMALL = [
    # (hq, hkv, d, layout, mask, N, c)
    (2, 2, 128, C, 0, 3, 200),
    (2, 2, 128, C, 1, 4, 130),
    (4, 2, 128, S, 1, 3, 96),
    (4, 1, 128, C, 1, 2, 257),
    (2, 2, 128, S, 1, 4, 64),
    (2, 2, 64, C, 0, 2, 300),
    (4, 2, 64, S, 1, 3, 129),
    (2, 2, 128, Z, 1, 3, 256),
    (4, 2, 128, Z, 1, 4, 512),
    (4, 1, 64, Z, 1, 2, 256),
    (2, 2, 128, Z, 1, 1, 256),
    (2, 2, 128, Z, 0, 3, 130),
]


@pytest.mark.parametrize("hq,hkv,d,layout,mask,N,c", SMALL)
def test_ring_bwd_small_all_rows(torch, hq, hkv, d, layout, mask, N, c):
    import long_context_transformers_amd as ra
    w = rs.Workload("bwd_small", 95, 1, hq, hkv, d, N, c, rs.DT_BF16, mask, layout, 0, N)
    inp = rs.make_inputs(w, with_do=True)
    q, k, v, do = (H.dev_tensor(x, w.dtype) for x in (inp.q_dev, inp.k_dev, inp.v_dev, inp.do_dev))
    O, lse = _fwd(torch, w, q, k, v)
    cfg = H.cfg_of(w)
    dQ = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    dK = torch.empty(k.shape, dtype=torch.float32, device="cuda")
    dV = torch.empty(v.shape, dtype=torch.float32, device="cuda")
    ws = torch.empty(ra.ring_workspace_size(cfg, True), dtype=torch.uint8, device="cuda")
    stats = ra.ring_bwd(cfg, q, k, v, O, lse, do, dQ, dK, dV, ws, torch.cuda.current_stream(),
                        torch.cuda.Stream())
    torch.cuda.synchronize()
    assert stats["compute_steps"] == N and stats["transfers"] == N - 1
    rows = np.arange(c)
    dQr, dKr, dVr = _oracle_grads(w, inp, rows, rows, range(hkv))
    tag = f"{hq}/{hkv} d={d} layout={layout} mask={mask} N={N} c={c}"
    _compare(f"ring_bwd dQ {tag}", _gather(dQ, rows), dQr)
    _compare(f"ring_bwd dK {tag}", _gather(dK, rows), dKr)
    _compare(f"ring_bwd dV {tag}", _gather(dV, rows), dVr)


def test_block_bwd_accumulates(torch):
    """ra_block_bwd over a host's schedule, summed over hosts, equals the
    oracle's gradient (and dK/dV received through dk_in are carried)."""
    import long_context_transformers_amd as ra
    w = rs.Workload("blk_bwd", 96, 1, 2, 2, 64, 3, 100, rs.DT_BF16, 1, C, 0, 3)
    inp = rs.make_inputs(w, with_do=True)
    q, k, v, do = (H.dev_tensor(x, w.dtype) for x in (inp.q_dev, inp.k_dev, inp.v_dev, inp.do_dev))
    O, lse = _fwd(torch, w, q, k, v)
    dims = H.dims_of(w)
    D = torch.empty(lse.shape, dtype=torch.float32, device="cuda")
    for i in range(w.n_hosts):
        ra.bwd_preprocess(dims, O[i], do[i], D[i])
    dQ = torch.zeros(q.shape, dtype=torch.float32, device="cuda")
    dK = torch.zeros(k.shape, dtype=torch.float32, device="cuda")
    dV = torch.zeros(v.shape, dtype=torch.float32, device="cuda")
    for i in range(w.n_hosts):
        for st in ra.schedule(w.n_hosts, i, w.block_len, w.layout, w.mask):
            j = st["src"]
            ra.block_bwd(dims, q[i], k[j], v[j], do[i], lse[i], D[i], w.mask, st["q_offset"],
                         st["kv_offset"], st["stride"], dQ[i], dK[j], dV[j])
    torch.cuda.synchronize()
    rows = np.arange(w.block_len)
    dQr, dKr, dVr = _oracle_grads(w, inp, rows, rows, range(w.heads_kv))
    _compare("block_bwd dQ", _gather(dQ, rows), dQr)
    _compare("block_bwd dK", _gather(dK, rows), dKr)
    _compare("block_bwd dV", _gather(dV, rows), dVr)


@pytest.mark.parametrize("layout", [C, Z])
def test_ring_bwd_concurrent_equals_serialized(torch, layout):
    import long_context_transformers_amd as ra
    w = rs.Workload("bwd_race", 97, 1, 4, 4, 128, 8, 512, rs.DT_BF16, 1, layout, 0, 8)
    inp = rs.make_inputs(w, with_do=True)
    q, k, v, do = (H.dev_tensor(x, w.dtype) for x in (inp.q_dev, inp.k_dev, inp.v_dev, inp.do_dev))
    O, lse = _fwd(torch, w, q, k, v)
    outs = []
    for flags, delay in ((0, 0), (ra.RA_FLAG_SERIALIZE, 0), (0, 200)):
        cfg = H.cfg_of(w, flags, delay)
        dQ = torch.empty(q.shape, dtype=torch.float32, device="cuda")
        dK = torch.empty(k.shape, dtype=torch.float32, device="cuda")
        dV = torch.empty(v.shape, dtype=torch.float32, device="cuda")
        ws = torch.empty(ra.ring_workspace_size(cfg, True), dtype=torch.uint8, device="cuda")
        ra.ring_bwd(cfg, q, k, v, O, lse, do, dQ, dK, dV, ws, torch.cuda.current_stream(),
                    torch.cuda.Stream())
        torch.cuda.synchronize()
        outs.append((dQ, dK, dV))
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert torch.equal(a, b)


@pytest.mark.timeout(900)
def test_ring_bwd_64k_causal(torch):
    """Backward workload at full size: 32 heads, d = 128, 8 hosts x 8192.
    dQ on 1024 seeded rows of every head; dK, dV on 1024 seeded key rows of
    4 seeded heads (their LSE and D need the oracle's full forward)."""
    import long_context_transformers_amd as ra
    w = rs.workloads()["bwd_64k"]
    inp = H.inputs(w, with_do=True)
    q, k, v, do = (H.dev_tensor(x, w.dtype) for x in (inp.q_dev, inp.k_dev, inp.v_dev, inp.do_dev))
    O, lse = _fwd(torch, w, q, k, v)
    # forward of the backward workload, sampled
    rows = rs.row_sample(w, 1024)
    Os, Ls = H.sampled(O, lse, w, rows)
    O_ref, lse_ref = H.oracle_rows(w, inp, rows)
    H.report("ring_fwd bwd_64k", tol={"max_abs_O": 2e-2, "max_abs_lse": 1e-3}, max_abs_O=float(np.abs(Os - O_ref).max()),
             max_abs_lse=float(np.abs(Ls - lse_ref).max()))
    assert np.abs(Os - O_ref).max() <= 2e-2 and np.abs(Ls - lse_ref).max() <= 1e-3
    cfg = H.cfg_of(w)
    dQ = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    dK = torch.empty(k.shape, dtype=torch.float32, device="cuda")
    dV = torch.empty(v.shape, dtype=torch.float32, device="cuda")
    ws = torch.empty(ra.ring_workspace_size(cfg, True), dtype=torch.uint8, device="cuda")
    ra.ring_bwd(cfg, q, k, v, O, lse, do, dQ, dK, dV, ws, torch.cuda.current_stream(),
                torch.cuda.Stream())
    torch.cuda.synchronize()
    krows = rs.row_sample(w, 1024, seed=9500 + w.cfg)
    heads = sorted(np.random.default_rng(9600 + w.cfg).choice(w.heads_kv, 4, replace=False).tolist())
    dQr, dKr, dVr = _oracle_grads(w, inp, rows, krows, heads)
    _compare("ring_bwd bwd_64k dQ", _gather(dQ, rows), dQr)
    _compare("ring_bwd bwd_64k dK", _gather(dK, krows, heads), dKr)
    _compare("ring_bwd bwd_64k dV", _gather(dV, krows, heads), dVr)


@pytest.mark.timeout(600)
def test_ring_bwd_zigzag_mid_sampled(torch):
    """Causal zigzag backward, 8 hosts x 2048 (each half spans 8 key tiles
    of 128), 8 query heads on 4 KV heads, d = 128: dQ on 512 seeded rows of
    every head, dK and dV on 512 seeded key rows of 2 seeded KV heads."""
    import long_context_transformers_amd as ra
    w = rs.Workload("bwd_zz_mid", 98, 1, 8, 4, 128, 8, 2048, rs.DT_BF16, 1, Z, 0, 8)
    inp = H.inputs(w, with_do=True)
    q, k, v, do = (H.dev_tensor(x, w.dtype) for x in (inp.q_dev, inp.k_dev, inp.v_dev, inp.do_dev))
    O, lse = _fwd(torch, w, q, k, v)
    cfg = H.cfg_of(w)
    dQ = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    dK = torch.empty(k.shape, dtype=torch.float32, device="cuda")
    dV = torch.empty(v.shape, dtype=torch.float32, device="cuda")
    ws = torch.empty(ra.ring_workspace_size(cfg, True), dtype=torch.uint8, device="cuda")
    stats = ra.ring_bwd(cfg, q, k, v, O, lse, do, dQ, dK, dV, ws, torch.cuda.current_stream(),
                        torch.cuda.Stream())
    torch.cuda.synchronize()
    assert stats["skipped_blocks"] == 0
    rows = rs.row_sample(w, 512)
    krows = rs.row_sample(w, 512, seed=9500 + w.cfg)
    heads = [1, 3]
    dQr, dKr, dVr = _oracle_grads(w, inp, rows, krows, heads)
    _compare("ring_bwd zigzag mid dQ", _gather(dQ, rows), dQr)
    _compare("ring_bwd zigzag mid dK", _gather(dK, krows, heads), dKr)
    _compare("ring_bwd zigzag mid dV", _gather(dV, krows, heads), dVr)


@pytest.mark.timeout(900)
def test_ring_bwd_64k_closed_form_zero_keys(torch):
    """Backward workload at full size with K = 0, every row checked.
    All scores are 0, so each visible key gets probability 1 / (t_q + 1)
    (causal contiguous: token t_q sees tokens 0..t_q).  The gradient of
    softmax attention then has closed forms in token order:
      dQ = scale dS K = 0 exactly (every product has a zero factor);
      dV_k = sum over q >= k of dO_q / (q + 1), a reverse cumulative sum;
      dK_k = scale sum over q >= k of (dO_q . v_k - D_q) Q_q / (q + 1),
    with D_q = dO_q . O_q and O_q the prefix mean of V.  dV is compared on
    every key row of every head, dK on 256 seeded key rows of 4 seeded
    heads (the d x d suffix sums of Q_q dO_q^T are evaluated only there)."""
    import long_context_transformers_amd as ra
    w = rs.workloads()["bwd_64k"]
    N, Hq, c, d = w.n_hosts, w.heads_q, w.block_len, w.head_dim
    S = N * c
    inp = H.inputs(w, with_do=True)
    q, v, do = (H.dev_tensor(x, w.dtype) for x in (inp.q_dev, inp.v_dev, inp.do_dev))
    k = torch.zeros_like(q)
    O, lse = _fwd(torch, w, q, k, v)
    cfg = H.cfg_of(w)
    dQ = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    dK = torch.empty(k.shape, dtype=torch.float32, device="cuda")
    dV = torch.empty(v.shape, dtype=torch.float32, device="cuda")
    ws = torch.empty(ra.ring_workspace_size(cfg, True), dtype=torch.uint8, device="cuda")
    ra.ring_bwd(cfg, q, k, v, O, lse, do, dQ, dK, dV, ws, torch.cuda.current_stream(),
                torch.cuda.Stream())
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(dQ)) == 0, "dQ must be exactly zero when K = 0"

    def tok(x, h):        # host-major [N][1][H][c][d] -> token-ordered [S, d] of head h (fp64)
        return np.ascontiguousarray(x[:, 0, h]).reshape(S, d).astype(np.float64)

    inv = 1.0 / np.arange(1, S + 1, dtype=np.float64)
    scale = 1.0 / np.sqrt(d)
    err_v = 0.0
    for h in range(Hq):
        dOh = tok(inp.do_f32, h)
        want = np.cumsum((dOh * inv[:, None])[::-1], axis=0)[::-1]
        got = dV[:, 0, h].float().cpu().numpy().reshape(S, d)
        err_v = max(err_v, float(np.abs(got - want).max()))
        assert np.all(np.isfinite(got))
    H.report("ring_bwd bwd_64k K=0 dV (all rows)", tol=TOL_BWD, max_abs=err_v)
    assert err_v <= TOL_BWD, err_v

    rng = np.random.default_rng(9700 + w.cfg)
    heads = sorted(rng.choice(Hq, 4, replace=False).tolist())
    err_k = 0.0
    for h in heads:
        Qh, Vh, dOh = tok(inp.q_f32, h), tok(inp.v_f32, h), tok(inp.do_f32, h)
        Oh = np.cumsum(Vh, axis=0) * inv[:, None]
        Dq = (dOh * Oh).sum(axis=1)
        ks = np.sort(np.unique(np.concatenate([[0, 1, S - 1], rng.choice(S, 253, replace=False)])))[::-1]
        M = np.zeros((d, d))          # sum over q >= k of Q_q dO_q^T / (q + 1)
        u = np.zeros(d)               # sum over q >= k of D_q Q_q / (q + 1)
        hi = S
        want = np.empty((len(ks), d))
        for i, kr in enumerate(ks):
            wq = Qh[kr:hi] * inv[kr:hi, None]
            M += wq.T @ dOh[kr:hi]
            u += (wq * Dq[kr:hi, None]).sum(axis=0)
            hi = kr
            want[i] = scale * (M @ Vh[kr] - u)
        got = dK[:, 0, h].float().cpu().numpy().reshape(S, d)[ks]
        err_k = max(err_k, float(np.abs(got - want).max()))
    H.report("ring_bwd bwd_64k K=0 dK (sampled rows)", tol=TOL_BWD, max_abs=err_k, heads=heads)
    assert err_k <= TOL_BWD, err_k
