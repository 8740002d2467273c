"""GPU parity of the forward path against the fp64 oracle (calls go through
the C ABI).  Tolerances: bf16 O max-abs 2e-2 and LSE max-abs 1e-3; fp32
1e-4 on both.  Large workloads are checked on 1024 seeded rows per head."""
import math

import numpy as np
import pytest

import ra_synth as rs
from oracle import cref, npref
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

TOL = {rs.DT_BF16: (2e-2, 1e-3), rs.DT_F32: (1e-4, 1e-4)}
C, S = rs.LAYOUT_CONTIGUOUS, rs.LAYOUT_STRIPED


@pytest.fixture(scope="module")
def torch():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import long_context_transformers_amd as ra
    ra.version()
    return torch


@pytest.fixture(autouse=True)
def _seed(torch):
    torch.manual_seed(1234)


def _check(name, w, O, lse, O_ref, lse_ref):
    tol_o, tol_l = TOL[w.dtype]
    eo = float(np.abs(O - O_ref).max())
    el = float(np.abs(lse - lse_ref).max())
    H.report(name, tol={"max_abs_O": tol_o, "max_abs_lse": tol_l}, max_abs_O=eo, max_abs_lse=el, rows=O.shape[0])
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(lse))
    assert eo <= tol_o and el <= tol_l


# ---------------------------------------------------------------------------
# block-level: drive one host through ra_block_fwd in ring order
# ---------------------------------------------------------------------------

SMALL = [
    # (dtype, d, hq, hkv, layout, mask, N, c)
    (rs.DT_BF16, 128, 2, 2, C, 0, 3, 200),
    (rs.DT_BF16, 128, 4, 1, C, 1, 3, 200),
    (rs.DT_BF16, 128, 8, 2, S, 1, 4, 130),
    (rs.DT_BF16, 64, 2, 2, S, 1, 3, 96),
    (rs.DT_BF16, 64, 4, 2, C, 1, 2, 257),
    (rs.DT_BF16, 128, 2, 2, C, 1, 2, 1),
    (rs.DT_F32, 64, 2, 2, C, 1, 3, 70),
    (rs.DT_F32, 128, 4, 2, S, 1, 3, 65),
    (rs.DT_F32, 64, 2, 1, C, 0, 2, 33),
]


@pytest.mark.parametrize("dtype,d,hq,hkv,layout,mask,N,c", SMALL)
def test_block_fwd_ring_order_small(torch, dtype, d, hq, hkv, layout, mask, N, c):
    import long_context_transformers_amd as ra
    w = rs.Workload("small", 90, 2, hq, hkv, d, N, c, dtype, mask, layout, 0, N)
    inp = rs.make_inputs(w)
    dims = H.dims_of(w)
    q = H.dev_tensor(inp.q_dev, dtype)
    k = H.dev_tensor(inp.k_dev, dtype)
    v = H.dev_tensor(inp.v_dev, dtype)
    rows_all = cref.row_desc(range(N), range(w.batch), range(hq), range(c))
    O_ref, lse_ref, _, _ = cref.attn_rows(inp.q_f32, inp.k_f32, inp.v_f32, n_hosts=N, layout=layout,
                                          causal=mask, rows=rows_all)
    O_out = torch.empty((N, w.batch, hq, c, d), dtype=H.torch_dtype(dtype), device="cuda")
    lse = torch.empty((N, w.batch, hq, c), dtype=torch.float32, device="cuda")
    for i in range(N):
        m = torch.empty((w.batch, hq, c), dtype=torch.float32, device="cuda")
        l = torch.empty_like(m)
        O = torch.empty((w.batch, hq, c, d), dtype=torch.float32, device="cuda")
        ra.state_init(dims, m, l, O)
        for st in ra.schedule(N, i, c, layout, mask):
            ra.block_fwd(dims, q[i], k[st["src"]], v[st["src"]], mask, st["q_offset"],
                         st["kv_offset"], st["stride"], m, l, O)
        ra.finalize(dims, m, l, O, O_out[i], lse[i])
    torch.cuda.synchronize()
    _check(f"block_fwd {dtype=} {d=} {hq}/{hkv} {layout=} {mask=} {N=} {c=}", w,
           O_out.float().cpu().numpy().reshape(-1, d).astype(np.float64),
           lse.cpu().numpy().reshape(-1).astype(np.float64), O_ref, lse_ref)


@pytest.mark.parametrize("layout,mask", [(C, 0), (C, 1), (S, 1)])
def test_block_fwd_growing_logits(torch, layout, mask):
    """Keys scaled up with their token index (x0.5 .. x6) and Q x 2, so a
    row's running max keeps climbing across the key tiles and the lazy
    rescale fires again and again along the ring; all rows against the
    oracle at the bf16 tolerances."""
    import long_context_transformers_amd as ra
    N, c, d, hq, hkv = 3, 320, 128, 2, 2
    w = rs.Workload("growing", 92, 1, hq, hkv, d, N, c, rs.DT_BF16, mask, layout, 0, N, q_scale=2.0)
    inp = rs.make_inputs(w)
    S_len = N * c
    for h in range(N):
        t = np.array([npref.token_index(layout, N, c, h, r) for r in range(c)], dtype=np.float32)
        f = (0.5 + 5.5 * t / S_len).astype(np.float32)
        bits = rs.f32_to_bf16_bits(inp.k_f32[h] * f[None, None, :, None])
        inp.k_dev[h] = bits
        inp.k_f32[h] = rs.bf16_bits_to_f32(bits)
    dims = H.dims_of(w)
    q, k, v = (H.dev_tensor(x, w.dtype) for x in (inp.q_dev, inp.k_dev, inp.v_dev))
    rows_all = cref.row_desc(range(N), range(w.batch), range(hq), range(c))
    O_ref, lse_ref, _, _ = cref.attn_rows(inp.q_f32, inp.k_f32, inp.v_f32, n_hosts=N, layout=layout,
                                          causal=mask, rows=rows_all)
    # within a block the keys' scale grows tile by tile: the row max of the
    # last 64-key tile of host 0's block exceeds that of its first tile by far
    # more than the rescale threshold (8 in log2 units) on most rows
    s0 = np.einsum("hrd,hkd->hrk", inp.q_f32[0, 0].astype(np.float64),
                   inp.k_f32[0, 0].astype(np.float64)) / np.sqrt(d) * 1.4426950408889634
    grow = s0[:, :, -64:].max(axis=2) - s0[:, :, :64].max(axis=2)
    assert np.median(grow) > 8
    O_out = torch.empty((N, w.batch, hq, c, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((N, w.batch, hq, c), dtype=torch.float32, device="cuda")
    for i in range(N):
        m = torch.empty((w.batch, hq, c), dtype=torch.float32, device="cuda")
        l = torch.empty_like(m)
        O = torch.empty((w.batch, hq, c, d), dtype=torch.float32, device="cuda")
        ra.state_init(dims, m, l, O)
        for st in ra.schedule(N, i, c, layout, mask):
            ra.block_fwd(dims, q[i], k[st["src"]], v[st["src"]], mask, st["q_offset"],
                         st["kv_offset"], st["stride"], m, l, O)
        ra.finalize(dims, m, l, O, O_out[i], lse[i])
    torch.cuda.synchronize()
    _check(f"block_fwd growing logits {layout=} {mask=}", w,
           O_out.float().cpu().numpy().reshape(-1, d).astype(np.float64),
           lse.cpu().numpy().reshape(-1).astype(np.float64), O_ref, lse_ref)


def test_block_fwd_any_order_and_empty_rows(torch):
    """Order invariance on the GPU, and a striped strict block alone leaves
    row 0 (no visible key) at the initial state without NaN."""
    import long_context_transformers_amd as ra
    N, c, d = 4, 96, 128
    w = rs.Workload("order", 91, 1, 2, 2, d, N, c, rs.DT_BF16, 1, S, 0, N)
    inp = rs.make_inputs(w)
    dims = H.dims_of(w)
    q, k, v = (H.dev_tensor(x, w.dtype) for x in (inp.q_dev, inp.k_dev, inp.v_dev))
    host = 1
    rows = cref.row_desc([host], [0], range(2), range(c))
    O_ref, lse_ref, _, _ = cref.attn_rows(inp.q_f32, inp.k_f32, inp.v_f32, n_hosts=N, layout=S,
                                          causal=1, rows=rows)
    steps = ra.schedule(N, host, c, S, 1)
    for order in ([0, 1, 2, 3], [3, 1, 0, 2], [2, 3, 1, 0]):
        m = torch.empty((1, 2, c), dtype=torch.float32, device="cuda")
        l = torch.empty_like(m)
        O = torch.empty((1, 2, c, d), dtype=torch.float32, device="cuda")
        ra.state_init(dims, m, l, O)
        for s in order:
            st = steps[s]
            ra.block_fwd(dims, q[host], k[st["src"]], v[st["src"]], 1, st["q_offset"], st["kv_offset"],
                         st["stride"], m, l, O)
        Ob = torch.empty((1, 2, c, d), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((1, 2, c), dtype=torch.float32, device="cuda")
        ra.finalize(dims, m, l, O, Ob, lse)
        torch.cuda.synchronize()
        _check(f"order {order}", w, Ob.float().cpu().numpy().reshape(-1, d).astype(np.float64),
               lse.cpu().numpy().reshape(-1).astype(np.float64), O_ref, lse_ref)
    # strict block alone (host 1 against block 2: r' < r)
    st = steps[3]
    assert st["src"] == 2 and st["cls"] == ra.RA_BLK_TRI_STRICT
    m = torch.empty((1, 2, c), dtype=torch.float32, device="cuda")
    l = torch.empty_like(m)
    O = torch.empty((1, 2, c, d), dtype=torch.float32, device="cuda")
    ra.state_init(dims, m, l, O)
    ra.block_fwd(dims, q[host], k[2], v[2], 1, st["q_offset"], st["kv_offset"], st["stride"], m, l, O)
    torch.cuda.synchronize()
    mc, lc, Oc = m.cpu().numpy(), l.cpu().numpy(), O.cpu().numpy()
    assert np.all(mc[:, :, 0] == -np.inf) and np.all(lc[:, :, 0] == 0) and np.all(Oc[:, :, 0] == 0)
    assert np.all(np.isfinite(mc[:, :, 1:])) and np.all(np.isfinite(Oc))
    # every other row r sees exactly r keys (Q = anything, count via l with Q = 0 below)


# ---------------------------------------------------------------------------
# ring driver on the five workloads
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "tiny_bigq"])
def test_ring_fwd_tiny_f32_all_rows(torch, name):
    w = rs.workloads()[name]
    inp = H.inputs(w)
    O, lse, stats = H.run_ring_fwd(w, inp)
    rows = np.arange(w.block_len)
    Os, Ls = H.sampled(O, lse, w, rows)
    O_ref, lse_ref = H.oracle_rows(w, inp, rows)
    _check(f"ring_fwd {name}", w, Os, Ls, O_ref, lse_ref)
    assert stats["compute_steps"] == w.n_hosts and stats["transfers"] == w.n_hosts - 1


def _check_residency(w, stats):
    """Per simulated host the forward holds its query block, its output
    block, the K/V block being folded and the incoming K/V block -- the 6
    blocks of [P2] 5.3 (6bch with Hq = Hkv; grouped heads make K/V blocks
    smaller) -- plus the fp32 numerator O and the m, l rows.  The ring
    buffers the library holds per host (resident_bytes_per_host) are the
    receive double buffer (2 slots x K, V) and that fp32 state."""
    el = 2 if w.dtype == rs.DT_BF16 else 4
    rows = w.batch * w.heads_q * w.block_len
    q_blk = rows * w.head_dim * el
    kv_blk = w.batch * w.heads_kv * w.block_len * w.head_dim * el
    fp32_state = 4 * (2 * rows + rows * w.head_dim)
    assert stats["resident_bytes_per_host"] == 4 * kv_blk + fp32_state
    blocks = q_blk + q_blk + (stats["resident_bytes_per_host"] - fp32_state)   # Q, O out, K/V x 2
    assert blocks <= 6 * q_blk
    H.report(f"residency {w.name}", blocks_of_6=blocks / q_blk, fp32_state_bytes=fp32_state)


def test_ring_fwd_noncausal_32k(torch):
    w = rs.workloads()["noncausal_32k"]
    inp = H.inputs(w)
    O, lse, stats = H.run_ring_fwd(w, inp)
    rows = rs.row_sample(w, 1024)
    Os, Ls = H.sampled(O, lse, w, rows)
    O_ref, lse_ref = H.oracle_rows(w, inp, rows)
    _check("ring_fwd noncausal_32k", w, Os, Ls, O_ref, lse_ref)
    assert stats["compute_steps"] == 8 and stats["transfers"] == 7
    assert stats["copy_kind"] == 1, "ring transfers must run on the DMA engines on MI355X"
    _check_residency(w, stats)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["causal_256k_contig", "causal_256k_striped"])
def test_ring_fwd_causal_256k(torch, name):
    w = rs.workloads()[name]
    inp = H.inputs(w, q_hosts_only=True)
    O, lse, stats = H.run_ring_fwd(w, inp)
    rows = rs.row_sample(w, 1024)
    Os, Ls = H.sampled(O, lse, w, rows)
    O_ref, lse_ref = H.oracle_rows(w, inp, rows)
    _check(f"ring_fwd {name}", w, Os, Ls, O_ref, lse_ref)
    assert stats["skipped_blocks"] == 0   # host 7 is the last host: nothing above it
    _check_residency(w, stats)


@pytest.mark.timeout(900)
def test_ring_fwd_striped_786k_gqa(torch):
    w = rs.workloads()["striped_786k_gqa"]
    inp = H.inputs(w, q_hosts_only=True)
    O, lse, stats = H.run_ring_fwd(w, inp)
    rows = rs.row_sample(w, 1024)
    Os, Ls = H.sampled(O, lse, w, rows)
    O_ref, lse_ref = H.oracle_rows(w, inp, rows)
    _check("ring_fwd striped_786k_gqa", w, Os, Ls, O_ref, lse_ref)


# ---------------------------------------------------------------------------
# closed forms at full scale: every row, no sampling
# ---------------------------------------------------------------------------

@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["causal_256k_contig", "causal_256k_striped", "striped_786k_gqa"])
def test_index_digit_closed_form_full_scale(torch, name):
    """Q = 0 and V = base-16 digits of each key's token index: every score is
    exactly 0, so the fp32 state holds l = number of visible keys and O = sum
    of their digits, both exact.  count = t + 1 and sum = t (t + 1) / 2 for
    every row prove that the visible set is exactly {0 .. t}."""
    import long_context_transformers_amd as ra
    w = rs.workloads()[name]
    N, c, d, i = w.n_hosts, w.block_len, w.head_dim, w.host_begin
    dims = H.dims_of(w)
    k = torch.randn((N, 1, w.heads_kv, c, d), device="cuda").to(torch.bfloat16)
    v = torch.zeros((N, 1, w.heads_kv, c, d), dtype=torch.float32, device="cuda")
    for h in range(N):
        t = torch.as_tensor(npref.token_index(w.layout, N, c, h, np.arange(c)), device="cuda")
        for ch in range(5):
            v[h, :, :, :, ch] = ((t >> (4 * ch)) & 15).float()[None, None, :]
    v = v.to(torch.bfloat16)
    q = torch.zeros((1, w.heads_q, c, d), dtype=torch.bfloat16, device="cuda")
    m = torch.empty((1, w.heads_q, c), dtype=torch.float32, device="cuda")
    l = torch.empty_like(m)
    O = torch.empty((1, w.heads_q, c, d), dtype=torch.float32, device="cuda")
    ra.state_init(dims, m, l, O)
    for st in ra.schedule(N, i, c, w.layout, w.mask):
        ra.block_fwd(dims, q, k[st["src"]], v[st["src"]], w.mask, st["q_offset"], st["kv_offset"],
                     st["stride"], m, l, O)
    torch.cuda.synchronize()
    t = torch.as_tensor(npref.token_index(w.layout, N, c, i, np.arange(c)), device="cuda",
                        dtype=torch.float64)
    lc = l.double()
    num = O[..., :5].double()
    s = sum(num[..., ch] * 16 ** ch for ch in range(5))
    assert torch.equal(lc, (t + 1)[None, None, :].expand_as(lc))
    assert torch.equal(s, (t * (t + 1) / 2)[None, None, :].expand_as(s))
    assert torch.all(m == 0)
    H.report(f"closed form {name}", rows=int(lc.numel()))


# ---------------------------------------------------------------------------
# the kernels' mask predicate, bit-exact
# ---------------------------------------------------------------------------

def test_mask_tile_bit_exact(torch):
    import long_context_transformers_amd as ra
    for layout in (C, S):
        for N, c in ((4, 64), (8, 100), (3, 7)):
            for i in range(N):
                for st in ra.schedule(N, i, c, layout, 1):
                    out = torch.empty(c * c, dtype=torch.uint8, device="cuda")
                    ra.mask_tile(st["q_offset"], st["kv_offset"], st["stride"], c, c, out)
                    got = out.cpu().numpy().reshape(c, c)
                    want = cref.block_mask(layout, 1, N, c, i, st["src"])
                    assert np.array_equal(got, want), (layout, N, c, i, st)


# ---------------------------------------------------------------------------
# HBM-bound kernels
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d", [64, 128])
def test_merge_lse(torch, d):
    """LogSumExp merge against the oracle's, out of place and in place
    (O_out and lse_out aliasing the first operand), with empty partials
    (lse = -inf) on either side; 300 rows, a ragged last workgroup pass."""
    import long_context_transformers_amd as ra
    rng = np.random.default_rng(5 + d)
    B, Hq, c = 2, 3, 50
    dims = ra.Dims(B, Hq, Hq, d, c, rs.DT_F32)
    Oa = rng.standard_normal((B, Hq, c, d)).astype(np.float32)
    Ob = rng.standard_normal((B, Hq, c, d)).astype(np.float32)
    la = (rng.standard_normal((B, Hq, c)) * 5).astype(np.float32)
    lb = (rng.standard_normal((B, Hq, c)) * 5).astype(np.float32)
    la[0, 0, :5] = -np.inf
    lb[0, 0, 3:8] = -np.inf
    Om_ref, lm_ref = npref.lse_merge(Oa.astype(np.float64), la.astype(np.float64),
                                     Ob.astype(np.float64), lb.astype(np.float64))
    tOa, tOb, tla, tlb = (torch.from_numpy(x).cuda() for x in (Oa, Ob, la, lb))
    Oo = torch.empty_like(tOa)
    lo = torch.empty_like(tla)
    ra.merge_lse(dims, tOa, tla, tOb, tlb, Oo, lo)
    ra.merge_lse(dims, tOa, tla, tOb, tlb, tOa, tla)     # in place
    torch.cuda.synchronize()
    for O_, l_ in ((Oo, lo), (tOa, tla)):
        assert np.allclose(O_.cpu().numpy(), Om_ref, atol=1e-5, rtol=1e-5)
        lg = l_.cpu().numpy()
        assert np.array_equal(np.isinf(lg), np.isinf(lm_ref))
        fin = np.isfinite(lm_ref)
        assert np.allclose(lg[fin], lm_ref[fin], atol=1e-5)


@pytest.mark.parametrize("dtype", [rs.DT_BF16, rs.DT_F32])
def test_finalize_and_bwd_preprocess(torch, dtype):
    import long_context_transformers_amd as ra
    rng = np.random.default_rng(6)
    B, Hq, c, d = 1, 2, 70, 128
    dims = ra.Dims(B, Hq, Hq, d, c, dtype)
    m = rng.standard_normal((B, Hq, c)).astype(np.float32)
    l = (rng.random((B, Hq, c)) * 10 + 0.5).astype(np.float32)
    l[0, 1, :3] = 0
    m[0, 1, :3] = -np.inf
    O = rng.standard_normal((B, Hq, c, d)).astype(np.float32)
    O[0, 1, :3] = 0
    tm, tl, tO = (torch.from_numpy(x).cuda() for x in (m, l, O))
    out = torch.empty((B, Hq, c, d), dtype=H.torch_dtype(dtype), device="cuda")
    lse = torch.empty((B, Hq, c), dtype=torch.float32, device="cuda")
    ra.finalize(dims, tm, tl, tO, out, lse)
    torch.cuda.synchronize()
    with np.errstate(divide="ignore", invalid="ignore"):
        want = np.where(l[..., None] > 0, O / l[..., None], 0)
        want_lse = np.where(l > 0, m + np.log(l), -np.inf)
    got = out.float().cpu().numpy()
    tol = 1e-6 if dtype == rs.DT_F32 else 2 ** -8
    assert np.all(np.abs(got - want) <= tol * np.maximum(1, np.abs(want)))
    assert np.allclose(lse.cpu().numpy()[l > 0], want_lse[l > 0], atol=1e-6)
    assert np.all(lse.cpu().numpy()[l == 0] == -np.inf)
    # D = rowsum(dO * O) on the finalized output
    dO = torch.randn((B, Hq, c, d), device="cuda").to(H.torch_dtype(dtype))
    D = torch.empty((B, Hq, c), dtype=torch.float32, device="cuda")
    ra.bwd_preprocess(dims, out, dO, D)
    torch.cuda.synchronize()
    ref = (dO.double() * out.double()).sum(-1)
    assert torch.allclose(D.double(), ref, atol=1e-4, rtol=1e-5)


@pytest.mark.parametrize("layout", [C, S])
def test_layout_permute_bit_exact(torch, layout):
    import long_context_transformers_amd as ra
    B, H_, N, c, d = 2, 3, 4, 9, 64
    dims = ra.Dims(B, H_, H_, d, c, rs.DT_BF16)
    full = torch.randn((B, H_, N * c, d), device="cuda").to(torch.bfloat16)
    hm = torch.empty((N, B, H_, c, d), dtype=torch.bfloat16, device="cuda")
    ra.layout_permute(dims, H_, N, layout, True, full, hm)
    back = torch.empty_like(full)
    ra.layout_permute(dims, H_, N, layout, False, hm, back)
    torch.cuda.synchronize()
    for h in range(N):
        t = torch.as_tensor(npref.token_index(layout, N, c, h, np.arange(c)), device="cuda")
        assert torch.equal(hm[h], full[:, :, t])
    assert torch.equal(back, full)


# ---------------------------------------------------------------------------
# ordering: the side-stream double buffer gives the same bits as one stream
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("layout,mask", [(C, 0), (C, 1), (S, 1)])
def test_ring_concurrent_equals_serialized(torch, layout, mask):
    import long_context_transformers_amd as ra
    w = rs.Workload("race", 92, 1, 4, 2, 128, 8, 1024, rs.DT_BF16, mask, layout, 0, 8)
    inp = H.inputs(w)
    t = tuple(H.dev_tensor(x, w.dtype) for x in (inp.q_dev, inp.k_dev, inp.v_dev))
    O1, l1, s1 = H.run_ring_fwd(w, inp, tensors=t)
    O2, l2, _ = H.run_ring_fwd(w, inp, flags=ra.RA_FLAG_SERIALIZE, tensors=t)
    O3, l3, _ = H.run_ring_fwd(w, inp, delay_us=300, tensors=t)
    assert torch.equal(O1, O2) and torch.equal(l1, l2)
    assert torch.equal(O1, O3) and torch.equal(l1, l3)
    assert s1["transfers"] == 7 and s1["copy_bytes"] == 7 * 8 * 2 * (2 * 1024 * 128 * 2)
    # single host with copy elision equals the full ring's host 7
    w7 = w.replace(host_begin=7, host_end=8)
    t7 = (t[0][7:8].contiguous(), t[1], t[2])
    O4, l4, s4 = H.run_ring_fwd(w7, inp, tensors=t7, flags=ra.RA_FLAG_ELIDE_SKIPPED_COPIES)
    assert torch.equal(O4[0], O1[7]) and torch.equal(l4[0], l1[7])


def test_ring_transfers_wait_for_inputs_on_compute_stream(torch):
    """K and V produced on the compute stream just before the call (behind a
    long matmul) reach the side-stream transfers intact: forward and backward
    equal a run on inputs that were ready long before."""
    import long_context_transformers_amd as ra
    w = rs.Workload("order", 99, 1, 4, 2, 128, 4, 512, rs.DT_BF16, 1, C, 0, 4)
    inp = rs.make_inputs(w, with_do=True)
    q, k, v, do = (H.dev_tensor(x, w.dtype) for x in (inp.q_dev, inp.k_dev, inp.v_dev, inp.do_dev))
    O1, l1, _ = H.run_ring_fwd(w, inp, tensors=(q, k, v))
    k2, v2 = torch.zeros_like(k), torch.zeros_like(v)
    a = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
    torch.cuda.synchronize()
    for _ in range(8):
        b = torch.matmul(a, a)                  # a few ms of work ahead of the copies below
    k2.copy_(k)
    v2.copy_(v)
    O2, l2, _ = H.run_ring_fwd(w, inp, tensors=(q, k2, v2))
    assert torch.equal(O1, O2) and torch.equal(l1, l2)
    del b
    cfg = H.cfg_of(w)
    grads = []
    for kk, vv in ((k, v), (None, None)):
        if kk is None:
            kk, vv = torch.zeros_like(k), torch.zeros_like(v)
            torch.cuda.synchronize()
            for _ in range(8):
                b = torch.matmul(a, a)
            kk.copy_(k)
            vv.copy_(v)
        dQ = torch.empty(q.shape, dtype=torch.float32, device="cuda")
        dK = torch.empty(k.shape, dtype=torch.float32, device="cuda")
        dV = torch.empty(v.shape, dtype=torch.float32, device="cuda")
        ws = torch.empty(ra.ring_workspace_size(cfg, True), dtype=torch.uint8, device="cuda")
        ra.ring_bwd(cfg, q, kk, vv, O1, l1, do, dQ, dK, dV, ws, torch.cuda.current_stream(),
                    torch.cuda.Stream())
        torch.cuda.synchronize()
        grads.append((dQ, dK, dV))
    for x, y in zip(*grads):
        assert torch.equal(x, y)
