"""GPU parity of one decode step against a ring-sharded KV cache (calls
through the C ABI) with the fp64 oracle.  Tolerances as for the forward:
bf16 O max-abs 2e-2, LSE max-abs 1e-3; the fp32-output path and the merge of
per-shard partials are checked against the all-shard call to 1e-5."""
import numpy as np
import pytest

import ra_synth as rs
from oracle import npref
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

TOL_O, TOL_L = 2e-2, 1e-3


@pytest.fixture(scope="module")
def torch():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import long_context_transformers_amd as ra
    ra.version()
    return torch


def _inputs(seed, N, B, Hq, Hkv, d, c, full=False):
    q = rs.f32_to_bf16_bits(rs.normal_f32((seed, 1), (B, Hq, d)))
    k = rs.f32_to_bf16_bits(rs.normal_f32((seed, 2), (N, B, Hkv, c, d)))
    v = rs.f32_to_bf16_bits(rs.normal_f32((seed, 3), (N, B, Hkv, c, d)))
    lens = rs.decode_lens(N, B, c, seed, full=full)
    return q, k, v, lens


def _run(torch, dims, N, q, k, v, lens, o_dtype):
    import long_context_transformers_amd as ra
    B, Hq, d = dims.batch, dims.heads_q, dims.head_dim
    tq, tk, tv = (H.dev_tensor(x, rs.DT_BF16) for x in (q, k, v))
    tl = torch.as_tensor(np.ascontiguousarray(lens, dtype=np.int32)).cuda()
    O = torch.empty((B, Hq, d), dtype=o_dtype, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    ws = torch.empty(ra.decode_workspace_size(dims, N), dtype=torch.uint8, device="cuda")
    ra.ring_decode(dims, N, tq, tk, tv, tl, O, lse, ws)
    torch.cuda.synchronize()
    return O, lse


def _check(name, O, lse, O_ref, lse_ref):
    Og = O.float().cpu().numpy().astype(np.float64)
    lg = lse.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isinf(lg), np.isinf(lse_ref)), name
    fin = np.isfinite(lse_ref)
    eo = float(np.abs(Og - O_ref).max())
    el = float(np.abs(lg[fin] - lse_ref[fin]).max()) if fin.any() else 0.0
    H.report(name, tol={"max_abs_O": TOL_O, "max_abs_lse": TOL_L}, max_abs_O=eo, max_abs_lse=el)
    assert np.all(np.isfinite(Og))
    assert eo <= TOL_O and el <= TOL_L, (name, eo, el)


SMALL = [
    # (N, B, Hq, Hkv, d, c)
    (1, 1, 4, 4, 128, 1),
    (3, 2, 8, 2, 128, 100),
    (4, 3, 16, 1, 64, 1000),
    (2, 2, 6, 3, 128, 4096),
    (5, 1, 32, 32, 128, 333),
    (8, 2, 4, 4, 64, 129),
]


@pytest.mark.parametrize("N,B,Hq,Hkv,d,c", SMALL)
def test_ring_decode_small_all_outputs(torch, N, B, Hq, Hkv, d, c):
    import long_context_transformers_amd as ra
    q, k, v, lens = _inputs(500 + N * 7 + c, N, B, Hq, Hkv, d, c)
    dims = ra.Dims(B, Hq, Hkv, d, c, rs.DT_BF16)
    O_ref, lse_ref = npref.decode_attention(rs.bf16_bits_to_f32(q), rs.bf16_bits_to_f32(k),
                                            rs.bf16_bits_to_f32(v), lens, d ** -0.5)
    O, lse = _run(torch, dims, N, q, k, v, lens, torch.bfloat16)
    _check(f"decode N={N} B={B} {Hq}/{Hkv} d={d} c={c}", O, lse, O_ref, lse_ref)
    O32, lse32 = _run(torch, dims, N, q, k, v, lens, torch.float32)
    _check(f"decode fp32 out N={N} c={c}", O32, lse32, O_ref, lse_ref)
    assert torch.equal(lse, lse32)


def test_decode_partials_merge_to_ring_result(torch):
    """Each shard's call (n_hosts = 1, fp32 O) merged with ra_merge_lse in
    ring order gives the all-shard result: the form in which N GPUs would
    run the step, one shard each."""
    import long_context_transformers_amd as ra
    N, B, Hq, Hkv, d, c = 4, 2, 8, 2, 128, 700
    q, k, v, lens = _inputs(77, N, B, Hq, Hkv, d, c)
    dims = ra.Dims(B, Hq, Hkv, d, c, rs.DT_BF16)
    O_all, lse_all = _run(torch, dims, N, q, k, v, lens, torch.float32)
    mdims = ra.Dims(B, Hq, Hq, d, 1, rs.DT_F32)
    Om = lm = None
    for h in range(N):
        O_h, l_h = _run(torch, dims, 1, q, k[h:h + 1], v[h:h + 1], lens[h:h + 1], torch.float32)
        if Om is None:
            Om, lm = O_h, l_h
        else:
            ra.merge_lse(mdims, Om, lm, O_h, l_h, Om, lm)
    torch.cuda.synchronize()
    assert torch.allclose(Om, O_all, atol=1e-5, rtol=1e-5)
    assert torch.allclose(lm, lse_all, atol=1e-5, rtol=0)


def test_decode_empty_and_deterministic(torch):
    import long_context_transformers_amd as ra
    N, B, Hq, Hkv, d, c = 3, 2, 4, 2, 64, 300
    q, k, v, lens = _inputs(88, N, B, Hq, Hkv, d, c)
    dims = ra.Dims(B, Hq, Hkv, d, c, rs.DT_BF16)
    O0, l0 = _run(torch, dims, N, q, k, v, np.zeros_like(lens), torch.float32)
    assert torch.all(O0 == 0) and torch.all(torch.isinf(l0)) and torch.all(l0 < 0)
    O1, l1 = _run(torch, dims, N, q, k, v, lens, torch.bfloat16)
    O2, l2 = _run(torch, dims, N, q, k, v, lens, torch.bfloat16)
    assert torch.equal(O1, O2) and torch.equal(l1, l2)


@pytest.mark.timeout(600)
def test_decode_512k_gqa_all_outputs(torch):
    """Every output of the grouped-head decode over a 512K-token cache per
    sequence (8 shards x 64K rows, the last shard partly filled), against the
    oracle reading every valid key."""
    import long_context_transformers_amd as ra
    w = rs.decode_workloads()["decode_512k_gqa"]
    N, B, Hq, Hkv, d, c = w.n_hosts, w.batch, w.heads_q, w.heads_kv, w.head_dim, w.block_len
    g = torch.Generator(device="cuda")
    g.manual_seed(w.cfg)
    q = torch.randn((B, Hq, d), generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn((N, B, Hkv, c, d), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((N, B, Hkv, c, d), generator=g, device="cuda").to(torch.bfloat16)
    lens = rs.decode_lens(N, B, c, w.cfg, full=True)
    dims = ra.Dims(B, Hq, Hkv, d, c, rs.DT_BF16)
    tl = torch.as_tensor(lens).cuda()
    O = torch.empty((B, Hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    ws = torch.empty(ra.decode_workspace_size(dims, N), dtype=torch.uint8, device="cuda")
    ra.ring_decode(dims, N, q, k, v, tl, O, lse, ws)
    torch.cuda.synchronize()
    O_ref, lse_ref = npref.decode_attention(q.float().cpu().numpy(), k.float().cpu().numpy(),
                                            v.float().cpu().numpy(), lens, d ** -0.5)
    _check(w.name, O, lse, O_ref, lse_ref)


@pytest.mark.timeout(600)
def test_decode_8m_closed_form(torch):
    """The 8M-token cache (32 shards x 256K rows, 32 heads, d = 128) with
    Q = 0: every score is exactly 0, so O is the mean of all cached V rows
    and LSE = ln(number of rows) = ln(T).  l is a sum of ones in fp32, exact
    below 2^24 rows."""
    import long_context_transformers_amd as ra
    w = rs.decode_workloads()["decode_8m"]
    N, B, Hq, Hkv, d, c = w.n_hosts, w.batch, w.heads_q, w.heads_kv, w.head_dim, w.block_len
    g = torch.Generator(device="cuda")
    g.manual_seed(w.cfg)
    k = torch.empty((N, B, Hkv, c, d), dtype=torch.bfloat16, device="cuda")
    v = torch.empty_like(k)
    for h in range(N):
        k[h].copy_(torch.randn((B, Hkv, c, d), generator=g, device="cuda"))
        v[h].copy_(torch.randn((B, Hkv, c, d), generator=g, device="cuda"))
    lens = rs.decode_lens(N, B, c, w.cfg, full=True)
    T = int(lens.sum())
    dims = ra.Dims(B, Hq, Hkv, d, c, rs.DT_BF16)
    q = torch.zeros((B, Hq, d), dtype=torch.bfloat16, device="cuda")
    O = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    ws = torch.empty(ra.decode_workspace_size(dims, N), dtype=torch.uint8, device="cuda")
    ra.ring_decode(dims, N, q, k, v, torch.as_tensor(lens).cuda(), O, lse, ws)
    torch.cuda.synchronize()
    want_l = torch.log(torch.tensor(float(T), dtype=torch.float64)).float()
    ulp = float(torch.nextafter(want_l, torch.tensor(np.inf)) - want_l)
    err_l = float((lse - want_l.cuda()).abs().max())
    mean = torch.zeros((Hkv, d), dtype=torch.float64, device="cuda")
    for h in range(N):
        n = int(lens[h, 0])
        mean += v[h, 0, :, :n].sum(dim=1, dtype=torch.float64)
    mean /= T
    err_o = float((O[0].double() - mean).abs().max())
    H.report(w.name + " Q = 0", tokens=T, max_abs_O=err_o, lse_err_ulps=err_l / ulp)
    assert err_l <= 2 * ulp
    assert err_o <= 1e-5
    del k, v
    torch.cuda.empty_cache()
