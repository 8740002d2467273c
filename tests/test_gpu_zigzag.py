"""GPU parity of the zigzag layout (two chunks of c/2 tokens per host, chunk h
and chunk 2N-1-h) against the fp64 oracle, through the C ABI.  Tolerances as
for the other forward tests: bf16 O max-abs 2e-2, LSE max-abs 1e-3."""
import numpy as np
import pytest

import ra_synth as rs
from oracle import npref
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

Z = rs.LAYOUT_ZIGZAG
TOL_O, TOL_L = 2e-2, 1e-3


@pytest.fixture(scope="module")
def torch():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import long_context_transformers_amd as ra
    ra.version()
    return torch


def _check(name, O, lse, O_ref, lse_ref):
    eo = float(np.abs(O - O_ref).max())
    el = float(np.abs(lse - lse_ref).max())
    H.report(name, tol={"max_abs_O": TOL_O, "max_abs_lse": TOL_L}, max_abs_O=eo, max_abs_lse=el, rows=O.shape[0])
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(lse))
    assert eo <= TOL_O and el <= TOL_L


SMALL = [
    # (d, hq, hkv, mask, N, c, host_begin, host_end)
    (128, 2, 2, 1, 1, 256, 0, 1),
    (128, 2, 2, 1, 2, 256, 0, 2),
    (128, 4, 2, 1, 3, 512, 0, 3),
    (64, 4, 1, 1, 4, 256, 0, 4),
    (128, 2, 2, 1, 4, 768, 1, 3),
    (64, 2, 2, 0, 3, 130, 0, 3),       # non-causal zigzag: a plain permutation of tokens
    (128, 2, 1, 0, 2, 6, 0, 2),
]


@pytest.mark.parametrize("d,hq,hkv,mask,N,c,hb,he", SMALL)
def test_ring_fwd_zigzag_small_all_rows(torch, d, hq, hkv, mask, N, c, hb, he):
    w = rs.Workload(f"zz_d{d}_h{hq}x{hkv}_m{mask}_N{N}_c{c}", 80 + N, 1, hq, hkv, d, N, c,
                    rs.DT_BF16, mask, Z, hb, he)
    inp = H.inputs(w)
    O, lse, stats = H.run_ring_fwd(w, inp)
    rows = np.arange(c)
    Os, Ls = H.sampled(O, lse, w, rows)
    O_ref, lse_ref = H.oracle_rows(w, inp, rows)
    _check(f"ring_fwd {w.name} hosts {hb}..{he - 1}", Os, Ls, O_ref, lse_ref)
    assert stats["compute_steps"] == N


def test_ring_fwd_zigzag_mid_sampled(torch):
    """c = 4096 (each half spans 32 key tiles), N = 4, GQA, sampled rows on
    every host."""
    w = rs.Workload("zz_mid_N4_c4096", 86, 1, 8, 2, 128, 4, 4096, rs.DT_BF16, 1, Z, 0, 4)
    inp = H.inputs(w)
    O, lse, _ = H.run_ring_fwd(w, inp)
    rows = rs.row_sample(w, 512)
    Os, Ls = H.sampled(O, lse, w, rows)
    O_ref, lse_ref = H.oracle_rows(w, inp, rows)
    _check("ring_fwd zz_mid_N4_c4096", Os, Ls, O_ref, lse_ref)


@pytest.mark.timeout(600)
def test_ring_fwd_zigzag_causal_256k(torch):
    w = rs.workloads()["causal_256k_zigzag"]
    inp = H.inputs(w, q_hosts_only=True)
    O, lse, stats = H.run_ring_fwd(w, inp)
    rows = rs.row_sample(w, 1024)
    Os, Ls = H.sampled(O, lse, w, rows)
    O_ref, lse_ref = H.oracle_rows(w, inp, rows)
    _check(f"ring_fwd {w.name}", Os, Ls, O_ref, lse_ref)
    assert stats["skipped_blocks"] == 0    # every zigzag host sees keys on every other host


@pytest.mark.timeout(600)
def test_zigzag_closed_forms_full_scale(torch):
    """Two closed forms on all 8 hosts of the 256K causal zigzag workload,
    every row of every host.  K holds the base-16 digits of each key's token
    index t' in channels 0..4.

    Q = 0: every score is exactly 0, so row t's LSE is log(number of visible
    keys) = log(t + 1).  The device logf is within 2 fp32 ulps; counts t and
    t + 2 lie at least 8 ulps away for t < 2^17 (so the count is exact there)
    and at least 4 ulps away above.

    Q = (1, 16, 256, 4096, 65536, 0, ...): the score of key t' is exactly t'
    before the softmax scale a = 1/sqrt(d), so row t's LSE is
    a t + log(sum_{j=0..t} exp(-a j)).  Making key t + 1 visible or hiding key
    t moves it by about a = 0.088; the tolerance is a/4."""
    w = rs.workloads()["causal_256k_zigzag"].replace(host_begin=0, host_end=8)
    N, c, d = w.n_hosts, w.block_len, w.head_dim
    t = torch.as_tensor(np.stack([npref.token_index(Z, N, c, h, np.arange(c)) for h in range(N)]),
                        device="cuda")
    k = torch.zeros((N, 1, w.heads_kv, c, d), dtype=torch.float32, device="cuda")
    for ch in range(5):
        k[..., ch] = ((t >> (4 * ch)) & 15).float()[:, None, None, :]
    k = k.to(torch.bfloat16)
    v = torch.randn((N, 1, w.heads_kv, c, d), device="cuda").to(torch.bfloat16)
    q = torch.zeros((N, 1, w.heads_q, c, d), dtype=torch.bfloat16, device="cuda")
    O, lse, stats = H.run_ring_fwd(w, None, tensors=(q, k, v))
    assert stats["skipped_blocks"] == 0
    want = torch.log((t + 1).double()).float()[:, None, None, :].expand_as(lse)
    ulp = torch.abs(torch.nextafter(want, torch.full_like(want, np.inf)) - want)
    err = torch.abs(lse - want)
    H.report("closed form zigzag 256k, Q = 0", rows=int(lse.numel()),
             max_err_ulps=float((err / ulp).max()))
    assert torch.all(err <= 2 * ulp)
    # O is the mean of the visible V rows: spot-check a few tokens per host
    hk = torch.arange(w.heads_q, device="cuda") // (w.heads_q // w.heads_kv)
    for h in range(N):
        for r in (0, 1, c // 2 - 1, c // 2, c - 1):
            src_h, src_r = torch.nonzero(t <= t[h, r], as_tuple=True)
            want_o = v[src_h, 0, :, src_r, :].sum(0, dtype=torch.float64) / src_h.numel()
            got = O[h, 0, :, r, :].double()
            assert float((got - want_o[hk]).abs().max()) <= 2e-2, (h, r)
    del O
    for ch in range(5):
        q[..., ch] = float(16 ** ch)
    _, lse, _ = H.run_ring_fwd(w, None, tensors=(q, k, v))
    a = 1.0 / np.sqrt(d)
    n = N * c
    tail = np.log(np.cumsum(np.exp(-a * np.arange(n, dtype=np.float64))))   # log sum_{j<=t}
    want = torch.as_tensor(a * np.arange(n) + tail, device="cuda")[t][:, None, None, :]
    err = float((lse.double() - want).abs().max())
    H.report("closed form zigzag 256k, score = token index", tol=a / 4, rows=int(lse.numel()), max_abs_lse=err)
    assert err <= a / 4


@pytest.mark.parametrize("mask", [0, 1])
def test_ring_zigzag_concurrent_equals_serialized(torch, mask):
    import long_context_transformers_amd as ra
    w = rs.Workload("race_zz", 93, 1, 4, 2, 128, 8, 1024, rs.DT_BF16, mask, Z, 0, 8)
    inp = H.inputs(w)
    t = tuple(H.dev_tensor(x, w.dtype) for x in (inp.q_dev, inp.k_dev, inp.v_dev))
    O1, l1, _ = H.run_ring_fwd(w, inp, tensors=t)
    O2, l2, _ = H.run_ring_fwd(w, inp, flags=ra.RA_FLAG_SERIALIZE, tensors=t)
    O3, l3, _ = H.run_ring_fwd(w, inp, delay_us=300, tensors=t)
    assert torch.equal(O1, O2) and torch.equal(l1, l2)
    assert torch.equal(O1, O3) and torch.equal(l1, l3)


def test_layout_permute_zigzag_bit_exact(torch):
    import long_context_transformers_amd as ra
    B, H_, N, c, d = 2, 3, 4, 10, 64
    dims = ra.Dims(B, H_, H_, d, c, rs.DT_BF16)
    full = torch.randn((B, H_, N * c, d), device="cuda").to(torch.bfloat16)
    hm = torch.empty((N, B, H_, c, d), dtype=torch.bfloat16, device="cuda")
    ra.layout_permute(dims, H_, N, Z, True, full, hm)
    back = torch.empty_like(full)
    ra.layout_permute(dims, H_, N, Z, False, hm, back)
    torch.cuda.synchronize()
    for h in range(N):
        t = torch.as_tensor(npref.token_index(Z, N, c, h, np.arange(c)), device="cuda")
        assert torch.equal(hm[h], full[:, :, t])
    assert torch.equal(back, full)
