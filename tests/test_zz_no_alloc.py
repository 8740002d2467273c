"""The allocation-free decode entry point (ra_ring_decode_noalloc), called
through the C ABI: its output must equal ra_ring_decode's (same kernels, same
split of the keys, so bit for bit) and meet the decode tolerances against the
fp64 oracle, over two calls in a row on the shared scratch, the second with a
smaller input (so a stale partial from the first call would show).  A request
whose partials exceed the scratch is refused before any HIP call."""
import ctypes

import numpy as np
import pytest

import ra_synth as rs
from oracle import npref
from tests import gpu_helpers as H

TOL_O, TOL_L = 2e-2, 1e-3


def test_noalloc_refuses_oversized_request():
    """64 sequences x 64 hosts x 32 query heads need far more than the 32 MiB
    scratch: RA_ERR_WORKSPACE from the host-side check (fake pointers are
    never touched)."""
    import long_context_transformers_amd as ra
    from long_context_transformers_amd import _lib as L
    d = L.RaDims(64, 32, 8, 128, 256, 0, 0.0)
    need = ra.decode_workspace_size(ra.Dims(64, 32, 8, 128, 256, 0), 64)
    assert need > (32 << 20)
    fake = 0x100000
    rc = ra.raw_call("ra_ring_decode_noalloc", ctypes.byref(d), 64, fake, fake, fake, fake, fake, 0, fake, None)
    assert rc == L.RA_ERR_WORKSPACE and "scratch" in ra.last_error()
    rc = ra.raw_call("ra_ring_decode_noalloc", ctypes.byref(L.RaDims(1, 4, 2, 96, 8, 0, 0.0)), 1, fake, fake,
                     fake, fake, fake, 0, fake, None)
    assert rc == L.RA_ERR_UNSUPPORTED


def _case(seed, N, B, Hq, Hkv, d, c):
    q = rs.f32_to_bf16_bits(rs.normal_f32((seed, 1), (B, Hq, d)))
    k = rs.f32_to_bf16_bits(rs.normal_f32((seed, 2), (N, B, Hkv, c, d)))
    v = rs.f32_to_bf16_bits(rs.normal_f32((seed, 3), (N, B, Hkv, c, d)))
    lens = rs.decode_lens(N, B, c, seed, full=False)
    return q, k, v, lens


@pytest.mark.gpu
def test_noalloc_matches_workspace_call_twice():
    import torch
    import long_context_transformers_amd as ra
    assert torch.cuda.is_available()
    cases = [(601, 8, 2, 32, 8, 128, 4096),     # first call: the larger one
             (602, 3, 1, 4, 2, 64, 300)]        # second call: smaller, other head_dim
    for seed, N, B, Hq, Hkv, d, c in cases:
        print(f"[no-alloc] seed={seed} N={N} B={B} Hq={Hq} Hkv={Hkv} d={d} c={c}", flush=True)
        q, k, v, lens = _case(seed, N, B, Hq, Hkv, d, c)
        dims = ra.Dims(B, Hq, Hkv, d, c, rs.DT_BF16)
        tq, tk, tv = (H.dev_tensor(x, rs.DT_BF16) for x in (q, k, v))
        tl = torch.as_tensor(np.ascontiguousarray(lens, dtype=np.int32)).cuda()
        for o_dt in (torch.bfloat16, torch.float32):
            O_ws = torch.empty((B, Hq, d), dtype=o_dt, device="cuda")
            lse_ws = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
            ws = torch.empty(ra.decode_workspace_size(dims, N), dtype=torch.uint8, device="cuda")
            ra.ring_decode(dims, N, tq, tk, tv, tl, O_ws, lse_ws, ws)
            O_na = torch.full((B, Hq, d), float("nan"), dtype=o_dt, device="cuda")
            lse_na = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
            ra.ring_decode_noalloc(dims, N, tq, tk, tv, tl, O_na, lse_na)
            torch.cuda.synchronize()
            assert torch.equal(O_na, O_ws) and torch.equal(lse_na, lse_ws), (seed, o_dt)
        O_ref, lse_ref = npref.decode_attention(rs.bf16_bits_to_f32(q), rs.bf16_bits_to_f32(k),
                                                rs.bf16_bits_to_f32(v), lens, d ** -0.5)
        Og = O_na.double().cpu().numpy()
        lg = lse_na.double().cpu().numpy()
        assert np.array_equal(np.isinf(lg), np.isinf(lse_ref))
        fin = np.isfinite(lse_ref)
        eo = float(np.abs(Og - O_ref).max())
        el = float(np.abs(lg[fin] - lse_ref[fin]).max()) if fin.any() else 0.0
        H.report(f"decode no-alloc seed={seed}", tol={"max_abs_O": TOL_O, "max_abs_lse": TOL_L},
                 max_abs_O=eo, max_abs_lse=el)
        assert eo <= TOL_O and el <= TOL_L
