"""GPU parity of the blockwise feedforward Y = GELU(X W1^T) W2^T (calls
through the C ABI) with the fp64 oracle.  Tolerance: max-abs 2e-2 on Y
(bf16 inputs, bf16 GELU output between the layers, bf16 Y), with weights
scaled by 1/sqrt(fan-in) so Y is O(1)."""
import numpy as np
import pytest

import ra_synth as rs
from oracle import npref
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu
TOL = 2e-2


@pytest.fixture(scope="module")
def torch():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import long_context_transformers_amd as ra
    ra.version()
    return torch


def _bf16(seed, shape, scale=1.0):
    return rs.f32_to_bf16_bits(rs.normal_f32(seed, shape, scale))


def _run(torch, x, w1, w2, block_rows):
    import long_context_transformers_amd as ra
    tx, t1, t2 = (H.dev_tensor(a, rs.DT_BF16) for a in (x, w1, w2))
    y = torch.empty((x.shape[0], x.shape[1]), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(ra.ffn_workspace_size(block_rows, x.shape[1], w1.shape[0]), dtype=torch.uint8, device="cuda")
    ra.block_ffn(tx, t1, t2, y, block_rows, ws)
    torch.cuda.synchronize()
    return y


SMALL = [
    # (rows, h, f, block_rows)
    (1, 64, 64, 1),
    (100, 128, 256, 64),
    (300, 64, 448, 300),
    (513, 320, 192, 256),
    (257, 128, 512, 1000),
    (1024, 256, 1024, 1024),     # few tiles per layer: K split over 4 and 8 workgroups
    (1100, 256, 1024, 1024),     # and a ragged last row block
]


@pytest.mark.parametrize("rows,h,f,block_rows", SMALL)
def test_block_ffn_small_all_rows(torch, rows, h, f, block_rows):
    seed = 700 + rows
    x = _bf16((seed, 1), (rows, h))
    w1 = _bf16((seed, 2), (f, h), h ** -0.5)
    w2 = _bf16((seed, 3), (h, f), f ** -0.5)
    y = _run(torch, x, w1, w2, block_rows)
    want = npref.blockwise_ffn(rs.bf16_bits_to_f32(x), rs.bf16_bits_to_f32(w1), rs.bf16_bits_to_f32(w2))
    got = y.float().cpu().numpy().astype(np.float64)
    err = float(np.abs(got - want).max())
    H.report(f"block_ffn rows={rows} h={h} f={f} block={block_rows}", tol=TOL, max_abs=err)
    assert np.all(np.isfinite(got)) and err <= TOL


def test_block_ffn_block_size_does_not_change_bits(torch):
    """Every output row depends on its own row only: row blockings that split
    K the same way (here every block gives each layer 2 K splits) give the
    same bits."""
    rows, h, f = 700, 128, 320
    x = _bf16((71, 1), (rows, h))
    w1 = _bf16((71, 2), (f, h), h ** -0.5)
    w2 = _bf16((71, 3), (h, f), f ** -0.5)
    ys = [_run(torch, x, w1, w2, b) for b in (64, 256, 700, 4096)]
    for y in ys[1:]:
        assert torch.equal(y, ys[0])


@pytest.mark.timeout(600)
def test_block_ffn_7b_block_sampled(torch):
    """A 7B-like layer's feedforward (h = 4096, f = 4h = 16384) on one host's
    block of 4096 tokens, as one row block (a full tile grid) and in row
    blocks of 1024 (the second layer splits K over 4 workgroups); 64 seeded
    rows of both against the oracle."""
    import long_context_transformers_amd as ra
    w = rs.ffn_workloads()["ffn_7b_c4096"]
    g = torch.Generator(device="cuda")
    g.manual_seed(w.cfg)
    x = torch.randn((w.rows, w.h), generator=g, device="cuda").to(torch.bfloat16)
    w1 = (torch.randn((w.f, w.h), generator=g, device="cuda") * w.h ** -0.5).to(torch.bfloat16)
    w2 = (torch.randn((w.h, w.f), generator=g, device="cuda") * w.f ** -0.5).to(torch.bfloat16)
    y = torch.empty_like(x)
    ws = torch.empty(max(ra.ffn_workspace_size(b, w.h, w.f) for b in (w.block_rows, 1024)), dtype=torch.uint8,
                     device="cuda")
    ra.block_ffn(x, w1, w2, y, w.block_rows, ws)
    y2 = torch.empty_like(x)
    ra.block_ffn(x, w1, w2, y2, 1024, ws)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(w.cfg).choice(w.rows, 64, replace=False))
    idx = torch.as_tensor(rows, device="cuda")
    xs = x[idx].float().cpu().numpy()
    want = npref.blockwise_ffn(xs, w1.float().cpu().numpy(), w2.float().cpu().numpy())
    for tag, out in (("one block", y), ("blocks of 1024", y2)):
        got = out[idx].float().cpu().numpy().astype(np.float64)
        err = float(np.abs(got - want).max())
        H.report(f"{w.name} {tag}", tol=TOL, max_abs=err, rows=len(rows))
        assert np.all(np.isfinite(got)) and err <= TOL
