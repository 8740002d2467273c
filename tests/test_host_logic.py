"""Host-side logic of libringattn, checked on the CPU (no GPU calls).

- every function include/ringattn.h declares is exported by the library;
- the ring schedule (source block, class and offsets per step) is bit-exact
  against the oracle's explicit per-element masks;
- printed examples: ring holdings, striped token lists, block counts;
- argument checks fail before any HIP call;
- the c >= F/B reporter against the pages' table.
"""
import ctypes
import json
import os
import re
import subprocess
import sys

import numpy as np
import pytest

import long_context_transformers_amd as ra
from long_context_transformers_amd import _lib as L
import ra_synth as rs
from oracle import cref

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
C, S = ra.RA_LAYOUT_CONTIGUOUS, ra.RA_LAYOUT_STRIPED


def test_header_symbols_exported():
    hdr = open(os.path.join(ROOT, "include", "ringattn.h")).read()
    declared = set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(ra_[a-z_0-9]+)\s*\(", hdr, re.M))
    assert len(declared) >= 17, declared
    lib = L.load()
    for name in declared:
        assert hasattr(lib, name), name
    assert declared == {n for n, _, _ in L.SIGNATURES}


def _implied_mask(step, c, mask):
    r = np.arange(c)[:, None]
    rk = np.arange(c)[None, :]
    if mask == ra.RA_MASK_NONE:
        return np.ones((c, c), dtype=bool)
    return step["kv_offset"] + rk * step["stride"] <= step["q_offset"] + r * step["stride"]


_CLASS_PATTERN = {
    ra.RA_BLK_FULL: lambda c: np.ones((c, c), dtype=bool),
    ra.RA_BLK_SKIP: lambda c: np.zeros((c, c), dtype=bool),
    ra.RA_BLK_TRI_INCL: lambda c: np.tril(np.ones((c, c), dtype=bool)),
    ra.RA_BLK_TRI_STRICT: lambda c: np.tril(np.ones((c, c), dtype=bool), -1),
}


@pytest.mark.parametrize("layout", [C, S])
@pytest.mark.parametrize("mask", [ra.RA_MASK_NONE, ra.RA_MASK_CAUSAL])
def test_schedule_bit_exact_vs_oracle_masks(layout, mask):
    for N in (1, 2, 3, 4, 5, 8, 16):
        for c in (2, 3, 8, 64):
            for i in range(N):
                steps = ra.schedule(N, i, c, layout, mask)
                assert [s["src"] for s in steps] == [(i - s) % N for s in range(N)]
                for s in steps:
                    want = cref.block_mask(layout, mask, N, c, i, s["src"]).astype(bool)
                    got = _implied_mask(s, c, mask)
                    assert np.array_equal(got, want), (layout, mask, N, c, i, s)
                    assert np.array_equal(_CLASS_PATTERN[s["cls"]](c), want), (N, c, i, s)


@pytest.mark.parametrize("mask", [ra.RA_MASK_NONE, ra.RA_MASK_CAUSAL])
def test_schedule_zigzag(mask):
    """Zigzag steps: ring order, first-chunk offsets (stride 1), class
    QUADRANTS under the causal mask; quadrant (0, 0) -- chunk i against
    chunk src -- is exactly the oracle's mask on those rows and keys."""
    Z = ra.RA_LAYOUT_ZIGZAG
    for N in (1, 2, 3, 4, 8):
        for c in (2, 4, 8, 64):
            h = c // 2
            for i in range(N):
                steps = ra.schedule(N, i, c, Z, mask)
                assert [s["src"] for s in steps] == [(i - s) % N for s in range(N)]
                for s in steps:
                    j = s["src"]
                    assert (s["q_offset"], s["kv_offset"], s["stride"]) == (i * h, j * h, 1)
                    assert s["cls"] == (ra.RA_BLK_FULL if mask == ra.RA_MASK_NONE else ra.RA_BLK_QUADRANTS)
                    want = cref.block_mask(Z, mask, N, c, i, j).astype(bool)
                    assert np.array_equal(_implied_mask(s, h, mask), want[:h, :h]), (N, c, i, s)


def test_schedule_ring_holdings(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "ring_holdings_N4.json")))
    for step, held in g["held"].items():
        for host, blk in enumerate(held):
            assert ra.schedule(4, host, 16, C, ra.RA_MASK_NONE)[int(step)]["src"] == blk


def test_schedule_block_counts(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "contiguous_split_4dev_100tok.json")))
    N, c = g["n_hosts"], g["block_len"]
    for i in range(N):
        steps = ra.schedule(N, i, c, C, ra.RA_MASK_CAUSAL)
        live = [s for s in steps if s["cls"] != ra.RA_BLK_SKIP]
        assert len(live) * c == g["attention_shape"][str(i)][1]
        # N compute steps including the host's own block, own block first
        assert steps[0]["src"] == i and steps[0]["cls"] == ra.RA_BLK_TRI_INCL
    for i in range(N):
        steps = ra.schedule(N, i, c, S, ra.RA_MASK_CAUSAL)
        assert all(s["cls"] in (ra.RA_BLK_TRI_INCL, ra.RA_BLK_TRI_STRICT) for s in steps)


def test_token_index_golden(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "striped_tokens_N4.json")))
    for dev, toks in g["tokens_per_device_prefix"].items():
        assert [ra.token_index(S, 4, 100, int(dev), r) for r in range(4)] == toks
    for h in range(5):
        for r in (0, 1, 6):
            assert ra.token_index(C, 5, 7, h, r) == cref.token_index(C, 5, 7, h, r)
            assert ra.token_index(S, 5, 7, h, r) == cref.token_index(S, 5, 7, h, r)
    assert ra.token_index(S, 4, 10, 4, 0) == -1 and ra.token_index(C, 4, 10, 0, 10) == -1
    Z = ra.RA_LAYOUT_ZIGZAG
    for N, c in ((1, 2), (3, 6), (4, 8), (8, 256)):
        got = [ra.token_index(Z, N, c, h, r) for h in range(N) for r in range(c)]
        assert got == [cref.token_index(Z, N, c, h, r) for h in range(N) for r in range(c)]
    assert ra.token_index(Z, 4, 7, 0, 0) == -1                       # odd block_len


def test_block_class_general_offsets():
    # a band: key row r' visible iff r' - r <= 5
    assert ra.block_class_of(ra.RA_MASK_CAUSAL, 5, 0, 1, 64) == ra.RA_BLK_BAND
    assert ra.block_class_of(ra.RA_MASK_CAUSAL, 0, 64, 1, 64) == ra.RA_BLK_SKIP
    assert ra.block_class_of(ra.RA_MASK_CAUSAL, 63, 0, 1, 64) == ra.RA_BLK_FULL
    assert ra.block_class_of(ra.RA_MASK_CAUSAL, 0, 63, 1, 64) == ra.RA_BLK_BAND
    assert ra.block_class_of(ra.RA_MASK_CAUSAL, 0, 64, 1, 64) == ra.RA_BLK_SKIP
    # striped: floor division for negative offsets
    assert ra.block_class_of(ra.RA_MASK_CAUSAL, 2, 3, 4, 8) == ra.RA_BLK_TRI_STRICT
    assert ra.block_class_of(ra.RA_MASK_CAUSAL, 3, 2, 4, 8) == ra.RA_BLK_TRI_INCL
    # c = 1: the diagonal block is a single visible pair
    assert ra.block_class_of(ra.RA_MASK_CAUSAL, 0, 0, 1, 1) == ra.RA_BLK_FULL
    assert ra.block_class_of(ra.RA_MASK_NONE, 0, 99, 1, 8) == ra.RA_BLK_FULL
    assert ra.block_class_of(ra.RA_MASK_CAUSAL, 0, 0, 0, 8) == -1


# ---------------------------------------------------------------------------
# argument checks: every call below has a bad argument and must fail before
# any HIP call (fake device addresses are never dereferenced)
# ---------------------------------------------------------------------------

FAKE = 0x10000          # aligned, never touched
MIS = 0x10004           # misaligned


def _dims(**kw):
    d = dict(batch=1, heads_q=4, heads_kv=2, head_dim=128, block_len=64, dtype=0, scale=0.0)
    d.update(kw)
    return L.RaDims(**d)


def _call_block_fwd(dims, q=FAKE, k=FAKE, v=FAKE, mask=0, stride=1, m=FAKE, l=FAKE, o=FAKE):
    return ra.raw_call("ra_block_fwd", ctypes.byref(dims), q, k, v, mask, 0, 0, stride, m, l, o, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(heads_q=3, heads_kv=2), L.RA_ERR_INVALID_ARG),
    (dict(head_dim=96), L.RA_ERR_UNSUPPORTED),
    (dict(block_len=0), L.RA_ERR_INVALID_ARG),
    (dict(batch=0), L.RA_ERR_INVALID_ARG),
    (dict(dtype=7), L.RA_ERR_INVALID_ARG),
    (dict(scale=-1.0), L.RA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), L.RA_ERR_INVALID_ARG),
])
def test_bad_dims(kw, expect):
    assert _call_block_fwd(_dims(**kw)) == expect
    assert ra.last_error()


def test_bad_pointers_and_modes():
    d = _dims()
    assert _call_block_fwd(d, q=None) == L.RA_ERR_INVALID_ARG
    assert _call_block_fwd(d, k=MIS) == L.RA_ERR_INVALID_ARG and "aligned" in ra.last_error()
    assert _call_block_fwd(d, mask=5) == L.RA_ERR_INVALID_ARG
    assert _call_block_fwd(d, stride=0) == L.RA_ERR_INVALID_ARG
    assert ra.raw_call("ra_merge_lse", ctypes.byref(d), FAKE, FAKE, FAKE, None, FAKE, FAKE, None) == L.RA_ERR_INVALID_ARG
    assert ra.raw_call("ra_finalize", ctypes.byref(d), FAKE, FAKE, FAKE, MIS, FAKE, None) == L.RA_ERR_INVALID_ARG
    assert ra.raw_call("ra_bwd_preprocess", ctypes.byref(d), FAKE, None, FAKE, None) == L.RA_ERR_INVALID_ARG
    assert ra.raw_call("ra_state_init", None, FAKE, FAKE, FAKE, None) == L.RA_ERR_INVALID_ARG
    assert ra.raw_call("ra_layout_permute", ctypes.byref(d), 2, 4, 0, 1, FAKE, FAKE, None) == L.RA_ERR_INVALID_ARG
    assert ra.raw_call("ra_layout_permute", ctypes.byref(d), 2, 4, 9, 1, FAKE, FAKE + 256, None) == L.RA_ERR_INVALID_ARG
    assert ra.raw_call("ra_mask_tile", 0, 0, 0, 4, 4, FAKE, None) == L.RA_ERR_INVALID_ARG
    assert ra.raw_call("ra_block_bwd", ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0, 0, 1,
                       FAKE, FAKE, None, None) == L.RA_ERR_INVALID_ARG
    out = (L.RaStep * 4)()
    assert ra.raw_call("ra_schedule", 4, 4, 8, 0, 1, out) == L.RA_ERR_INVALID_ARG
    assert ra.raw_call("ra_schedule", 4, 0, 8, 3, 1, out) == L.RA_ERR_INVALID_ARG
    assert ra.raw_call("ra_schedule", 4, 0, 8, 0, 1, None) == L.RA_ERR_INVALID_ARG


def _cfg(**kw):
    c = dict(dims=_dims(), n_hosts=8, host_begin=0, host_end=8, layout=0, mask=0, flags=0,
             debug_copy_delay_us=0)
    c.update(kw)
    return L.RaRingCfg(**c)


def _ring_fwd(cfg, ws_bytes, ws=0x100000):
    st = L.RaRingStats()
    return ra.raw_call("ra_ring_fwd", ctypes.byref(cfg), FAKE, FAKE, FAKE, FAKE, FAKE, ws, ws_bytes,
                       None, None, ctypes.byref(st))


def test_ring_argument_checks():
    cfg = _cfg()
    n = ctypes.c_size_t(0)
    assert ra.raw_call("ra_ring_workspace_size", ctypes.byref(cfg), 0, ctypes.byref(n)) == 0
    need = n.value
    assert _ring_fwd(cfg, need - 1) == L.RA_ERR_WORKSPACE
    assert _ring_fwd(cfg, need, ws=0x100010) == L.RA_ERR_INVALID_ARG   # not 256-aligned
    assert _ring_fwd(_cfg(host_begin=3, host_end=3), need) == L.RA_ERR_INVALID_ARG
    assert _ring_fwd(_cfg(host_end=9), need) == L.RA_ERR_INVALID_ARG
    assert _ring_fwd(_cfg(layout=7), need) == L.RA_ERR_INVALID_ARG
    assert _ring_fwd(_cfg(flags=0x80), need) == L.RA_ERR_INVALID_ARG
    assert _ring_fwd(_cfg(n_hosts=0), need) == L.RA_ERR_INVALID_ARG
    # zigzag: even block_len; the causal ring forward needs bf16 and c % 256 == 0
    Z = ra.RA_LAYOUT_ZIGZAG
    big = 1 << 40
    assert _ring_fwd(_cfg(layout=Z, dims=_dims(block_len=63)), big) == L.RA_ERR_INVALID_ARG
    assert _ring_fwd(_cfg(layout=Z, mask=1, dims=_dims(block_len=64)), big) == L.RA_ERR_UNSUPPORTED
    assert _ring_fwd(_cfg(layout=Z, mask=1, dims=_dims(block_len=256, dtype=1)), big) == L.RA_ERR_UNSUPPORTED
    st = L.RaRingStats()
    # backward: causal zigzag with block_len % 256 != 0 is not supported;
    # copy elision only applies to a subset of the hosts
    assert ra.raw_call("ra_ring_bwd", ctypes.byref(_cfg(flags=1)), *([FAKE] * 10), 1 << 40,
                       None, None, ctypes.byref(st)) == L.RA_ERR_INVALID_ARG
    assert ra.raw_call("ra_ring_bwd", ctypes.byref(_cfg(layout=Z, mask=1, dims=_dims(block_len=128))),
                       *([FAKE] * 10), 1 << 40, None, None, ctypes.byref(st)) == L.RA_ERR_UNSUPPORTED
    assert ra.raw_call("ra_ring_bwd", ctypes.byref(_cfg(layout=Z, dims=_dims(block_len=63))),
                       *([FAKE] * 10), 1 << 40, None, None, ctypes.byref(st)) == L.RA_ERR_INVALID_ARG
    # fp32 causal zigzag is refused by the synchronous checks (not after the
    # first enqueue): the status is UNSUPPORTED and the stats stay untouched
    st.kernel_launches = -7
    assert ra.raw_call("ra_ring_bwd", ctypes.byref(_cfg(layout=Z, mask=1, dims=_dims(block_len=256, dtype=1))),
                       *([FAKE] * 10), 1 << 40, None, None, ctypes.byref(st)) == L.RA_ERR_UNSUPPORTED
    assert "bf16" in ra.last_error() and st.kernel_launches == -7


def _gpu_visible():
    import torch
    return torch.cuda.device_count() > 0


def test_ring_bwd_fp32_passes_checks():
    """fp32 ring backward is supported: with valid arguments the call gets
    past every check to its first HIP call, which on a machine without a GPU
    fails with RA_ERR_HIP (never RA_ERR_UNSUPPORTED after enqueueing work).
    Only run where no GPU is visible: the pointers are fake."""
    if _gpu_visible():
        pytest.skip("fake device pointers: run only where no GPU is visible")
    st = L.RaRingStats()
    rc = ra.raw_call("ra_ring_bwd", ctypes.byref(_cfg(mask=1, dims=_dims(dtype=1))), *([FAKE] * 10), 1 << 40,
                     None, None, ctypes.byref(st))
    assert rc == L.RA_ERR_HIP, (rc, ra.last_error())


def test_ring_bwd_host_subset_workspace_and_checks():
    """One host's share of the backward needs D and the K/V double buffer
    only (no rotating dK/dV slots); a too-small workspace is refused before
    any HIP call."""
    d = _dims(batch=1, heads_q=8, heads_kv=4, head_dim=128, block_len=4096)
    n = ctypes.c_size_t(0)
    assert ra.raw_call("ra_ring_workspace_size", ctypes.byref(_cfg(dims=d, host_begin=7, host_end=8)), 1,
                       ctypes.byref(n)) == 0
    rows, kv = 8 * 4096, 4 * 4096 * 128
    assert n.value == rows * 4 + 4 * kv * 2
    assert ra.raw_call("ra_ring_workspace_size", ctypes.byref(_cfg(dims=d)), 1, ctypes.byref(n)) == 0
    assert n.value == 8 * (rows * 4 + 4 * kv * 2 + 4 * kv * 4)
    st = L.RaRingStats()
    rc = ra.raw_call("ra_ring_bwd", ctypes.byref(_cfg(dims=d, host_begin=7, host_end=8)), *([FAKE] * 10),
                     rows * 4 + 4 * kv * 2 - 1, None, None, ctypes.byref(st))
    assert rc == L.RA_ERR_WORKSPACE


def test_workspace_size_formula():
    # per simulated host: m, l (fp32 rows), O (fp32), 2 slots x (K, V) blocks
    d = _dims(batch=1, heads_q=8, heads_kv=8, head_dim=128, block_len=4096)
    cfg = _cfg(dims=d)
    n = ctypes.c_size_t(0)
    assert ra.raw_call("ra_ring_workspace_size", ctypes.byref(cfg), 0, ctypes.byref(n)) == 0
    rows = 8 * 4096
    want = 8 * (2 * rows * 4 + rows * 128 * 4 + 4 * 8 * 4096 * 128 * 2)
    assert n.value == want
    cfg1 = _cfg(dims=d, host_begin=7, host_end=8)
    assert ra.raw_call("ra_ring_workspace_size", ctypes.byref(cfg1), 0, ctypes.byref(n)) == 0
    assert n.value == want // 8


def test_missing_library_fails_loudly(tmp_path):
    code = ("import long_context_transformers_amd._lib as L; L.LIB_PATH='/nonexistent/libringattn.so';\n"
            "try:\n L.load()\nexcept ImportError as e:\n print('raised', e)\n")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT)
    assert "raised" in out.stdout


def test_overlap_threshold_table(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "min_block_size_table.json")))
    tol = g["tolerance_rel"]
    for row in g["rows"]:
        F = row["flops"] * 1e12
        B = row["bandwidth"] * 1e9
        c = ra.overlap.min_block_size(F, B)
        assert abs(c / 1000 - row["min_block"]) <= tol * row["min_block"] + 0.05, row
        assert abs(ra.overlap.min_local_sequence(F, B) / 1000 - row["min_seq"]) <= tol * row["min_seq"], row
    # the time model: a block pair's 4 d c^2 FLOPs against 4 c d bytes
    assert ra.overlap.block_flops(128, 1024) == 4 * 128 * 1024 ** 2
    assert ra.overlap.kv_transfer_bytes(128, 1024) == 4 * 1024 * 128
    assert ra.overlap.ring_time(8, 2.0, 3.0) == 24.0


def test_bench_pair_count_matches_oracle_masks():
    """bench.py counts visible (query, key) pairs in closed form per layout;
    the oracle's block masks summed over the ring must give the same."""
    import bench
    for layout in (rs.LAYOUT_CONTIGUOUS, rs.LAYOUT_STRIPED, rs.LAYOUT_ZIGZAG):
        for mask in (rs.MASK_NONE, rs.MASK_CAUSAL):
            for N, c in ((1, 8), (3, 6), (4, 10)):
                w = rs.Workload("count", 0, 1, 1, 1, 64, N, c, rs.DT_BF16, mask, layout, 0, N)
                for h in range(N):
                    want = sum(int(cref.block_mask(layout, mask, N, c, h, j).sum()) for j in range(N))
                    assert bench.counted_pairs(w, h) == want, (layout, mask, N, c, h)


def test_decode_argument_checks():
    """ra_ring_decode rejects bad arguments before any HIP call."""
    d = _dims(batch=2, heads_q=8, heads_kv=2, block_len=1000)
    n = ctypes.c_size_t(0)
    assert ra.raw_call("ra_decode_workspace_size", ctypes.byref(d), 4, ctypes.byref(n)) == L.RA_OK
    ws = n.value
    assert ws >= 4 * 2 * 8 * (2 + 128) * 4
    big = 1 << 40

    def call(dims=d, nh=4, q=FAKE, k=FAKE, v=FAKE, lens=FAKE, o=FAKE, odt=0, lse=FAKE, w=FAKE, wb=big):
        return ra.raw_call("ra_ring_decode", ctypes.byref(dims), nh, q, k, v, lens, o, odt, lse, w, wb, None)

    assert call(dims=_dims(batch=2, heads_q=8, heads_kv=2, block_len=1000, dtype=1)) == L.RA_ERR_UNSUPPORTED
    assert call(dims=_dims(heads_q=32, heads_kv=1)) == L.RA_ERR_UNSUPPORTED
    assert call(dims=_dims(head_dim=96)) == L.RA_ERR_UNSUPPORTED
    assert call(nh=0) == L.RA_ERR_INVALID_ARG
    assert call(lens=None) == L.RA_ERR_INVALID_ARG
    assert call(lens=FAKE + 2) == L.RA_ERR_INVALID_ARG
    assert call(q=None) == L.RA_ERR_INVALID_ARG
    assert call(odt=5) == L.RA_ERR_INVALID_ARG
    assert call(lse=None) == L.RA_ERR_INVALID_ARG
    assert call(w=FAKE + 16) == L.RA_ERR_INVALID_ARG
    assert call(wb=ws - 1) == L.RA_ERR_WORKSPACE
    assert ra.raw_call("ra_decode_workspace_size", ctypes.byref(d), 0, ctypes.byref(n)) == L.RA_ERR_INVALID_ARG
    assert ra.raw_call("ra_decode_workspace_size", ctypes.byref(d), 4, None) == L.RA_ERR_INVALID_ARG


def test_ffn_argument_checks():
    """ra_block_ffn rejects bad arguments before any HIP call."""
    n = ctypes.c_size_t(0)
    assert ra.raw_call("ra_ffn_workspace_size", 4096, 4096, 16384, ctypes.byref(n)) == L.RA_OK
    assert n.value == 4096 * 16384 * 2                # a full grid: no split-K partials
    assert ra.raw_call("ra_ffn_workspace_size", 256, 128, 512, ctypes.byref(n)) == L.RA_OK
    assert n.value >= 256 * 512 * 2 + 2 * 256 * 512 * 4   # GELU output + split-K partials
    assert ra.raw_call("ra_ffn_workspace_size", 256, 128, 500, ctypes.byref(n)) == L.RA_ERR_INVALID_ARG
    assert ra.raw_call("ra_ffn_workspace_size", 0, 128, 512, ctypes.byref(n)) == L.RA_ERR_INVALID_ARG
    big = 1 << 40

    def call(x=FAKE, w1=FAKE, w2=FAKE, y=FAKE, rows=100, h=128, f=256, br=64, w=FAKE, wb=big):
        return ra.raw_call("ra_block_ffn", x, w1, w2, y, rows, h, f, br, w, wb, None)

    assert call(h=100) == L.RA_ERR_INVALID_ARG
    assert call(f=0) == L.RA_ERR_INVALID_ARG
    assert call(rows=-1) == L.RA_ERR_INVALID_ARG
    assert call(br=0) == L.RA_ERR_INVALID_ARG
    assert call(x=None) == L.RA_ERR_INVALID_ARG
    assert call(w2=FAKE + 2) == L.RA_ERR_INVALID_ARG
    assert call(w=FAKE + 64) == L.RA_ERR_INVALID_ARG
    assert ra.raw_call("ra_ffn_workspace_size", 64, 128, 256, ctypes.byref(n)) == L.RA_OK
    assert call(wb=n.value - 1) == L.RA_ERR_WORKSPACE
    assert call(h=1 << 21) == L.RA_ERR_UNSUPPORTED
    assert call(br=(1 << 24) + 1) == L.RA_ERR_UNSUPPORTED
