#!/usr/bin/env python3
"""Benchmark of the Ring Attention hot path on one MI355X.

One step = one pass of the ring over one batch of synthetic input: the ring
forward (scheduler, side-stream K/V transfers, block kernels, finalize) and
the ring backward (preprocess, block backward kernels, K/V and dK/dV
rotation), on the striped causal 256K workload with every host of the ring
simulated: batch 1, 32 heads, d = 128, 8 virtual hosts of c = 32768 tokens in
the striped layout (host h holds tokens h, h + 8, ...), bf16 inputs
([P1] "Ring Attention如何让大模型突破百万token上下文", 因果掩码的负载均衡挑战).

Throughput is attention TFLOP/s counting only computed work: 4 d per visible
(query, key) pair in the forward, 10 d in the backward ([P2] "Ring Attention
with Blockwise Transformers for Near Infinite Context" reading notes, 5.4:
4 d c^2 per block pair).  Inputs are drawn on the device (seeded) and are
resident in HBM before the timed region.

Prints ONE JSON line.  Extra measurements (the non-causal 32K ring with its
60 %-of-peak target row, one host's share of the causal 256K and 786K
workloads, t_calc(c) sweep, merge/finalize bandwidth, decode, feedforward)
ride along under "extra".
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import ra_synth as rs  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
METRIC = "ring-attention TFLOP/s per GPU (bf16, causal/striped) and % of MFMA peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def counted_pairs(w, host):
    """Visible (query, key) pairs of one host's query block over the ring, per head."""
    c, N = w.block_len, w.n_hosts
    if w.mask == rs.MASK_NONE:
        return N * c * c
    if w.layout == rs.LAYOUT_CONTIGUOUS:
        return host * c * c + c * (c + 1) // 2
    if w.layout == rs.LAYOUT_ZIGZAG:       # chunks h and 2N-1-h of c/2 tokens: the same on every host
        return c * (N * c + 1) // 2
    return (host + 1) * c * (c + 1) // 2 + (N - 1 - host) * c * (c - 1) // 2


def counted_flops(w, per_pair):
    heads = w.batch * w.heads_q
    return per_pair * w.head_dim * heads * sum(counted_pairs(w, h) for h in range(w.host_begin, w.host_end))


class Ring:
    """Device buffers and calls for one workload."""

    def __init__(self, w, torch, ra, inp=None, seed=0, with_bwd=False):
        self.w, self.torch, self.ra = w, torch, ra
        dt = torch.bfloat16 if w.dtype == rs.DT_BF16 else torch.float32
        na = w.n_active
        if inp is not None:
            def up(a):
                return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
            q0 = w.host_begin - inp.q_host_base
            self.q = up(inp.q_dev[q0:q0 + na])
            self.k = up(inp.k_dev)
            self.v = up(inp.v_dev)
        else:
            g = torch.Generator(device="cuda")
            g.manual_seed(seed)
            self.q = torch.randn(rs.q_shape(w, na), generator=g, device="cuda").to(dt)
            self.k = torch.randn(rs.kv_shape(w), generator=g, device="cuda").to(dt)
            self.v = torch.randn(rs.kv_shape(w), generator=g, device="cuda").to(dt)
        self.O = torch.empty(rs.q_shape(w, na), dtype=dt, device="cuda")
        self.lse = torch.empty((na, w.batch, w.heads_q, w.block_len), dtype=torch.float32, device="cuda")
        self.dims = ra.Dims(w.batch, w.heads_q, w.heads_kv, w.head_dim, w.block_len, w.dtype)
        cfg = ra.RingCfg(self.dims, w.n_hosts, w.host_begin, w.host_end, w.layout, w.mask)
        self.ws = torch.empty(ra.ring_workspace_size(cfg), dtype=torch.uint8, device="cuda")
        self.comm = torch.cuda.Stream()
        self.with_bwd = with_bwd
        if with_bwd:
            g = torch.Generator(device="cuda")
            g.manual_seed(seed + 1)
            self.dO = torch.randn(rs.q_shape(w, na), generator=g, device="cuda").to(dt)
            self.dQ = torch.empty(rs.q_shape(w, na), dtype=torch.float32, device="cuda")
            self.dK = torch.empty(rs.kv_shape(w), dtype=torch.float32, device="cuda")
            self.dV = torch.empty(rs.kv_shape(w), dtype=torch.float32, device="cuda")
            self.wsb = torch.empty(ra.ring_workspace_size(cfg, True), dtype=torch.uint8, device="cuda")

    def cfg(self, events=None):
        w = self.w
        return self.ra.RingCfg(self.dims, w.n_hosts, w.host_begin, w.host_end, w.layout, w.mask,
                               step_events=events)

    def fwd(self, events=None):
        return self.ra.ring_fwd(self.cfg(events), self.q, self.k, self.v, self.O, self.lse, self.ws,
                                self.torch.cuda.current_stream(), self.comm)

    def bwd(self, events=None):
        return self.ra.ring_bwd(self.cfg(events), self.q, self.k, self.v, self.O, self.lse, self.dO,
                                self.dQ, self.dK, self.dV, self.wsb, self.torch.cuda.current_stream(),
                                self.comm)


def make_events(torch, n):
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in ev:
        e.record()
    return ev


def time_ring(ring, steps, warmup, bwd):
    """Warm up, then time `steps` ring passes; per-launch kernel times from
    the library's step events (recorded on the compute stream)."""
    torch = ring.torch
    N = ring.w.n_hosts
    for _ in range(warmup):
        ring.fwd()
        if bwd:
            ring.bwd()
    torch.cuda.synchronize()
    fev = [make_events(torch, 2 * N) for _ in range(steps)]
    bev = [make_events(torch, 2 * N) for _ in range(steps)] if bwd else None
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for i in range(steps):
        ring.fwd(fev[i])
        if bwd:
            ring.bwd(bev[i])
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = start.elapsed_time(end)
    f_ms = [fev[i][2 * s].elapsed_time(fev[i][2 * s + 1]) for i in range(steps) for s in range(N)]
    b_ms = [bev[i][2 * s].elapsed_time(bev[i][2 * s + 1]) for i in range(steps) for s in range(N)] if bwd else []
    return wall, gpu_ms, f_ms, b_ms


def cpu_baseline(w, ring, target_s=15.0):
    """Time the fp64 oracle on a bounded sample of the workload's query rows
    (evenly spaced rows of every host and head), on the bench's own inputs
    (the device tensors, widened to float32 on the host).  Counted work: 4 d
    per visible (query, key) pair of the sampled rows."""
    from oracle import cref
    hosts = list(range(w.host_begin, w.host_end))
    q = ring.q.float().cpu().numpy()
    k = ring.k.float().cpu().numpy()
    v = ring.v.float().cpu().numpy()

    def visible_keys(h, r):
        if w.mask == rs.MASK_NONE:
            return w.n_hosts * w.block_len
        return cref.token_index(w.layout, w.n_hosts, w.block_len, h, int(r)) + 1

    def run(n_rows):
        rows = np.arange(n_rows) * (w.block_len // n_rows)
        desc = cref.row_desc(hosts, range(w.batch), range(w.heads_q), rows)
        t0 = time.perf_counter()
        cref.attn_rows(q, k, v, n_hosts=w.n_hosts, layout=w.layout, causal=w.mask, rows=desc,
                       q_host_base=w.host_begin)
        dt = time.perf_counter() - t0
        pairs = w.batch * w.heads_q * sum(visible_keys(h, r) for h in hosts for r in rows)
        return dt, pairs, len(desc)

    dt, pairs, n = run(4)
    n_rows = int(max(4, min(w.block_len, 4 * target_s / max(dt, 1e-3))))
    n_rows = 4 * max(1, n_rows // 4)
    if n_rows > 4:
        dt, pairs, n = run(n_rows)
    flops = 4.0 * w.head_dim * pairs
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cref.num_threads(),
            "kind": "oracle",
            "sample": f"{n} query rows ({n_rows} evenly spaced rows x {w.heads_q} heads x "
                      f"{len(hosts)} hosts) of {w.name}, forward only, fp64, {dt:.1f} s wall"}


def tcalc_sweep(torch, ra, reps=5):
    """t_calc(c): one FULL and one TRI_INCL block through ra_block_fwd, H=32, d=128."""
    out = {}
    for c in (512, 1024, 2048, 4096, 8192, 16384, 32768):
        dims = ra.Dims(1, 32, 32, 128, c, rs.DT_BF16)
        g = torch.Generator(device="cuda")
        g.manual_seed(c)
        q = torch.randn((1, 32, c, 128), generator=g, device="cuda").to(torch.bfloat16)
        k = torch.randn((1, 32, c, 128), generator=g, device="cuda").to(torch.bfloat16)
        v = torch.randn((1, 32, c, 128), generator=g, device="cuda").to(torch.bfloat16)
        m = torch.empty((1, 32, c), dtype=torch.float32, device="cuda")
        l = torch.empty_like(m)
        O = torch.empty((1, 32, c, 128), dtype=torch.float32, device="cuda")
        res = {}
        for cls, qoff in (("full", c), ("tri_incl", 0)):
            ra.state_init(dims, m, l, O)
            ts = []
            for r in range(reps + 2):
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record()
                ra.block_fwd(dims, q, k, v, ra.RA_MASK_CAUSAL, qoff, 0, 1, m, l, O)
                b.record()
                b.synchronize()
                if r >= 2:
                    ts.append(a.elapsed_time(b))
            med = statistics.median(ts) / 1e3
            pairs = c * c if cls == "full" else c * (c + 1) // 2
            res[cls] = {"t_calc_s": med, "tflops": 4 * 128 * 32 * pairs / med / 1e12}
        out[c] = res
        del q, k, v, m, l, O
    # overlap crossing: smallest c with t_calc(c) >= t_comm(c) = 4 c d H_kv / B
    cross = {}
    for name, B in (("xgmi_153GBs", 153e9), ("nvlink_300GBs", 300e9), ("ib_12.5GBs", 12.5e9)):
        tc = {c: v["full"]["t_calc_s"] for c, v in out.items()}
        cross[name] = ra.overlap.crossing_block_len(tc, 32, 128, B)
    f_meas = max(v["full"]["tflops"] for v in out.values()) * 1e12
    return {"t_calc": {str(c): v for c, v in out.items()},
            "crossing_c": cross,
            "F_meas_over_B": {"153GBs": f_meas / 153e9, "300GBs": f_meas / 300e9, "12.5GBs": f_meas / 12.5e9}}


def elementwise_bw(torch, ra, reps=10):
    """Finalize, merge and the backward preprocess at one 256K-host shape
    (32 heads, c = 32768, d = 128)."""
    B, Hq, c, d = 1, 32, 32768, 128
    dims = ra.Dims(B, Hq, Hq, d, c, rs.DT_BF16)
    rows = B * Hq * c
    m = torch.randn((B, Hq, c), device="cuda")
    l = torch.rand((B, Hq, c), device="cuda") + 1
    O = torch.randn((B, Hq, c, d), device="cuda")
    Ob = torch.empty((B, Hq, c, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq, c), device="cuda")
    O2 = torch.randn_like(O)
    l2 = torch.randn_like(m)
    Om = torch.empty_like(O)
    lm = torch.empty_like(m)

    def timeit(fn):
        fn()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        b.synchronize()
        return a.elapsed_time(b) / reps / 1e3

    dO = torch.randn((B, Hq, c, d), device="cuda").to(torch.bfloat16)
    Dd = torch.empty((B, Hq, c), device="cuda")
    tf = timeit(lambda: ra.finalize(dims, m, l, O, Ob, lse))
    tm = timeit(lambda: ra.merge_lse(dims, O, m, O2, l2, Om, lm))
    tp = timeit(lambda: ra.bwd_preprocess(dims, Ob, dO, Dd))
    fin_bytes = rows * (6 * d + 12)     # O fp32 read, m, l read, bf16 out, lse out
    mer_bytes = rows * (12 * d + 12)    # two fp32 O in, one out, three lse
    pre_bytes = rows * (4 * d + 4)      # bf16 O and dO in, D out
    # reference: torch's device copy of the same O array (read + write), the
    # plain read/write stream these kernels are measured beside
    src = O.view(torch.uint8)
    dst = torch.empty_like(src)
    tc = timeit(lambda: dst.copy_(src))
    del src, dst
    out = {}
    for key, t, nbytes, per_row in (("finalize", tf, fin_bytes, 6 * d + 12), ("merge", tm, mer_bytes, 12 * d + 12),
                                     ("bwd_preprocess", tp, pre_bytes, 4 * d + 4)):
        out[key] = {"s": t, "GBs": nbytes / t / 1e9, "bytes_per_row": per_row,
                    "frac_hbm_peak": nbytes / t / 1e9 / PEAK_HBM_GBS}
    out["reference_copy_GBs"] = 2 * O.numel() * 4 / tc / 1e9
    out["peak_GBs"] = PEAK_HBM_GBS
    return out


def reference_gemm(torch, n=8192, reps=20):
    """This GPU's bf16 GEMM rate (torch.matmul, n^3, N(0,1) operands): a
    measured practical ceiling for dense bf16 contractions on random data,
    reported beside the published peak."""
    g = torch.Generator(device="cuda")
    g.manual_seed(1234)
    a = torch.randn((n, n), device="cuda", dtype=torch.bfloat16, generator=g)
    b = torch.randn((n, n), device="cuda", dtype=torch.bfloat16, generator=g)
    for _ in range(3):
        c = a @ b
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        c = a @ b
    e1.record()
    e1.synchronize()
    del c
    ms = e0.elapsed_time(e1) / reps
    return {"tflops": 2.0 * n ** 3 / (ms / 1e3) / 1e12, "shape": [n, n, n], "operands": "randn bf16",
            "ms": ms}


def causal_rates(torch, ra, steps=2):
    """One host's share of the causal 256K workload (host 7; contiguous,
    striped and zigzag layouts) and of the 786K striped GQA workload (host
    15): ring forward and ring backward of that host (seeded device-side
    inputs), TFLOP/s over the host's visible pairs (4 d forward, 10 d
    backward) from the per-step kernel times, and the whole-call time."""
    out = {}
    wl = rs.workloads()
    for key in ("causal_256k_contig", "causal_256k_striped", "causal_256k_zigzag", "striped_786k_gqa"):
        w = wl[key]
        ring = Ring(w, torch, ra, seed=w.cfg, with_bwd=True)
        ring.fwd()
        ring.bwd()
        torch.cuda.synchronize()
        wall, gpu_ms, f_ms, b_ms = time_ring(ring, steps, 0, True)
        f_pass, b_pass = sum(f_ms) / steps, sum(b_ms) / steps
        out[key] = {"fwd_ms": f_pass, "fwd_tflops": counted_flops(w, 4) / (f_pass / 1e3) / 1e12,
                    "bwd_ms": b_pass, "bwd_tflops": counted_flops(w, 10) / (b_pass / 1e3) / 1e12,
                    "gpu_event_ms_per_step": gpu_ms / steps}
        del ring
        torch.cuda.empty_cache()
    return out


BWD_SOURCES = [os.path.join(ROOT, "long_context_transformers_amd", "csrc", n)
               for n in ("ra_bwd.hip", "ra_tile.h")]   # the backward kernels' code


def traffic_profile(w):
    """Committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary of the backward
    step of workload w."""
    return os.path.join(ROOT, "profiles", f"ring_bwd_step_{w.name}_hbm_traffic.md")


def bwd_sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for p in BWD_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(w):
    """HBM bytes per backward ring step (dK/dV + dQ kernels) from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary, or None when the kernel sources
    have changed since the counters were taken (or no summary exists)."""
    import re
    try:
        text = open(traffic_profile(w)).read()
    except OSError:
        return None
    vals = dict(re.findall(r"^- (\w+): `([^`]+)`", text, re.M))
    if vals.get("sources_sha256") != bwd_sources_sha256():
        return None
    return float(vals["fetch_bytes_per_step"]) + float(vals["write_bytes_per_step"])


def bwd_algorithmic_bytes(w):
    """Compulsory bytes of one backward ring step for all hosts, averaged over
    a ring pass: the dK/dV kernel reads Q, dO, K, V (bf16), lse, D (fp32) and
    the received dK/dV partial sums (fp32; none at the first step) and writes
    the new sums; the dQ kernel reads Q, dO, K, V, lse, D and the fp32 dQ sum
    (none at the first step) and writes it.  Every block pair of the
    non-causal and striped rings touches every row, so each is read once."""
    N, c, d = w.n_hosts, w.block_len, w.head_dim
    hq, hkv = w.batch * w.heads_q, w.batch * w.heads_kv
    qo = 2 * hq * c * d * 2 + 2 * hq * c * 4         # Q, dO, lse, D
    kv = 2 * hkv * c * d * 2                         # K, V
    dkdv = 2 * hkv * c * d * 4                       # dK and dV sums, one direction
    dq = hq * c * d * 4                              # dQ sum, one direction
    per_host = 2 * (qo + kv) + (dkdv + dq) * (1 + (N - 1) / N)
    return N * per_host


def copy_calibration(torch, mib, reps=5):
    """Plain device copy of a known size, for scaling the HBM counters."""
    n = mib << 20
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "reps": reps}), flush=True)


def bwd_rates(torch, ra, steps=2):
    """Ring forward + backward of the causal 64K workload (32 heads, d = 128,
    8 hosts x 8192) in the contiguous and zigzag layouts: counted TFLOP/s of
    the forward (4 d per visible pair) and of the backward (10 d)."""
    out = {}
    base = rs.workloads()["bwd_64k"]
    for key, w in (("bwd_64k_contig", base),
                   ("bwd_64k_zigzag", base.replace(name=base.name + "_zigzag", layout=rs.LAYOUT_ZIGZAG))):
        ring = Ring(w, torch, ra, seed=w.cfg, with_bwd=True)
        _, gpu_ms, f_ms, b_ms = time_ring(ring, steps, 1, True)
        f_step, b_step = sum(f_ms) / steps, sum(b_ms) / steps
        out[key] = {"fwd_ms": f_step, "bwd_ms": b_step,
                    "fwd_tflops": counted_flops(w, 4) / (f_step / 1e3) / 1e12,
                    "bwd_tflops": counted_flops(w, 10) / (b_step / 1e3) / 1e12,
                    "gpu_event_ms_per_step": gpu_ms / steps}
        del ring
        torch.cuda.empty_cache()
    return out


def decode_rates(torch, ra, reps=10):
    """One decode step (ra_ring_decode) on the decode workloads: ms per step,
    new tokens per second, and HBM GB/s counting the valid K and V rows read
    once (the step's algorithmic bytes; q, the partials and O are < 0.01 %)
    against the 8 TB/s peak.  Inputs are drawn on the device, seeded."""
    out = {}
    for key, w in rs.decode_workloads().items():
        N, B, Hq, Hkv, d, c = w.n_hosts, w.batch, w.heads_q, w.heads_kv, w.head_dim, w.block_len
        g = torch.Generator(device="cuda")
        g.manual_seed(w.cfg)
        k = torch.empty((N, B, Hkv, c, d), dtype=torch.bfloat16, device="cuda")
        v = torch.empty_like(k)
        for h in range(N):
            k[h].normal_(generator=g)
            v[h].normal_(generator=g)
        q = torch.randn((B, Hq, d), generator=g, device="cuda").to(torch.bfloat16)
        lens = rs.decode_lens(N, B, c, w.cfg, full=True)
        tl = torch.as_tensor(lens).cuda()
        dims = ra.Dims(B, Hq, Hkv, d, c, rs.DT_BF16)
        O = torch.empty((B, Hq, d), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
        ws = torch.empty(ra.decode_workspace_size(dims, N), dtype=torch.uint8, device="cuda")
        for _ in range(3):
            ra.ring_decode(dims, N, q, k, v, tl, O, lse, ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            ra.ring_decode(dims, N, q, k, v, tl, O, lse, ws)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        nbytes = int(lens.sum()) * Hkv * d * 2 * 2
        out[key] = {"workload": w.name, "cache_tokens_per_seq": int(lens.sum() // B), "ms": ms,
                    "tokens_per_s": B / (ms / 1e3), "GBs": nbytes / (ms / 1e3) / 1e9,
                    "frac_hbm_peak": nbytes / (ms / 1e3) / 1e9 / PEAK_HBM_GBS,
                    "algorithmic_bytes": nbytes}
        del k, v
        torch.cuda.empty_cache()
    return out


def ffn_rates(torch, ra, reps=10):
    """Blockwise feedforward (ra_block_ffn) of one host's block: TFLOP/s
    counting the two products (4 rows h f), beside torch.matmul (hipBLASLt)
    running the same two products with torch's GELU between them."""
    out = {}
    for key, w in rs.ffn_workloads().items():
        g = torch.Generator(device="cuda")
        g.manual_seed(w.cfg)
        x = torch.randn((w.rows, w.h), generator=g, device="cuda").to(torch.bfloat16)
        w1 = (torch.randn((w.f, w.h), generator=g, device="cuda") * w.h ** -0.5).to(torch.bfloat16)
        w2 = (torch.randn((w.h, w.f), generator=g, device="cuda") * w.f ** -0.5).to(torch.bfloat16)
        y = torch.empty_like(x)
        ws = torch.empty(ra.ffn_workspace_size(w.block_rows, w.h, w.f), dtype=torch.uint8, device="cuda")
        flops = 4.0 * w.rows * w.h * w.f

        def timed(fn):
            for _ in range(2):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps

        ms = timed(lambda: ra.block_ffn(x, w1, w2, y, w.block_rows, ws))
        w1t, w2t = w1.t().contiguous(), w2.t().contiguous()
        ms_ref = timed(lambda: torch.matmul(torch.nn.functional.gelu(torch.matmul(x, w1t)), w2t))
        out[key] = {"workload": w.name, "ms": ms, "tflops": flops / (ms / 1e3) / 1e12,
                    "torch_matmul_ms": ms_ref, "torch_matmul_tflops": flops / (ms_ref / 1e3) / 1e12}
        del x, w1, w2, y, ws, w1t, w2t
        torch.cuda.empty_cache()
    return out


def headline_workload():
    """Striped causal 256K over all 8 hosts: 32 heads, d = 128, c = 32768,
    bf16 -- the causal 256K workload with every host of the ring simulated."""
    base = rs.workloads()["causal_256k_striped"]
    return base.replace(name="causal_256k_striped_H32_N8_c32768_all_hosts", host_begin=0,
                        host_end=base.n_hosts)


def step_rates(w, f_ms, b_ms, steps):
    """Per-launch kernel rates from the step events: forward (one launch per
    ring step, all hosts) and backward (dK/dV + dQ launches of one ring step)."""
    N = w.n_hosts
    out = {"fwd_kernel_avg_launch_ms": statistics.mean(f_ms),
           "fwd_kernel_tflops": counted_flops(w, 4) / N / (statistics.mean(f_ms) / 1e3) / 1e12,
           "fwd_ms_per_pass": sum(f_ms) / steps}
    if b_ms:
        out.update({"bwd_step_avg_launch_ms": statistics.mean(b_ms),
                    "bwd_step_tflops": counted_flops(w, 10) / N / (statistics.mean(b_ms) / 1e3) / 1e12,
                    "bwd_ms_per_pass": sum(b_ms) / steps})
    out["fwd_kernel_frac_of_peak"] = out["fwd_kernel_tflops"] / PEAK_BF16_TFLOPS
    if b_ms:
        out["bwd_step_frac_of_peak"] = out["bwd_step_tflops"] / PEAK_BF16_TFLOPS
    return out


def first_pass(ring):
    """Event-timed first ring forward and backward on fresh buffers (the
    cold pass: first touch of the workspace and output pages)."""
    torch = ring.torch
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    e[0].record()
    st_f = ring.fwd()
    e[1].record()
    st_b = ring.bwd() if ring.with_bwd else None
    e[2].record()
    torch.cuda.synchronize()
    return {"fwd_ms": e[0].elapsed_time(e[1]), "bwd_ms": e[1].elapsed_time(e[2]) if st_b else None}, st_f, st_b


def noncausal_32k(torch, ra, steps, warmup):
    """The non-causal 32K ring (8 hosts x 4096, 8 heads): whole-step rate,
    the forward kernel and backward step against the bf16 peak (the 60 %
    target row) -- same timing as the headline."""
    w = rs.workloads()["noncausal_32k"]
    ring = Ring(w, torch, ra, seed=w.cfg, with_bwd=True)
    ring.fwd()
    ring.bwd()
    torch.cuda.synchronize()
    wall, gpu_ms, f_ms, b_ms = time_ring(ring, steps, warmup, True)
    out = {"workload": w.name + " ring fwd+bwd",
           "tflops": counted_flops(w, 14) / (wall / steps) / 1e12, "ms_per_step": wall * 1e3 / steps}
    out.update(step_rates(w, f_ms, b_ms, steps))
    out["target_frac"] = 0.60
    del ring
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--workload", choices=["headline", "noncausal_32k"], default="headline",
                    help="what the timed steps run (profiling runs may pick the non-causal 32K ring)")
    ap.add_argument("--ffn-only", action="store_true",
                    help="only measure the blockwise feedforward and print its JSON")
    ap.add_argument("--decode-only", action="store_true",
                    help="only measure the decode workloads and print their JSON")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (HBM counter scaling) and exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "the ring runs on one GPU: its N virtual hosts share it; "
                                   "--gpus above 1 is not supported", "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import long_context_transformers_amd as ra
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    ra.version()
    if args.copy_calibration:
        copy_calibration(torch, args.copy_calibration)
        return
    if args.decode_only:
        print(json.dumps(decode_rates(torch, ra)), flush=True)
        return
    if args.ffn_only:
        print(json.dumps(ffn_rates(torch, ra)), flush=True)
        return

    w = headline_workload() if args.workload == "headline" else rs.workloads()["noncausal_32k"]
    log(f"[bench] workload {w.name}: drawing inputs on the device")
    ring = Ring(w, torch, ra, seed=w.cfg, with_bwd=True)
    cold, st_f, st_b = first_pass(ring)     # also checks that forward and backward run
    log(f"[bench] first pass: forward {cold['fwd_ms']:.1f} ms, backward {cold['bwd_ms']:.1f} ms")
    log(f"[bench] timing {args.steps} steps (ring forward + backward) after {args.warmup} warm-up steps")
    wall, gpu_ms, f_ms, b_ms = time_ring(ring, args.steps, args.warmup, True)
    ms_per_step = wall * 1e3 / args.steps
    N = w.n_hosts
    fwd_flops = counted_flops(w, 4)
    bwd_flops = counted_flops(w, 10)
    value = (fwd_flops + bwd_flops) / (ms_per_step / 1e3) / 1e12
    rates = step_rates(w, f_ms, b_ms, args.steps)

    # dominant kernel: the block kernels with the most time per step -- the
    # backward (dK/dV + dQ launches of one ring step, all hosts)
    f_launch, b_launch = statistics.mean(f_ms), statistics.mean(b_ms)
    if b_launch >= f_launch:
        dom = {"kernel": "block backward (dK/dV + dQ kernels of one ring step, all hosts)",
               "flops_per_launch": bwd_flops / N, "avg_launch_ms": b_launch,
               "traffic": measured_traffic(w), "algorithmic_bytes_per_launch": bwd_algorithmic_bytes(w)}
    else:
        dom = {"kernel": "fwd_bf16_kernel (one ring step, all hosts)",
               "flops_per_launch": fwd_flops / N, "avg_launch_ms": f_launch, "traffic": None,
               "algorithmic_bytes_per_launch": None}
    achieved = dom["flops_per_launch"] / (dom["avg_launch_ms"] / 1e3) / 1e12
    roofline = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS, "traffic": dom["traffic"],
                "kernel": dom["kernel"], "avg_launch_ms": dom["avg_launch_ms"],
                "algorithmic_flops_per_launch": dom["flops_per_launch"],
                "algorithmic_bytes_per_launch": dom["algorithmic_bytes_per_launch"],
                "traffic_source": os.path.relpath(traffic_profile(w), ROOT)}

    extra = dict(rates)
    extra["gpu_event_ms_per_step"] = gpu_ms / args.steps
    extra["first_pass"] = cold
    extra["copy_kind"] = {0: "none", 1: "dma_engines", 2: "fallback_device_copy"}[st_f["copy_kind"]]
    extra["copy_kind_bwd"] = {0: "none", 1: "dma_engines", 2: "fallback_device_copy"}[st_b["copy_kind"]]
    extra["resident_bytes_per_host"] = {"fwd": st_f["resident_bytes_per_host"],
                                        "bwd": st_b["resident_bytes_per_host"]}
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (fp64 oracle)")
        cpu = cpu_baseline(w, ring, args.cpu_seconds)
    del ring
    torch.cuda.empty_cache()
    if not args.no_extra:
        if w.name.startswith("noncausal_32k"):
            extra["noncausal_32k"] = dict(rates, workload=w.name, target_frac=0.60)
        else:
            log("[bench] non-causal 32K ring (60 % target row)")
            extra["noncausal_32k"] = noncausal_32k(torch, ra, max(3, args.steps), 2)
            nc = extra["noncausal_32k"]
            # like for like: per-launch kernel rates of whole ring steps over all hosts
            extra["striped_vs_noncausal_per_flop"] = {
                "fwd": rates["fwd_kernel_tflops"] / nc["fwd_kernel_tflops"],
                "bwd": rates["bwd_step_tflops"] / nc["bwd_step_tflops"]}
        log("[bench] one host's share: causal 256K (contiguous, striped, zigzag) and 786K striped GQA forward + backward")
        extra["causal"] = causal_rates(torch, ra)
        log("[bench] causal 64K forward + backward")
        extra["causal_bwd"] = bwd_rates(torch, ra)
        log("[bench] decode against a ring-sharded KV cache")
        extra["decode"] = decode_rates(torch, ra)
        log("[bench] blockwise feedforward")
        extra["ffn"] = ffn_rates(torch, ra)
        log("[bench] t_calc(c) sweep")
        extra["overlap"] = tcalc_sweep(torch, ra)
        log("[bench] finalize / merge bandwidth")
        extra["elementwise"] = elementwise_bw(torch, ra)
        log("[bench] reference bf16 GEMM")
        extra["reference_gemm"] = reference_gemm(torch)
        extra["dominant_kernel_vs_reference_gemm"] = achieved / extra["reference_gemm"]["tflops"]

    line = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name + " ring fwd+bwd", "global_batch": w.batch,
                   "seq_len": w.seq_len, "heads": w.heads_q, "head_dim": w.head_dim,
                   "virtual_hosts": w.n_hosts, "block_len": w.block_len,
                   "layout": {0: "contiguous", 1: "striped", 2: "zigzag"}[w.layout],
                   "mask": "causal" if w.mask else "none",
                   "parallelism": f"ring of {w.n_hosts} virtual hosts on 1 GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
